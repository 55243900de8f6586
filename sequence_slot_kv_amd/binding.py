"""ctypes binding of ``libslot_kv.so`` (the C ABI in include/slot_kv.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Torch is used for device memory and streams; tensors are passed by
their data pointers after shape, dtype, device and contiguity checks.  The
library must be built (``python -m sequence_slot_kv_amd.build``); importing
this module without it raises ImportError -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libslot_kv.so")

SLOT_KV_OK = 0
SLOT_KV_FLAG_V_NORM, SLOT_KV_FLAG_ROPE_INTERLEAVED, SLOT_KV_FLAG_NORM_ONE_PLUS_W = 1, 2, 4
SLOT_KV_EINVAL = -1
SLOT_KV_ERANGE = -2
SLOT_KV_ENOTALLOC = -3
SLOT_KV_ENOMEM = -4
SLOT_KV_EDUP = -5
SLOT_KV_EDEVICE = -6
SLOT_KV_ESCRATCH = -7

# Every symbol include/slot_kv.h declares.
EXPORTS = ("slot_kv_create", "slot_kv_destroy", "slot_kv_alloc", "slot_kv_set_layer",
           "slot_kv_set_layer_flags", "slot_kv_offset_bytes", "slot_reset", "slot_decode_attn",
           "slot_decode_attn_noalloc",
           "slot_prefill_attn",
           "slot_verify_attn", "slot_state_alloc", "slot_conv_offset_bytes",
           "slot_ssm_offset_bytes", "slot_state_ptrs", "slot_reset_batch",
           "slot_kv_layer_ptrs",
           "slot_kv_write_rows", "slot_kv_read_rows", "slot_kv_check_batch",
           "slot_kv_chunk_keys", "slot_kv_profile_begin", "slot_kv_profile_end",
           "slot_kv_strerror")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m sequence_slot_kv_amd.build` (hipcc, gfx950)")

# torch ships its own HIP runtime under the same soname as /opt/rocm's.  Load
# torch first so that the library binds to that one runtime: the streams and
# device pointers torch hands over are then valid in the library's calls.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_u32 = ctypes.c_uint32
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)

_lib.slot_kv_create.argtypes = [ctypes.POINTER(_vp)]
_lib.slot_kv_destroy.argtypes = [_vp]
_lib.slot_kv_destroy.restype = None
_lib.slot_kv_alloc.argtypes = [_vp, _u32, _u32, _u32p, _u32]
_lib.slot_kv_set_layer.argtypes = [_vp, _u32, _u32, _u32, _u32, _f32p, _f32p, _f32p, _f32p,
                                   ctypes.c_float, ctypes.c_float]
_lib.slot_kv_offset_bytes.argtypes = [_vp, _u32, _u32, _u32, ctypes.POINTER(ctypes.c_uint64)]
_lib.slot_reset.argtypes = [_vp, _u32, _vp]
_lib.slot_reset_batch.argtypes = [_vp, _u32p, _u32, _vp]
_lib.slot_state_alloc.argtypes = [_vp, _u32, _u32, _u32p, _u32, _u32p, _u32p, _u32]
_lib.slot_conv_offset_bytes.argtypes = [_vp, _u32, _u32, ctypes.POINTER(ctypes.c_uint64)]
_lib.slot_ssm_offset_bytes.argtypes = [_vp, _u32, _u32, ctypes.POINTER(ctypes.c_uint64)]
_lib.slot_state_ptrs.argtypes = [_vp, _u32, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]
_lib.slot_kv_set_layer_flags.argtypes = [_vp, _u32, _u32]
_lib.slot_decode_attn.argtypes = [_vp, _u32, _vp, _vp, _vp, _u32p, _u32p, _u32, _vp, _vp]
_lib.slot_decode_attn_noalloc.argtypes = _lib.slot_decode_attn.argtypes
_lib.slot_prefill_attn.argtypes = [_vp, _u32, _vp, _vp, _vp, _u32, _u32, _u32, _vp, _vp]
_lib.slot_verify_attn.argtypes = [_vp, _u32, _vp, _vp, _vp, _u32p, _u32p, _u32p, _u32, _vp, _vp]
_lib.slot_kv_layer_ptrs.argtypes = [_vp, _u32, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]
_lib.slot_kv_write_rows.argtypes = [_vp, _u32, _u32, _u32, _u32, _vp, _vp, _vp]
_lib.slot_kv_read_rows.argtypes = [_vp, _u32, _u32, _u32, _u32, _vp, _vp, _vp]
_lib.slot_kv_check_batch.argtypes = [_u32, _u32, _u32p, _u32p, _u32, _u32, _u32p, _u32p]
_lib.slot_kv_chunk_keys.argtypes = []
_lib.slot_kv_chunk_keys.restype = _u32
_lib.slot_kv_profile_begin.argtypes = [_vp]
_lib.slot_kv_profile_end.argtypes = [_vp, ctypes.POINTER(ctypes.c_double), _u32p]
_lib.slot_kv_strerror.argtypes = [ctypes.c_int]
_lib.slot_kv_strerror.restype = ctypes.c_char_p
for _name in EXPORTS:
    if _name not in ("slot_kv_destroy", "slot_kv_chunk_keys", "slot_kv_strerror"):
        getattr(_lib, _name).restype = ctypes.c_int


class SlotKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {slot_kv_strerror(status)} ({status})")
        self.status = status


def _check(status: int, what: str) -> int:
    if status != SLOT_KV_OK:
        raise SlotKVError(status, what)
    return status


def _host_u32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint32))


def _host_f32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr_u32(a: np.ndarray):
    return a.ctypes.data_as(_u32p)


def _ptr_f32(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_f32p)


def _dev_ptr(t, name: str, numel: Optional[int] = None) -> int:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a GPU tensor, got {t.device}")
    if t.dtype != torch.float32:
        raise TypeError(f"{name}: expected float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---------------------------------------------------------------- raw C names
def slot_kv_create() -> int:
    h = _vp()
    _check(_lib.slot_kv_create(ctypes.byref(h)), "slot_kv_create")
    return h.value


def slot_kv_destroy(h: int) -> None:
    _lib.slot_kv_destroy(h)


def slot_kv_alloc(h: int, n_slots: int, slot_ctx: int, kv_dims: Sequence[int]) -> int:
    dims = _host_u32(kv_dims)
    return _lib.slot_kv_alloc(h, n_slots, slot_ctx, _ptr_u32(dims), len(dims))


def slot_kv_set_layer(h, layer, n_heads, n_kv_heads, head_dim, q_norm_w, k_norm_w, inv_freq,
                      sinks=None, eps=1e-6, scale=None) -> int:
    qw, kw, fr, sk = (_host_f32(x) for x in (q_norm_w, k_norm_w, inv_freq, sinks))
    if qw is None or kw is None or fr is None:
        return SLOT_KV_EINVAL
    if qw.size != head_dim or kw.size != head_dim or fr.size != head_dim // 2:
        return SLOT_KV_EINVAL
    if sk is not None and sk.size != n_heads:
        return SLOT_KV_EINVAL
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    return _lib.slot_kv_set_layer(h, layer, n_heads, n_kv_heads, head_dim, _ptr_f32(qw),
                                  _ptr_f32(kw), _ptr_f32(fr), _ptr_f32(sk), float(eps),
                                  float(scale))


def slot_kv_offset_bytes(h, layer, slot, pos):
    """Returns (status, offset)."""
    out = ctypes.c_uint64(0)
    rc = _lib.slot_kv_offset_bytes(h, layer, slot, pos, ctypes.byref(out))
    return rc, int(out.value)


def slot_reset(h, slot, stream=None) -> int:
    return _lib.slot_reset(h, slot, _stream_handle(stream))


def slot_reset_batch(h, slots, stream=None) -> int:
    sv = _host_u32(slots)
    return _lib.slot_reset_batch(h, _ptr_u32(sv), sv.size, _stream_handle(stream))


def slot_state_alloc(h, n_slots, slot_ctx, kv_dims, conv_state_len, ssm_state_len) -> int:
    dims, cl, sl = (_host_u32(x) for x in (kv_dims, conv_state_len, ssm_state_len))
    if cl.size != sl.size:
        return SLOT_KV_EINVAL
    return _lib.slot_state_alloc(h, n_slots, slot_ctx, _ptr_u32(dims) if dims.size else None,
                                 dims.size, _ptr_u32(cl) if cl.size else None,
                                 _ptr_u32(sl) if sl.size else None, cl.size)


def slot_conv_offset_bytes(h, ssm_layer, slot):
    """Returns (status, offset)."""
    out = ctypes.c_uint64(0)
    rc = _lib.slot_conv_offset_bytes(h, ssm_layer, slot, ctypes.byref(out))
    return rc, int(out.value)


def slot_ssm_offset_bytes(h, ssm_layer, slot):
    """Returns (status, offset)."""
    out = ctypes.c_uint64(0)
    rc = _lib.slot_ssm_offset_bytes(h, ssm_layer, slot, ctypes.byref(out))
    return rc, int(out.value)


def slot_state_ptrs(h, ssm_layer):
    """Returns (status, conv pointer, recurrent-state pointer)."""
    c, s_ = _vp(), _vp()
    rc = _lib.slot_state_ptrs(h, ssm_layer, ctypes.byref(c), ctypes.byref(s_))
    return rc, c.value, s_.value


def slot_decode_attn(h, layer, q, k_new, v_new, positions, slots, out, stream=None) -> int:
    """Raw call: q/k_new/v_new/out are GPU float32 tensors, positions/slots
    host integer sequences.  Returns the status code."""
    pos = _host_u32(positions)
    sl = _host_u32(slots)
    if pos.shape != sl.shape or pos.ndim != 1:
        return SLOT_KV_EINVAL
    B = int(pos.shape[0])
    ptrs = [_dev_ptr(t, n) for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out"))]
    return _lib.slot_decode_attn(h, layer, ptrs[0], ptrs[1], ptrs[2], _ptr_u32(pos), _ptr_u32(sl),
                                 B, ptrs[3], _stream_handle(stream))


def slot_decode_attn_noalloc(h, layer, q, k_new, v_new, positions, slots, out,
                             stream=None) -> int:
    """Raw call of the allocation-free decode (scratch in the library's fixed
    per-GPU array); same arguments as slot_decode_attn."""
    pos = _host_u32(positions)
    sl = _host_u32(slots)
    if pos.shape != sl.shape or pos.ndim != 1:
        return SLOT_KV_EINVAL
    B = int(pos.shape[0])
    ptrs = [_dev_ptr(t, n) for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out"))]
    return _lib.slot_decode_attn_noalloc(h, layer, ptrs[0], ptrs[1], ptrs[2], _ptr_u32(pos),
                                         _ptr_u32(sl), B, ptrs[3], _stream_handle(stream))


def slot_prefill_attn(h, layer, q, k_new, v_new, slot, pos0, out, stream=None) -> int:
    """Raw call: q/k_new/v_new/out are GPU float32 tensors of T rows (T is
    taken from q's leading dimension).  Returns the status code."""
    T = int(q.shape[0]) if q.dim() > 0 else 0
    ptrs = [_dev_ptr(t, n) for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out"))]
    return _lib.slot_prefill_attn(h, layer, ptrs[0], ptrs[1], ptrs[2], slot, pos0, T, ptrs[3],
                                  _stream_handle(stream))


def slot_verify_attn(h, layer, q, k_new, v_new, slots, pos0, ks, out, stream=None) -> int:
    """Raw call: q/k_new/v_new/out are GPU float32 tensors of sum(ks) rows,
    slots/pos0/ks host integer sequences of one entry per sequence."""
    sl, p0, k = _host_u32(slots), _host_u32(pos0), _host_u32(ks)
    if not (sl.shape == p0.shape == k.shape) or sl.ndim != 1:
        return SLOT_KV_EINVAL
    ptrs = [_dev_ptr(t, n) for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out"))]
    return _lib.slot_verify_attn(h, layer, ptrs[0], ptrs[1], ptrs[2], _ptr_u32(sl), _ptr_u32(p0),
                                 _ptr_u32(k), int(sl.shape[0]), ptrs[3], _stream_handle(stream))


def slot_kv_set_layer_flags(h, layer, flags) -> int:
    return _lib.slot_kv_set_layer_flags(h, layer, flags)


def slot_kv_layer_ptrs(h, layer):
    """Returns (status, k_ptr, v_ptr)."""
    k, v = _vp(), _vp()
    rc = _lib.slot_kv_layer_ptrs(h, layer, ctypes.byref(k), ctypes.byref(v))
    return rc, k.value, v.value


def slot_kv_write_rows(h, layer, slot, pos0, k_src=None, v_src=None, n_rows=None,
                       stream=None) -> int:
    src = k_src if k_src is not None else v_src
    if n_rows is None:
        n_rows = int(src.shape[0]) if src is not None else 0
    kp = _dev_ptr(k_src, "k_src") if k_src is not None else None
    vp = _dev_ptr(v_src, "v_src") if v_src is not None else None
    return _lib.slot_kv_write_rows(h, layer, slot, pos0, n_rows, kp, vp, _stream_handle(stream))


def slot_kv_read_rows(h, layer, slot, pos0, n_rows, k_dst=None, v_dst=None, stream=None) -> int:
    kp = _dev_ptr(k_dst, "k_dst") if k_dst is not None else None
    vp = _dev_ptr(v_dst, "v_dst") if v_dst is not None else None
    return _lib.slot_kv_read_rows(h, layer, slot, pos0, n_rows, kp, vp, _stream_handle(stream))


def slot_kv_check_batch(n_slots, slot_ctx, positions, slots, chunk_keys=None):
    """Host-only precondition check.  Returns (status, n_items, n_split_rows)."""
    pos = _host_u32(positions)
    sl = _host_u32(slots)
    if pos.shape != sl.shape:
        return SLOT_KV_EINVAL, 0, 0
    ni, ns = _u32(0), _u32(0)
    rc = _lib.slot_kv_check_batch(n_slots, slot_ctx, _ptr_u32(pos), _ptr_u32(sl), pos.shape[0],
                                  slot_kv_chunk_keys() if chunk_keys is None else chunk_keys,
                                  ctypes.byref(ni), ctypes.byref(ns))
    return rc, int(ni.value), int(ns.value)


def slot_kv_chunk_keys() -> int:
    return int(_lib.slot_kv_chunk_keys())


def slot_kv_profile_begin(h) -> int:
    return _lib.slot_kv_profile_begin(h)


def slot_kv_profile_end(h):
    """Returns (status, summed fused-kernel milliseconds, launches)."""
    ms, n = ctypes.c_double(0.0), _u32(0)
    rc = _lib.slot_kv_profile_end(h, ctypes.byref(ms), ctypes.byref(n))
    return rc, float(ms.value), int(n.value)


def slot_kv_strerror(status: int) -> str:
    return _lib.slot_kv_strerror(status).decode()


# ---------------------------------------------------------------- convenience
def _device_view(ptr, shape):
    """A torch float32 tensor over device memory the handle owns (no copy)."""
    import torch

    class _Arr:
        def __init__(self):
            self.__cuda_array_interface__ = {
                "shape": tuple(shape), "typestr": "<f4", "data": (ptr, False), "version": 2,
                "strides": None}

    return torch.as_tensor(_Arr(), device=torch.device("cuda", torch.cuda.current_device()))


class SlotKV:
    """Owning wrapper of one handle; raises SlotKVError on any failure."""

    def __init__(self):
        self.h = slot_kv_create()
        self.n_slots = self.slot_ctx = 0
        self.kv_dims: list = []
        self.state_lens: list = []  # (conv_state_len, ssm_state_len) per ssm layer
        self.layers: dict = {}

    def close(self):
        if self.h:
            slot_kv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n_slots, slot_ctx, kv_dims):
        _check(slot_kv_alloc(self.h, n_slots, slot_ctx, kv_dims), "slot_kv_alloc")
        self.n_slots, self.slot_ctx, self.kv_dims = n_slots, slot_ctx, list(kv_dims)
        self.state_lens, self.layers = [], {}

    def alloc_state(self, n_slots, slot_ctx, kv_dims, conv_state_len, ssm_state_len):
        """Slot KV for the attention layers and a conv ring and recurrent state
        per slot for each ssm layer (slot_state_alloc)."""
        _check(slot_state_alloc(self.h, n_slots, slot_ctx, kv_dims, conv_state_len,
                                ssm_state_len), "slot_state_alloc")
        self.n_slots, self.slot_ctx, self.kv_dims = n_slots, slot_ctx, list(kv_dims)
        self.state_lens = list(zip(conv_state_len, ssm_state_len))
        self.layers = {}

    def state_view(self, ssm_layer):
        """torch views of ssm layer ``ssm_layer``'s conv ring [n_slots, conv_state_len]
        and recurrent state [n_slots, ssm_state_len] (device memory owned by the handle)."""
        rc, cp, sp = slot_state_ptrs(self.h, ssm_layer)
        _check(rc, "slot_state_ptrs")
        cl, sl = self.state_lens[ssm_layer]
        return _device_view(cp, (self.n_slots, cl)), _device_view(sp, (self.n_slots, sl))

    def conv_offset_bytes(self, ssm_layer, slot) -> int:
        rc, off = slot_conv_offset_bytes(self.h, ssm_layer, slot)
        _check(rc, "slot_conv_offset_bytes")
        return off

    def ssm_offset_bytes(self, ssm_layer, slot) -> int:
        rc, off = slot_ssm_offset_bytes(self.h, ssm_layer, slot)
        _check(rc, "slot_ssm_offset_bytes")
        return off

    def reset_batch(self, slots, stream=None):
        _check(slot_reset_batch(self.h, slots, stream), "slot_reset_batch")

    def set_layer(self, layer, params):
        """``params`` has the fields of workloads.LayerParams."""
        P = params
        _check(slot_kv_set_layer(self.h, layer, P.n_heads, P.n_kv_heads, P.head_dim, P.q_norm_w,
                                 P.k_norm_w, P.inv_freq, P.sinks, P.eps, P.scale),
               "slot_kv_set_layer")
        flags = int(getattr(P, "flags", 0))
        if flags:
            _check(slot_kv_set_layer_flags(self.h, layer, flags), "slot_kv_set_layer_flags")
        self.layers[layer] = P

    def offset_bytes(self, layer, slot, pos) -> int:
        rc, off = slot_kv_offset_bytes(self.h, layer, slot, pos)
        _check(rc, "slot_kv_offset_bytes")
        return off

    def reset(self, slot, stream=None):
        _check(slot_reset(self.h, slot, stream), "slot_reset")

    def decode_attn(self, layer, q, k_new, v_new, positions, slots, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        P = self.layers.get(layer)
        if P is not None:
            B = len(positions)
            for t, n, w in ((q, "q", P.n_heads * P.head_dim), (k_new, "k_new", P.kv_dim),
                            (v_new, "v_new", P.kv_dim), (out, "out", P.n_heads * P.head_dim)):
                if t.numel() != B * w:
                    raise ValueError(f"{n}: expected {B}x{w} elements, got {tuple(t.shape)}")
        _check(slot_decode_attn(self.h, layer, q, k_new, v_new, positions, slots, out, stream),
               "slot_decode_attn")
        return out

    def prefill_attn(self, layer, q, k_new, v_new, slot, pos0, out=None, stream=None):
        """T tokens (rows of q / k_new / v_new) of one sequence at positions
        pos0 .. pos0+T-1 of ``slot``; returns out [T, n_heads*head_dim]."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        P = self.layers.get(layer)
        if P is not None:
            T = int(q.shape[0])
            for t, n, w in ((q, "q", P.n_heads * P.head_dim), (k_new, "k_new", P.kv_dim),
                            (v_new, "v_new", P.kv_dim), (out, "out", P.n_heads * P.head_dim)):
                if t.numel() != T * w:
                    raise ValueError(f"{n}: expected {T}x{w} elements, got {tuple(t.shape)}")
        _check(slot_prefill_attn(self.h, layer, q, k_new, v_new, slot, pos0, out, stream),
               "slot_prefill_attn")
        return out

    def verify_attn(self, layer, q, k_new, v_new, slots, pos0, ks, out=None, stream=None):
        """ks[i] rows for each sequence i at positions pos0[i].. of slots[i]
        (rows sequence-major); returns out [sum ks, n_heads*head_dim]."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        P = self.layers.get(layer)
        if P is not None:
            rows = int(np.asarray(ks, np.int64).sum())
            for t, n, w in ((q, "q", P.n_heads * P.head_dim), (k_new, "k_new", P.kv_dim),
                            (v_new, "v_new", P.kv_dim), (out, "out", P.n_heads * P.head_dim)):
                if t.numel() != rows * w:
                    raise ValueError(f"{n}: expected {rows}x{w} elements, got {tuple(t.shape)}")
        _check(slot_verify_attn(self.h, layer, q, k_new, v_new, slots, pos0, ks, out, stream),
               "slot_verify_attn")
        return out

    def layer_view(self, layer):
        """torch views of the layer's K and V buffers, [n_slots, slot_ctx, kv_dim]
        (device memory owned by the handle)."""
        import torch
        rc, kp, vp = slot_kv_layer_ptrs(self.h, layer)
        _check(rc, "slot_kv_layer_ptrs")
        shape = (self.n_slots, self.slot_ctx, self.kv_dims[layer])
        return _device_view(kp, shape), _device_view(vp, shape)

    def write_rows(self, layer, slot, pos0, k_src=None, v_src=None, stream=None):
        _check(slot_kv_write_rows(self.h, layer, slot, pos0, k_src, v_src, stream=stream),
               "slot_kv_write_rows")

    def read_rows(self, layer, slot, pos0, n_rows, stream=None):
        import torch
        kd = self.kv_dims[layer]
        k = torch.empty((n_rows, kd), dtype=torch.float32, device="cuda")
        v = torch.empty((n_rows, kd), dtype=torch.float32, device="cuda")
        _check(slot_kv_read_rows(self.h, layer, slot, pos0, n_rows, k, v, stream=stream),
               "slot_kv_read_rows")
        return k, v
