"""CPU oracle for the slot-indexed batched decode-attention step.

TEST INFRASTRUCTURE ONLY: the plain, slow, double-precision definition that
the HIP library is checked against.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this package; the library itself
never does, and this package imports nothing from the library.

The arithmetic lives in ``slot_kv_oracle.c`` (plain C, compiled with gcc, no
fast-math, no FP contraction); this module only marshals numpy arrays into it.
Definitions follow the ZINC "Forward Cuda Gemma" page (sections decodeBatch,
allocSlotKv, slotKvOffsetBytes) and the "Forward Cuda" page (init: upload of
inv_freq and sinks; slot byte offsets).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "slot_kv_oracle.c")
_LIB_DEFAULT = os.path.join(_HERE, "liboracle.so")
# The mutation test points this at deliberately broken copies of the oracle.
_LIB = os.environ.get("SLOT_KV_ORACLE_LIB", _LIB_DEFAULT)

OK, EINVAL, ERANGE, EDUP = 0, -1, -2, -5


def build(force: bool = True, src: str = _SRC, out: str = _LIB_DEFAULT) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) and _LIB == _LIB_DEFAULT:
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u32, u64 = ctypes.c_uint32, ctypes.c_uint64
        lib.oracle_slot_kv_offset_bytes.argtypes = [u32, u32, u32, u32]
        lib.oracle_slot_kv_offset_bytes.restype = u64
        lib.oracle_rms_norm.argtypes = [f32p, f32p, u32, ctypes.c_double, f64p]
        lib.oracle_rms_norm.restype = None
        lib.oracle_rope.argtypes = [f64p, f32p, u32, u32]
        lib.oracle_rope.restype = None
        lib.oracle_decode_row.argtypes = [
            u32, u32, u32, f32p, f32p, f32p, f32p, ctypes.c_float, ctypes.c_float,
            u32, f32p, f32p, f32p, f32p, f32p, u64, f32p, f32p, f32p, u32]
        lib.oracle_decode_row.restype = ctypes.c_int
        lib.oracle_check_batch.argtypes = [u32, u32, u32p, u32p, u32]
        lib.oracle_check_batch.restype = ctypes.c_int
        lib.oracle_decode_batch.argtypes = [
            u32, u32, u32, f32p, f32p, f32p, f32p, ctypes.c_float, ctypes.c_float,
            f32p, f32p, u32, u32, f32p, f32p, f32p, u32p, u32p, u32, f32p, u32]
        lib.oracle_decode_batch.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [
            u32, u32, u32, f32p, f32p, f32p, f32p, ctypes.c_float, ctypes.c_float,
            f32p, f32p, u32, u32, f32p, f32p, f32p, u32, u32, u32, f32p, u32]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_verify.argtypes = [
            u32, u32, u32, f32p, f32p, f32p, f32p, ctypes.c_float, ctypes.c_float,
            f32p, f32p, u32, u32, f32p, f32p, f32p, u32p, u32p, u32p, u32, f32p, u32]
        lib.oracle_verify.restype = ctypes.c_int
        lib.oracle_rms_norm_1pw.argtypes = [f32p, f32p, u32, ctypes.c_double, f64p]
        lib.oracle_rms_norm_1pw.restype = None
        lib.oracle_rms_norm_plain.argtypes = [f32p, u32, ctypes.c_double, f64p]
        lib.oracle_rms_norm_plain.restype = None
        lib.oracle_rope_interleaved.argtypes = [f64p, f32p, u32, u32]
        lib.oracle_rope_interleaved.restype = None
        lib.oracle_slot_state_offset_bytes.argtypes = [u32, u32]
        lib.oracle_slot_state_offset_bytes.restype = u64
        lib.oracle_slot_reset.argtypes = [ctypes.POINTER(f32p), ctypes.POINTER(f32p), u32p, u32p,
                                          u32, u32, u32p, u32]
        lib.oracle_slot_reset.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a, name):
    if a.dtype != np.float32 or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name}: expected C-contiguous float32 array")
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _u32(a, name):
    if a.dtype != np.uint32 or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name}: expected C-contiguous uint32 array")
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def _opt_f32(a, name):
    return None if a is None else _f32(a, name)


# Convention flags of a layer (LayerParams.flags): see slot_kv_oracle.c.
V_NORM, ROPE_INTERLEAVED, NORM_ONE_PLUS_W = 1, 2, 4


def _flags(layer) -> int:
    return int(getattr(layer, "flags", 0))


def slot_kv_offset_bytes(slot: int, pos: int, slot_ctx: int, kv_dim: int) -> int:
    """(slot * slot_ctx + pos) * kv_dim * 4, in 64-bit arithmetic."""
    return int(_load().oracle_slot_kv_offset_bytes(slot, pos, slot_ctx, kv_dim))


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-vector RMSNorm in float64 (returns float64)."""
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    y = np.empty(x.shape[0], np.float64)
    _load().oracle_rms_norm(_f32(x, "x"), _f32(w, "w"), x.shape[0], float(eps),
                            y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return y


def rms_norm_1pw(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with (1 + w) weights, float64."""
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    y = np.empty(x.shape[0], np.float64)
    _load().oracle_rms_norm_1pw(_f32(x, "x"), _f32(w, "w"), x.shape[0], float(eps),
                                y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return y


def rms_norm_plain(x: np.ndarray, eps: float) -> np.ndarray:
    """Weightless RMSNorm, float64."""
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty(x.shape[0], np.float64)
    _load().oracle_rms_norm_plain(_f32(x, "x"), x.shape[0], float(eps),
                                  y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return y


def rope_interleaved(x: np.ndarray, inv_freq: np.ndarray, pos: int) -> np.ndarray:
    """Interleaved-pair RoPE of one float64 head vector at position ``pos``."""
    y = np.array(x, dtype=np.float64, copy=True)
    inv_freq = np.ascontiguousarray(inv_freq, np.float32)
    _load().oracle_rope_interleaved(y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                    _f32(inv_freq, "inv_freq"), pos, y.shape[0])
    return y


def rope(x: np.ndarray, inv_freq: np.ndarray, pos: int) -> np.ndarray:
    """Rotate-half RoPE of one float64 head vector at position ``pos``."""
    y = np.array(x, dtype=np.float64, copy=True)
    inv_freq = np.ascontiguousarray(inv_freq, np.float32)
    _load().oracle_rope(y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                        _f32(inv_freq, "inv_freq"), pos, y.shape[0])
    return y


def decode_row(layer, pos, q_row, k_new_row, v_new_row, hist_k, hist_v):
    """One row of the step.  ``layer`` carries n_heads, n_kv_heads, head_dim,
    q_norm_w, k_norm_w, inv_freq, sinks (or None), eps, scale.  ``hist_k`` /
    ``hist_v`` are [>=pos, kv_dim] float32 (rows 0..pos-1 are read).
    Returns (k_written, v_written, out_row)."""
    L = layer
    kv_dim = L.n_kv_heads * L.head_dim
    k_w = np.empty(kv_dim, np.float32)
    v_w = np.empty(kv_dim, np.float32)
    out = np.empty(L.n_heads * L.head_dim, np.float32)
    if pos > 0:
        hist_k = np.ascontiguousarray(hist_k, np.float32)
        hist_v = np.ascontiguousarray(hist_v, np.float32)
        if hist_k.shape[0] < pos or hist_v.shape[0] < pos:
            raise ValueError("history shorter than pos")
        hk, hv, stride = _f32(hist_k, "hist_k"), _f32(hist_v, "hist_v"), hist_k.shape[1]
    else:
        hk = hv = None
        stride = kv_dim
    rc = _load().oracle_decode_row(
        L.n_heads, L.n_kv_heads, L.head_dim, _f32(L.q_norm_w, "q_norm_w"),
        _f32(L.k_norm_w, "k_norm_w"), _f32(L.inv_freq, "inv_freq"),
        _opt_f32(L.sinks, "sinks"), float(L.eps), float(L.scale), int(pos),
        _f32(np.ascontiguousarray(q_row, np.float32), "q"),
        _f32(np.ascontiguousarray(k_new_row, np.float32), "k_new"),
        _f32(np.ascontiguousarray(v_new_row, np.float32), "v_new"),
        hk, hv, stride, _f32(k_w, "k_w"), _f32(v_w, "v_w"), _f32(out, "out"), _flags(layer))
    if rc != OK:
        raise ValueError(f"oracle_decode_row failed: {rc}")
    return k_w, v_w, out


def check_batch(n_slots, slot_ctx, positions, slots) -> int:
    positions = np.ascontiguousarray(positions, np.uint32)
    slots = np.ascontiguousarray(slots, np.uint32)
    return int(_load().oracle_check_batch(n_slots, slot_ctx, _u32(positions, "positions"),
                                          _u32(slots, "slots"), positions.shape[0]))


def decode_batch(layer, cache_k, cache_v, q, k_new, v_new, positions, slots):
    """The whole step over host mirrors ``cache_k`` / ``cache_v`` of shape
    [n_slots, slot_ctx, kv_dim] float32 (updated in place).  Returns
    (status, out[B, n_heads*head_dim])."""
    L = layer
    n_slots, slot_ctx, kv_dim = cache_k.shape
    if kv_dim != L.n_kv_heads * L.head_dim or cache_v.shape != cache_k.shape:
        raise ValueError("cache shape does not match the layer")
    positions = np.ascontiguousarray(positions, np.uint32)
    slots = np.ascontiguousarray(slots, np.uint32)
    B = positions.shape[0]
    out = np.zeros((B, L.n_heads * L.head_dim), np.float32)
    rc = _load().oracle_decode_batch(
        L.n_heads, L.n_kv_heads, L.head_dim, _f32(L.q_norm_w, "q_norm_w"),
        _f32(L.k_norm_w, "k_norm_w"), _f32(L.inv_freq, "inv_freq"),
        _opt_f32(L.sinks, "sinks"), float(L.eps), float(L.scale),
        _f32(cache_k, "cache_k"), _f32(cache_v, "cache_v"), n_slots, slot_ctx,
        _f32(np.ascontiguousarray(q, np.float32), "q"),
        _f32(np.ascontiguousarray(k_new, np.float32), "k_new"),
        _f32(np.ascontiguousarray(v_new, np.float32), "v_new"),
        _u32(positions, "positions"), _u32(slots, "slots"), B, _f32(out, "out"), _flags(L))
    return rc, out


def prefill(layer, cache_k, cache_v, q, k_new, v_new, slot, pos0):
    """Slot prefill over host mirrors ``cache_k`` / ``cache_v``
    [n_slots, slot_ctx, kv_dim] float32 (updated in place): the T rows of q,
    k_new, v_new are tokens at positions pos0 .. pos0+T-1 of ``slot``.
    Returns (status, out[T, n_heads*head_dim])."""
    L = layer
    n_slots, slot_ctx, kv_dim = cache_k.shape
    if kv_dim != L.n_kv_heads * L.head_dim or cache_v.shape != cache_k.shape:
        raise ValueError("cache shape does not match the layer")
    q = np.ascontiguousarray(q, np.float32)
    T = q.shape[0]
    out = np.zeros((T, L.n_heads * L.head_dim), np.float32)
    rc = _load().oracle_prefill(
        L.n_heads, L.n_kv_heads, L.head_dim, _f32(L.q_norm_w, "q_norm_w"),
        _f32(L.k_norm_w, "k_norm_w"), _f32(L.inv_freq, "inv_freq"),
        _opt_f32(L.sinks, "sinks"), float(L.eps), float(L.scale),
        _f32(cache_k, "cache_k"), _f32(cache_v, "cache_v"), n_slots, slot_ctx,
        _f32(q, "q"), _f32(np.ascontiguousarray(k_new, np.float32), "k_new"),
        _f32(np.ascontiguousarray(v_new, np.float32), "v_new"), slot, pos0, T, _f32(out, "out"),
        _flags(L))
    return rc, out


def verify(layer, cache_k, cache_v, q, k_new, v_new, slots, pos0, ks):
    """ks[i] rows for each sequence i (rows sequence-major in q / k_new /
    v_new) at positions pos0[i] .. of slot slots[i], over host mirrors
    [n_slots, slot_ctx, kv_dim] (updated in place).  Returns (status,
    out[sum ks, n_heads*head_dim])."""
    L = layer
    n_slots, slot_ctx, kv_dim = cache_k.shape
    if kv_dim != L.n_kv_heads * L.head_dim or cache_v.shape != cache_k.shape:
        raise ValueError("cache shape does not match the layer")
    slots = np.ascontiguousarray(slots, np.uint32)
    pos0 = np.ascontiguousarray(pos0, np.uint32)
    ks = np.ascontiguousarray(ks, np.uint32)
    rows = int(ks.astype(np.int64).sum())
    q = np.ascontiguousarray(q, np.float32).reshape(rows, -1) if rows else np.zeros((1, L.n_heads * L.head_dim), np.float32)
    k_new = np.ascontiguousarray(k_new, np.float32) if rows else np.zeros((1, kv_dim), np.float32)
    v_new = np.ascontiguousarray(v_new, np.float32) if rows else np.zeros((1, kv_dim), np.float32)
    out = np.zeros((max(rows, 1), L.n_heads * L.head_dim), np.float32)
    rc = _load().oracle_verify(
        L.n_heads, L.n_kv_heads, L.head_dim, _f32(L.q_norm_w, "q_norm_w"),
        _f32(L.k_norm_w, "k_norm_w"), _f32(L.inv_freq, "inv_freq"),
        _opt_f32(L.sinks, "sinks"), float(L.eps), float(L.scale),
        _f32(cache_k, "cache_k"), _f32(cache_v, "cache_v"), n_slots, slot_ctx,
        _f32(q, "q"), _f32(k_new, "k_new"), _f32(v_new, "v_new"),
        _u32(slots, "slots"), _u32(pos0, "pos0"), _u32(ks, "ks"), slots.shape[0], _f32(out, "out"),
        _flags(L))
    return rc, out[:rows]


# ---------------------------------------------------------------- per-slot SSM state
def slot_state_offset_bytes(slot: int, state_len: int) -> int:
    """Byte offset of slot ``slot`` in a [slot][state_len] f32 buffer: the conv
    ring (state_len = conv_state_len) or the recurrent state (ssm_state_len)."""
    return int(_load().oracle_slot_state_offset_bytes(slot, state_len))


def slot_reset(conv, ssm, slots, n_slots=None) -> int:
    """Reset of reused slots on admit: zeroes, in place, each listed slot's conv
    ring and recurrent state in every ssm layer.  ``conv`` / ``ssm`` are lists
    (one entry per ssm layer) of C-contiguous float32 arrays of shape
    [n_slots, state_len].  Returns the status (ERANGE writes nothing)."""
    lib = _load()
    n_layers = len(conv)
    if len(ssm) != n_layers:
        raise ValueError("conv and ssm need one buffer per ssm layer each")
    if n_slots is None:
        n_slots = conv[0].shape[0] if n_layers else 0
    for a in list(conv) + list(ssm):
        if a.ndim != 2 or a.shape[0] != n_slots:
            raise ValueError("state buffers must be [n_slots, state_len]")
    f32p = ctypes.POINTER(ctypes.c_float)
    cp = (f32p * max(n_layers, 1))(*[_f32(a, "conv") for a in conv])
    sp = (f32p * max(n_layers, 1))(*[_f32(a, "ssm") for a in ssm])
    cl = np.array([a.shape[1] for a in conv] or [0], np.uint32)
    sl = np.array([a.shape[1] for a in ssm] or [0], np.uint32)
    sv = np.ascontiguousarray(np.asarray(slots, np.uint32).reshape(-1))
    return int(lib.oracle_slot_reset(cp, sp, _u32(cl, "conv_len"), _u32(sl, "ssm_len"), n_layers,
                                     n_slots, _u32(sv, "slots"), sv.size))
