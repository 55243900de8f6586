"""GPU parity of the convention flags (SLOT_KV_FLAG_*: V-norm, interleaved
RoPE, (1 + w) norm weights) on every entry point, against the oracle run with
the same flags."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from sequence_slot_kv_amd import binding as b
from sequence_slot_kv_amd import workloads as wl

from _gpu_util import assert_close

pytestmark = pytest.mark.gpu

FLAG_SETS = [oracle.V_NORM, oracle.ROPE_INTERLEAVED, oracle.NORM_ONE_PLUS_W,
             oracle.V_NORM | oracle.ROPE_INTERLEAVED | oracle.NORM_ONE_PLUS_W]


def _layer(rng, H, Hkv, D, flags, sinks):
    L = wl.make_layer(rng, H, Hkv, D, 1e4, sinks)
    return dataclasses.replace(L, flags=flags)


def _cache(rng, n_slots, slot_ctx, kv_dim):
    return (rng.standard_normal((n_slots, slot_ctx, kv_dim), dtype=np.float32),
            rng.standard_normal((n_slots, slot_ctx, kv_dim), dtype=np.float32))


def _handle(n_slots, slot_ctx, L, ck, cv):
    kv = b.SlotKV()
    kv.alloc(n_slots, slot_ctx, [L.kv_dim])
    kv.set_layer(0, L)
    for s in range(n_slots):
        kv.write_rows(0, s, 0, torch.from_numpy(ck[s]).cuda(), torch.from_numpy(cv[s]).cuda())
    return kv


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("H,Hkv,D", [(4, 2, 64), (8, 2, 128), (4, 2, 256)])
def test_decode_with_flags(flags, H, Hkv, D):
    rng = np.random.default_rng(50 + flags + D)
    C = b.slot_kv_chunk_keys()
    n_slots, slot_ctx, B = 6, C + 188, 5   # rows of one and of two split-K chunks
    L = _layer(rng, H, Hkv, D, flags, sinks=True)
    ck, cv = _cache(rng, n_slots, slot_ctx, L.kv_dim)
    slots = rng.permutation(n_slots)[:B].astype(np.uint32)
    positions = np.array([0, 1, 37, C - 1, C + 187], np.uint32)
    q = rng.standard_normal((B, H * D), dtype=np.float32)
    kn = rng.standard_normal((B, L.kv_dim), dtype=np.float32)
    vn = rng.standard_normal((B, L.kv_dim), dtype=np.float32)
    kv = _handle(n_slots, slot_ctx, L, ck, cv)
    out = kv.decode_attn(0, *(torch.from_numpy(x).cuda() for x in (q, kn, vn)), positions, slots)
    gk, gv = (x.cpu().numpy() for x in kv.layer_view(0))
    out = out.cpu().numpy()
    kv.close()
    rc, ref = oracle.decode_batch(L, ck, cv, q, kn, vn, positions, slots)
    assert rc == 0
    assert_close(out, ref, f"decode out flags={flags}")
    for p_, s_ in zip(positions, slots):
        assert_close(gk[s_, p_], ck[s_, p_], "written K")
        assert_close(gv[s_, p_], cv[s_, p_], "written V")


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("H,Hkv,D", [(4, 2, 64), (8, 2, 128), (4, 2, 256)])
def test_prefill_and_verify_with_flags(flags, H, Hkv, D):
    rng = np.random.default_rng(60 + flags + D)
    n_slots, slot_ctx = 4, 96
    L = _layer(rng, H, Hkv, D, flags, sinks=True)
    ck, cv = _cache(rng, n_slots, slot_ctx, L.kv_dim)
    slots, pos0, ks = [2, 0, 3], [10, 0, 50], [21, 5, 9]
    rows = sum(ks)
    q = rng.standard_normal((rows, H * D), dtype=np.float32)
    kn = rng.standard_normal((rows, L.kv_dim), dtype=np.float32)
    vn = rng.standard_normal((rows, L.kv_dim), dtype=np.float32)
    kv = _handle(n_slots, slot_ctx, L, ck, cv)
    q_d, k_d, v_d = (torch.from_numpy(x).cuda() for x in (q, kn, vn))
    # the first sequence by prefill, the others by one verify call
    out_p = kv.prefill_attn(0, q_d[:ks[0]], k_d[:ks[0]], v_d[:ks[0]], slots[0], pos0[0]).cpu().numpy()
    out_v = kv.verify_attn(0, q_d[ks[0]:], k_d[ks[0]:], v_d[ks[0]:], slots[1:], pos0[1:],
                           ks[1:]).cpu().numpy()
    gk, gv = (x.cpu().numpy() for x in kv.layer_view(0))
    kv.close()
    rc, ref = oracle.verify(L, ck, cv, q, kn, vn, slots, pos0, ks)
    assert rc == 0
    assert_close(out_p, ref[:ks[0]], f"prefill out flags={flags}")
    assert_close(out_v, ref[ks[0]:], f"verify out flags={flags}")
    for s_, p0, k in zip(slots, pos0, ks):
        assert_close(gk[s_, p0:p0 + k], ck[s_, p0:p0 + k], "written K")
        assert_close(gv[s_, p0:p0 + k], cv[s_, p0:p0 + k], "written V")


@pytest.mark.parametrize("H,Hkv,D", [(8, 4, 256), (16, 4, 128)])
def test_prefill_and_verify_flags_far_positions(H, Hkv, D):
    """All three flags at positions past 20,000, where the RoPE angles are
    large: a key-chunked tiled prefill (more than 64 query rows per kv head)
    and a split-K verify, against the oracle."""
    flags = oracle.V_NORM | oracle.ROPE_INTERLEAVED | oracle.NORM_ONE_PLUS_W
    rng = np.random.default_rng(70 + D)
    n_slots, slot_ctx = 3, 24576
    L = _layer(rng, H, Hkv, D, flags, sinks=True)
    ck, cv = _cache(rng, n_slots, slot_ctx, L.kv_dim)
    slots, pos0, ks = [1, 2, 0], [slot_ctx - 48, 20011, 23999], [48, 4, 3]
    rows = sum(ks)
    q = rng.standard_normal((rows, H * D), dtype=np.float32)
    kn = rng.standard_normal((rows, L.kv_dim), dtype=np.float32)
    vn = rng.standard_normal((rows, L.kv_dim), dtype=np.float32)
    kv = _handle(n_slots, slot_ctx, L, ck, cv)
    q_d, k_d, v_d = (torch.from_numpy(x).cuda() for x in (q, kn, vn))
    out_p = kv.prefill_attn(0, q_d[:ks[0]], k_d[:ks[0]], v_d[:ks[0]], slots[0], pos0[0]).cpu().numpy()
    out_v = kv.verify_attn(0, q_d[ks[0]:], k_d[ks[0]:], v_d[ks[0]:], slots[1:], pos0[1:],
                           ks[1:]).cpu().numpy()
    written = [(kv.read_rows(0, s_, p0, k)) for s_, p0, k in zip(slots, pos0, ks)]
    written = [(a.cpu().numpy(), c.cpu().numpy()) for a, c in written]
    kv.close()
    rc, ref = oracle.verify(L, ck, cv, q, kn, vn, slots, pos0, ks)
    assert rc == 0
    assert_close(out_p, ref[:ks[0]], f"prefill out, far positions, D={D}")
    assert_close(out_v, ref[ks[0]:], f"verify out, far positions, D={D}")
    for (gk, gv), s_, p0, k in zip(written, slots, pos0, ks):
        assert_close(gk, ck[s_, p0:p0 + k], "written K")
        assert_close(gv, cv[s_, p0:p0 + k], "written V")
