"""GPU parity of the HIP decode step against the CPU oracle, through the C ABI.

Bar: KV-write placement and V bytes bit-exact; K rows and attention outputs
within |gpu - oracle| <= 1e-4 + 1e-5 |oracle| (f32 kernel vs f64 oracle).
Workloads: the five seeded configurations (tiny, mid, long, many short,
8-layer stack); tiny, mid and many are checked on every row, long and the
layer stack on a seeded sample that holds the longest and shortest row.
"ZINC Forward Cuda Gemma", decodeBatch / allocSlotKv / slotKvOffsetBytes /
slotKvSmoke; "Forward Cuda", slot reset on admit and the serial reference.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sequence_slot_kv_amd import binding as b  # noqa: E402
from sequence_slot_kv_amd import workloads as wl  # noqa: E402

from _gpu_util import (assert_close, device_inputs, fill_history_device,  # noqa: E402
                       handle_for, oracle_rows, sample_rows, snapshot_rows, upload_history)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- smoke
def test_slot_kv_smoke_sentinels():
    # "Forward Cuda Gemma", slotKvSmoke: a sentinel at (slot 0, pos 0) and a
    # distinct pattern at the LAST (slot, pos) of layer 0's K cache survive
    # each other's writes.  Generalised: every (layer, slot, pos) row of a
    # tiny 2-layer cache gets a unique pattern through the library's offsets,
    # and the whole buffer reads back exactly.
    kv = b.SlotKV()
    n_slots, slot_ctx, dims = 4, 128, [128, 96]
    kv.alloc(n_slots, slot_ctx, dims)
    for L, kd in enumerate(dims):
        kbuf, vbuf = kv.layer_view(L)
        assert kbuf.shape == (n_slots, slot_ctx, kd)
        assert int(kbuf.abs().sum().item()) == 0 and int(vbuf.abs().sum().item()) == 0  # zeroed
        ids = torch.arange(n_slots * slot_ctx, device="cuda", dtype=torch.float32)
        pat = (ids[:, None] * 1000 + torch.arange(kd, device="cuda", dtype=torch.float32)[None])
        for s in range(n_slots):
            rows = pat[s * slot_ctx:(s + 1) * slot_ctx].contiguous()
            kv.write_rows(L, s, 0, k_src=rows, v_src=(-rows).contiguous())
        torch.cuda.synchronize()
        flat_k = kbuf.reshape(-1)
        for s in range(n_slots):
            for p in (0, 1, slot_ctx - 1):
                off = kv.offset_bytes(L, s, p)
                assert off == oracle.slot_kv_offset_bytes(s, p, slot_ctx, kd)
                got = flat_k[off // 4: off // 4 + kd]
                assert torch.equal(got, pat[s * slot_ctx + p])
        assert torch.equal(kbuf.reshape(-1, kd), pat) and torch.equal(vbuf.reshape(-1, kd), -pat)
    kv.close()


def test_offsets_beyond_32_bits():
    # A 128 x 8192 cache of 1024- and 2048-float rows (the layer-stack shape):
    # the last row of the 2048-wide layer starts at 2^33 - 2^13 bytes.
    kv = b.SlotKV()
    kv.alloc(128, 8192, [1024, 2048])
    assert kv.offset_bytes(1, 127, 8191) == 2**33 - 2**13
    assert kv.offset_bytes(0, 127, 8191) == 2**32 - 2**12
    row = torch.arange(2048, device="cuda", dtype=torch.float32)[None].contiguous()
    kv.write_rows(1, 127, 8191, k_src=row, v_src=(row + 1).contiguous())
    k, v = kv.read_rows(1, 127, 8191, 1)
    assert torch.equal(k, row) and torch.equal(v, row + 1)
    kbuf, _ = kv.layer_view(1)
    assert torch.equal(kbuf[127, 8191], row[0]) and float(kbuf[127, 8190].abs().sum()) == 0.0
    kv.close()


# ---------------------------------------------------------------- tiny
def _run_tiny(kv, w, out=None):
    q, k_new, v_new = device_inputs(w, 0)
    out = kv.decode_attn(0, q, k_new, v_new, w.positions, w.slots, out=out)
    torch.cuda.synchronize()
    return out


def test_tiny_full_parity_and_placement():
    w = wl.tiny()
    _say(f"tiny: positions {w.positions.tolist()} slots {w.slots.tolist()}")
    hk, hv = wl.history_host(w, 0)
    kv = handle_for(w)
    upload_history(kv, 0, hk, hv)
    out = _run_tiny(kv, w).cpu().numpy()
    ck, cv = hk.copy(), hv.copy()
    rc, ref = oracle.decode_batch(w.layers[0], ck, cv, w.inputs[0].q, w.inputs[0].k_new,
                                  w.inputs[0].v_new, w.positions, w.slots)
    assert rc == 0
    assert_close(out, ref, "tiny out")
    gk, gv = (t.cpu().numpy() for t in kv.layer_view(0))
    # exactly the B written rows changed; V bytes verbatim; K within tolerance
    changed_k = {tuple(x) for x in np.argwhere((gk != hk).any(-1))}
    changed_v = {tuple(x) for x in np.argwhere((gv != hv).any(-1))}
    expect = {(int(s), int(p)) for s, p in zip(w.slots, w.positions)}
    assert changed_k == expect and changed_v == expect
    assert gv.tobytes() == cv.tobytes()
    assert_close(gk, ck, "tiny K cache")
    kv.close()


def test_tiny_multi_step_decode_matches_oracle():
    # Serving pattern ("Forward Cuda Gemma", decodeBatch: the caller advances
    # pos and feeds back): several steps in a row, each row at its own
    # position, the cache carried from step to step on both sides.
    w = wl.tiny()
    L = w.layers[0]
    hk, hv = wl.history_host(w, 0)
    kv = handle_for(w)
    upload_history(kv, 0, hk, hv)
    ck, cv = hk.copy(), hv.copy()
    rng = np.random.default_rng(11)
    pos = np.minimum(w.positions.astype(np.int64), w.slot_ctx - 8)
    for step in range(6):
        q = rng.standard_normal((w.B, L.q_dim), dtype=np.float32)
        kn = rng.standard_normal((w.B, L.kv_dim), dtype=np.float32)
        vn = rng.standard_normal((w.B, L.kv_dim), dtype=np.float32)
        out = kv.decode_attn(0, torch.from_numpy(q).cuda(), torch.from_numpy(kn).cuda(),
                             torch.from_numpy(vn).cuda(), pos, w.slots)
        rc, ref = oracle.decode_batch(L, ck, cv, q, kn, vn, pos, w.slots)
        assert rc == 0
        assert_close(out.cpu().numpy(), ref, f"step {step}")
        pos = pos + 1
    gk, gv = (t.cpu().numpy() for t in kv.layer_view(0))
    assert gv.tobytes() == cv.tobytes()
    assert_close(gk, ck, "K cache after 6 steps")
    kv.close()


def test_reused_slot_needs_no_reset():
    # "Forward Cuda", reset on admit: a reused slot keeps the previous
    # request's rows, yet a new sequence prefilled token by token from pos 0
    # (B=1 decode calls, as the pages' per-token prefill into a slot) reads
    # only what it wrote: the result equals the same sequence on a zeroed
    # cache.
    w = wl.tiny()
    L = w.layers[0]
    kv = handle_for(w)
    stale_k = np.full((w.n_slots, w.slot_ctx, L.kv_dim), 7.5, np.float32)
    upload_history(kv, 0, stale_k, -stale_k)
    kv.reset(2)
    rng = np.random.default_rng(12)
    ck = np.zeros((w.n_slots, w.slot_ctx, L.kv_dim), np.float32)
    cv = np.zeros_like(ck)
    for p in range(40):
        q = rng.standard_normal((1, L.q_dim), dtype=np.float32)
        kn = rng.standard_normal((1, L.kv_dim), dtype=np.float32)
        vn = rng.standard_normal((1, L.kv_dim), dtype=np.float32)
        out = kv.decode_attn(0, torch.from_numpy(q).cuda(), torch.from_numpy(kn).cuda(),
                             torch.from_numpy(vn).cuda(), [p], [2])
        rc, ref = oracle.decode_batch(L, ck, cv, q, kn, vn, [p], [2])
        assert rc == 0
        assert_close(out.cpu().numpy(), ref, f"prefill pos {p}")
    kv.close()


# ---------------------------------------------------------------- errors
def test_error_paths_write_nothing():
    w = wl.tiny()
    kv = handle_for(w)
    hk, hv = wl.history_host(w, 0)
    upload_history(kv, 0, hk, hv)
    q, k_new, v_new = device_inputs(w, 0)
    out = torch.full_like(q, 3.0)
    h = kv.h
    call = lambda pos, sl: b.slot_decode_attn(h, 0, q[:len(pos)], k_new[:len(pos)],  # noqa: E731
                                              v_new[:len(pos)], pos, sl, out[:len(pos)])
    assert call([128], [0]) == b.SLOT_KV_ERANGE
    assert call([5], [4]) == b.SLOT_KV_ERANGE
    assert call([5, 6], [1, 1]) == b.SLOT_KV_EDUP
    assert b.slot_decode_attn(h, 1, q, k_new, v_new, w.positions, w.slots, out) == b.SLOT_KV_EINVAL
    assert call([], []) == b.SLOT_KV_OK  # B = 0 is a no-op
    assert b.slot_kv_offset_bytes(h, 0, 4, 0)[0] == b.SLOT_KV_ERANGE
    assert b.slot_kv_offset_bytes(h, 0, 0, 128)[0] == b.SLOT_KV_ERANGE
    assert b.slot_reset(h, 4) == b.SLOT_KV_ERANGE and b.slot_reset(h, 3) == b.SLOT_KV_OK
    P = w.layers[0]
    bad = b.slot_kv_set_layer(h, 0, 4, 4, 64, P.q_norm_w, P.k_norm_w, P.inv_freq)
    assert bad == b.SLOT_KV_EINVAL  # 4 x 64 != kv_dim 128
    assert b.slot_kv_set_layer(h, 0, 6, 2, 64, P.q_norm_w, P.k_norm_w,
                               P.inv_freq) == b.SLOT_KV_EINVAL  # group of 3 unsupported
    torch.cuda.synchronize()
    assert float(out.min()) == 3.0 and float(out.max()) == 3.0
    gk, gv = (t.cpu().numpy() for t in kv.layer_view(0))
    assert gk.tobytes() == hk.tobytes() and gv.tobytes() == hv.tobytes()
    # a layer that was never configured
    kv2 = b.SlotKV()
    kv2.alloc(4, 128, [128])
    assert b.slot_decode_attn(kv2.h, 0, q, k_new, v_new, w.positions, w.slots,
                              out) == b.SLOT_KV_EINVAL
    # alloc is idempotent: a second alloc frees the first and re-zeroes
    kv2.alloc(4, 128, [128])
    assert float(kv2.layer_view(0)[0].abs().sum()) == 0.0
    kv2.close()
    kv.close()


# ---------------------------------------------------------------- mid (bench config)
@pytest.fixture(scope="module")
def mid_setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = wl.mid()
    kv = handle_for(w)
    fill_history_device(kv, w, 0)
    hist = {bi: snapshot_rows(kv, 0, int(w.slots[bi]), int(w.positions[bi])) for bi in range(w.B)}
    ref = oracle_rows(w, 0, range(w.B), hist)
    yield w, kv, hist, ref
    kv.close()


def test_mid_full_parity(mid_setup):
    w, kv, hist, ref = mid_setup
    _say(f"mid: B={w.B} kv_bytes={w.kv_bytes()}")
    q, k_new, v_new = device_inputs(w, 0)
    out = kv.decode_attn(0, q, k_new, v_new, w.positions, w.slots).cpu().numpy()
    for bi in range(w.B):
        assert_close(out[bi], ref[bi][2], f"mid row {bi} pos {w.positions[bi]}")
        s, p = int(w.slots[bi]), int(w.positions[bi])
        k, v = kv.read_rows(0, s, p, 1)
        assert v.cpu().numpy().tobytes() == ref[bi][1].tobytes()
        assert_close(k.cpu().numpy()[0], ref[bi][0], f"mid K row {bi}")
        # history rows untouched
        if p > 0:
            k1, v1 = kv.read_rows(0, s, p - 1, 1)
            assert k1.cpu().numpy().tobytes() == hist[bi][0][p - 1].tobytes()


def test_mid_batch_equals_serial_bit_exact(mid_setup):
    # "Forward Cuda", serial reference; "Forward Cuda Gemma", decodeBatch: the
    # batched step equals each sequence run alone (B = 1), here bit for bit.
    w, kv, _, _ = mid_setup
    q, k_new, v_new = device_inputs(w, 0)
    out = kv.decode_attn(0, q, k_new, v_new, w.positions, w.slots)
    out2 = kv.decode_attn(0, q, k_new, v_new, w.positions, w.slots)
    assert torch.equal(out, out2), "two runs differ"
    for bi in range(w.B):
        o1 = kv.decode_attn(0, q[bi:bi + 1].contiguous(), k_new[bi:bi + 1].contiguous(),
                            v_new[bi:bi + 1].contiguous(), w.positions[bi:bi + 1],
                            w.slots[bi:bi + 1])
        assert torch.equal(o1[0], out[bi]), f"row {bi} differs from its B=1 run"
    perm = np.random.default_rng(3).permutation(w.B)
    pt = torch.from_numpy(perm).cuda()
    op = kv.decode_attn(0, q[pt].contiguous(), k_new[pt].contiguous(), v_new[pt].contiguous(),
                        w.positions[perm], w.slots[perm])
    assert torch.equal(op, out[pt])


# ---------------------------------------------------------------- many short
def test_many_short_full_parity_with_poison():
    # 256 rows, 26 of them at pos 0 in reused slots whose later rows hold
    # stale data: every cell a row may not read, from its own position on, is
    # poisoned (qNaN, then +-1e30); outputs stay finite and equal the
    # oracle's, and the poison outside the written rows survives the step.
    w = wl.many_short()
    _say(f"many: B={w.B} pos0 rows={(w.positions == 0).sum()}")
    kv = handle_for(w)
    fill_history_device(kv, w, 0)
    hist = {bi: snapshot_rows(kv, 0, int(w.slots[bi]), int(w.positions[bi])) for bi in range(w.B)}
    ref = oracle_rows(w, 0, range(w.B), hist)
    q, k_new, v_new = device_inputs(w, 0)
    kbuf, vbuf = kv.layer_view(0)
    used = np.zeros(w.n_slots, bool)
    used[w.slots] = True
    for poison in (float("nan"), 1e30, -1e30):
        # the row at pos itself too: the step must overwrite it, and must not
        # read what it held
        for bi in range(w.B):
            s, p = int(w.slots[bi]), int(w.positions[bi])
            kbuf[s, p:] = poison
            vbuf[s, p:] = poison
        idle = torch.from_numpy(np.nonzero(~used)[0]).cuda()
        if idle.numel():
            kbuf[idle] = poison
            vbuf[idle] = poison
        k_snap, v_snap = kbuf.clone(), vbuf.clone()
        out = kv.decode_attn(0, q, k_new, v_new, w.positions, w.slots).cpu().numpy()
        for bi in range(w.B):
            assert_close(out[bi], ref[bi][2], f"many row {bi} poison {poison}")
        # every poisoned cell still holds the poison: exactly the B written
        # rows changed, bit for bit; those rows hold the rotated key (within
        # tolerance) and v_new's bytes
        changed = {tuple(x) for x in
                   ((kbuf.view(torch.int32) != k_snap.view(torch.int32)).any(-1) |
                    (vbuf.view(torch.int32) != v_snap.view(torch.int32)).any(-1))
                   .nonzero().cpu().tolist()}
        assert changed == {(int(s), int(p)) for s, p in zip(w.slots, w.positions)}
        del k_snap, v_snap
        for bi in range(w.B):
            s, p = int(w.slots[bi]), int(w.positions[bi])
            assert vbuf[s, p].cpu().numpy().tobytes() == ref[bi][1].tobytes()
            assert_close(kbuf[s, p].cpu().numpy(), ref[bi][0], f"many K row {bi}")
    kv.close()


# ---------------------------------------------------------------- long context
def test_long_context_sampled_parity():
    w = wl.long_ctx()
    rows = sample_rows(w, 6, seed=31)
    _say(f"long: rows {rows} positions {[int(w.positions[r]) for r in rows]}")
    kv = handle_for(w)
    fill_history_device(kv, w, 0)
    hist = {bi: snapshot_rows(kv, 0, int(w.slots[bi]), int(w.positions[bi])) for bi in rows}
    ref = oracle_rows(w, 0, rows, hist)
    q, k_new, v_new = device_inputs(w, 0)
    out = kv.decode_attn(0, q, k_new, v_new, w.positions, w.slots).cpu().numpy()
    for bi in rows:
        assert_close(out[bi], ref[bi][2], f"long row {bi} pos {w.positions[bi]}")
        k, v = kv.read_rows(0, int(w.slots[bi]), int(w.positions[bi]), 1)
        assert v.cpu().numpy().tobytes() == ref[bi][1].tobytes()
        assert_close(k.cpu().numpy()[0], ref[bi][0], f"long K row {bi}")
    kv.close()


# ---------------------------------------------------------------- layer stack
def test_layer_stack_sampled_parity():
    # 8 layers alternating 8x128 and 8x256 kv heads, per-head sinks, one
    # decode step through every layer on one stream (96 GiB of slot KV).
    w = wl.layer_stack()
    rows = sample_rows(w, 4, seed=41)
    _say(f"layer_stack: rows {rows}")
    kv = handle_for(w)
    outs, refs = [], []
    for l in range(len(w.layers)):
        fill_history_device(kv, w, l)
        hist = {bi: snapshot_rows(kv, l, int(w.slots[bi]), int(w.positions[bi])) for bi in rows}
        refs.append(oracle_rows(w, l, rows, hist))
    for l in range(len(w.layers)):
        q, k_new, v_new = device_inputs(w, l)
        outs.append(kv.decode_attn(l, q, k_new, v_new, w.positions, w.slots))
    torch.cuda.synchronize()
    for l in range(len(w.layers)):
        o = outs[l].cpu().numpy()
        for bi in rows:
            assert_close(o[bi], refs[l][bi][2], f"layer {l} row {bi}")
            k, v = kv.read_rows(l, int(w.slots[bi]), int(w.positions[bi]), 1)
            assert v.cpu().numpy().tobytes() == refs[l][bi][1].tobytes()
    kv.close()


# ---------------------------------------------------------------- every head shape
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_shapes_full_parity(D, G):
    # Each (head_dim, group) instantiation of the decode kernel: rows of one
    # key, rows at both sides of the split-K chunk boundaries (split rows
    # merged by the last workgroup), every cache cell outside 0..pos poisoned.
    Hkv = 2
    H = G * Hkv
    rng = np.random.default_rng(300 + 10 * G + D)
    # Rows whose last chunk holds a few keys leave some of the waves that
    # split a chunk with no keys, others with one partial stage.
    C = b.slot_kv_chunk_keys()
    n_slots, slot_ctx = 12, 2 * C + 176
    L = wl.make_layer(rng, H, Hkv, D, 1e4, G % 2 == 0)
    positions = np.array([0, 1, 53, C - 1, C, C + 1, C + 8, 2 * C - 1, 2 * C + 175], np.uint32)
    slots = rng.permutation(n_slots)[:positions.size].astype(np.uint32)
    B = positions.size
    q = rng.standard_normal((B, H * D), dtype=np.float32)
    kn = rng.standard_normal((B, L.kv_dim), dtype=np.float32)
    vn = rng.standard_normal((B, L.kv_dim), dtype=np.float32)
    ck = np.full((n_slots, slot_ctx, L.kv_dim), np.nan, np.float32)
    cv = np.full_like(ck, np.nan)
    for s, p in zip(slots, positions):
        ck[s, :p] = rng.standard_normal((p, L.kv_dim), dtype=np.float32)
        cv[s, :p] = rng.standard_normal((p, L.kv_dim), dtype=np.float32)
    kv = b.SlotKV()
    kv.alloc(n_slots, slot_ctx, [L.kv_dim])
    kv.set_layer(0, L)
    upload_history(kv, 0, ck, cv)
    out = kv.decode_attn(0, *(torch.from_numpy(x).cuda() for x in (q, kn, vn)), positions, slots)
    out = out.cpu().numpy()
    gk = kv.layer_view(0)[0].cpu().numpy()
    kv.close()
    rc, ref = oracle.decode_batch(L, ck, cv, q, kn, vn, positions, slots)
    assert rc == 0
    assert_close(out, ref, f"decode D={D} G={G}")
    for s, p in zip(slots, positions):
        assert_close(gk[s, p], ck[s, p], "written K")


def test_decode_more_rows_than_one_launch():
    # 300 rows: the call is cut into launches of at most 256 rows, each with
    # its own row table; every row is checked against the oracle.
    rng = np.random.default_rng(400)
    H, Hkv, D = 8, 2, 64
    C = b.slot_kv_chunk_keys()
    n_slots, slot_ctx, B = 300, C + 128, 300  # rows of one and of two split-K chunks
    L = wl.make_layer(rng, H, Hkv, D, 1e4, True)
    positions = rng.integers(0, slot_ctx, size=B).astype(np.uint32)
    positions[:3] = [0, C - 1, slot_ctx - 1]
    slots = rng.permutation(n_slots)[:B].astype(np.uint32)
    q = rng.standard_normal((B, H * D), dtype=np.float32)
    kn = rng.standard_normal((B, L.kv_dim), dtype=np.float32)
    vn = rng.standard_normal((B, L.kv_dim), dtype=np.float32)
    ck = rng.standard_normal((n_slots, slot_ctx, L.kv_dim), dtype=np.float32)
    cv = rng.standard_normal((n_slots, slot_ctx, L.kv_dim), dtype=np.float32)
    kv = b.SlotKV()
    kv.alloc(n_slots, slot_ctx, [L.kv_dim])
    kv.set_layer(0, L)
    upload_history(kv, 0, ck, cv)
    b.slot_kv_profile_begin(kv.h)
    out = kv.decode_attn(0, *(torch.from_numpy(x).cuda() for x in (q, kn, vn)), positions, slots)
    rc, _, launches = b.slot_kv_profile_end(kv.h)
    assert rc == 0 and launches == 2
    out = out.cpu().numpy()
    kv.close()
    rc, ref = oracle.decode_batch(L, ck, cv, q, kn, vn, positions, slots)
    assert rc == 0
    assert_close(out, ref, "300-row decode")
