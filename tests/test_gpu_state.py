"""GPU checks of the per-slot SSM state through the C ABI ("Forward Cuda":
allocation of the per-sequence slot state, the conv-ring and recurrent-state
byte offsets, the reset of a reused slot on admit, and the sub-step 4a smoke).

Bar: bit-exact.  After a reset, every buffer equals the oracle's reset of a
host copy of the same seeded contents, byte for byte; at the full benchmark
size the same is checked as a property (the listed slots read +0.0, every
other byte is unchanged).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from sequence_slot_kv_amd import binding as b  # noqa: E402
from sequence_slot_kv_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def _handle(n_slots, conv_lens, ssm_lens, kv_dims=(), slot_ctx=16):
    kv = b.SlotKV()
    kv.alloc_state(n_slots, slot_ctx, list(kv_dims), list(conv_lens), list(ssm_lens))
    return kv


def _fill_host(kv, rng):
    """Seeded N(0,1) contents for every state buffer; returns the host copies."""
    conv, ssm = [], []
    for l in range(len(kv.state_lens)):
        cv, sv = kv.state_view(l)
        c = rng.standard_normal(tuple(cv.shape)).astype(np.float32)
        s = rng.standard_normal(tuple(sv.shape)).astype(np.float32)
        cv.copy_(torch.from_numpy(c))
        sv.copy_(torch.from_numpy(s))
        conv.append(c)
        ssm.append(s)
    torch.cuda.synchronize()
    return conv, ssm


def _read_all(kv):
    torch.cuda.synchronize()
    out = [kv.state_view(l) for l in range(len(kv.state_lens))]
    return [c.cpu().numpy() for c, _ in out], [s.cpu().numpy() for _, s in out]


def _same_bytes(a_list, b_list):
    return all(x.tobytes() == y.tobytes() for x, y in zip(a_list, b_list))


def test_alloc_zeroes_and_realloc_frees_first():
    kv = _handle(5, [27, 8], [4099, 7], kv_dims=[64])
    try:
        for l in range(2):
            c, s = kv.state_view(l)
            assert tuple(c.shape) == (5, [27, 8][l]) and tuple(s.shape) == (5, [4099, 7][l])
            assert not bool(c.any()) and not bool(s.any())
        _fill_host(kv, np.random.default_rng(1))
        kv.alloc_state(3, 16, [], [12], [40])  # re-callable: frees first, new shape, zeroed
        c, s = kv.state_view(0)
        assert tuple(c.shape) == (3, 12) and not bool(c.any()) and not bool(s.any())
        with pytest.raises(b.SlotKVError):
            kv.state_view(1)
        with pytest.raises(b.SlotKVError):
            kv.layer_view(0)  # no attention layer in this allocation
    finally:
        kv.close()


def test_offsets_match_oracle_and_address_the_buffers():
    conv_lens, ssm_lens = [27, 8, 3], [4099, 10000, 7]
    n_slots = 6
    kv = _handle(n_slots, conv_lens, ssm_lens, kv_dims=[128], slot_ctx=32)
    try:
        for l in range(3):
            cp = b.slot_state_ptrs(kv.h, l)
            for s in range(n_slots):
                oc = kv.conv_offset_bytes(l, s)
                os_ = kv.ssm_offset_bytes(l, s)
                assert oc == oracle.slot_state_offset_bytes(s, conv_lens[l])
                assert os_ == oracle.slot_state_offset_bytes(s, ssm_lens[l])
                # the view's row s starts at the offset the library reports
                cv, sv = kv.state_view(l)
                assert cv[s].data_ptr() == cp[1] + oc and sv[s].data_ptr() == cp[2] + os_
            assert b.slot_conv_offset_bytes(kv.h, l, n_slots)[0] == b.SLOT_KV_ERANGE
            assert b.slot_ssm_offset_bytes(kv.h, l, n_slots)[0] == b.SLOT_KV_ERANGE
        assert b.slot_conv_offset_bytes(kv.h, 3, 0)[0] == b.SLOT_KV_EINVAL
        assert b.slot_state_ptrs(kv.h, 3)[0] == b.SLOT_KV_EINVAL
    finally:
        kv.close()


def test_substep_4a_smoke_sentinels():
    # "Forward Cuda", sub-step 4a smoke: with n_slots >= 2, sentinels written
    # through the library's offsets into slot 0 and slot n_slots-1 of the
    # attention KV and of every ssm layer's conv ring and recurrent state
    # survive each other's writes.
    n_slots, slot_ctx, dims, conv_lens, ssm_lens = 2, 8, [64], [5, 24], [33, 4096]
    kv = _handle(n_slots, conv_lens, ssm_lens, kv_dims=dims, slot_ctx=slot_ctx)
    try:
        kbuf, _ = kv.layer_view(0)
        flat = kbuf.reshape(-1)
        first = kv.offset_bytes(0, 0, 0) // 4
        last = kv.offset_bytes(0, n_slots - 1, slot_ctx - 1) // 4
        flat[first:first + dims[0]] = 1.5
        flat[last:last + dims[0]] = -2.5
        for l in range(2):
            for view, off, n in ((kv.state_view(l)[0], kv.conv_offset_bytes, conv_lens[l]),
                                 (kv.state_view(l)[1], kv.ssm_offset_bytes, ssm_lens[l])):
                f = view.reshape(-1)
                a, z = off(l, 0) // 4, off(l, n_slots - 1) // 4
                f[a:a + n] = 3.0 + l
                f[z:z + n] = -4.0 - l
        torch.cuda.synchronize()
        assert bool((flat[first:first + dims[0]] == 1.5).all())
        assert bool((flat[last:last + dims[0]] == -2.5).all())
        for l in range(2):
            for view in kv.state_view(l):
                assert bool((view[0] == 3.0 + l).all()) and bool((view[-1] == -4.0 - l).all())
    finally:
        kv.close()


@pytest.mark.parametrize("slots", [[0], [3, 1, 5], [2, 2], [5, 0, 1, 2, 3, 4], []])
def test_reset_matches_oracle(slots):
    w = wl.state_tiny()
    _say(f"reset {slots} lens {w.conv_state_len} {w.ssm_state_len}")
    kv = _handle(w.n_slots, w.conv_state_len, w.ssm_state_len, kv_dims=[64])
    try:
        rng = np.random.default_rng(90 + len(slots))
        conv, ssm = _fill_host(kv, rng)
        kb, vb = kv.layer_view(0)
        kb.normal_()
        vb.normal_()
        k0, v0 = kb.clone(), vb.clone()
        kv.reset_batch(slots)
        gc, gs = _read_all(kv)
        assert oracle.slot_reset(conv, ssm, slots) == 0
        assert _same_bytes(gc, conv) and _same_bytes(gs, ssm)
        # the attention KV is left alone
        assert bool(torch.equal(kb, k0)) and bool(torch.equal(vb, v0))
    finally:
        kv.close()


def test_single_slot_reset_and_stream_order():
    w = wl.state_tiny()
    kv = _handle(w.n_slots, w.conv_state_len, w.ssm_state_len)
    try:
        conv, ssm = _fill_host(kv, np.random.default_rng(5))
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            # refill slot 4 on the side stream, then reset it on the same stream
            for l in range(len(w.conv_state_len)):
                c, s = kv.state_view(l)
                c[4].fill_(7.0)
                s[4].fill_(7.0)
            kv.reset(4, stream=side)
        side.synchronize()
        gc, gs = _read_all(kv)
        assert oracle.slot_reset(conv, ssm, [4]) == 0
        assert _same_bytes(gc, conv) and _same_bytes(gs, ssm)
    finally:
        kv.close()


def test_reset_errors_write_nothing():
    w = wl.state_tiny()
    kv = _handle(w.n_slots, w.conv_state_len, w.ssm_state_len)
    try:
        conv, ssm = _fill_host(kv, np.random.default_rng(6))
        assert b.slot_reset_batch(kv.h, [1, w.n_slots]) == b.SLOT_KV_ERANGE
        assert b.slot_reset(kv.h, w.n_slots) == b.SLOT_KV_ERANGE
        gc, gs = _read_all(kv)
        assert _same_bytes(gc, conv) and _same_bytes(gs, ssm)
        assert oracle.slot_reset(conv, ssm, [1, w.n_slots]) == oracle.ERANGE
    finally:
        kv.close()
    # attention KV only: the reset validates and leaves the cache alone
    kv = b.SlotKV()
    try:
        kv.alloc(3, 8, [64])
        kb, _ = kv.layer_view(0)
        kb.fill_(2.0)
        kv.reset(2)
        assert b.slot_reset(kv.h, 3) == b.SLOT_KV_ERANGE
        torch.cuda.synchronize()
        assert bool((kb == 2.0).all())
    finally:
        kv.close()


def test_reset_more_slots_than_one_launch():
    # 300 slots and duplicates: two launches of at most 256 slots
    n_slots, conv_lens, ssm_lens = 300, [5, 3], [9, 1030]
    kv = _handle(n_slots, conv_lens, ssm_lens)
    try:
        conv, ssm = _fill_host(kv, np.random.default_rng(7))
        rng = np.random.default_rng(8)
        slots = np.concatenate([rng.permutation(n_slots)[:270], [0, 0, 299]]).astype(np.uint32)
        b.slot_kv_profile_begin(kv.h)
        kv.reset_batch(slots)
        rc, _, launches = b.slot_kv_profile_end(kv.h)
        assert rc == 0
        assert launches == 2
        gc, gs = _read_all(kv)
        assert oracle.slot_reset(conv, ssm, slots) == 0
        assert _same_bytes(gc, conv) and _same_bytes(gs, ssm)
    finally:
        kv.close()


def test_state_admit_full_size_property():
    # The benchmark's workload at full size (36 ssm layers, 64 slots, 5 GB of
    # state), launched as the benchmark launches it: the listed slots read +0.0
    # everywhere and every other slot is bit-identical to before.
    w = wl.state_admit()
    _say(f"state_admit: {w.n_slots} slots, {len(w.conv_state_len)} layers, reset {list(w.slots)}")
    kv = _handle(w.n_slots, w.conv_state_len, w.ssm_state_len)
    try:
        g = torch.Generator(device="cuda")
        g.manual_seed(w.state_seed)
        views = [kv.state_view(l) for l in range(len(w.conv_state_len))]
        for c, s in views:
            c.normal_(generator=g)
            s.normal_(generator=g)
        before = [(c.clone(), s.clone()) for c, s in views]
        kv.reset_batch(w.slots)
        torch.cuda.synchronize()
        keep = torch.ones(w.n_slots, dtype=torch.bool, device="cuda")
        keep[torch.from_numpy(w.slots.astype(np.int64)).cuda()] = False
        for (c, s), (c0, s0) in zip(views, before):
            for x, x0 in ((c, c0), (s, s0)):
                assert bool(torch.equal(x[keep], x0[keep]))
                gone = x[~keep]
                assert bool((gone.view(torch.int32) == 0).all())  # +0.0 bit patterns
    finally:
        kv.close()
