"""Batch-level invariants of the HIP decode step at full size, through the C ABI.

"Forward Cuda Gemma", decodeBatch: each row writes its new K/V at its own
slot and position and attends over that slot's positions 0..pos only, and
the batched step is the per-row loop fused ("the looped form ... is already
correct for mixed positions"); "Forward Cuda": the serial per-sequence
reference of the batch harness, and a reused slot that is never read past
its positions.  For the 64-row, long-context, many-short and 8-layer (with
sinks) workloads:
  - exactly the B written rows of every layer change, bit for bit against a
    device snapshot taken just before the step, and each written V row holds
    v_new's bytes;
  - a second run of the step gives the same bits;
  - every row equals its own B = 1 call bit for bit, and a permuted batch
    gives the permuted rows bit for bit (the result of a row does not depend
    on the rest of the batch).
Values against the oracle are checked by test_gpu_parity.py; these checks
need no oracle, since each side of every comparison is a run of the kernel.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from sequence_slot_kv_amd import workloads as wl  # noqa: E402

from _gpu_util import device_inputs, fill_history_device, handle_for  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(msg):
    print(msg, flush=True)


def changed_rows(buf, snap):
    """(slot, pos) rows whose bits differ (NaN-safe: compares bit patterns)."""
    diff = (buf.view(torch.int32) != snap.view(torch.int32)).any(dim=-1)
    return {tuple(x) for x in diff.nonzero().cpu().tolist()}


def check_exact_writes(kv, w, layer, k_snap, v_snap, v_new):
    kbuf, vbuf = kv.layer_view(layer)
    expect = {(int(s), int(p)) for s, p in zip(w.slots, w.positions)}
    assert changed_rows(kbuf, k_snap) <= expect, f"layer {layer}: stray K writes"
    assert changed_rows(vbuf, v_snap) <= expect, f"layer {layer}: stray V writes"
    sl = torch.from_numpy(w.slots.astype(np.int64)).cuda()
    ps = torch.from_numpy(w.positions.astype(np.int64)).cuda()
    assert torch.equal(vbuf[sl, ps].view(torch.int32), v_new.view(torch.int32)), \
        f"layer {layer}: written V rows are not v_new's bytes"
    # every written K row changed (a new rotated key, not the history value)
    assert changed_rows(kbuf, k_snap) == expect, f"layer {layer}: a K row was not written"


def run_invariants(w, n_serial=None):
    n_layers = len(w.layers)
    kv = handle_for(w)
    for l in range(n_layers):
        fill_history_device(kv, w, l)
    ins = [device_inputs(w, l) for l in range(n_layers)]
    # the history rows at the written positions are N(0,1) values that the
    # step overwrites; snapshot every layer, step, then diff
    outs = []
    for l in range(n_layers):
        k_snap, v_snap = (t.clone() for t in kv.layer_view(l))
        q, kn, vn = ins[l]
        outs.append(kv.decode_attn(l, q, kn, vn, w.positions, w.slots))
        torch.cuda.synchronize()
        check_exact_writes(kv, w, l, k_snap, v_snap, vn)
        del k_snap, v_snap
        torch.cuda.empty_cache()
    _say(f"{w.name}: exact writes ok on {n_layers} layer(s)")
    # the same step again (it rewrites the same rows with the same values)
    for l in range(n_layers):
        q, kn, vn = ins[l]
        assert torch.equal(kv.decode_attn(l, q, kn, vn, w.positions, w.slots), outs[l]), \
            f"{w.name} layer {l}: two runs differ"
    # each row alone
    rows = range(w.B) if n_serial is None else \
        sorted(np.random.default_rng(7).choice(w.B, size=n_serial, replace=False).tolist())
    for l in range(n_layers):
        q, kn, vn = ins[l]
        for bi in rows:
            o1 = kv.decode_attn(l, q[bi:bi + 1].contiguous(), kn[bi:bi + 1].contiguous(),
                                vn[bi:bi + 1].contiguous(), w.positions[bi:bi + 1],
                                w.slots[bi:bi + 1])
            assert torch.equal(o1[0], outs[l][bi]), \
                f"{w.name} layer {l} row {bi} (pos {w.positions[bi]}) differs from its B=1 run"
    _say(f"{w.name}: batch == serial on {len(rows)} rows x {n_layers} layer(s)")
    # a permuted batch
    perm = np.random.default_rng(3).permutation(w.B)
    pt = torch.from_numpy(perm).cuda()
    for l in range(n_layers):
        q, kn, vn = ins[l]
        op = kv.decode_attn(l, q[pt].contiguous(), kn[pt].contiguous(), vn[pt].contiguous(),
                            w.positions[perm], w.slots[perm])
        assert torch.equal(op, outs[l][pt]), f"{w.name} layer {l}: permuted batch differs"
    kv.close()


def test_mid_invariants():
    run_invariants(wl.mid())


def test_many_short_invariants():
    # G = 8 (4-wave workgroups), 26 rows at pos 0
    run_invariants(wl.many_short())


def test_long_context_invariants():
    # head_dim 256, rows of up to 32 chunks merged by their last workgroup
    run_invariants(wl.long_ctx())


def test_layer_stack_invariants():
    # 8 layers alternating head_dim 128 / 256, per-head sinks; 96 GiB of KV
    # plus one layer's snapshot at a time.  The serial check takes a seeded
    # 32 of the 128 rows (a B = 1 call per row and layer); the other checks
    # cover every row.
    run_invariants(wl.layer_stack(), n_serial=32)
