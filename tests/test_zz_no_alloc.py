"""The allocation-free decode entry point (slot_decode_attn_noalloc) against
the allocating one (slot_decode_attn), through the C ABI.

Both run the same kernels; only where the split rows' partials and the work
queue's counters live differs (the library's fixed per-GPU array against the
handle's own buffers).  Two calls in a row, the second with a smaller batch:
the outputs and the written K/V rows must agree bit for bit (so also within
the oracle tolerance), and the small call's rows are also checked against the
oracle.  A call whose partials or counters would not fit the array returns
SLOT_KV_ESCRATCH and writes nothing.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from sequence_slot_kv_amd import binding as b  # noqa: E402
from sequence_slot_kv_amd import workloads as wl  # noqa: E402

from _gpu_util import (assert_close, device_inputs, fill_history_device,  # noqa: E402
                       handle_for, oracle_rows, snapshot_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _both(kv, q, kn, vn, positions, slots, noalloc_first):
    """Runs both entry points on the same inputs, in the given order; returns
    their outputs and checks that the second call rewrote the written rows
    with the same bits."""
    outs = {}
    order = ("noalloc", "alloc") if noalloc_first else ("alloc", "noalloc")
    k_buf, v_buf = kv.layer_view(0)
    snap = None
    for i, which in enumerate(order):
        out = torch.full_like(q, float("nan"))
        fn = b.slot_decode_attn_noalloc if which == "noalloc" else b.slot_decode_attn
        rc = fn(kv.h, 0, q, kn, vn, positions, slots, out)
        assert rc == b.SLOT_KV_OK, f"{which}: {b.slot_kv_strerror(rc)}"
        torch.cuda.synchronize()
        outs[which] = out
        if i == 0:
            snap = (k_buf.clone(), v_buf.clone())
    assert torch.equal(k_buf.view(torch.int32), snap[0].view(torch.int32))
    assert torch.equal(v_buf.view(torch.int32), snap[1].view(torch.int32))
    return outs["alloc"], outs["noalloc"]


def test_noalloc_equals_decode_on_two_calls():
    w = wl.mid()  # 64 rows at positions U{1..4095}: rows of 1 to 4 chunks
    print(f"noalloc: mid B={w.B}", flush=True)
    kv = handle_for(w)
    fill_history_device(kv, w, 0)
    q, kn, vn = device_inputs(w, 0)
    a, n = _both(kv, q, kn, vn, w.positions, w.slots, noalloc_first=False)
    assert torch.equal(a, n), "first call: outputs differ"
    # a smaller second call, the array keeping the first call's contents:
    # the shortest and longest rows, a row of one chunk and a split row
    C = b.slot_kv_chunk_keys()
    pos = w.positions.astype(np.int64)
    sel = sorted({int(np.argmin(pos)), int(np.argmax(pos)), int(np.argmax(pos < C)),
                  int(np.argmax(pos >= 2 * C)), 5})
    print(f"noalloc: second call rows {sel} positions {pos[sel].tolist()}", flush=True)
    hist = {i: snapshot_rows(kv, 0, int(w.slots[r]), int(w.positions[r])) for i, r in enumerate(sel)}
    idx = torch.tensor(sel, device="cuda")
    q2, kn2, vn2 = (x[idx].contiguous() for x in (q, kn, vn))
    a2, n2 = _both(kv, q2, kn2, vn2, w.positions[sel], w.slots[sel], noalloc_first=True)
    assert torch.equal(a2, n2), "second call: outputs differ"
    assert torch.equal(n2, n[idx]), "a row's result depends on the batch"
    # the small call against the oracle (history read back before the call's
    # rows were rewritten: rows 0..pos-1 only, which no call writes)
    sub = wl.Workload(name="sub", seed=w.seed, n_slots=w.n_slots, slot_ctx=w.slot_ctx,
                      layers=w.layers, positions=w.positions[sel], slots=w.slots[sel],
                      inputs=[wl.LayerInputs(w.inputs[0].q[sel], w.inputs[0].k_new[sel],
                                             w.inputs[0].v_new[sel])], theta=w.theta)
    ref = oracle_rows(sub, 0, range(len(sel)), hist)
    got = n2.cpu().numpy()
    for i in range(len(sel)):
        assert_close(got[i], ref[i][2], f"noalloc row {sel[i]}")
    kv.close()


def test_noalloc_rejects_what_does_not_fit():
    # 128 kv heads: the counters of a full launch (1 + 256 * 128 words) pass
    # the array's 256 KiB counter region; nothing may be written.
    rng = np.random.default_rng(5)
    H = Hkv = 128
    D = 64
    L = wl.make_layer(rng, H, Hkv, D, 1e4, False)
    kv = b.SlotKV()
    kv.alloc(2, 64, [L.kv_dim])
    kv.set_layer(0, L)
    q = torch.randn((1, H * D), device="cuda")
    kn = torch.randn((1, L.kv_dim), device="cuda")
    vn = torch.randn((1, L.kv_dim), device="cuda")
    out = torch.full_like(q, 3.0)
    rc = b.slot_decode_attn_noalloc(kv.h, 0, q, kn, vn, [7], [1], out)
    assert rc == b.SLOT_KV_ESCRATCH
    torch.cuda.synchronize()
    assert float(out.min()) == 3.0 and float(out.max()) == 3.0
    assert float(kv.layer_view(0)[0].abs().sum()) == 0.0
    # the allocating entry point takes the same call
    assert b.slot_decode_attn(kv.h, 0, q, kn, vn, [7], [1], out) == b.SLOT_KV_OK
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    kv.close()
