"""Helpers of the GPU tests: set a workload up on the device through the C ABI
and run the oracle on exactly the rows a test checks.  History K/V that a test
compares against is read back from the device BEFORE the decode call, so the
oracle's inputs are the seeded generator's values, never a kernel's output."""
import numpy as np
import torch

import oracle
from sequence_slot_kv_amd import binding as b
from sequence_slot_kv_amd import workloads as wl

ATOL, RTOL = 1e-4, 1e-5  # |gpu - oracle| <= ATOL + RTOL * |oracle|


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref) - (ATOL + RTOL * np.abs(ref))
    worst = int(np.argmax(err))
    assert err.max() <= 0, (f"{what}: max violation {err.max():.3e} at {worst}: "
                            f"gpu {gpu.flat[worst]!r} oracle {ref.flat[worst]!r}")


def handle_for(w: wl.Workload, layers=None):
    kv = b.SlotKV()
    kv.alloc(w.n_slots, w.slot_ctx, w.kv_dims)
    for l in (range(len(w.layers)) if layers is None else layers):
        kv.set_layer(l, w.layers[l])
    return kv


def upload_history(kv, layer, hk: np.ndarray, hv: np.ndarray):
    for s in range(hk.shape[0]):
        kv.write_rows(layer, s, 0, torch.from_numpy(hk[s]).cuda(), torch.from_numpy(hv[s]).cuda())
    torch.cuda.synchronize()


def fill_history_device(kv, w: wl.Workload, layer: int):
    """N(0,1) history for every slot of one layer from seeded torch generators."""
    kd = w.layers[layer].kv_dim
    for which in (0, 1):
        g = torch.Generator(device="cuda")
        g.manual_seed(wl.device_history_seed(w, layer, which))
        for s in range(w.n_slots):
            rows = torch.randn((w.slot_ctx, kd), generator=g, device="cuda", dtype=torch.float32)
            if which == 0:
                kv.write_rows(layer, s, 0, k_src=rows)
            else:
                kv.write_rows(layer, s, 0, v_src=rows)
    torch.cuda.synchronize()


def snapshot_rows(kv, layer, slot, n):
    """Rows 0..n-1 of one slot as host arrays (K, V)."""
    if n == 0:
        kd = kv.kv_dims[layer]
        return np.zeros((0, kd), np.float32), np.zeros((0, kd), np.float32)
    k, v = kv.read_rows(layer, slot, 0, n)
    torch.cuda.synchronize()
    return k.cpu().numpy(), v.cpu().numpy()


def device_inputs(w: wl.Workload, layer: int):
    li = w.inputs[layer]
    return (torch.from_numpy(li.q).cuda(), torch.from_numpy(li.k_new).cuda(),
            torch.from_numpy(li.v_new).cuda())


def oracle_rows(w: wl.Workload, layer: int, rows, hist):
    """Oracle (k_written, v_written, out) for batch rows `rows`; hist[b] is the
    (K, V) history snapshot of row b's slot, rows 0..pos-1."""
    L, li = w.layers[layer], w.inputs[layer]
    res = {}
    for bi in rows:
        p = int(w.positions[bi])
        hk, hv = hist[bi]
        res[bi] = oracle.decode_row(L, p, li.q[bi], li.k_new[bi], li.v_new[bi], hk, hv)
    return res


def sample_rows(w: wl.Workload, n: int, seed: int):
    """A seeded sample of batch rows that always holds the longest and the
    shortest row."""
    rng = np.random.default_rng(seed)
    pos = w.positions
    pick = {int(np.argmax(pos)), int(np.argmin(pos))}
    rest = [i for i in range(w.B) if i not in pick]
    pick.update(int(i) for i in rng.choice(rest, size=min(n, len(rest)), replace=False))
    return sorted(pick)
