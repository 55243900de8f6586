#!/usr/bin/env python3
"""Benchmark of the batched slot-KV decode-attention step on one MI355X.

One "step" is one pass of the whole hot path over one batch: host validation
and staging, the fused norm + RoPE + KV-write + split-K attention + merge
kernel (``slot_decode_attn``), for every layer of the workload.  Default
workload: 1 layer, 32 query / 8 kv heads of 128, 64 slots x 4096 positions,
B = 64 rows at seeded positions U{1..4095}.

Prints ONE JSON line on stdout:
  value        rows/s (B / step time), inputs resident in HBM
  kv_gbps      algorithmic KV bytes per step / step time, where the KV bytes
               are sum_b (pos_b + 1) * kv_dim * 4 for K and again for V
  roofline     the fused kernel's achieved GB/s vs 8 TB/s: KV bytes per
               launch / mean launch time, the time from HIP events recorded
               on the launch stream around the timed region (K steps back to
               back, so it also holds the short gaps between launches);
               beside it the mean of per-launch event pairs (which also span
               the dispatch in front of each launch), the launch time with
               L2 and the Infinity Cache emptied before every step, the
               rocprofv3 kernel average and the HBM traffic from rocprofv3
               counters, the last two only when the committed records were
               taken from the current kernel sources
  cpu_baseline the CPU oracle on the host over rows of the same step: one
               thread, and as many threads as the job's CPU share

    python bench.py [--steps K] [--warmup W] [--workload mid]

With --workload prefill_prompt or prefill_chunk it measures the slot prefill
instead (one slot_prefill_attn call per step: the norm / RoPE / KV-write
kernel and the causal attention kernel on the matrix cores):
  value        prompt tokens/s
  roofline     the attention kernel's f32 matrix-core rate (attention flops /
               mean kernel time from the library's HIP events) vs the
               157.3 TFLOP/s dense f32 MFMA peak
  cpu_baseline the CPU oracle's prefill over the first tokens of the prompt

With --workload verify_mid it measures the multi-row verify (one
slot_verify_attn call per step: 4 rows for each of 64 sequences):
  value        rows/s
  roofline     KV bytes (each sequence's keys 0..pos0+k-1, K and V, once) /
               mean attention-kernel time vs 8 TB/s

With --workload state_admit it measures the reset of reused slots on admit
(one slot_reset_batch call per step: 8 slots of a 36-ssm-layer state):
  value        slot resets/s
  roofline     bytes zeroed (every listed slot's conv ring and recurrent state)
               / mean reset-kernel time vs 8 TB/s
  cpu_baseline the CPU oracle's reset of the same slots' state in host memory
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn rows/sec and achieved KV HBM GB/s (% of peak) at B=64, ctx 4096"
HBM_PEAK_GBPS = 8000.0
MFMA_F32_PEAK_TFLOPS = 157.3
PREFILL_METRIC = "slot prefill tokens/s and attention TFLOP/s (f32 matrix cores)"
VERIFY_METRIC = "multi-row verify rows/s and achieved KV HBM GB/s (% of peak)"
STATE_METRIC = "slot resets/s on admit and achieved HBM write GB/s (% of peak)"
CSRC = os.path.join(ROOT, "sequence_slot_kv_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "slot_kv_kernels.hip")
PREFILL_SRC = os.path.join(CSRC, "slot_kv_prefill.hip")
STATE_SRC = os.path.join(CSRC, "slot_kv_state.hip")
DEVICE_H = os.path.join(CSRC, "slot_kv_device.h")
# launch-shaping constants (chunk size, waves per workgroup, row tables) that
# every kernel is built with
INTERNAL_H = os.path.join(CSRC, "slot_kv_internal.h")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_counters.json")
TRACE_RECORD = os.path.join(ROOT, "profiles", "kernel_trace.json")



def gc_off():
    """Warm-up and timed passes run with Python's cyclic collector off, after
    one full collection: a collection of the interpreter's objects (tens of
    milliseconds with torch loaded) landing in the timed region would stall
    the launch loop, and when it lands depends on everything allocated
    before.  The caller turns it back on after its last timed pass."""
    gc.collect()
    gc.disable()

def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(src: str = KERNEL_SRC) -> str:
    """Hash of a kernel's source file and of the internal headers it is built
    with: a profiler record stays valid only while all are unchanged."""
    h = hashlib.sha256()
    for path in (src, INTERNAL_H, DEVICE_H):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _record(path: str, workload: str, src: str):
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_sha256_16") != kernel_hash(src):
        return None
    return entry


def measured_traffic(workload: str, src: str = KERNEL_SRC):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter record, or None when there is none for this
    workload or the kernel source `src` changed since it was taken."""
    entry = _record(TRAFFIC_RECORD, workload, src)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def rocprof_kernel_us(workload: str, src: str = KERNEL_SRC):
    """Mean duration (us) of the workload's dominant kernel in the committed
    rocprofv3 kernel trace, or None when the kernel source changed since."""
    entry = _record(TRACE_RECORD, workload, src)
    return None if entry is None else entry.get("avg_us")


def cpu_share() -> tuple:
    """(threads for the multi-threaded oracle leg, CPUs visible, where the
    count comes from): the CPUs this process may run on, cut to the job's CPU
    share when the environment states one in OMP_NUM_THREADS."""
    visible = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and 0 < int(share) < visible:
        return int(share), visible, "the job's CPU share, from OMP_NUM_THREADS"
    return visible, visible, "every CPU visible"


def cpu_rows(w, sample_max: int = 8, seed: int = 5):
    """Rows the oracle is timed on: every row of the 64-row workload, else a
    seeded sample that holds the longest and the shortest row."""
    import numpy as np
    if w.B <= 64 and len(w.layers) == 1:
        return list(range(w.B)), False
    rng = np.random.default_rng(seed)
    pick = {int(np.argmax(w.positions)), int(np.argmin(w.positions))}
    rest = [i for i in range(w.B) if i not in pick]
    pick.update(int(i) for i in rng.choice(rest, size=min(sample_max - 2, len(rest)),
                                           replace=False))
    return sorted(pick), True


def cpu_baseline(w, rows, sampled, hist, target_s: float = 6.0):
    """The oracle on (row, layer) tasks of one step, rows given, timed twice:
    on one thread, then on the job's CPU share of threads (ctypes releases the
    GIL, so the threads run in parallel); each leg repeats the tasks until
    about target_s seconds of wall time have passed."""
    import oracle
    tasks = [(bi, l) for bi in rows for l in range(len(w.layers))]

    def one(t):
        bi, l = t
        L, li = w.layers[l], w.inputs[l]
        hk, hv = hist[(bi, l)]
        oracle.decode_row(L, int(w.positions[bi]), li.q[bi], li.k_new[bi], li.v_new[bi], hk, hv)

    def leg(threads, batch):
        passes, t0 = 0, time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            while True:
                list(ex.map(one, tasks * batch))
                passes += batch
                wall = time.perf_counter() - t0
                if wall >= target_s:
                    return passes, wall

    n_threads, visible, why = cpu_share()
    keys = sum(int(w.positions[bi]) + 1 for bi in rows)
    kv_bytes = sum(keys * L.kv_dim * 8 for L in w.layers)  # per pass of every row and layer
    p1, t1 = leg(1, 1)
    # several passes per submission, about a quarter of the leg each, so that
    # the threads rarely wait on the longest row at the end of a pass
    batch = max(1, round(target_s / 4 * n_threads / (t1 / p1)))
    pn, tn = leg(n_threads, batch)
    what = (f"a seeded sample of {len(rows)} of the step's {w.B} rows (the longest and shortest "
            f"among them)" if sampled else f"all {w.B} rows of the step")
    if len(w.layers) > 1:
        what += f", each through all {len(w.layers)} layers"
    return {"value": len(rows) * pn / tn, "unit": "rows/s", "cores": n_threads, "kind": "oracle",
            "sample": f"{what}; {n_threads} threads ({why}; {visible} CPUs visible): "
                      f"{pn} passes in {tn:.1f} s; 1 thread: {p1} passes in {t1:.1f} s",
            "value_1_thread": len(rows) * p1 / t1, "cores_visible": visible,
            "kv_gbps": kv_bytes * pn / tn / 1e9, "kv_gbps_1_thread": kv_bytes * p1 / t1 / 1e9,
            "sampled": sampled}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mid",
                    choices=["tiny", "mid", "long", "many", "layer_stack", "prefill_prompt",
                             "prefill_chunk", "verify_mid", "state_admit"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel that scales the rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the step shards by "
              "slot with no exchange, so more GPUs are not exercised here", file=sys.stderr)
        sys.exit(2)

    import torch
    from sequence_slot_kv_amd import binding as b
    from sequence_slot_kv_amd import workloads as wl

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.calibrate_copy:
        src = torch.ones(2**28, device="cuda")  # 1 GiB of f32
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB x 5")
        return
    if args.workload.startswith("prefill"):
        return prefill_bench(args, wl.PREFILL_WORKLOADS[args.workload](), b)
    if args.workload.startswith("verify"):
        return verify_bench(args, wl.VERIFY_WORKLOADS[args.workload](), b)
    if args.workload.startswith("state"):
        return state_bench(args, wl.STATE_WORKLOADS[args.workload](), b)
    return decode_bench(args, wl.WORKLOADS[args.workload](), b)


def decode_bench(args, w, b):
    import numpy as np
    import torch
    from sequence_slot_kv_amd import workloads as wl
    n_layers = len(w.layers)
    log(f"[bench] workload {w.name}: B={w.B} n_slots={w.n_slots} slot_ctx={w.slot_ctx} "
        f"layers={n_layers} kv_bytes/step={w.kv_bytes()}")

    kv = b.SlotKV()
    kv.alloc(w.n_slots, w.slot_ctx, w.kv_dims)
    for l, P in enumerate(w.layers):
        kv.set_layer(l, P)
    for l, P in enumerate(w.layers):  # N(0,1) history from seeded device generators
        for which in (0, 1):
            g = torch.Generator(device="cuda")
            g.manual_seed(wl.device_history_seed(w, l, which))
            for s in range(w.n_slots):
                rows = torch.randn((w.slot_ctx, P.kv_dim), generator=g, device="cuda")
                if which == 0:
                    kv.write_rows(l, s, 0, k_src=rows)
                else:
                    kv.write_rows(l, s, 0, v_src=rows)
    torch.cuda.synchronize()
    log("[bench] history filled")

    ins = [tuple(torch.from_numpy(a).cuda() for a in (li.q, li.k_new, li.v_new)) for li in w.inputs]
    outs = [torch.empty_like(x[0]) for x in ins]
    positions, slots = w.positions, w.slots
    stream = torch.cuda.current_stream()  # the library launches on this stream

    def step():
        for l in range(n_layers):
            q, kn, vn = ins[l]
            kv.decode_attn(l, q, kn, vn, positions, slots, out=outs[l], stream=stream)

    gc_off()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, nothing else enqueued; HIP events on the launch
    # stream bracket it
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    t_enq = time.perf_counter()  # the host's share: validation, staging, launch calls
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    region_ms = ev0.elapsed_time(ev1)
    # per-launch event pairs (the library records one around every launch on
    # its stream; the start event sits before the launch, so a pair also
    # spans the dispatch), in a second pass of the same K steps
    rc = b.slot_kv_profile_begin(kv.h)
    assert rc == 0
    for _ in range(args.steps):
        step()
    rc, pair_ms, launches = b.slot_kv_profile_end(kv.h)
    torch.cuda.synchronize()
    assert rc == 0 and launches == args.steps * n_layers
    # and once more with the caches emptied before every step: a 1 GiB
    # write (outside the event pairs) evicts the KV rows from L2 and the
    # 256 MB Infinity Cache, so no launch can be served from there
    flush = torch.empty(2**28, dtype=torch.float32, device="cuda")
    cold_ms = 0.0
    cold_steps = []  # per step: the median and the best are reported too
    for _ in range(args.steps):
        flush.fill_(1.0)
        rc = b.slot_kv_profile_begin(kv.h)
        assert rc == 0
        step()
        rc, ms, n = b.slot_kv_profile_end(kv.h)
        assert rc == 0 and n == n_layers
        cold_ms += ms
        cold_steps.append(ms / n_layers)
    del flush
    torch.cuda.synchronize()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kv_bytes = w.kv_bytes()
    rows_per_s = w.B / (ms_per_step / 1e3)
    kv_gbps = kv_bytes / (ms_per_step / 1e3) / 1e9
    n_launch = args.steps * n_layers
    launch_ms = region_ms / n_launch
    bytes_per_launch = kv_bytes / n_layers
    achieved = bytes_per_launch / (launch_ms / 1e3) / 1e9
    cold_launch_ms = cold_ms / n_launch
    traffic = measured_traffic(w.name)
    prof_us = rocprof_kernel_us(w.name)
    host_us = (t_enq - t0) * 1e6 / args.steps
    log(f"[bench] host enqueue {host_us:.1f} us/step")
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step; fused kernel {launch_ms * 1e3:.1f} us/launch "
        f"(events over the timed region), {achieved:.0f} GB/s; event pairs "
        f"{pair_ms / n_launch * 1e3:.1f} us; {cold_launch_ms * 1e3:.1f} us/launch with caches "
        f"flushed; rocprofv3 record {prof_us}")

    gc.enable()
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's rows and their history, copied to the host only now:
        # a step writes row pos of each row's slot and never rows 0..pos-1,
        # and host work of this size before the timed region has slowed the
        # launch loop that follows it
        cpu_rows_, sampled = cpu_rows(w)
        hist = {}
        for bi in cpu_rows_:
            p = int(w.positions[bi])
            for l, P in enumerate(w.layers):
                if p == 0:
                    z = np.zeros((0, P.kv_dim), np.float32)
                    hist[(bi, l)] = (z, z)
                else:
                    k, v = kv.read_rows(l, int(w.slots[bi]), 0, p)
                    hist[(bi, l)] = (k.cpu().numpy(), v.cpu().numpy())
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(w, cpu_rows_, sampled, hist)

    res = {
        "metric": METRIC, "value": rows_per_s, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "n_slots": w.n_slots, "slot_ctx": w.slot_ctx,
                   "layers": n_layers, "n_heads": w.layers[0].n_heads,
                   "n_kv_heads": w.layers[0].n_kv_heads,
                   "head_dims": sorted({L.head_dim for L in w.layers}), "seed": w.seed,
                   "chunk_keys": b.slot_kv_chunk_keys()},
        "kv_bytes_per_step": kv_bytes, "kv_gbps": kv_gbps,
        "kv_pct_of_hbm_peak": 100.0 * kv_gbps / HBM_PEAK_GBPS,
        "host_enqueue_us_per_step": host_us,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "decode_attn_kernel", "kernel_us": launch_ms * 1e3,
                     "kernel_us_from": "HIP events on the launch stream around the timed "
                                       "region, per launch",
                     "algorithmic_bytes_per_launch": bytes_per_launch,
                     "kernel_us_event_pairs": pair_ms / n_launch * 1e3,
                     "kernel_us_rocprof": prof_us,
                     "kernel_us_caches_flushed": cold_launch_ms * 1e3,
                     "kernel_us_caches_flushed_median": statistics.median(cold_steps) * 1e3,
                     "kernel_us_caches_flushed_best": min(cold_steps) * 1e3,
                     "achieved_caches_flushed": bytes_per_launch / (cold_launch_ms / 1e3) / 1e9},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    kv.close()


def prefill_bench(args, w, b):
    import numpy as np
    import torch
    L, li = w.layer, w.inputs
    log(f"[bench] prefill {w.name}: T={w.T} pos0={w.pos0} slot={w.slot} heads {L.n_heads}/"
        f"{L.n_kv_heads}/{L.head_dim}, attention {w.attn_flops() / 1e9:.1f} GFLOP per step")
    kv = b.SlotKV()
    kv.alloc(w.n_slots, w.slot_ctx, [L.kv_dim])
    kv.set_layer(0, L)
    hist_k = hist_v = np.zeros((0, L.kv_dim), np.float32)
    hist_dev = None  # copied to the host after the timed passes
    if w.pos0:
        g = torch.Generator(device="cuda")
        g.manual_seed(77 + w.seed)
        hk = torch.randn((w.pos0, L.kv_dim), generator=g, device="cuda")
        hv = torch.randn((w.pos0, L.kv_dim), generator=g, device="cuda")
        kv.write_rows(0, w.slot, 0, hk, hv)
        if not args.no_cpu_baseline:
            hist_dev = (hk, hv)
    q, kn, vn = (torch.from_numpy(x).cuda() for x in (li.q, li.k_new, li.v_new))
    out = torch.empty_like(q)

    def step():
        kv.prefill_attn(0, q, kn, vn, w.slot, w.pos0, out=out)

    gc_off()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rc = b.slot_kv_profile_begin(kv.h)
    assert rc == 0
    for _ in range(args.steps):
        step()
    rc, attn_ms, launches = b.slot_kv_profile_end(kv.h)
    torch.cuda.synchronize()
    assert rc == 0 and launches == args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_us = attn_ms / launches * 1e3
    tflops = w.attn_flops() / (attn_us * 1e-6) / 1e12
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, attention kernel {attn_us:.1f} us, "
        f"{tflops:.1f} TFLOP/s")
    if hist_dev is not None:
        hist_k, hist_v = (x.cpu().numpy() for x in hist_dev)

    gc.enable()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the first n tokens of the prompt, run by the oracle in order (the
        # rest of the prompt does not change them)
        n = 1
        while True:
            ck = np.zeros((1, w.pos0 + n, L.kv_dim), np.float32)
            cv = np.zeros_like(ck)
            ck[0, :w.pos0], cv[0, :w.pos0] = hist_k, hist_v
            c0 = time.perf_counter()
            rc, _ = oracle.prefill(L, ck, cv, li.q[:n], li.k_new[:n], li.v_new[:n], 0, w.pos0)
            dt = time.perf_counter() - c0
            assert rc == 0
            if dt >= 2.0 or n >= w.T:
                break
            n = min(w.T, n * 4)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"the first {n} tokens of the prompt in order, {dt:.1f} s on one thread "
                         f"(later tokens attend over more keys, so this overstates the "
                         f"whole prompt's rate)"}
    res = {
        "metric": PREFILL_METRIC, "value": w.T / (ms_per_step / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "pos0": w.pos0, "slot_ctx": w.slot_ctx,
                   "n_heads": L.n_heads, "n_kv_heads": L.n_kv_heads, "head_dim": L.head_dim,
                   "seed": w.seed},
        "attn_flops_per_step": w.attn_flops(),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_F32_PEAK_TFLOPS, "traffic": None,
                     "kernel": "prefill_attn_kernel", "kernel_us": attn_us},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    kv.close()


def verify_bench(args, w, b):
    import numpy as np
    import torch
    L, li = w.layer, w.inputs
    log(f"[bench] verify {w.name}: {len(w.ks)} sequences x {int(w.ks[0])} rows, heads "
        f"{L.n_heads}/{L.n_kv_heads}/{L.head_dim}, KV bytes per step {w.kv_bytes()}")
    kv = b.SlotKV()
    kv.alloc(w.n_slots, w.slot_ctx, [L.kv_dim])
    kv.set_layer(0, L)
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    hist = {}  # per slot, on the device until the timed passes are over
    for s, p0 in zip(w.slots.tolist(), w.pos0.tolist()):
        hk = torch.randn((p0, L.kv_dim), generator=g, device="cuda")
        hv = torch.randn((p0, L.kv_dim), generator=g, device="cuda")
        kv.write_rows(0, s, 0, hk, hv)
        if not args.no_cpu_baseline:
            hist[s] = (hk, hv)
    q, kn, vn = (torch.from_numpy(x).cuda() for x in (li.q, li.k_new, li.v_new))
    out = torch.empty_like(q)

    def step():
        kv.verify_attn(0, q, kn, vn, w.slots, w.pos0, w.ks, out=out)

    gc_off()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rc = b.slot_kv_profile_begin(kv.h)
    assert rc == 0
    for _ in range(args.steps):
        step()
    rc, attn_ms, launches = b.slot_kv_profile_end(kv.h)
    torch.cuda.synchronize()
    assert rc == 0 and launches == args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_us = attn_ms / launches * 1e3
    achieved = w.kv_bytes() / (attn_us * 1e-6) / 1e9
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, attention kernel {attn_us:.1f} us, "
        f"{achieved:.0f} GB/s")
    hist = {s: (hk.cpu().numpy(), hv.cpu().numpy()) for s, (hk, hv) in hist.items()}
    gc.enable()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # whole sequences, in order, until ~10 s of one thread
        c0, done, n_seq = time.perf_counter(), 0, 0
        row_off = [0] + np.cumsum(w.ks.astype(np.int64)).tolist()
        for i in range(len(w.ks)):
            s, p0, k = int(w.slots[i]), int(w.pos0[i]), int(w.ks[i])
            ck = np.zeros((1, p0 + k, L.kv_dim), np.float32)
            cv = np.zeros_like(ck)
            ck[0, :p0], cv[0, :p0] = hist[s]
            r0 = row_off[i]
            rc, _ = oracle.prefill(L, ck, cv, li.q[r0:r0 + k], li.k_new[r0:r0 + k],
                                   li.v_new[r0:r0 + k], 0, p0)
            assert rc == 0
            done += k
            n_seq += 1
            if time.perf_counter() - c0 >= 10.0:
                break
        dt = time.perf_counter() - c0
        cpu = {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"the first {n_seq} sequences ({done} rows) in order, {dt:.1f} s on "
                         f"one thread"}
    res = {
        "metric": VERIFY_METRIC, "value": w.rows / (ms_per_step / 1e3), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n_seq": len(w.ks), "rows_per_seq": int(w.ks[0]),
                   "n_slots": w.n_slots, "slot_ctx": w.slot_ctx, "n_heads": L.n_heads,
                   "n_kv_heads": L.n_kv_heads, "head_dim": L.head_dim, "seed": w.seed},
        "kv_bytes_per_step": w.kv_bytes(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, PREFILL_SRC),
                     "kernel": "split_attn_kernel + split_merge_kernel", "kernel_us": attn_us},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    kv.close()


def state_bench(args, w, b):
    import numpy as np
    import torch
    n_layers = len(w.conv_state_len)
    log(f"[bench] state reset {w.name}: {len(w.slots)} of {w.n_slots} slots, {n_layers} ssm "
        f"layers, {w.bytes_per_slot()} bytes per slot, {w.write_bytes()} bytes per step")
    kv = b.SlotKV()
    kv.alloc_state(w.n_slots, 1, [], w.conv_state_len, w.ssm_state_len)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.state_seed)
    for l in range(n_layers):
        for view in kv.state_view(l):
            view.normal_(generator=g)
    torch.cuda.synchronize()

    def step():
        kv.reset_batch(w.slots)

    gc_off()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rc = b.slot_kv_profile_begin(kv.h)
    assert rc == 0
    for _ in range(args.steps):
        step()
    rc, k_ms, launches = b.slot_kv_profile_end(kv.h)
    torch.cuda.synchronize()
    assert rc == 0 and launches == args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    k_us = k_ms / launches * 1e3
    achieved = w.write_bytes() / (k_us * 1e-6) / 1e9
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, reset kernel {k_us:.1f} us, "
        f"{achieved:.0f} GB/s")
    kv.close()
    gc.enable()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the oracle's reset of the same slots, each held in its own host
        # state (one slot per entry, so only the listed slots are allocated)
        n = len(w.slots)
        conv = [np.ones((n, c), np.float32) for c in w.conv_state_len]
        ssm = [np.ones((n, s_), np.float32) for s_ in w.ssm_state_len]
        idx = np.arange(n, dtype=np.uint32)
        c0, reps = time.perf_counter(), 0
        while True:
            assert oracle.slot_reset(conv, ssm, idx) == 0
            reps += 1
            if time.perf_counter() - c0 >= 10.0:
                break
        dt = time.perf_counter() - c0
        cpu = {"value": reps * n / dt, "unit": "slot resets/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} resets of {n} slots ({w.write_bytes()} bytes each) in host "
                         f"memory, {dt:.1f} s on one thread"}
    res = {
        "metric": STATE_METRIC, "value": len(w.slots) / (ms_per_step / 1e3),
        "unit": "slot resets/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "n_reset": len(w.slots), "n_slots": w.n_slots,
                   "n_ssm_layers": n_layers, "conv_state_len": w.conv_state_len[0],
                   "ssm_state_len": w.ssm_state_len[0], "seed": w.seed},
        "write_bytes_per_step": w.write_bytes(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, STATE_SRC),
                     "kernel": "state_reset_kernel", "kernel_us": k_us},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
