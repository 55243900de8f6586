"""Address and undefined-behaviour sanitizer builds of the host-side C and C++
(no GPU).

- The CPU oracle (oracle/slot_kv_oracle.c) is rebuilt with
  -fsanitize=address,undefined and every oracle pin test runs against that
  build in a child interpreter (the oracle loader takes the library path
  from SLOT_KV_ORACLE_LIB; the sanitizer runtime is preloaded, since the
  interpreter itself is not instrumented).  Any invalid access, overflow or
  other undefined behaviour ends the run with an error.
- The decode planner (sequence_slot_kv_amd/csrc/slot_kv_plan.cpp: batch
  validation, the split-K row table and the queue lookup the kernel uses)
  and the per-wave key split of the shared header are rebuilt the same way
  and driven over the work-queue and shape cases of test_queue_plan.py and
  test_decode_shape.py.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_slot_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
PIN_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_prefill_pins.py",
             "tests/test_oracle_conventions.py", "tests/test_oracle_state_pins.py"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded into this process tree")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's address sanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", *SAN, "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", "-Wall", "-Wextra", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "slot_kv_oracle.c"), "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=runtime, SLOT_KV_ORACLE_LIB=str(lib), **SAN_ENV)
    # -s: a sanitizer report goes straight to the child's stderr (captured
    # output would be lost when the report ends the process)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PIN_TESTS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail
    assert "runtime error" not in tail  # UBSan's report line


def _build(tmp_path, name, driver, extra_sources=()):
    src = tmp_path / f"{name}.cpp"
    src.write_text(driver)
    exe = tmp_path / name
    subprocess.run(["g++", *SAN, "-std=c++17", "-I", INCLUDE, "-I", CSRC, str(src),
                    *extra_sources, "-o", str(exe)], check=True, capture_output=True)
    return exe


def test_planner_under_asan_ubsan(tmp_path):
    import test_queue_plan as qp
    exe = _build(tmp_path, "plan", qp.DRIVER, [os.path.join(CSRC, "slot_kv_plan.cpp")])
    env = dict(os.environ, **SAN_ENV)

    def run(positions, chunk):
        inp = f"{len(positions)} {chunk}\n" + " ".join(str(int(p)) for p in positions) + "\n"
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, env=env)
        assert r.returncode == 0, r.stderr[-3000:]
        lines = r.stdout.split("\n")
        n_full, n_items, max_chunks = map(int, lines[0].split())
        items = [tuple(map(int, ln.split())) for ln in lines[1:1 + n_items]]
        return n_full, max_chunks, items

    rng = np.random.default_rng(13)
    qp.check_plan([0, 511, 512, 1023, 8 * 512 - 1, 8 * 512, 9 * 512 - 1, 9 * 512, 65535], 512,
                  run)
    qp.check_plan([0], 512, run)
    qp.check_plan(rng.integers(0, 1 << 17, 256), 512, run)  # a full 256-row table
    qp.check_plan(rng.integers(0, 64, 256), 64, run)
    pos = np.floor(np.exp(rng.uniform(0, np.log(32768), 16))).astype(np.int64).clip(1, 32767)
    qp.check_plan(pos, 1024, run)


def test_split_map_and_shapes_under_asan_ubsan(tmp_path):
    import test_decode_shape as ds
    import test_queue_plan as qp
    env = dict(os.environ, **SAN_ENV)
    exe = _build(tmp_path, "shape", ds.DRIVER)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr[-3000:]
    exe = _build(tmp_path, "split", qp.SPLIT_DRIVER)
    rng = np.random.default_rng(21)
    for G, hkv, sk in ((4, 8, 256), (8, 4, 512), (1, 2, 256)):
        seqs = [(int(rng.integers(0, 40000)), int(rng.integers(1, 64 // G + 1)))
                for _ in range(128)]
        inp = f"{len(seqs)} {G} {hkv} {sk}\n" + " ".join(f"{p} {t}" for p, t in seqs) + "\n"
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, env=env)
        assert r.returncode == 0, r.stderr[-3000:]
        out = r.stdout.split()
        items = int(out[0])
        assert sorted(map(int, out[2:2 + items])) == list(range(items))
