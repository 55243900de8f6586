"""Host checks of the decode kernel's per-wave key split and its LDS bound
(no GPU).

A decode work unit is one chunk of a row's history keys against one kv head;
the waves of a workgroup split the chunk's keys in whole pipeline stages
(wave_keys in slot_kv_internal.h, the function the kernel calls), and each
wave keeps one score per key and head of every stage of its share in an LDS
buffer sized for decode_stage_bound(D, G, chunk) stages.  A wave given more
stages than that would write past its buffer, so this compiles the shared
header with g++ and, for every head shape the kernel is built for, every
chunk size from 256 to 2048 keys in steps of 64 and several build settings
of the shape constants, walks every key count a chunk can hold and every
wave: the waves' ranges must tile the chunk's keys exactly once, each in
whole stages but the last, and no wave's even-padded stage count may pass the
bound.  (The kernel also asserts the bound at compile time for the chunk it
is built with.)
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_slot_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

DRIVER = r"""
#include <cstdio>
#include "slot_kv_internal.h"
using namespace slotkv;
int main() {
  const int Ds[] = {64, 128, 256}, Gs[] = {1, 2, 4, 8};
  long checked = 0;
  for (int chunk = 256; chunk <= 2048; chunk += 64)
    for (int D : Ds)
      for (int G : Gs) {
        const uint32_t nw = decode_waves(D, G), step = decode_step(D, G);
        const uint32_t bound = decode_stage_bound(D, G, chunk);
        if (chunk % nw) continue;  // the kernel requires an even split (asserted there)
        for (uint32_t n = 0; n <= uint32_t(chunk); ++n) {
          uint32_t next = 0;
          for (uint32_t w = 0; w < nw; ++w) {
            const WaveKeys k = wave_keys(n, step, nw, w);
            if (k.begin != next || k.begin % step) {
              std::printf("FAIL tiling D=%d G=%d C=%d n=%u w=%u begin=%u\n", D, G, chunk, n, w,
                          k.begin);
              return 1;
            }
            next = k.begin + k.len;
            const uint32_t whole = k.len / step, part = k.len % step != 0;
            if (k.n_full != whole || k.n_st % 2 || k.n_st < whole + part ||
                k.n_st > whole + part + 1 || (w + 1 < nw && part && next != n)) {
              std::printf("FAIL stages D=%d G=%d C=%d n=%u w=%u len=%u n_st=%u\n", D, G, chunk,
                          n, w, k.len, k.n_st);
              return 1;
            }
            if (k.n_st > bound) {
              std::printf("FAIL bound D=%d G=%d C=%d n=%u w=%u n_st=%u > %u\n", D, G, chunk, n,
                          w, k.n_st, bound);
              return 1;
            }
            ++checked;
          }
          if (next != n) {
            std::printf("FAIL cover D=%d G=%d C=%d n=%u end=%u\n", D, G, chunk, n, next);
            return 1;
          }
        }
      }
  std::printf("ok %ld\n", checked);
  return 0;
}
"""

# build settings of the shape constants: the defaults, then the knobs the
# kernel exposes (waves per workgroup, lanes per key row, keys per group and
# stage, which shapes run on the matrix cores)
SETTINGS = [[], ["-DSLOT_KV_WG_WAVES=2"], ["-DSLOT_KV_WG_WAVES=4"], ["-DSLOT_KV_WG_WAVES=16"],
            ["-DSLOT_KV_LPK=8"], ["-DSLOT_KV_LPK=4"], ["-DSLOT_KV_UNROLL=2"],
            ["-DSLOT_KV_UNROLL=1"], ["-DSLOT_KV_MFMA_SHAPES=0"],
            ["-DSLOT_KV_MFMA_SHAPES=0", "-DSLOT_KV_WG_WAVES=4"], ["-DSLOT_KV_MFMA_SHAPES=0xfff"]]


@pytest.mark.parametrize("flags", SETTINGS, ids=lambda f: " ".join(f) or "default")
def test_wave_split_tiles_chunk_within_score_buffer(flags, tmp_path):
    src = tmp_path / "shape.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "shape"
    subprocess.run(["g++", "-O2", "-std=c++17", *flags, "-I", INCLUDE, "-I", CSRC, str(src),
                    "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")


def test_bound_is_tight_where_it_was_once_too_small():
    # In the vector-ALU form, a 768-key chunk at head_dim 64, G = 1 splits
    # into 24 stages of 32 keys over 8 waves: 3 each, padded to 4.  The
    # unpadded bound (3) was once too small; the bound must be 4 there.
    drv = r"""
#include <cstdio>
#include "slot_kv_internal.h"
int main() {
  std::printf("%d %d %u\n", slotkv::decode_step(64, 1), slotkv::decode_stage_bound(64, 1, 768),
              slotkv::wave_keys(768, slotkv::decode_step(64, 1), 8, 7).n_st);
}
"""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "t.cpp"), os.path.join(d, "t")
        open(src, "w").write(drv)
        subprocess.run(["g++", "-std=c++17", "-DSLOT_KV_MFMA_SHAPES=0", "-I", INCLUDE, "-I", CSRC,
                        src, "-o", exe], check=True, capture_output=True)
        step, bound, n_st = map(int, subprocess.run([exe], capture_output=True, text=True,
                                                    check=True).stdout.split())
    assert (step, bound, n_st) == (32, 4, 4)
