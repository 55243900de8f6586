"""Host logic of the decode kernel's work queue (no GPU).

The decode kernel cuts each row b of a call into ceil((pos_b + 1) / C) key
chunks and each chunk into one unit per kv head; workgroups take the units
in queue order.  Whatever the order, every (row, chunk) must be queued
exactly once, or a part of some row's history would be skipped or counted
twice.  This compiles the library's plain C++ planner (slot_kv_plan.cpp)
with a small driver that walks the queue through the same lookup the kernel
uses (locate_item) and checks coverage and the stated order: every full
chunk, row by row, then each row's shorter last chunk, longest first.

The split-K kernel of prefill / verify maps its workgroups to partial items
the same way (split_item_of_block): the mapping must be a bijection onto the
items, with every group of whole chunk spans before any tile's last group.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_slot_kv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

DRIVER = r"""
#include <cstdio>
#include <vector>
#include "slot_kv_internal.h"
int main() {
  unsigned n, chunk;
  if (std::scanf("%u %u", &n, &chunk) != 2) return 2;
  std::vector<uint32_t> pos(n), slot(n);
  for (unsigned b = 0; b < n; ++b) { if (std::scanf("%u", &pos[b]) != 1) return 2; slot[b] = b; }
  static slotkv::LaunchRows rows;
  slotkv::LaunchWork w = slotkv::fill_rows(rows, pos.data(), slot.data(), n, chunk);
  std::printf("%u %u %u\n", w.n_full, w.n_items, w.max_chunks);
  for (uint32_t it = 0; it < w.n_items; ++it) {
    uint32_t b, c;
    slotkv::locate_item(rows, n, w.n_full, chunk, it, &b, &c);
    std::printf("%u %u\n", b, c);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    d = tmp_path_factory.mktemp("plan")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", INCLUDE, "-I", CSRC, str(src),
                    os.path.join(CSRC, "slot_kv_plan.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)

    def run(positions, chunk):
        inp = f"{len(positions)} {chunk}\n" + " ".join(str(int(p)) for p in positions) + "\n"
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
        lines = r.stdout.split("\n")
        n_full, n_items, max_chunks = map(int, lines[0].split())
        items = [tuple(map(int, ln.split())) for ln in lines[1:1 + n_items]]
        return n_full, max_chunks, items
    return run


def check_plan(positions, chunk, run):
    positions = np.asarray(positions, dtype=np.int64)
    n_full, max_chunks, items = run(positions, chunk)
    n_chunks = positions // chunk + 1
    tail = (positions + 1) % chunk
    # coverage: every (row, chunk) exactly once
    want = sorted((b, c) for b in range(len(positions)) for c in range(n_chunks[b]))
    assert sorted(items) == want
    assert max_chunks == (n_chunks.max() if len(positions) else 0)
    assert n_full == int(((positions + 1) // chunk).sum())
    full, late = items[:n_full], items[n_full:]
    # full chunks: row-major, each row's chunks in order
    assert full == sorted(full)
    for b, c in full:
        assert (c + 1) * chunk <= positions[b] + 1
    # then every partial last chunk, longest first (ties in row order)
    for b, c in late:
        assert c == n_chunks[b] - 1 and tail[b] > 0
    assert [b for b, _ in late] == sorted((b for b, _ in late), key=lambda b: (-tail[b], b))


def test_plan_mixed_lengths(planner):
    rng = np.random.default_rng(11)
    pos = np.floor(np.exp(rng.uniform(0, np.log(32768), 16))).astype(np.int64).clip(1, 32767)
    for C in (512, 1024):
        check_plan(pos, C, planner)


def test_plan_uniform_rows(planner):
    rng = np.random.default_rng(12)
    for C in (512, 1024):
        check_plan(rng.integers(1, 4096, 64), C, planner)


def test_plan_edges(planner):
    # pos 0, exact multiples of the chunk (no partial chunk), one key short
    # of a multiple, the largest launch
    check_plan([0, 511, 512, 1023, 8 * 512 - 1, 8 * 512, 9 * 512 - 1, 9 * 512, 65535], 512, planner)
    check_plan([0], 512, planner)
    rng = np.random.default_rng(13)
    check_plan(rng.integers(0, 1 << 17, 256), 512, planner)
    check_plan(rng.integers(0, 64, 256), 64, planner)


SPLIT_DRIVER = r"""
#include <cstdio>
#include "slot_kv_internal.h"
using namespace slotkv;
int main() {
  unsigned n, G, hkv, sk;
  if (std::scanf("%u %u %u %u", &n, &G, &hkv, &sk) != 4 || n > kMaxSeqPerLaunch) return 2;
  static PrefillSeqs s;
  uint32_t items = 0;
  for (unsigned i = 0; i < n; ++i) {
    if (std::scanf("%u %u", &s.pos0[i], &s.len[i]) != 2) return 2;
    const uint32_t tiles = (s.len[i] * G + 15) / 16;
    s.item_off[i] = items;
    items += tiles * split_groups(s.pos0[i] + s.len[i], sk) * hkv;
  }
  s.item_off[n] = items;
  order_split_groups(s, n, G, hkv, sk);
  std::printf("%u %u\n", items, s.grp_off[n]);
  for (uint32_t b = 0; b < items; ++b) {
    const SplitItem si = split_item_of_block(s, n, items, sk, b);
    // the sequence returned is the one whose items hold the item
    if (si.seq >= n || si.item < s.item_off[si.seq] || si.item >= s.item_off[si.seq + 1]) return 3;
    std::printf("%u\n", si.item);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def split_map(tmp_path_factory):
    d = tmp_path_factory.mktemp("split")
    src = d / "split.cpp"
    src.write_text(SPLIT_DRIVER)
    exe = d / "split"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", INCLUDE, "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)

    def run(seqs, G, hkv, sk):
        inp = f"{len(seqs)} {G} {hkv} {sk}\n" + " ".join(f"{p} {t}" for p, t in seqs) + "\n"
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
        lines = r.stdout.split()
        items, last = int(lines[0]), int(lines[1])
        return items, last, [int(x) for x in lines[2:2 + items]]
    return run


def _groups(keys, sk):
    return ((keys + sk - 1) // sk + 3) // 4  # four chunks of sk keys per group


def test_split_item_mapping(split_map):
    rng = np.random.default_rng(21)
    for G, hkv, sk in ((4, 8, 256), (8, 4, 512), (1, 2, 256), (2, 8, 1024)):
        seqs = [(int(rng.integers(0, 40000)), int(rng.integers(1, 64 // G + 1)))
                for _ in range(int(rng.integers(1, 129)))]
        items, last, order = split_map(seqs, G, hkv, sk)
        assert sorted(order) == list(range(items)), "a bijection onto the items"
        # which items are a tile's last group, and the keys of each group
        is_last, gkeys, seq_of = [], [], []
        for s, (p0, t) in enumerate(seqs):
            ng = _groups(p0 + t, sk)
            for _ in range((t * G + 15) // 16 * hkv):
                is_last += [g == ng - 1 for g in range(ng)]
                gkeys += [min(p0 + t - g * 4 * sk, 4 * sk) for g in range(ng)]
                seq_of += [s] * ng
        assert len(is_last) == items and sum(is_last) == last
        flags = [is_last[i] for i in order]
        assert flags == sorted(flags), "whole-span groups first, last groups after"
        whole = [i for i in order if not is_last[i]]
        assert whole == sorted(whole), "whole-span groups in item order"
        tail = [i for i in order if is_last[i]]
        keys = [gkeys[i] for i in tail]
        assert keys == sorted(keys, reverse=True), "longest last group first"
        # ties keep sequence order, and a sequence's last groups stay in item order
        ranked = [(-gkeys[i], seq_of[i], i) for i in tail]
        assert ranked == sorted(ranked)


# Tiled prefill / verify launches: the launch-band order of tile groups and
# the even cut of a tile group's keys into chunks (both used on the device
# through the same header).
TILED_DRIVER = r"""
#include <cstdio>
#include "slot_kv_internal.h"
using namespace slotkv;
int main() {
  char what;
  unsigned a, b, c;
  while (std::scanf(" %c %u %u %u", &what, &a, &b, &c) == 4) {
    if (what == 'r') {  // band n_groups (third unused): the order
      for (unsigned f = 0; f < b; ++f) std::printf("%u ", tiled_rank(f, a, b));
    } else {            // n_keys n_ck split_keys: the chunk length
      std::printf("%u", group_chunk_keys(a, b, c));
    }
    std::printf("\n");
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def tiled(tmp_path_factory):
    d = tmp_path_factory.mktemp("tiled")
    src = d / "tiled.cpp"
    src.write_text(TILED_DRIVER)
    exe = d / "tiled"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", INCLUDE, "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)

    def run(queries):
        inp = "".join(f"{q[0]} {q[1]} {q[2]} {q[3]}\n" for q in queries)
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
        return [list(map(int, ln.split())) for ln in r.stdout.strip("\n").split("\n")]
    return run


def test_tiled_rank_bands(tiled):
    cases = [(0, 37), (1, 9), (32, 32), (32, 100), (32, 64), (32, 65), (256, 1000), (7, 3)]
    outs = tiled([("r", band, n, 0) for band, n in cases])
    for (band, n), order in zip(cases, outs):
        assert sorted(order) == list(range(n)), "a permutation"
        if band == 0:
            assert order == list(range(n))
            continue
        for b0 in range(0, n, band):
            seg = list(range(b0, min(b0 + band, n)))
            want = seg[::-1] if (b0 // band) % 2 else seg
            assert order[b0:b0 + band] == want


def test_group_chunk_cut(tiled):
    """Each tile group's n_ck chunks tile its keys in whole 16-key blocks,
    every chunk the merge reads for any tile of the group is one the
    attention kernel wrote, and no chunk exceeds the sequence's own chunk."""
    rng = np.random.default_rng(5)
    cases = []
    for sk in (256, 1024):
        for _ in range(150):
            seq_keys = int(rng.integers(1, 20000))
            n_keys = int(rng.integers(1, seq_keys + 1))  # a tile group's keys
            cases.append((n_keys, (seq_keys + sk - 1) // sk, sk))
    cases += [(1, 1, 256), (16, 1, 256), (17, 2, 256), (256, 1, 256), (257, 2, 256),
              (3584, 4, 1024), (3073, 4, 1024)]
    outs = tiled([("c", *c) for c in cases])
    for (n_keys, n_ck, sk), (ln,) in zip(cases, outs):
        assert ln % 16 == 0 and ln > 0
        assert ln <= ((sk + 15) // 16) * 16 or n_ck * sk < n_keys
        # the kernel's chunks: [c*ln, min((c+1)*ln, n_keys)) for c < n_ck, empty past n_keys
        covered = 0
        for c in range(n_ck):
            lo, hi = c * ln, min((c + 1) * ln, n_keys)
            if lo >= n_keys:
                continue
            assert lo == covered
            covered = hi
        assert covered == n_keys, "every key in exactly one chunk"
        # the merge of a tile with t_keys <= n_keys reads ceil(t_keys / ln) chunks,
        # each one the kernel wrote (start below n_keys, index below n_ck)
        for t_keys in {1, n_keys, max(1, n_keys // 2), max(1, n_keys - 15)}:
            nck = (t_keys + ln - 1) // ln
            assert nck <= n_ck and (nck - 1) * ln < n_keys


# The kernels' table lookups (row of a queue item, sequence of a launch row or
# workgroup, segment of a reset tile) all go through last_le: the last index
# whose non-decreasing key is <= x.
SEARCH_DRIVER = r"""
#include <cstdio>
#include <vector>
#include "slot_kv_internal.h"
int main() {
  unsigned n, x;
  while (std::scanf("%u %u", &n, &x) == 2) {
    std::vector<uint32_t> v(n);
    for (unsigned i = 0; i < n; ++i) if (std::scanf("%u", &v[i]) != 1) return 2;
    std::printf("%u\n", slotkv::last_le(n, x, [&](uint32_t i) { return v[i]; }));
  }
  return 0;
}
"""


def test_last_le_matches_brute_force(tmp_path):
    src = tmp_path / "search.cpp"
    src.write_text(SEARCH_DRIVER)
    exe = tmp_path / "search"
    subprocess.run(["g++", "-O1", "-std=c++17", "-fsanitize=address,undefined", "-I", INCLUDE,
                    "-I", CSRC, str(src), "-o", str(exe)], check=True, capture_output=True)
    rng = np.random.default_rng(17)
    cases = []
    for n in list(range(1, 40)) + [63, 64, 65, 127, 128, 129, 255, 256, 257, 300]:
        for _ in range(6):
            # non-decreasing keys from 0 with plateaus (empty sequences, zero-length rows)
            steps = rng.integers(0, 4, n) * (rng.random(n) < 0.7)
            keys = np.concatenate([[0], np.cumsum(steps[1:])]).astype(np.int64)
            for x in {0, int(keys[-1]), int(keys[-1]) + 5, int(rng.integers(0, keys[-1] + 2)),
                      int(keys[n // 2])}:
                cases.append((keys, x))
    inp = "".join(f"{len(k)} {x} " + " ".join(map(str, k.tolist())) + "\n" for k, x in cases)
    r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
    got = list(map(int, r.stdout.split()))
    want = [int(np.nonzero(k <= x)[0].max()) for k, x in cases]
    assert got == want


SHARE_DRIVER = r"""
#include <cstdio>
#include "slot_kv_internal.h"
int main() {
  unsigned lo, hi;
  while (std::scanf("%u %u", &lo, &hi) == 2) {
    for (uint32_t w = 0; w < slotkv::kSplitChunksPerGroup; ++w) {
      const slotkv::WaveShare s = slotkv::split_wave_share(lo, hi, w);
      std::printf("%u %u %u ", s.k0, s.k1, s.n_blk);
    }
    std::printf("\n");
  }
  return 0;
}
"""


def test_split_wave_shares_tile_the_group(tmp_path):
    """The split-K waves of a workgroup cut its group's keys [lo, hi) evenly:
    the active waves' ranges tile [lo, hi) in order, each of whole 16-key
    blocks but the last, every active wave but the last takes the same
    number of blocks (the last at most that many), and a wave past the keys
    has none (it issues no load)."""
    src = tmp_path / "share.cpp"
    src.write_text(SHARE_DRIVER)
    exe = tmp_path / "share"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", INCLUDE, "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    rng = np.random.default_rng(23)
    groups = [(0, n) for n in range(0, 1100)]
    groups += [(int(lo) * 1024, int(lo) * 1024 + int(rng.integers(0, 1025))) for lo in rng.integers(0, 40, 400)]
    inp = "".join(f"{lo} {hi}\n" for lo, hi in groups)
    r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
    for (lo, hi), line in zip(groups, r.stdout.strip("\n").split("\n")):
        v = list(map(int, line.split()))
        shares = [tuple(v[i:i + 3]) for i in range(0, len(v), 3)]
        pos, blocks = lo, []
        for k0, k1, nb in shares:
            if nb == 0:
                assert k1 == k0 + 1 and k0 >= hi, (lo, hi, shares)
                continue
            assert k0 == pos and k1 > k0 and nb == (k1 - k0 + 15) // 16
            assert (k0 - lo) % 16 == 0
            if k1 != hi:
                assert (k1 - k0) % 16 == 0, (lo, hi, shares)
            pos = k1
            blocks.append(nb)
        assert pos == max(lo, hi), (lo, hi, shares)
        if blocks:
            assert len(set(blocks[:-1])) <= 1 and blocks[-1] <= blocks[0], (lo, hi, shares)
            # even: no more waves idle than a cut of ceil(blocks / waves) each leaves
            total = -(-(hi - lo) // 16)
            per = -(-total // len(shares))
            assert blocks[0] == per and len(blocks) == -(-total // per)
