// slot_kv_internal.h -- types shared by the host runtime and the kernels of
// the slot-KV decode step.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "slot_kv.h"

#ifndef SLOT_KV_CHUNK
#define SLOT_KV_CHUNK 1024  // keys per split-K chunk (a multiple of 64)
#endif
#ifndef SLOT_KV_WG_WAVES
#define SLOT_KV_WG_WAVES 0  // waves of one decode workgroup; 0: by head group size
#endif

namespace slotkv {

// Rows of one launch travel inside the kernel arguments (no staging copy).
constexpr uint32_t kMaxRowsPerLaunch = 256;

// The launch's work items are the (row, chunk) pairs: first every full chunk
// (row-major), then each row's shorter last chunk, longest first.
// The first kFirstItems full-chunk items also have their row listed, so that
// a workgroup finds its first unit (and any unit among them) with one load
// instead of a halving search.
constexpr uint32_t kFirstItems = 256;
struct LaunchRows {
  uint32_t pos[kMaxRowsPerLaunch];    // position written and attended up to (inclusive)
  uint32_t slot[kMaxRowsPerLaunch];   // slot index
  uint32_t full_prefix[kMaxRowsPerLaunch + 1];  // full chunks of the rows before b
  uint8_t tail_row[kMaxRowsPerLaunch];          // rows owning a partial chunk, longest first
  uint8_t first_row[kFirstItems];               // row of full-chunk item i < kFirstItems
};
static_assert(offsetof(LaunchRows, tail_row) % 4 == 0, "tail_row is read through 32-bit words");
static_assert(offsetof(LaunchRows, first_row) % 4 == 0, "first_row is read through 32-bit words");

#if defined(__HIPCC__)
#define SLOTKV_HD __host__ __device__
#else
#define SLOTKV_HD
#endif

// The last index i in [0, n) with key(i) <= x, for key non-decreasing over
// [0, n) and key(0) <= x (n >= 1), by halving.  (Probing 15 indices per round
// instead, two rounds for 256 entries, measured slower in every kernel: the
// extra scalar loads cost more than the shorter chain saves.)
template <class Key>
SLOTKV_HD inline uint32_t last_le(uint32_t n, uint32_t x, Key key) {
  uint32_t lo = 0, hi = n;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (key(mid) <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Byte k of a row table, through its aligned word (on the device the read
// stays a scalar load).
SLOTKV_HD inline uint32_t row_byte(const uint8_t* table, uint32_t k) {
  const uint32_t word = reinterpret_cast<const uint32_t*>(table)[k / 4];
  return (word >> (8 * (k % 4))) & 0xffu;
}

// Row and chunk of queue item `item` (< n_full + the rows' partial chunks).
SLOTKV_HD inline void locate_item(const LaunchRows& rows, uint32_t n_rows, uint32_t n_full,
                                  uint32_t chunk, uint32_t item, uint32_t* row,
                                  uint32_t* chunk_index) {
  if (item < n_full) {
    // full chunk: the last row whose first full chunk is <= item
    const uint32_t b = item < kFirstItems
                           ? row_byte(rows.first_row, item)
                           : last_le(n_rows, item, [&](uint32_t i) { return rows.full_prefix[i]; });
    *row = b;
    *chunk_index = item - rows.full_prefix[b];
  } else {
    *row = row_byte(rows.tail_row, item - n_full);
    *chunk_index = rows.pos[*row] / chunk;  // the partial last chunk
  }
}

// ---------------------------------------------------------------- decode kernel shape
// The decode kernel's per-shape constants, visible to host code so that the
// bound of its LDS score buffer can be checked for every shape and chunk
// size on the CPU.
#ifndef SLOT_KV_LPK
#define SLOT_KV_LPK 0  // lanes per key row; 0: derive from the shape
#endif
#ifndef SLOT_KV_UNROLL
#define SLOT_KV_UNROLL 0  // keys per key group per stage; 0: derive from the shape
#endif
constexpr int kWaveLanes = 64;

// Head shapes whose scores and weighted sums run on the matrix cores
// (v_mfma_f32_16x16x4f32, the kv head's G query heads as the columns of a
// 16-column tile); the others on the vector ALUs.  A bit per (head_dim,
// group): bit 4 * log2(head_dim / 64) + log2(G).  G = 8 at head_dim 64 and
// 128: there the vector form spends most of its time in the per-score
// reductions, while the tile wastes half its columns; with smaller groups
// the tile is mostly padding, and that arithmetic measured slower than the
// vector form under sustained load.  (head_dim 256 would need more
// registers than two waves per SIMD leave.)
#ifndef SLOT_KV_MFMA_SHAPES
#define SLOT_KV_MFMA_SHAPES 0x088u
#endif
constexpr bool decode_mfma(int D, int G) {
  const int di = D == 64 ? 0 : (D == 128 ? 1 : 2);
  const int gi = G == 1 ? 0 : (G == 2 ? 1 : (G == 4 ? 2 : 3));
  return (SLOT_KV_MFMA_SHAPES >> (4 * di + gi)) & 1u;
}
// Waves per workgroup.  Eight waves share a unit's keys in the vector-ALU
// form; G = 8 and the matrix-core form keep four (two workgroups per CU),
// which measured faster there.
constexpr int decode_waves(int D, int G) {
  return SLOT_KV_WG_WAVES ? SLOT_KV_WG_WAVES : (G >= 8 || decode_mfma(D, G) ? 4 : 8);
}
// Lanes per key row: enough that each lane holds about 32 floats of query
// (G heads) and as many of accumulator, at most 16 (one DPP row).
constexpr int decode_lpk(int D, int G) {
  const int want = SLOT_KV_LPK ? SLOT_KV_LPK : G * D / 32;
  int lpk = want < 4 ? 4 : (want > 16 ? 16 : want);
  while (D / (4 * lpk) < 1) lpk /= 2;
  return lpk;
}
// Keys per key group per pipeline stage: about 8 float4 loads per lane, and
// at most 16 scores (G per key) per lane, which leaves G = 8 with 64 floats
// each of query and accumulator room for two waves per SIMD.
constexpr int decode_unroll(int D, int G) {
  const int nv4 = D / (4 * decode_lpk(D, G));
  int u = nv4 >= 8 ? 1 : 8 / nv4;
  while (u > 1 && G * u > 16) u /= 2;
  return SLOT_KV_UNROLL ? SLOT_KV_UNROLL : u;
}
// 16-key tiles per pipeline stage of the matrix-core form: a stage of
// about 16 KB per wave (a wave issues a stage's loads one stage ahead, so
// this sets the bytes it has in flight).
#ifndef SLOT_KV_MFMA_TILES
#define SLOT_KV_MFMA_TILES 0  // 0: by head_dim
#endif
constexpr int decode_mfma_tiles(int D) {
  return SLOT_KV_MFMA_TILES ? SLOT_KV_MFMA_TILES : (D <= 64 ? 2 : 1);
}
// Keys one wave streams per pipeline stage: 16-key tiles on the matrix
// cores, else (64 / lanes per key) key groups of `unroll` keys.
constexpr int decode_step(int D, int G) {
  return decode_mfma(D, G) ? 16 * decode_mfma_tiles(D)
                           : kWaveLanes / decode_lpk(D, G) * decode_unroll(D, G);
}
// Stages per pass that the LDS score buffer of one wave holds: a wave's
// share of a full chunk of `chunk` keys, padded to even as the stage count
// of every pass is.
constexpr int decode_stage_bound(int D, int G, int chunk) {
  const int kpw = chunk / decode_waves(D, G);
  const int step = decode_step(D, G);
  return ((kpw + step - 1) / step + 1) & ~1;
}

// The history keys [begin, begin + len) of a chunk that wave w of nw streams
// when the chunk holds n_keys (<= chunk) history keys: the chunk's stages of
// `step` keys split as evenly as whole stages allow, so a short last chunk
// keeps every wave busy (a full chunk gives each wave chunk / nw keys).
// n_st counts the wave's stages per pass, rounded up to even (the stages past
// n_full whole ones are masked) so that each pass ends in the same buffer.
struct WaveKeys {
  uint32_t begin, len, n_full, n_st;
};
SLOTKV_HD constexpr inline WaveKeys wave_keys(uint32_t n_keys, uint32_t step, uint32_t nw,
                                              uint32_t w) {
  const uint32_t steps = (n_keys + step - 1) / step;
  const uint32_t k0 = steps * w / nw * step;
  const uint32_t k1 = steps * (w + 1) / nw * step;
  WaveKeys r{};
  r.begin = k0 < n_keys ? k0 : n_keys;
  r.len = (k1 < n_keys ? k1 : n_keys) - r.begin;
  r.n_full = r.len / step;
  const uint32_t n_st = r.n_full + (r.len % step != 0 ? 1u : 0u);
  r.n_st = (n_st + 1) & ~1u;
  return r;
}

// Work-queue and split-row counter words are 64-bit: the launch's epoch in
// the bits from kEpochShift up, a count below.  Every launch takes a new
// epoch, larger than any earlier one in the process, and raises a word to
// its own epoch (an atomic max of epoch << kEpochShift, which sets the count
// to zero when the word still holds an older epoch) before the first
// increment it makes; so no launch needs the words cleared, and a word left
// behind by any earlier launch, finished or not, is never counted on.
constexpr uint32_t kEpochShift = 24;
constexpr uint64_t kCountMask = (uint64_t(1) << kEpochShift) - 1;
constexpr uint64_t kMaxEpoch = (uint64_t(1) << (64 - kEpochShift)) - 1;

// Kernel-side parameters of one decode launch (rows 0..n_rows-1 of it).
struct AttnParams {
  float* k_cache;          // layer K buffer [n_slots][slot_ctx][kv_dim]
  float* v_cache;          // layer V buffer
  const float* q;          // [n_rows][n_heads*D]
  const float* k_new;      // [n_rows][kv_dim]
  const float* v_new;      // [n_rows][kv_dim]
  float* out;              // [n_rows][n_heads*D]
  float* part_acc;         // [n_rows][max_chunks][n_heads][D]  unnormalised partial outputs
  float* part_ml;          // [n_rows][max_chunks][n_heads][2]  max (log2 units), sum
  uint64_t* sched;         // [1]: the work queue (epoch | dynamic units handed out)
  uint64_t* counters;      // [n_rows][n_kv_heads]: (epoch | chunks finished) of split rows
  uint64_t epoch_tag;      // this launch's epoch << kEpochShift
  const float* q_norm_w;   // [D]
  const float* k_norm_w;   // [D]
  const float* inv_freq;   // [D/2]
  const float* sinks;      // [n_heads] or nullptr
  uint64_t slot_stride;    // slot_ctx * kv_dim (floats)
  uint32_t kv_dim;
  uint32_t n_kv_heads;
  uint32_t n_heads;
  uint32_t n_rows;
  uint32_t n_full;         // full-chunk items
  uint32_t n_units;        // (full + partial items) * n_kv_heads, below 2^kEpochShift
  uint32_t max_chunks;     // largest chunk count of a row (partial-result stride)
  uint32_t chunk;
  float eps;
  float qk_scale_log2;     // scale * log2(e)
  uint32_t flags;          // SLOT_KV_FLAG_*
};

constexpr uint32_t kArgsMagic = 0x534c4b56u;  // last word of the kernel arguments

struct AttnArgs {
  AttnParams p;
  LaunchRows rows;
  uint32_t magic;  // kArgsMagic; the kernel does nothing if it reads another value
};
static_assert(sizeof(AttnArgs) < 4000, "kernel arguments must stay below 4 KiB");

// Sequences of one prefill / verify launch: sequence i has len[i] token rows
// (rows row_off[i] .. row_off[i+1]-1 of the launch, sequence-major) at
// positions pos0[i] .. pos0[i]+len[i]-1 of slot slot[i].
constexpr uint32_t kMaxSeqPerLaunch = 128;

struct PrefillParams {
  float* k_cache;          // layer K buffer
  float* v_cache;          // layer V buffer
  const float* q;          // [n_rows][n_heads*D]
  const float* k_new;      // [n_rows][kv_dim]
  const float* v_new;      // [n_rows][kv_dim]
  float* rope;             // [n_rows][D][2] (scratch): per query element d the factors A, B
                           // of its norm weight, rotation and scale (prep kernel)
  float* part;             // split-K partials (scratch): acc [n_items][16][D], then
                           // (max, sum) [n_items][16][2]
  float* out;              // [n_rows][n_heads*D]
  const float* q_norm_w;   // [D]
  const float* k_norm_w;   // [D]
  const float* inv_freq;   // [D/2]
  const float* sinks;      // [n_heads] or nullptr
  uint64_t slot_stride;    // slot_ctx * kv_dim (floats)
  uint32_t kv_dim;
  uint32_t n_heads;
  uint32_t n_kv_heads;
  uint32_t n_seq;          // sequences of this launch
  uint32_t n_rows;         // token rows of this launch
  uint32_t n_groups;       // attention workgroups per kv head (all sequences)
  uint32_t n_items;        // key-chunked: partial items of this launch
  uint32_t split_keys;     // keys per chunk (a multiple of 64); 0: the tiled attention
                           // runs over whole key ranges and normalises itself
  float eps;
  float qk_scale_log2;     // scale * log2(e)
  uint32_t flags;          // SLOT_KV_FLAG_*
  uint32_t prep_vpw;       // head vectors per wave of the prep kernel
  uint32_t band;           // tiled: groups per launch band, every other band reversed (0: none)
};

struct PrefillSeqs {
  uint32_t slot[kMaxSeqPerLaunch];
  uint32_t pos0[kMaxSeqPerLaunch];
  uint32_t len[kMaxSeqPerLaunch];
  uint32_t row_off[kMaxSeqPerLaunch + 1];  // first row of each sequence (and the total)
  uint32_t grp_off[kMaxSeqPerLaunch + 1];  // tiled: first workgroup of by_work[k] (per kv head);
                                           // split-K: the last-group items of sequences before i
  uint32_t item_off[kMaxSeqPerLaunch + 1]; // key-chunked: first partial item of each sequence
  uint32_t last_off[kMaxSeqPerLaunch + 1]; // split-K: the last-group items of by_work[0..k)
  uint8_t by_work[kMaxSeqPerLaunch];       // tiled: the sequences, most attention work first;
                                           // split-K: longest last group first
};
static_assert(kMaxSeqPerLaunch <= 256, "by_work holds sequence indices in bytes");

struct PrefillArgs {
  PrefillParams p;
  PrefillSeqs s;
  uint32_t magic;  // kArgsMagic; the kernels do nothing if they read another value
};
static_assert(sizeof(PrefillArgs) < 4000, "kernel arguments must stay below 4 KiB");

// Query rows per attention workgroup of a prefill (4 waves x 16 rows).
constexpr uint32_t kPrefillRowsPerGroup = 64;

// Tiled launches: the heaviest-first rank of the workgroup at launch index
// `flat` (< n_groups, per kv head).  Every other band of `band` ranks is
// taken in reverse, so that the workgroups a CU receives at once (about one
// from each band) add up to about the same work; band 0 leaves the order as
// it is.  A permutation of [0, n_groups).
SLOTKV_HD inline uint32_t tiled_rank(uint32_t flat, uint32_t band, uint32_t n_groups) {
  if (band == 0 || (flat / band) % 2 == 0) return flat;
  const uint32_t b0 = flat - flat % band;
  const uint32_t len = n_groups - b0 < band ? n_groups - b0 : band;
  return b0 + len - 1 - (flat - b0);
}

// Key-chunked tiled launches: a sequence's keys give n_ck chunks of
// split_keys, and each tile group cuts its own keys [0, n_keys) into n_ck
// even chunks of whole 16-key blocks, so that the group's workgroups carry
// equal work.  Chunk c covers [c * len, min((c + 1) * len, n_keys)); a
// chunk past n_keys is empty.
#ifndef SLOT_KV_EVEN_CHUNKS
#define SLOT_KV_EVEN_CHUNKS 1
#endif
SLOTKV_HD inline uint32_t group_chunk_keys(uint32_t n_keys, uint32_t n_ck, uint32_t split_keys) {
  return SLOT_KV_EVEN_CHUNKS ? ((n_keys + n_ck - 1) / n_ck + 15) / 16 * 16 : split_keys;
}

// Key-chunked attention.  The keys of a (sequence, kv head) are cut into
// chunks of split_keys keys, and each (chunk, 16-row tile) pair leaves a
// partial result (an item), ordered within a sequence
//   item_off[i] + (chunk * n_kv_heads + j) * n_tiles + tile,
// n_tiles = ceil(len * G / 16), so that neighbouring items read the kv heads
// of the same key rows; a merge kernel then combines each row's chunks.
// Sequences with at most kSplitMaxRows query rows per kv head (a multi-row
// verify) run one wave per item (split-K); longer ones keep the tiled
// workgroups, which are cut into key chunks only when they are too few to
// fill the chip (fewer than kChunkBelowGroups per launch).
constexpr uint32_t kSplitMaxRows = 64;
// Split-K workgroups take kSplitChunksPerGroup consecutive chunks (a build
// setting, 4 by default: one per wave) of one (sequence, kv head, tile),
// ordered item_off[i] + (j * n_tiles + tile) * groups + group, and leave one
// partial each.
#ifndef SLOT_KV_SPLIT_GROUP
#define SLOT_KV_SPLIT_GROUP 4
#endif
constexpr uint32_t kSplitChunksPerGroup = SLOT_KV_SPLIT_GROUP;
// Split-K launches: wave w's share [k0, k1) of a group's keys [g_lo, g_hi)
// (g_hi >= g_lo), cut evenly over the kSplitChunksPerGroup waves in whole
// 16-key blocks, and its block count; a wave past the keys gets k1 = k0 + 1
// and no block.
struct WaveShare {
  uint32_t k0, k1, n_blk;
};
SLOTKV_HD inline WaveShare split_wave_share(uint32_t g_lo, uint32_t g_hi, uint32_t w) {
  const uint32_t per =
      ((g_hi - g_lo + 15) / 16 + kSplitChunksPerGroup - 1) / kSplitChunksPerGroup * 16;
  WaveShare s;
  s.k0 = g_lo + w * per;
  const bool active = s.k0 < g_hi;
  s.k1 = active ? (s.k0 + per < g_hi ? s.k0 + per : g_hi) : s.k0 + 1;
  s.n_blk = active ? (s.k1 - s.k0 + 15) / 16 : 0;
  return s;
}
SLOTKV_HD inline uint32_t split_groups(uint32_t keys, uint32_t split_keys) {
  const uint32_t chunks = (keys + split_keys - 1) / split_keys;
  return (chunks + kSplitChunksPerGroup - 1) / kSplitChunksPerGroup;
}

// Split-K launches: the partial item that workgroup `block` (< n_items)
// computes, and its sequence.  Items stay sequence-major, (kv head, tile) then group, but the
// workgroups take every group of whole chunk spans first, in sequence order,
// and each tile's last group after them, the sequences of longer last groups
// first (seqs.by_work), so that the end of the grid holds the shortest work;
// seqs.grp_off[i] counts the last groups of the sequences before i, and
// seqs.last_off[k] those of by_work[0..k).
struct SplitItem {
  uint32_t item, seq;
};
SLOTKV_HD inline SplitItem split_item_of_block(const PrefillSeqs& seqs, uint32_t n_seq,
                                               uint32_t n_items, uint32_t split_keys,
                                               uint32_t block) {
  const uint32_t n_whole = n_items - seqs.grp_off[n_seq];
  if (block < n_whole) {
    // the sequence: the last i whose first whole-span item is <= block
    const uint32_t lo = last_le(n_seq, block, [&](uint32_t i) {
      return seqs.item_off[i] - seqs.grp_off[i];
    });
    const uint32_t ng = split_groups(seqs.pos0[lo] + seqs.len[lo], split_keys);
    const uint32_t r = block - (seqs.item_off[lo] - seqs.grp_off[lo]);
    return {seqs.item_off[lo] + r / (ng - 1) * ng + r % (ng - 1), lo};
  }
  // the rank k in by_work: the last k with last_off[k] <= f
  const uint32_t f = block - n_whole;
  const uint32_t k = last_le(n_seq, f, [&](uint32_t r) { return seqs.last_off[r]; });
  const uint32_t i = seqs.by_work[k];
  const uint32_t ng = split_groups(seqs.pos0[i] + seqs.len[i], split_keys);
  return {seqs.item_off[i] + (f - seqs.last_off[k]) * ng + ng - 1, i};
}
// Split-K launches, host side: fills seqs.grp_off, seqs.by_work and
// seqs.last_off for split_item_of_block from the sequences' pos0 and len
// (item_off is filled by the caller).  A sequence's last group holds its keys
// past the whole spans of kSplitChunksPerGroup * split_keys.
inline void order_split_groups(PrefillSeqs& seqs, uint32_t n_seq, uint32_t G,
                               uint32_t n_kv_heads, uint32_t split_keys) {
  uint32_t last_keys[kMaxSeqPerLaunch];
  uint32_t last = 0;
  for (uint32_t i = 0; i < n_seq; ++i) {
    seqs.grp_off[i] = last;
    last += (seqs.len[i] * G + 15) / 16 * n_kv_heads;
    const uint32_t keys = seqs.pos0[i] + seqs.len[i];
    last_keys[i] = keys - (split_groups(keys, split_keys) - 1) * split_keys * kSplitChunksPerGroup;
    seqs.by_work[i] = static_cast<uint8_t>(i);
  }
  seqs.grp_off[n_seq] = last;
  // stable insertion sort, longest last group first (n_seq <= kMaxSeqPerLaunch)
  for (uint32_t k = 1; k < n_seq; ++k) {
    const uint8_t v = seqs.by_work[k];
    uint32_t m = k;
    for (; m > 0 && last_keys[seqs.by_work[m - 1]] < last_keys[v]; --m)
      seqs.by_work[m] = seqs.by_work[m - 1];
    seqs.by_work[m] = v;
  }
  last = 0;
  for (uint32_t k = 0; k < n_seq; ++k) {
    seqs.last_off[k] = last;
    last += (seqs.len[seqs.by_work[k]] * G + 15) / 16 * n_kv_heads;
  }
  seqs.last_off[n_seq] = last;
}

#ifndef SLOT_KV_SPLIT_MIN_KEYS
#define SLOT_KV_SPLIT_MIN_KEYS 256
#endif
constexpr uint32_t kSplitMinKeys = SLOT_KV_SPLIT_MIN_KEYS;  // smallest split-K chunk
constexpr uint32_t kMaxSplitItems = 1u << 14; // per launch (bounds the partials)
constexpr uint32_t kChunkBelowGroups = 512;
#ifndef SLOT_KV_CHUNK_TARGET
#define SLOT_KV_CHUNK_TARGET 1024
#endif
constexpr uint32_t kChunkTargetGroups = SLOT_KV_CHUNK_TARGET;

// Launches of a prefill / verify: norm + RoPE + KV write, then the
// attention (tiled, or split-K and merge when `split`).  `before_attn` /
// `after_attn` (hipEvent_t or null) are recorded around the attention
// kernels.  Returns a hipError_t value.
int launch_prefill(const PrefillArgs& a, uint32_t head_dim, uint32_t group, bool split,
                   void* stream, void* before_attn, void* after_attn);

// Validation of one batch (no device access, no allocation).  Returns a
// SLOT_KV_* status.
int check_batch(uint32_t n_slots, uint32_t slot_ctx, const uint32_t* positions,
                const uint32_t* slots, uint32_t B);
// Whether a slot appears twice among slots[0..n) (no allocation).
bool has_duplicate(const uint32_t* slots, uint32_t n);

// Work of one launch over rows [0, n) of positions / slots.
struct LaunchWork {
  uint32_t n_full = 0;      // full-chunk items
  uint32_t n_items = 0;     // full + partial items
  uint32_t max_chunks = 0;  // largest chunk count of a row
};
// Fill the row table of one launch (n <= kMaxRowsPerLaunch).
LaunchWork fill_rows(LaunchRows& rows, const uint32_t* positions, const uint32_t* slots,
                     uint32_t n, uint32_t chunk);

// Launch of the fused decode kernel with `blocks` persistent workgroups;
// `after_decode` (a hipEvent_t or null) is recorded after it.  Returns a
// hipError_t value.
int launch_decode(const AttnArgs& a, uint32_t head_dim, uint32_t group, uint32_t blocks,
                  void* stream, void* after_decode);
// The next launch epoch (1, 2, ...; shared by every handle and device of
// the process, so that it grows on every word it is used with), or 0 once
// kMaxEpoch has been handed out.
uint64_t next_epoch();
// Workgroups of the decode kernel for this shape that are resident at once
// on the current device (0 on error).
uint32_t resident_blocks(uint32_t head_dim, uint32_t group);
bool decode_shape_supported(uint32_t head_dim, uint32_t group);

// ---------------------------------------------------------------- per-slot SSM state
// One [slot][len] f32 buffer of an ssm layer (its conv ring or its recurrent
// state).  The reset kernel cuts each slot's region of a segment into tiles
// of kResetTileUnits 16-byte units; `tile0` is the first tile of this segment
// within one slot's tiles (segments in table order), so a slot's tiles are
// [0, tiles_per_slot) and segment k holds [tile0_k, tile0_{k+1}).
constexpr uint32_t kResetThreads = 256;
constexpr uint32_t kResetUnitsPerThread = 2;
constexpr uint32_t kResetTileUnits = kResetThreads * kResetUnitsPerThread;  // 8 KiB
constexpr uint32_t kMaxResetPerLaunch = 256;

struct StateSeg {
  float* base;    // device buffer [n_slots][len]
  uint64_t len;   // floats per slot
  uint32_t tile0; // first tile of this segment in a slot's tile range
  uint32_t pad;
};

// Tiles covering one slot's region of `len` floats wherever it starts: the
// region spans at most ceil((len + 3) / 4) 16-byte units.
inline uint64_t reset_tiles(uint64_t len) {
  const uint64_t units = (len + 3) / 4 + (len ? 1 : 0);
  return (units + kResetTileUnits - 1) / kResetTileUnits;
}

struct ResetArgs {
  const StateSeg* segs;     // device table, n_seg entries
  uint32_t n_seg;
  uint32_t tiles_per_slot;  // tile0 of a one-past-the-end segment
  uint32_t n;               // slots in this launch
  uint32_t slots[kMaxResetPerLaunch];
};

// Zeroes the regions of a.slots[0..n) in every segment: n * tiles_per_slot
// workgroups.  `before` / `after` (hipEvent_t or null) are recorded around the
// kernel.  Returns a hipError_t value.
int launch_state_reset(const ResetArgs& a, void* stream, void* before, void* after);

}  // namespace slotkv
