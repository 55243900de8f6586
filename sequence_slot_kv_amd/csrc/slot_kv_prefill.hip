// slot_kv_prefill.hip -- gfx950 kernels of a slot prefill / multi-row verify:
// several token rows per sequence, each sequence in its own slot ("Forward
// Cuda": batched prefill that writes the KV cache into the slot's
// per-sequence region; "Forward Cuda Gemma", prefillBatched, equal to the
// one-token step run over the tokens in order; the other system's batched
// verify of ks[i] consecutive rows for each of n_seqs sequences).
//
// Launches on the caller's stream:
//   prep  one wave per key head of every token row: RMSNorm and RoPE, and
//         the key head and its value row go into the slot; per row, a table
//         of the query heads' norm-weight, rotation and scale factors.
//   attn  causal attention of every row over its slot's positions
//         0 .. pos0+t, now all in the cache; each wave first normalises and
//         rotates its raw query rows with the table.  Many query rows meet
//         each key block, so this is a dense contraction and runs on the
//         matrix cores:
//         v_mfma_f32_16x16x4f32 in its transposed form
//             S^T = K * Q^T   (16 keys x 16 query rows, summed over head_dim)
//             O^T += V^T * P^T (16 head_dim values x 16 rows, summed over keys)
//         With the key order chosen below, the score registers of S^T are
//         exactly the P^T operand of the second product, so no value ever
//         moves between lanes except the per-row max and sum.
#include <hip/hip_runtime.h>

#include "slot_kv_internal.h"

namespace slotkv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kPrepWaves = 4;
constexpr int kAttnWaves = 4;
static_assert(kAttnWaves * 16 == kPrefillRowsPerGroup, "rows per attention workgroup");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;  // tiled attention: max growth absorbed without a rescale

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// The sequence holding launch row `row`: the last i with row_off[i] <= row.
__device__ __forceinline__ uint32_t seq_of_row(const PrefillArgs& a, uint32_t row) {
  // row is wave-uniform.  Lane l tests entries l and 64 + l (both loads in
  // flight together, always inside the table); the count of entries below
  // n_seq at or below row (row_off rises from row_off[0] = 0) is one past
  // the sequence.  One round trip instead of a chain of dependent loads.
  static_assert(kMaxSeqPerLaunch <= 2 * kWave, "two entries per lane");
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t n = a.p.n_seq;
  const uint32_t r0 = a.s.row_off[lane], r1 = a.s.row_off[kWave + lane];
  const uint32_t cnt = __popcll(__ballot(lane < n && r0 <= row)) +
                       __popcll(__ballot(kWave + lane < n && r1 <= row));
  return __builtin_amdgcn_readfirstlane(cnt - 1);
}

// A workgroup takes 4 * prep_vpw key heads of a token row, wave w the heads
// w, w + 4, ...; prep_vpw is 1 for calls of a few hundred rows, so that they
// spread over the whole chip, and larger for long ones.  The workgroup first
// puts the cos / sin of the row's D/2 angles in LDS, and the row's first
// workgroup also writes the row's entry of the query table, from which the
// attention kernels normalise and rotate the row's query heads.  Lane l
// holds elements l*EPL .. l*EPL+EPL-1 of the vector; the RoPE partner
// d +- D/2 of an element sits in lane l ^ 32 with the same angle, and with
// interleaved pairs the partner d ^ 1 is the neighbouring element of the
// lane (lane l ^ 1 when a lane holds one) and the angle that of d / 2.
template <int D>
__global__ void __launch_bounds__(kWave * kPrepWaves) prefill_prep_kernel(const PrefillArgs a) {
  constexpr int EPL = D / kWave;
  __shared__ float cs[D / 2], sn[D / 2];
  if (a.magic != kArgsMagic) return;  // argument block not delivered whole
  const PrefillParams& p = a.p;
  const uint32_t per_wg = kPrepWaves * p.prep_vpw;
  const uint32_t per_row = (p.n_kv_heads + per_wg - 1) / per_wg;
  const uint32_t row = blockIdx.x / per_row;  // < n_rows
  const uint32_t part = blockIdx.x - row * per_row;
  const uint32_t v0 = part * per_wg + threadIdx.x / kWave;
  const uint32_t i = seq_of_row(a, row);
  const uint32_t t = row - a.s.row_off[i];
  const uint32_t pos = a.s.pos0[i] + t;
  const float fpos = static_cast<float>(pos);
  for (uint32_t e = threadIdx.x; e < D / 2; e += kWave * kPrepWaves) {
    const float ang = fpos * p.inv_freq[e];  // one f32 multiply
    float s_, c_;
    sincosf(ang, &s_, &c_);
    sn[e] = s_;
    cs[e] = c_;
  }
  __syncthreads();
  const float one = (p.flags & SLOT_KV_FLAG_NORM_ONE_PLUS_W) ? 1.f : 0.f;
  const bool inter = p.flags & SLOT_KV_FLAG_ROPE_INTERLEAVED;  // uniform
  if (part == 0) {  // workgroup-uniform: the row's query rotation table
    float2* tab = reinterpret_cast<float2*>(p.rope) + static_cast<size_t>(row) * D;
    for (uint32_t d = threadIdx.x; d < D; d += kWave * kPrepWaves) {
      const uint32_t k = inter ? d / 2 : d % (D / 2);            // the angle of d
      const uint32_t pd = inter ? d ^ 1u : (d + D / 2) % D;       // its partner
      const bool first = inter ? (d & 1u) == 0 : d < D / 2;
      const float wa = p.qk_scale_log2 * (one + p.q_norm_w[d]);
      const float wb = p.qk_scale_log2 * (one + p.q_norm_w[pd]);
      tab[d] = make_float2(wa * cs[k], first ? -wb * sn[k] : wb * sn[k]);
    }
  }
  const uint32_t lane = threadIdx.x % kWave;
  const uint64_t at_row = a.s.slot[i] * p.slot_stride + static_cast<uint64_t>(pos) * p.kv_dim;
  for (uint32_t kvh = v0; kvh < min(v0 + per_wg, p.n_kv_heads); kvh += kPrepWaves) {  // wave-uniform
    const float* src = p.k_new + static_cast<size_t>(row) * p.kv_dim + kvh * D;
    float x[EPL];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      x[e] = src[lane * EPL + e];
      ss += x[e] * x[e];
    }
    ss = wave_sum(ss);
    const float rn = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
    float xn[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) xn[e] = x[e] * rn * (one + p.k_norm_w[lane * EPL + e]);
    float y[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float partner;
      bool first;
      uint32_t k;
      if (inter) {
        if constexpr (EPL >= 2) partner = xn[e ^ 1];
        else partner = __shfl_xor(xn[e], 1);
        first = ((lane * EPL + e) & 1u) == 0;
        k = (lane * EPL + e) / 2;
      } else {
        partner = __shfl_xor(xn[e], 32);
        first = lane < 32;
        k = (lane & 31) * EPL + e;
      }
      y[e] = first ? xn[e] * cs[k] - partner * sn[k] : xn[e] * cs[k] + partner * sn[k];
    }
    const uint64_t at = at_row + kvh * D + lane * EPL;
    const float* vsrc = p.v_new + static_cast<size_t>(row) * p.kv_dim + kvh * D + lane * EPL;
    float vw[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) vw[e] = vsrc[e];
    if (p.flags & SLOT_KV_FLAG_V_NORM) {  // uniform: weightless RMSNorm of the value
      float sv = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sv += vw[e] * vw[e];
      const float rv = 1.0f / sqrtf(wave_sum(sv) * (1.0f / D) + p.eps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) vw[e] *= rv;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      p.k_cache[at + e] = y[e];
      p.v_cache[at + e] = vw[e];
    }
  }
}

// The query heads of a row are normalised and rotated by the attention waves
// that use them.  With xn = x * r * (one + w) the normalised query (r the
// reciprocal RMS of the head vector x) and p(d) the RoPE partner of element d
// at the angle a(d), the rotated, scaled element is
//   q[d] = s * (xn[d] cos a(d) -+ xn[p(d)] sin a(d))
//        = r * (x[d] * A[d] + x[p(d)] * B[d]),
//   A[d] = s (one + w[d]) cos a(d),  B[d] = -+ s (one + w[p(d)]) sin a(d),
// minus for the first element of a pair, s = scale * log2(e) (so that the
// scores come out in log2 units).  A and B depend on the row's position and
// the weights only: the prep kernel writes them per row ([row][d] (A, B)), and
// a lane then needs the raw query, its elements' (A, B) and the partners.
// The sum of squares of a query row is spread over lanes l, l ^ 16, l ^ 32 and
// l ^ 48 in both layouts below.
__device__ __forceinline__ float row_rms(const PrefillParams& p, float ss, int D) {
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  return 1.0f / sqrtf(ss * (1.0f / static_cast<float>(D)) + p.eps);
}

// Tiled layout: lane group g holds d = (D/4)*g + i, i < D/4.  With
// rotate-half pairs the partner d +- D/2 is element i of lane l ^ 32; with
// interleaved pairs the partner d ^ 1 is element i ^ 1 of the lane.
template <int D>
__device__ __forceinline__ void tiled_query(const PrefillParams& p, uint32_t row, uint32_t h,
                                            uint32_t g, float (&qv)[D / 4]) {
  constexpr int DQ = D / 4;
  const float* src = p.q + (static_cast<size_t>(row) * p.n_heads + h) * D + DQ * g;
  const f4* tab = reinterpret_cast<const f4*>(p.rope + (static_cast<size_t>(row) * D + DQ * g) * 2);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < DQ; i += 4) {
    const f4 v = *reinterpret_cast<const f4*>(src + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[i + e] = v[e];
      ss += v[e] * v[e];
    }
  }
  const bool inter = p.flags & SLOT_KV_FLAG_ROPE_INTERLEAVED;  // uniform
  const float rn = row_rms(p, ss, D);
  // the table in two halves (the registers of a whole one would spill)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f4 ab[DQ / 4];  // (A, B) of elements 2k and 2k + 1 of this half
#pragma unroll
    for (int k = 0; k < DQ / 4; ++k) ab[k] = tab[hf * DQ / 4 + k];
    if (inter) {
#pragma unroll
      for (int k = 0; k < DQ / 4; ++k) {
        const int i = hf * DQ / 2 + 2 * k;
        const float x0 = qv[i], x1 = qv[i + 1];
        qv[i] = rn * (x0 * ab[k][0] + x1 * ab[k][1]);
        qv[i + 1] = rn * (x1 * ab[k][2] + x0 * ab[k][3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < DQ / 4; ++k) {
        const int i = hf * DQ / 2 + 2 * k;
        const float x0 = qv[i], x1 = qv[i + 1];
        const float p0 = __shfl_xor(x0, 32), p1 = __shfl_xor(x1, 32);
        qv[i] = rn * (x0 * ab[k][0] + p0 * ab[k][1]);
        qv[i + 1] = rn * (x1 * ab[k][2] + p1 * ab[k][3]);
      }
    }
  }
}

// Split-K layout: lane group g holds d = 16v + 4g + e as element 4v + e
// (v < D/16, e < 4).  With rotate-half pairs the partner d +- D/2 is element
// 4(v +- D/32) + e of the same lane; with interleaved pairs element
// 4v + (e ^ 1).
template <int D>
__device__ __forceinline__ void split_query(const PrefillParams& p, uint32_t row, uint32_t h,
                                            uint32_t g, float (&qv)[D / 4]) {
  constexpr int NK = D / 16;
  const float* src = p.q + (static_cast<size_t>(row) * p.n_heads + h) * D + 4 * g;
  const f4* tab = reinterpret_cast<const f4*>(p.rope + (static_cast<size_t>(row) * D + 4 * g) * 2);
  f4 ab[2 * NK];  // (A, B) of elements 4v + 2m and 4v + 2m + 1 at 2v + m
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NK; ++v) {
    const f4 x = *reinterpret_cast<const f4*>(src + 16 * v);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[4 * v + e] = x[e];
      ss += x[e] * x[e];
    }
  }
#pragma unroll
  for (int v = 0; v < NK; ++v) {
    ab[2 * v] = tab[8 * v];
    ab[2 * v + 1] = tab[8 * v + 1];
  }
  const float rn = row_rms(p, ss, D);
  float x[D / 4];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) x[e] = qv[e];
  const bool inter = p.flags & SLOT_KV_FLAG_ROPE_INTERLEAVED;  // uniform
#pragma unroll
  for (int v = 0; v < NK; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float partner = inter ? x[4 * v + (e ^ 1)] : x[(4 * v + e + D / 8) % (D / 4)];
      const f4 t = ab[2 * v + e / 2];
      qv[4 * v + e] = rn * (x[4 * v + e] * t[2 * (e % 2)] + partner * t[2 * (e % 2) + 1]);
    }
  }
}

// A workgroup of four waves takes four consecutive tiles of 16 query rows of
// one sequence and one kv head j; row r of tile k is row R = 16k + r of the
// head group: token R / G of the sequence, query head j*G + R % G.  The
// workgroup walks the key blocks of its last (longest) tile, 16 keys at a
// time: all 256 threads stage a block's K and V rows in LDS
// (double-buffered), then each wave takes its MFMA operands from there.  Lane
// l works on row c = l % 16 and lane group g = l / 16:
//   S^T block:  A = K[key c][d], B = Q[row c][d] with d = (D/4)*g + i for
//               MFMA i < D/4; result lane l, register r: key 4g + r, row c;
//   O^T tile u: MFMA m < 4 sums key 4g + m (A = V[key][d], d = 4c + 64(u/4)
//               + u%4, so that the sixteen lanes of a lane group read 256
//               contiguous bytes of a staged row, free of bank conflicts;
//               B = the score register m); result lane l, register r:
//               d = 16g + 4r + 64(u/4) + u%4, row c.
// So a lane's whole accumulator belongs to its own row.  Workgroup ranks run
// heaviest first: sequences by decreasing work, and inside a sequence its
// last tokens first.  The ranks are launched in bands of one workgroup per
// CU, every other band reversed: the CUs take their first workgroups about
// one from each band, so that each CU's resident set sums to about the same
// work (in plain heaviest-first order the first CU would hold the heaviest
// of every band), and the shortest ones fill in at the end.
constexpr int kLdsPad = 4;  // floats of padding per staged row: rows start 4 banks apart
template <int D>
struct PrefillLds {
  float k[2][16][D + kLdsPad];
  float v[2][16][D + kLdsPad];
};

template <int D, int G, bool CHUNKED>
__global__ void __launch_bounds__(kWave * kAttnWaves) prefill_attn_kernel(const PrefillArgs a) {
  constexpr int DQ = D / 4;   // head_dim values per lane group
  constexpr int TD = D / 16;  // output tiles of 16 head_dim values
  constexpr int NF4 = 16 * D / 4 / (kWave * kAttnWaves);  // staged float4 per thread per block
  static_assert(DQ % 4 == 0 && TD % 4 == 0 && NF4 >= 1, "float4 staging");
  __shared__ __attribute__((aligned(16))) PrefillLds<D> sh;
  if (a.magic != kArgsMagic) return;  // argument block not delivered whole
  const PrefillParams& p = a.p;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid % kWave;
  const uint32_t w = tid / kWave;
  const uint32_t g = lane / 16, c = lane % 16;
  // workgroup -> (kv head, sequence, tile group, key chunk)
  const uint32_t CK = CHUNKED ? p.split_keys : 0;  // 0: one chunk of all keys
  const uint32_t j = blockIdx.x % p.n_kv_heads;
  // the group's rank in the heaviest-first order, in launch bands
  const uint32_t flat = tiled_rank(blockIdx.x / p.n_kv_heads, p.band, p.n_groups);
  const uint32_t lo = last_le(p.n_seq, flat, [&](uint32_t k) { return a.s.grp_off[k]; });
  const uint32_t sq = a.s.by_work[lo];
  const uint32_t T = a.s.len[sq], pos0 = a.s.pos0[sq], row0 = a.s.row_off[sq];
  const uint32_t n_ck = CK ? (pos0 + T + CK - 1) / CK : 1;
  const uint32_t local = a.s.grp_off[lo + 1] - 1 - flat;  // the sequence's last group first
  const uint32_t grp = local / n_ck, chunk = local - grp * n_ck;
  const uint32_t n_tiles = (T * G + 15) / 16;
  // keys up to and including the last token of a tile's rows
  auto tile_keys = [&](uint32_t tl) { return pos0 + min((tl * 16 + 15) / G, T - 1) + 1; };
  // the wave's tile (one past the last tile only helps stage)
  const uint32_t tile = grp * kAttnWaves + w;
  const uint32_t n_keys = tile_keys(min(grp * kAttnWaves + kAttnWaves - 1, n_tiles - 1));
  // the workgroup's keys [k_lo, k_hi): its chunk of the keys of its last tile
  const uint32_t ckg = CK ? group_chunk_keys(n_keys, n_ck, CK) : 0;
  const uint32_t k_lo = chunk * ckg;
  if (CK && k_lo >= n_keys) return;  // workgroup-uniform, before any barrier
  const uint32_t k_hi = CK ? min(k_lo + ckg, n_keys) : n_keys;
  const uint32_t R = tile * 16 + c;
  const uint32_t t = R / G, h = j * G + R % G;
  const uint32_t tq = min(t, T - 1);  // rows past the last token compute on it, unused
  const uint32_t row_pos = pos0 + tq;

  float qv[DQ];  // the wave's query rows, prepared after the first fetch
  const uint64_t slot_base = a.s.slot[sq] * p.slot_stride;
  const float* kbase = p.k_cache + slot_base + j * D;
  const float* vbase = p.v_cache + slot_base + j * D;
  // Staging: float4 f = tid + 256*s of a block is row f / (D/4), column
  // 4 * (f % (D/4)).  Keys past the workgroup's range re-read its last key.
  f4 stk[NF4], stv[NF4];
  auto fetch = [&](f4* st, const float* base, uint32_t kb) {
#pragma unroll
    for (int s = 0; s < NF4; ++s) {
      const uint32_t f = tid + kWave * kAttnWaves * s;
      const uint32_t row = f / (D / 4), col = 4 * (f % (D / 4));
      st[s] = *reinterpret_cast<const f4*>(base + static_cast<size_t>(min(kb + row, k_hi - 1)) *
                                                      p.kv_dim + col);
    }
  };
  auto stage = [&](float (*buf)[D + kLdsPad], const f4* st) {
#pragma unroll
    for (int s = 0; s < NF4; ++s) {
      const uint32_t f = tid + kWave * kAttnWaves * s;
      *reinterpret_cast<f4*>(&buf[f / (D / 4)][4 * (f % (D / 4))]) = st[s];
    }
  };
  // S^T of a staged key block
  auto scores = [&](uint32_t buf) {
    f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f4 ka = *reinterpret_cast<const f4*>(&sh.k[buf][c][DQ * g + i]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], qv[i + e], sc, 0, 0, 0);
    }
    return sc;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f4 o[TD];
#pragma unroll
  for (int u = 0; u < TD; ++u) o[u] = f4{0.f, 0.f, 0.f, 0.f};
  // the block's weights: causal mask, running reference, exponentials
  auto weights = [&](f4 sc, uint32_t kb) {
    // key kb + 4g + r counts iff it is <= the row's position and inside the
    // workgroup's keys (keys >= n_keys are past every row)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (kb + 4 * g + r > row_pos || (CHUNKED && kb + 4 * g + r >= k_hi)) sc[r] = -INFINITY;
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    // m_run is the reference the exponentials are taken against; it moves
    // (rescaling the sum and accumulator) only when a block's max passes it
    // by more than kLazyLog2, so most blocks skip the rescale and every
    // weight stays below 2^kLazyLog2
    const bool up = mb > m_run + kLazyLog2;
    if (__any(up)) {  // wave-uniform
      const float m_new = up ? mb : m_run;
      const float corr = up ? fast_exp2(m_run - m_new) : 1.f;  // 0 from -inf
      l_run *= corr;
#pragma unroll
      for (int u = 0; u < TD; ++u) o[u] *= corr;
      m_run = m_new;
    }
    // finite from key 0 on; a later chunk may hold no key of a row yet
    const float m_use = (CHUNKED && m_run == -INFINITY) ? 0.f : m_run;
    f4 pr;
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - m_use);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    return pr;
  };
  // O^T += V^T P^T
  auto accumulate = [&](uint32_t buf, f4 pr) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int u = 0; u < TD; u += 4) {
        const f4 va = *reinterpret_cast<const f4*>(&sh.v[buf][4 * g + m][4 * c + 16 * u]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[u + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[e], pr[m], o[u + e], 0, 0, 0);
      }
    }
  };

  // Software pipeline over the key blocks b: the pass of block b takes the
  // weights of b (from the scores the previous pass left), the scores of
  // b + 1 and the accumulation of b, so that the matrix cores have
  // independent work while the weights are formed.  K runs one block ahead
  // of V: during pass b, K(b+1) and V(b) are read from LDS while K(b+2) and
  // V(b+1) are fetched into registers, then written into the buffers that
  // K(b) and V(b-1) held (read in the previous pass, before its barrier).
  const uint32_t n_blk = (k_hi - k_lo + 15) / 16;
  // the wave's blocks: those below its tile's last key (none past the last tile)
  const uint32_t wave_keys = tile_keys(tile);
  const uint32_t w_blk =
      tile < n_tiles && wave_keys > k_lo ? min(n_blk, (wave_keys - k_lo + 15) / 16) : 0;
  fetch(stk, kbase, k_lo);
  fetch(stv, vbase, k_lo);
  tiled_query<D>(p, row0 + tq, h, g, qv);
  stage(sh.k[0], stk);
  stage(sh.v[0], stv);
  if (n_blk > 1) {
    fetch(stk, kbase, k_lo + 16);
    stage(sh.k[1], stk);
  }
  // The query registers are read in every pass: their loads land (and the
  // norm and rotation are applied) here, so that no wait inside the loop
  // (where a fetch may or may not have been issued) has to wait for the
  // loop's fetches as well.
#pragma unroll
  for (int i = 0; i < DQ; ++i) asm volatile("" ::"v"(qv[i]));
  __syncthreads();
  f4 s_cur = f4{0.f, 0.f, 0.f, 0.f};
  if (w_blk > 0) s_cur = scores(0);
  __syncthreads();  // K buffer 0 is written again in pass 0
  for (uint32_t b = 0; b < n_blk; ++b) {  // workgroup-uniform
    const uint32_t kb = k_lo + b * 16;
    const bool next_k = b + 2 < n_blk, next_v = b + 1 < n_blk;
    if (next_k) fetch(stk, kbase, kb + 32);
    if (next_v) fetch(stv, vbase, kb + 16);
    if (b + 1 < w_blk) {  // wave-uniform
      const f4 s_next = scores((b + 1) & 1);
      accumulate(b & 1, weights(s_cur, kb));
      s_cur = s_next;
    } else if (b < w_blk) {
      accumulate(b & 1, weights(s_cur, kb));
    }
    if (next_k) stage(sh.k[b & 1], stk);
    if (next_v) stage(sh.v[(b + 1) & 1], stv);
    __syncthreads();
  }

  if (tile >= n_tiles) return;
  // the row's sum over its four lane groups, the sink, and the output
  float L = l_run + __shfl_xor(l_run, 16);
  L += __shfl_xor(L, 32);
  if (CHUNKED) {  // one chunk of several: leave the partial for the merge
    if (k_lo >= wave_keys) return;  // no key of this tile here: the merge skips it
    const uint32_t item = a.s.item_off[sq] + (chunk * p.n_kv_heads + j) * n_tiles + tile;
    float* acc = p.part + (static_cast<size_t>(item) * 16 + c) * D + 16 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < TD; u += 4)
        *reinterpret_cast<f4*>(acc + 4 * r + 16 * u) = f4{o[u][r], o[u + 1][r], o[u + 2][r], o[u + 3][r]};
    if (g == 0) {
      float* ml = p.part + static_cast<size_t>(p.n_items) * 16 * D + (static_cast<size_t>(item) * 16 + c) * 2;
      ml[0] = m_run;
      ml[1] = L;
    }
    return;
  }
  float sa = 1.f;
  if (p.sinks) {
    const float sk = p.sinks[h] * kLog2e;
    if (sk != -INFINITY) {
      const float mn = fmaxf(m_run, sk);
      sa = fast_exp2(m_run - mn);
      L = L * sa + fast_exp2(sk - mn);
    }
  }
  if (t >= T) return;
  const float rs = sa / L;
  float* dst = p.out + (static_cast<size_t>(row0 + t) * p.n_heads + h) * D + 16 * g;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int u = 0; u < TD; u += 4)
      *reinterpret_cast<f4*>(dst + 4 * r + 16 * u) =
          f4{o[u][r], o[u + 1][r], o[u + 2][r], o[u + 3][r]} * rs;
}

// Split-K attention for sequences with few query rows per kv head (a verify
// of k rows, a short prefill).  Every wave takes a 16-row tile of one
// sequence and kv head j against a range of keys (its share of the
// workgroup's group, below), loaded straight from the cache into registers
// (no other wave needs them), with the next 16-key block in flight while the
// current one is multiplied.  The MFMA forms are those of prefill_attn_kernel,
// except that the head_dim
// order of the score product is permuted so that each K load instruction
// reads 64 contiguous bytes per row: lane (c, g) multiplies
// d = 16v + 4g + e at MFMA (v, e), for K row c and for its query row c.
// The four waves of a workgroup take a group of four chunks of the same
// (sequence, kv head, tile), its keys cut evenly between them in 16-key
// blocks, and combine their results through LDS, so that one unnormalised
// partial per workgroup (per row: running max m in log2 units, sum l, and
// acc[D]) goes to memory; split_merge_kernel combines the partials of a row.
// Two waves per SIMD where the registers allow it without spilling (head_dim
// up to 128); head_dim 256 takes the whole register file.
template <int D>
constexpr int split_waves_per_eu() { return D <= 128 ? 2 : 1; }

// LDS of a split-K workgroup: waves 1..3 hand their results to wave 0,
// element-major ([float][lane]) so that the 16-byte stores of a wave fall on
// consecutive banks.
constexpr int kSplitWaves = kSplitChunksPerGroup;  // waves per split-K workgroup
template <int D>
struct SplitLds {
  f4 acc[kSplitWaves > 1 ? kSplitWaves - 1 : 1][D / 16][kWave];
  float m[kSplitWaves > 1 ? kSplitWaves - 1 : 1][kWave];
  float l[kSplitWaves > 1 ? kSplitWaves - 1 : 1][kWave];
  // per wave: a K block on its way to the A layout (head_dim up to 128)
  float kt[kSplitWaves][D <= 128 ? 16 * D : 4];
};

// Float offset of 16-byte segment s of row r in a wave's LDS K block: the
// segments are XOR-swizzled by row, so that the sixteen lanes of a lane
// group, writing one row each or reading sixteen rows, hit distinct banks.
template <int D>
__device__ __forceinline__ uint32_t kt_at(uint32_t r, uint32_t s) {
  return r * D + 4 * (s ^ (r % 16));
}

template <int D, int G>
__global__ void __launch_bounds__(kWave * kSplitWaves)
__attribute__((amdgpu_waves_per_eu(split_waves_per_eu<D>()))) split_attn_kernel(const PrefillArgs a) {
  constexpr int NK = D / 16;   // K float4 per lane per block
  constexpr int TD = D / 16;   // output tiles of 16 head_dim values
  constexpr int DQ = D / 4;
  constexpr int NV = TD / 4;   // V float4 per lane per key of a lane group
  __shared__ SplitLds<D> sh;
  if (a.magic != kArgsMagic) return;  // argument block not delivered whole
  const PrefillParams& p = a.p;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t g = lane / 16, c = lane % 16;
  // workgroup -> (sequence, kv head j, tile, chunk group); wave w takes the
  // w-th share of the group's keys.  All of it is uniform: scalar registers,
  // uniform loops.
  // Workgroups run the groups of whole chunk spans first and every tile's
  // last (shorter) group after them, so the end of the grid holds short work.
  if (blockIdx.x >= p.n_items) return;  // workgroup-uniform, before any barrier
  const SplitItem si = split_item_of_block(a.s, p.n_seq, p.n_items, p.split_keys, blockIdx.x);
  const uint32_t item = si.item, sq = si.seq;
  const uint32_t T = a.s.len[sq], pos0 = a.s.pos0[sq], row0 = a.s.row_off[sq];
  const uint32_t n_tiles = (T * G + 15) / 16;
  const uint32_t n_grp = split_groups(pos0 + T, p.split_keys);
  const uint32_t idx = item - a.s.item_off[sq];
  const uint32_t grp = idx % n_grp;
  const uint32_t ut = idx / n_grp;
  const uint32_t tile = ut % n_tiles;
  const uint32_t j = ut / n_tiles;
  const uint32_t tile_keys = pos0 + min((tile * 16 + 15) / G, T - 1) + 1;
  // the group's keys [g_lo, g_hi) of this tile, cut evenly over the waves
  // in whole 16-key blocks (a short last group keeps every wave streaming)
  const uint32_t g_lo = grp * kSplitWaves * p.split_keys;
  const uint32_t g_hi = max(g_lo, min(g_lo + kSplitWaves * p.split_keys, tile_keys));
  const WaveShare ws = split_wave_share(g_lo, g_hi, w);
  const uint32_t k0 = ws.k0, k1 = ws.k1, n_blk = ws.n_blk;
  const bool active = n_blk > 0;  // wave-uniform: else nothing of this tile here
  const uint32_t R = tile * 16 + c;
  const uint32_t t = R / G, h = j * G + R % G;
  const uint32_t tq = t < T ? t : T - 1;  // rows past the last token compute on it, unused
  const uint32_t row_pos = pos0 + tq;

  float qv[DQ];  // the wave's query rows, prepared with the first blocks in flight
  const uint64_t slot_base = a.s.slot[sq] * p.slot_stride;
  const float* kbase = p.k_cache + slot_base + j * D;
  const float* vbase = p.v_cache + slot_base + j * D;
  // Block b of the chunk: keys k0 + 16b .. k0 + 16b + 15.  Lane (g, c) loads
  // V rows k0 + 16b + 4g + m, floats 4c + 64x .. 4c + 64x + 3, so that the
  // sixteen lanes of a lane group read 256 contiguous bytes of one row.  K
  // rows are loaded the same way and go through the wave's LDS block into
  // the A layout (loading the operand in that layout would read 64 bytes of
  // each of sixteen rows per instruction, which streams measurably slower);
  // at head_dim 256 the registers leave no room for that, and K row
  // k0 + 16b + c is loaded in the A layout (floats 16v + 4g .. for v < D/16,
  // held as kr[v / NV][v % NV]).
  // Loads are issued unconditionally, so that the number in flight is known
  // where a block is consumed: rows past the chunk (a partial last block, or
  // the block after the last) re-read its last key, which the mask drops.
  // (an inactive wave issues no load: its loop runs no block, and its
  // prologue loads are skipped below)
  auto load_rows = [&](const float* base, f4 (&r)[4][NV], uint32_t b) {
    const uint32_t kb = k0 + 16 * b;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float* rp = base + static_cast<size_t>(min(kb + 4 * g + m, k1 - 1)) * p.kv_dim + 4 * c;
#pragma unroll
      for (int x = 0; x < NV; ++x)
        r[m][x] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(rp + 64 * x));
    }
  };
  constexpr bool kKTile = D <= 128;
  auto load_k = [&](f4 (&kr)[4][NV], uint32_t b) {
    if constexpr (kKTile) {
      load_rows(kbase, kr, b);
    } else {
      const uint32_t kb = k0 + 16 * b;
      const float* kp = kbase + static_cast<size_t>(min(kb + c, k1 - 1)) * p.kv_dim + 4 * g;
#pragma unroll
      for (int v = 0; v < NK; ++v)
        kr[v / NV][v % NV] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(kp + 16 * v));
    }
  };
  auto load_v = [&](f4 (&vr)[4][NV], uint32_t b) { load_rows(vbase, vr, b); };
  float* kt = sh.kt[w];

  float m_run = -INFINITY, l_run = 0.f;
  f4 o[TD];
#pragma unroll
  for (int u = 0; u < TD; ++u) o[u] = f4{0.f, 0.f, 0.f, 0.f};
  // scores of block b (from its K rows), then its softmax weights
  f4 pr;
  float corr;
  auto scores = [&](const f4 (&kr)[4][NV], uint32_t b) {
    const uint32_t kb = k0 + 16 * b;
    // the block's K rows into the LDS block (row 4g + m, segment c + 16x),
    // then back as the A operand: lane (g, c) takes row c, d = 16v + 4g + e
    if constexpr (kKTile) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int x = 0; x < NV; ++x)
          *reinterpret_cast<f4*>(kt + kt_at<D>(4 * g + m, c + 16 * x)) = kr[m][x];
    }
    f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < NK; ++v) {
      const f4 ka_v = kKTile ? *reinterpret_cast<const f4*>(kt + kt_at<D>(c, 4 * v + g))
                             : kr[v / NV][v % NV];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka_v[e], qv[4 * v + e], s, 0, 0, 0);
    }
    // key kb + 4g + r counts iff it is in the chunk and not after the row
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t key = kb + 4 * g + r;
      if (key >= k1 || key > row_pos) s[r] = -INFINITY;
    }
    float mb = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);
    // a row may have no key yet in this chunk: keep everything at zero
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    corr = fast_exp2(m_run - m_use);
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(s[r] - m_use);
    l_run = l_run * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
  };
  // the weighted V rows of the block whose scores were taken last
  auto accumulate = [&](const f4 (&vr)[4][NV]) {
#pragma unroll
    for (int u = 0; u < TD; ++u) o[u] *= corr;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int x = 0; x < NV; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[4 * x + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[m][x][e], pr[m], o[4 * x + e], 0, 0, 0);
  };

  // Two register sets, A for even blocks and B for odd ones.  A set's K
  // rows are reloaded (for the block two ahead) as soon as its scores are
  // taken and its V rows as soon as they are accumulated, so about three
  // half-blocks are in flight while a block is multiplied.
  f4 ka[4][NV], va[4][NV], kb_[4][NV], vb[4][NV];
  if (active) {
    load_k(ka, 0);
    load_v(va, 0);
    load_k(kb_, 1);
    load_v(vb, 1);
  }
  split_query<D>(p, row0 + tq, h, g, qv);  // with the first blocks in flight
  // The query registers are read in every block: their loads land (and the
  // norm and rotation are applied) here.
  // Left to the loop, the wait for them would sit where the loads in flight
  // are those of the next blocks, and would wait for those as well.
#pragma unroll
  for (int i = 0; i < DQ; ++i) asm volatile("" ::"v"(qv[i]));
  uint32_t b = 0;
  for (; b + 2 <= n_blk; b += 2) {
    __builtin_amdgcn_sched_barrier(0);
    scores(ka, b);
    __builtin_amdgcn_sched_barrier(0);
    load_k(ka, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(va);
    __builtin_amdgcn_sched_barrier(0);
    load_v(va, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    scores(kb_, b + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_k(kb_, b + 3);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(vb);
    __builtin_amdgcn_sched_barrier(0);
    load_v(vb, b + 3);
  }
  if (b < n_blk) {
    scores(ka, b);
    accumulate(va);
  }

  float L = l_run + __shfl_xor(l_run, 16);
  L += __shfl_xor(L, 32);
  // waves 1..3 hand (acc, m, l) to wave 0, which rescales all four to their
  // common maximum (an empty chunk, m = -inf, weighs 0) and adds them in
  // wave order
  if constexpr (kSplitWaves > 1) {
    if (w > 0) {
#pragma unroll
      for (int u = 0; u < TD; ++u) sh.acc[w - 1][u][lane] = o[u];
      sh.m[w - 1][lane] = m_run;
      sh.l[w - 1][lane] = L;
    }
    __syncthreads();
    if (w > 0) return;
  }
  float mx = m_run;
#pragma unroll
  for (int v = 0; v < kSplitWaves - 1; ++v) mx = fmaxf(mx, sh.m[v][lane]);
  const float base = mx == -INFINITY ? 0.f : mx;  // every chunk empty: all stays zero
  const float s0 = fast_exp2(m_run - base);
  L *= s0;
#pragma unroll
  for (int u = 0; u < TD; ++u) o[u] *= s0;
#pragma unroll
  for (int v = 0; v < kSplitWaves - 1; ++v) {
    const float sv = fast_exp2(sh.m[v][lane] - base);
    L += sh.l[v][lane] * sv;
#pragma unroll
    for (int u = 0; u < TD; ++u) o[u] += sh.acc[v][u][lane] * sv;
  }
  // register r of output tile u holds d = 16g + 4r + 64(u/4) + u%4 of row c
  float* acc = p.part + (static_cast<size_t>(item) * 16 + c) * D + 16 * g;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int u = 0; u < TD; u += 4)
      *reinterpret_cast<f4*>(acc + 4 * r + 16 * u) = f4{o[u][r], o[u + 1][r], o[u + 2][r], o[u + 3][r]};
  if (g == 0) {
    float* ml = p.part + static_cast<size_t>(p.n_items) * 16 * D + (static_cast<size_t>(item) * 16 + c) * 2;
    ml[0] = mx;
    ml[1] = L;
  }
}

// One wave per (row, query head) of the launch: combines the row's chunk
// partials (max over chunks, each rescaled by 2^(m_c - max)), adds the sink
// and writes the normalised output row.  Lane k reads the (max, sum) of
// chunk k (64 chunks per pass), so the weights take one round trip to
// memory; the accumulator slices of the chunks are then read four at a time.
template <int D, int G>
__global__ void __launch_bounds__(kWave * kAttnWaves) split_merge_kernel(const PrefillArgs a) {
  constexpr int EPL = D / kWave;
  if (a.magic != kArgsMagic) return;
  const PrefillParams& p = a.p;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wid = blockIdx.x * kAttnWaves + threadIdx.x / kWave;
  if (wid >= p.n_rows * p.n_heads) return;  // wave-uniform
  const uint32_t row = wid / p.n_heads, h = wid - row * p.n_heads;
  const uint32_t sq = seq_of_row(a, row);
  const uint32_t T = a.s.len[sq], pos0 = a.s.pos0[sq];
  const uint32_t t = row - a.s.row_off[sq];
  const uint32_t j = h / G, R = t * G + h % G, tile = R / 16, c = R % 16;
  const uint32_t n_tiles = (T * G + 15) / 16;
  const uint32_t tile_keys = pos0 + min((tile * 16 + 15) / G, T - 1) + 1;
  // split-K partials are per group of kSplitWaves chunks (j-major items);
  // chunked tiled ones per chunk (chunk-major items), each chunk of the
  // tile group's keys cut evenly
  const bool grouped = p.n_groups == 0;
  uint32_t span = p.split_keys * kSplitWaves;
  if (!grouped) {
    const uint32_t grp = tile / kAttnWaves;
    const uint32_t last = min(grp * kAttnWaves + kAttnWaves - 1, n_tiles - 1);
    const uint32_t n_keys = pos0 + min((last * 16 + 15) / G, T - 1) + 1;
    const uint32_t n_ck = (pos0 + T + p.split_keys - 1) / p.split_keys;
    span = group_chunk_keys(n_keys, n_ck, p.split_keys);
  }
  const uint32_t nck = (tile_keys + span - 1) / span;
  const uint32_t first = grouped ? a.s.item_off[sq] + (j * n_tiles + tile) * split_groups(pos0 + T, p.split_keys)
                                 : a.s.item_off[sq] + j * n_tiles + tile;
  const uint32_t stride = grouped ? 1 : p.n_kv_heads * n_tiles;  // from one partial to the next
  const float* ml = p.part + static_cast<size_t>(p.n_items) * 16 * D;
  auto at = [&](uint32_t k) { return static_cast<size_t>(first + k * stride) * 16 + c; };
  // the maximum over the chunks (finite: chunk 0 holds key 0) and the sink
  float mx = -INFINITY;
  for (uint32_t k0 = 0; k0 < nck; k0 += kWave)
    if (k0 + lane < nck) mx = fmaxf(mx, ml[at(k0 + lane) * 2]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float sk = p.sinks ? p.sinks[h] * kLog2e : -INFINITY;
  mx = fmaxf(mx, sk);
  float L = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (uint32_t k0 = 0; k0 < nck; k0 += kWave) {
    // lane k: chunk k0 + k's weight (0 for a chunk with no key of this row)
    float wgt = 0.f;
    if (k0 + lane < nck) {
      const float m = ml[at(k0 + lane) * 2];
      wgt = m == -INFINITY ? 0.f : fast_exp2(m - mx);
      L += ml[at(k0 + lane) * 2 + 1] * wgt;
    }
    const uint32_t n = min(nck - k0, static_cast<uint32_t>(kWave));
    uint32_t k = 0;
    for (; k + 4 <= n; k += 4) {
      float x[4][EPL];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[q][e] = p.part[at(k0 + k + q) * D + lane * EPL + e];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float wq = __shfl(wgt, k + q);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += x[q][e] * wq;
      }
    }
    for (; k < n; ++k) {
      const float wq = __shfl(wgt, k);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += p.part[at(k0 + k) * D + lane * EPL + e] * wq;
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) L += __shfl_xor(L, off);
  if (sk != -INFINITY) L += fast_exp2(sk - mx);
  const float rl = 1.f / L;
  float* dst = p.out + (static_cast<size_t>(row) * p.n_heads + h) * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * rl;
}

template <int D, int G>
hipError_t launch_split(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((split_attn_kernel<D, G>), dim3(a.p.n_items), dim3(kWave * kSplitWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t waves = a.p.n_rows * a.p.n_heads;
  hipLaunchKernelGGL((split_merge_kernel<D, G>), dim3((waves + kAttnWaves - 1) / kAttnWaves),
                     dim3(kWave * kAttnWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_attn(const PrefillArgs& a, hipStream_t s) {
  const uint32_t blocks = a.p.n_groups * a.p.n_kv_heads;
  if (a.p.split_keys == 0) {
    hipLaunchKernelGGL((prefill_attn_kernel<D, G, false>), dim3(blocks), dim3(kWave * kAttnWaves), 0,
                       s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_attn_kernel<D, G, true>), dim3(blocks), dim3(kWave * kAttnWaves), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t waves = a.p.n_rows * a.p.n_heads;
  hipLaunchKernelGGL((split_merge_kernel<D, G>), dim3((waves + kAttnWaves - 1) / kAttnWaves),
                     dim3(kWave * kAttnWaves), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, uint32_t G, bool split, hipStream_t s,
                    hipEvent_t before, hipEvent_t after) {
  const uint32_t per_wg = kPrepWaves * a.p.prep_vpw;
  const uint32_t per_row = (a.p.n_kv_heads + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((prefill_prep_kernel<D>), dim3(a.p.n_rows * per_row), dim3(kWave * kPrepWaves), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && before) e = hipEventRecord(before, s);
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: e = split ? launch_split<D, 1>(a, s) : launch_attn<D, 1>(a, s); break;
    case 2: e = split ? launch_split<D, 2>(a, s) : launch_attn<D, 2>(a, s); break;
    case 4: e = split ? launch_split<D, 4>(a, s) : launch_attn<D, 4>(a, s); break;
    case 8: e = split ? launch_split<D, 8>(a, s) : launch_attn<D, 8>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e == hipSuccess && after) e = hipEventRecord(after, s);
  return e;
}

}  // namespace

int launch_prefill(const PrefillArgs& a, uint32_t head_dim, uint32_t group, bool split,
                   void* stream, void* before_attn, void* after_attn) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t b = static_cast<hipEvent_t>(before_attn);
  hipEvent_t e = static_cast<hipEvent_t>(after_attn);
  switch (head_dim) {
    case 64: return launch_d<64>(a, group, split, s, b, e);
    case 128: return launch_d<128>(a, group, split, s, b, e);
    case 256: return launch_d<256>(a, group, split, s, b, e);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace slotkv
