// slot_kv_prefill.hip -- gfx950 kernels of a slot prefill: T tokens of one
// sequence into its slot ("Forward Cuda": batched prefill that writes the KV
// cache into the slot's per-sequence region; "Forward Cuda Gemma",
// prefillBatched, equal to the one-token step run over the tokens in order).
//
// Two launches on the caller's stream:
//   prep  one wave per head vector of a token: RMSNorm, then RoPE at the
//         token's position; a query head goes to a scratch buffer (times
//         scale*log2(e)), a key head and its value row go into the slot.
//   attn  causal attention of every token over positions 0 .. pos0+t, now
//         all in the cache.  Unlike decode this is a dense contraction
//         (T*G query rows against each key block), so it runs on the matrix
//         cores: v_mfma_f32_16x16x4f32 in its transposed form
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
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// One wave per head vector: vector v of token t is query head v (v < H) or
// kv head v - H.  Lane l holds elements l*EPL .. l*EPL+EPL-1, so the RoPE
// partner d +- D/2 of an element sits in lane l ^ 32.
template <int D>
__global__ void __launch_bounds__(kWave * kPrepWaves) prefill_prep_kernel(const PrefillParams p) {
  constexpr int EPL = D / kWave;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t vec = blockIdx.x * kPrepWaves + threadIdx.x / kWave;
  const uint32_t per_tok = p.n_heads + p.n_kv_heads;
  if (vec >= p.T * per_tok) return;  // wave-uniform
  const uint32_t t = vec / per_tok, v = vec % per_tok;
  const uint32_t pos = p.pos0 + t;
  const bool is_q = v < p.n_heads;
  const uint32_t kvh = v - p.n_heads;
  const float* src = is_q ? p.q + (static_cast<size_t>(t) * p.n_heads + v) * D
                          : p.k_new + static_cast<size_t>(t) * p.kv_dim + kvh * D;
  const float* w = is_q ? p.q_norm_w : p.k_norm_w;
  float x[EPL];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    x[e] = src[lane * EPL + e];
    ss += x[e] * x[e];
  }
  ss = wave_sum(ss);
  const float rn = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
  const float fpos = static_cast<float>(pos);
  float y[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float xn = x[e] * rn * w[lane * EPL + e];
    const float partner = __shfl_xor(xn, 32);
    const float ang = fpos * p.inv_freq[(lane & 31) * EPL + e];  // one f32 multiply
    float sn, cs;
    sincosf(ang, &sn, &cs);
    y[e] = lane < 32 ? xn * cs - partner * sn : xn * cs + partner * sn;
  }
  if (is_q) {
    float* dst = p.qs + (static_cast<size_t>(t) * p.n_heads + v) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = y[e] * p.qk_scale_log2;
  } else {
    const size_t at = p.slot_base + static_cast<size_t>(pos) * p.kv_dim + kvh * D + lane * EPL;
    const float* vsrc = p.v_new + static_cast<size_t>(t) * p.kv_dim + kvh * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      p.k_cache[at + e] = y[e];
      p.v_cache[at + e] = vsrc[e];
    }
  }
}

// One wave per tile of 16 query rows of one kv head j.  Row r of tile k is
// row R = 16k + r of the head group: token R / G, query head j*G + R % G.
// Lane l works on row c = l % 16 and lane group g = l / 16:
//   S^T block:  A = K[key c][d], B = Q[row c][d] with d = (D/4)*g + i for
//               MFMA i < D/4; result lane l, register r: key 4g + r, row c;
//   O^T tile u: MFMA m < 4 sums key 4g + m (A = V[key][d], d = (D/16)*c + u;
//               B = the score register m); result lane l, register r:
//               d = (D/16)*(4g + r) + u, row c.
// So a lane's whole accumulator belongs to its own row, and its output
// values are d = (D/4)*g .. (D/4)*g + D/4 - 1.  Tiles are launched heaviest
// first (last tokens first) so that the short ones fill in at the end.
template <int D, int G>
__global__ void __launch_bounds__(kWave * kAttnWaves) prefill_attn_kernel(const PrefillParams p) {
  constexpr int DQ = D / 4;   // head_dim values per lane group
  constexpr int TD = D / 16;  // output tiles of 16 head_dim values
  static_assert(DQ % 4 == 0 && TD % 4 == 0, "float4 loads");
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t g = lane / 16, c = lane % 16;
  const uint32_t wave = blockIdx.x * kAttnWaves + threadIdx.x / kWave;
  if (wave >= p.n_tiles * p.n_kv_heads) return;  // wave-uniform
  const uint32_t j = wave % p.n_kv_heads;
  const uint32_t tile = p.n_tiles - 1 - wave / p.n_kv_heads;
  const uint32_t R = tile * 16 + c;
  const uint32_t t = R / G, h = j * G + R % G;
  const bool row_ok = t < p.T;
  const uint32_t tq = row_ok ? t : p.T - 1;  // rows past the last token compute on it, unused
  const uint32_t row_pos = p.pos0 + tq;
  const uint32_t t_last = min((tile * 16 + 15) / G, p.T - 1);
  const uint32_t n_keys = p.pos0 + t_last + 1;  // keys 0 .. position of the tile's last token

  float qv[DQ];
  {
    const float* qsrc = p.qs + (static_cast<size_t>(tq) * p.n_heads + h) * D + DQ * g;
#pragma unroll
    for (int i = 0; i < DQ; i += 4) {
      const f4 v = *reinterpret_cast<const f4*>(qsrc + i);
      qv[i] = v[0];
      qv[i + 1] = v[1];
      qv[i + 2] = v[2];
      qv[i + 3] = v[3];
    }
  }
  const float* kbase = p.k_cache + p.slot_base + j * D;
  const float* vbase = p.v_cache + p.slot_base + j * D;

  float m_run = -INFINITY, l_run = 0.f;
  f4 o[TD];
#pragma unroll
  for (int u = 0; u < TD; ++u) o[u] = f4{0.f, 0.f, 0.f, 0.f};

  const uint32_t n_blk = (n_keys + 15) / 16;
  for (uint32_t blk = 0; blk < n_blk; ++blk) {
    const uint32_t kb = blk * 16;
    // keys past the tile's range re-read its last key (their scores are masked)
    float ka[DQ];
    {
      const float* kr = kbase + static_cast<size_t>(min(kb + c, n_keys - 1)) * p.kv_dim + DQ * g;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const f4 v = *reinterpret_cast<const f4*>(kr + i);
        ka[i] = v[0];
        ka[i + 1] = v[1];
        ka[i + 2] = v[2];
        ka[i + 3] = v[3];
      }
    }
    float va[4][TD];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float* vr =
          vbase + static_cast<size_t>(min(kb + 4 * g + m, n_keys - 1)) * p.kv_dim + TD * c;
#pragma unroll
      for (int u = 0; u < TD; u += 4) {
        const f4 v = *reinterpret_cast<const f4*>(vr + u);
        va[m][u] = v[0];
        va[m][u + 1] = v[1];
        va[m][u + 2] = v[2];
        va[m][u + 3] = v[3];
      }
    }
    f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DQ; ++i) s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[i], qv[i], s, 0, 0, 0);
    // causal mask: key kb + 4g + r is visible to the row iff it is <= the
    // row's position (every key >= n_keys is also past the row)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (kb + 4 * g + r > row_pos) s[r] = -INFINITY;
    float mb = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);  // finite: key 0 is visible to every row
    const float corr = fast_exp2(m_run - m_new);
    f4 pr;
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(s[r] - m_new);
    l_run = l_run * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
    for (int u = 0; u < TD; ++u) o[u] *= corr;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int u = 0; u < TD; ++u) o[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[m][u], pr[m], o[u], 0, 0, 0);
    m_run = m_new;
  }

  // the row's sum over its four lane groups, the sink, and the output
  float L = l_run + __shfl_xor(l_run, 16);
  L += __shfl_xor(L, 32);
  float sa = 1.f;
  if (p.sinks) {
    const float sk = p.sinks[h] * kLog2e;
    if (sk != -INFINITY) {
      const float mn = fmaxf(m_run, sk);
      sa = fast_exp2(m_run - mn);
      L = L * sa + fast_exp2(sk - mn);
    }
  }
  if (!row_ok) return;
  const float rs = sa / L;
  float* dst = p.out + (static_cast<size_t>(t) * p.n_heads + h) * D + DQ * g;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int u = 0; u < TD; u += 4)
      *reinterpret_cast<f4*>(dst + TD * r + u) =
          f4{o[u][r], o[u + 1][r], o[u + 2][r], o[u + 3][r]} * rs;
}

template <int D, int G>
hipError_t launch_attn(const PrefillParams& p, hipStream_t s) {
  const uint32_t waves = p.n_tiles * p.n_kv_heads;
  const uint32_t blocks = (waves + kAttnWaves - 1) / kAttnWaves;
  hipLaunchKernelGGL((prefill_attn_kernel<D, G>), dim3(blocks), dim3(kWave * kAttnWaves), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillParams& p, uint32_t G, hipStream_t s, hipEvent_t before,
                    hipEvent_t after) {
  const uint32_t vecs = p.T * (p.n_heads + p.n_kv_heads);
  hipLaunchKernelGGL((prefill_prep_kernel<D>), dim3((vecs + kPrepWaves - 1) / kPrepWaves),
                     dim3(kWave * kPrepWaves), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && before) e = hipEventRecord(before, s);
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: e = launch_attn<D, 1>(p, s); break;
    case 2: e = launch_attn<D, 2>(p, s); break;
    case 4: e = launch_attn<D, 4>(p, s); break;
    case 8: e = launch_attn<D, 8>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e == hipSuccess && after) e = hipEventRecord(after, s);
  return e;
}

}  // namespace

int launch_prefill(const PrefillParams& p, uint32_t head_dim, uint32_t group, void* stream,
                   void* before_attn, void* after_attn) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t b = static_cast<hipEvent_t>(before_attn);
  hipEvent_t a = static_cast<hipEvent_t>(after_attn);
  switch (head_dim) {
    case 64: return launch_d<64>(p, group, s, b, a);
    case 128: return launch_d<128>(p, group, s, b, a);
    case 256: return launch_d<256>(p, group, s, b, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace slotkv
