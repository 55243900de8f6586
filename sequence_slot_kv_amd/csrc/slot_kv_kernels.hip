// slot_kv_kernels.hip -- gfx950 kernels of the batched decode step over a
// slot-indexed KV cache ("Forward Cuda Gemma", decodeBatch: per-head Q/K
// norm, RoPE, KV write and causal softmax attention of every row against its
// own slot; "Forward Cuda", init: inv_freq and sinks).
//
// One fused split-K kernel does the whole step for one (row, key chunk, kv
// head) per 64-lane wave:
//   prologue  RMSNorm + RoPE of the row's G query heads of this kv head
//             (kept in registers, pre-multiplied by scale*log2(e));
//             the wave that owns the row's last chunk also normalises and
//             rotates the new key, stores it and v_new at
//             (slot*slot_ctx + pos)*kv_dim, and seeds its softmax state with
//             that key straight from registers (no read-after-write);
//   body      streams the chunk's history rows of K and V once, with 128-bit
//             non-temporal loads: LPK lanes own one key row (each lane four
//             floats per 4*LPK-float slice), 64/LPK keys per wave in flight,
//             dot products reduced over the LPK lanes with DPP, one online
//             softmax state per key group;
//   epilogue  the key groups of the wave are merged with cross-lane
//             shuffles; a row that fits one chunk is normalised (with its
//             sink) and written out, a longer row leaves an unnormalised
//             partial (acc, max, sum) per query head.
// A second kernel merges the partials of split rows in chunk order.  Chunk
// boundaries depend only on the row's position and the merge order is
// fixed, so a row's result does not depend on the rest of the batch.
#include <hip/hip_runtime.h>

#include "slot_kv_internal.h"

namespace slotkv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;

// Lanes per key row: enough that each lane holds about 64 floats of query
// (G heads) and as many of accumulator.  The lane's elements of a head
// vector are d = i*4*LPK + 4*r + c (slice i, lane r of the key group,
// component c), so the RoPE partner d + D/2 sits in the same lane, slice
// i + NV4/2.
constexpr int pick_lpk(int D, int G) {
  int want = G * D / 64;
  int lpk = want < 4 ? 4 : (want > 16 ? 16 : want);
  while (D / (4 * lpk) < 2) lpk /= 2;
  return lpk;
}
// Keys per key group per loop trip: about 16 float4 loads per lane in flight.
constexpr int pick_unroll(int D, int LPK) {
  int nv4 = D / (4 * LPK);
  return nv4 >= 8 ? 1 : 8 / nv4;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the LPK lanes of a key group; every lane of the group receives
// the same bits (each step adds a pair of values in both orders, and float
// addition is commutative).
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPK == 4 || LPK == 8 || LPK == 16, "lanes per key");
  v += dpp_mov<0xB1>(v);                         // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);                         // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPK >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror: i <-> 7-i
  if constexpr (LPK >= 16) v += dpp_mov<0x140>(v);  // row_mirror: i <-> 15-i
  return v;
}

__device__ __forceinline__ float dot4(f4 a, f4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 ld4_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rescale factor exp2(m_old - m_new) for a state that may still be empty.
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return m_old == -INFINITY ? 0.f : fast_exp2(m_old - m_new);
}

template <int D, int LPK>
__device__ __forceinline__ void rms_norm_lane(f4 (&x)[D / (4 * LPK)], const f4 (&w)[D / (4 * LPK)],
                                              float eps) {
  constexpr int NV4 = D / (4 * LPK);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV4; ++i) ss += dot4(x[i], x[i]);
  ss = group_sum<LPK>(ss);
  const float rn = 1.0f / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < NV4; ++i) x[i] = x[i] * rn * w[i];
}

template <int D, int LPK>
__device__ __forceinline__ void rope_lane(f4 (&x)[D / (4 * LPK)],
                                          const float (&cs)[D / (8 * LPK)][4],
                                          const float (&sn)[D / (8 * LPK)][4]) {
  constexpr int HALF = D / (8 * LPK);
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float a = x[i][c], b = x[i + HALF][c];
      x[i][c] = a * cs[i][c] - b * sn[i][c];
      x[i + HALF][c] = b * cs[i][c] + a * sn[i][c];
    }
  }
}

template <int D, int G>
__global__ void __launch_bounds__(kWave* kWavesPerBlock)
    decode_attn_kernel(const AttnParams p) {
  constexpr int LPK = pick_lpk(D, G);
  constexpr int U = pick_unroll(D, LPK);
  constexpr int NV4 = D / (4 * LPK);  // float4 per lane per head vector
  constexpr int HALF = NV4 / 2;
  constexpr int NG = kWave / LPK;     // key groups per wave
  constexpr int SL = 4 * LPK;         // floats per slice
  static_assert(NV4 >= 2 && NV4 % 2 == 0, "lane layout needs an even slice count");

  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (wave >= p.n_waves) return;  // wave-uniform
  const uint32_t j = wave % p.n_kv_heads;
  const WorkItem it = p.items[wave / p.n_kv_heads];
  const RowInfo row = p.rows[it.row];
  const uint32_t gi = lane / LPK;
  const uint32_t lo = 4 * (lane % LPK);  // lane's float offset inside a slice

  // ---- prologue: RoPE angles of this lane's first-half elements --------
  float cs[HALF][4], sn[HALF][4];
  {
    const float fpos = static_cast<float>(row.pos);
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const f4 f = ld4(p.inv_freq + i * SL + lo);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float ang = fpos * f[c];  // one f32 multiply
        sincosf(ang, &sn[i][c], &cs[i][c]);
      }
    }
  }

  // ---- query heads j*G .. j*G+G-1: norm, RoPE, fold in scale*log2(e) ----
  f4 q[G][NV4];
  {
    f4 w[NV4];
#pragma unroll
    for (int i = 0; i < NV4; ++i) w[i] = ld4(p.q_norm_w + i * SL + lo);
    const float* qrow = p.q + static_cast<size_t>(it.row) * p.n_heads * D +
                        static_cast<size_t>(j) * G * D + lo;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < NV4; ++i) q[g][i] = ld4(qrow + g * D + i * SL);
      rms_norm_lane<D, LPK>(q[g], w, p.eps);
      rope_lane<D, LPK>(q[g], cs, sn);
#pragma unroll
      for (int i = 0; i < NV4; ++i) q[g][i] *= p.qk_scale_log2;
    }
  }

  float m[G], l[G];
  f4 acc[G][NV4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < NV4; ++i) acc[g][i] = f4{0.f, 0.f, 0.f, 0.f};
  }

  const uint64_t slot_base = static_cast<uint64_t>(row.slot) * p.slot_stride + j * D + lo;

  // ---- the new key (last chunk of the row only) ---------------------------
  if (it.chunk == row.n_chunks - 1) {
    f4 kn[NV4], vn[NV4], w[NV4];
    const size_t nb = static_cast<size_t>(it.row) * p.kv_dim + j * D + lo;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      kn[i] = ld4(p.k_new + nb + i * SL);
      vn[i] = ld4(p.v_new + nb + i * SL);
      w[i] = ld4(p.k_norm_w + i * SL + lo);
    }
    rms_norm_lane<D, LPK>(kn, w, p.eps);
    rope_lane<D, LPK>(kn, cs, sn);
    if (gi == 0) {
      const uint64_t at = slot_base + static_cast<uint64_t>(row.pos) * p.kv_dim;
#pragma unroll
      for (int i = 0; i < NV4; ++i) {
        st4(p.k_cache + at + i * SL, kn[i]);
        st4(p.v_cache + at + i * SL, vn[i]);
      }
    }
    // Key group 0 starts its state from the new key: weight exp2(0) = 1.
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NV4; ++i) s += dot4(q[g][i], kn[i]);
      s = group_sum<LPK>(s);
      if (gi == 0) {
        m[g] = s;
        l[g] = 1.f;
#pragma unroll
        for (int i = 0; i < NV4; ++i) acc[g][i] = vn[i];
      }
    }
  }

  // ---- history keys [t0, min(t0 + C, pos)) --------------------------------
  const uint32_t t0 = it.chunk * p.chunk;
  const uint32_t t_end = min(t0 + p.chunk, row.pos);
  const float* kb = p.k_cache + slot_base;
  const float* vb = p.v_cache + slot_base;
  for (uint32_t base = t0; base < t_end; base += NG * U) {  // wave-uniform trip count
    f4 kr[U][NV4], vr[U][NV4];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t t = base + gi + NG * u;
      valid[u] = t < t_end;
      if (valid[u]) {
        const uint64_t o = static_cast<uint64_t>(t) * p.kv_dim;
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
          kr[u][i] = ld4_stream(kb + o + i * SL);
          vr[u][i] = ld4_stream(vb + o + i * SL);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
          kr[u][i] = f4{0.f, 0.f, 0.f, 0.f};
          vr[u][i] = f4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < NV4; ++i) d += dot4(q[g][i], kr[u][i]);
        s[u] = group_sum<LPK>(d);
      }
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (valid[u]) mx = fmaxf(mx, s[u]);
      const float corr = rescale(m[g], mx);
      float pu[U];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pu[u] = valid[u] ? fast_exp2(s[u] - mx) : 0.f;
        psum += pu[u];
      }
      l[g] = l[g] * corr + psum;
#pragma unroll
      for (int i = 0; i < NV4; ++i) {
        f4 a = acc[g][i] * corr;
#pragma unroll
        for (int u = 0; u < U; ++u) a += pu[u] * vr[u][i];
        acc[g][i] = a;
      }
      m[g] = mx;
    }
  }

  // ---- merge the wave's key groups (butterfly over lane ^ LPK .. ^ 32) ----
#pragma unroll
  for (int off = LPK; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo_ = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float c1 = rescale(m[g], mn), c2 = rescale(mo, mn);
      l[g] = l[g] * c1 + lo_ * c2;
#pragma unroll
      for (int i = 0; i < NV4; ++i) {
        f4 other;
#pragma unroll
        for (int c = 0; c < 4; ++c) other[c] = __shfl_xor(acc[g][i][c], off);
        acc[g][i] = acc[g][i] * c1 + other * c2;
      }
      m[g] = mn;
    }
  }

  // ---- epilogue ------------------------------------------------------------
  const uint32_t h0 = j * G;
  if (row.n_chunks == 1) {
    // the whole row lives in this item: add the sink and normalise
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mf = m[g], lf = l[g], sa = 1.f;
      if (p.sinks) {
        const float sk = p.sinks[h0 + g] * kLog2e;
        const float mn = fmaxf(mf, sk);
        sa = fast_exp2(mf - mn);
        lf = lf * sa + (sk == -INFINITY ? 0.f : fast_exp2(sk - mn));
      }
      const float inv = sa / lf;
      if (gi == 0) {
        float* o = p.out + (static_cast<size_t>(it.row) * p.n_heads + h0 + g) * D + lo;
#pragma unroll
        for (int i = 0; i < NV4; ++i) st4(o + i * SL, acc[g][i] * inv);
      }
    }
  } else {
    const size_t part = static_cast<size_t>(row.part_base) + it.chunk;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t ph = part * p.n_heads + h0 + g;
      if (gi == 0) {
        float* o = p.part_acc + ph * D + lo;
#pragma unroll
        for (int i = 0; i < NV4; ++i) st4(o + i * SL, acc[g][i]);
      }
      if (lane == 0) {
        p.part_ml[ph * 2 + 0] = m[g];
        p.part_ml[ph * 2 + 1] = l[g];
      }
    }
  }
}

// Merge of the partial results of rows cut into several chunks: one wave per
// (row, query head), chunks combined in index order.
template <int D>
__global__ void __launch_bounds__(kWave* kWavesPerBlock) merge_kernel(const AttnParams p) {
  constexpr int EPL = D / kWave;  // elements per lane
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const uint32_t b = wave / p.n_heads, h = wave % p.n_heads;
  if (b >= p.B) return;
  const RowInfo row = p.rows[b];
  if (row.n_chunks <= 1) return;
  const size_t first = static_cast<size_t>(row.part_base) * p.n_heads + h;
  float M = -INFINITY;
  for (uint32_t c = 0; c < row.n_chunks; ++c)
    M = fmaxf(M, p.part_ml[(first + static_cast<size_t>(c) * p.n_heads) * 2]);
  float sk = -INFINITY;
  if (p.sinks) {
    sk = p.sinks[h] * kLog2e;
    M = fmaxf(M, sk);
  }
  float L = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (uint32_t c = 0; c < row.n_chunks; ++c) {
    const size_t ph = first + static_cast<size_t>(c) * p.n_heads;
    const float w = fast_exp2(p.part_ml[ph * 2] - M);
    L += p.part_ml[ph * 2 + 1] * w;
    const float* a = p.part_acc + ph * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] += a[e] * w;
  }
  if (sk != -INFINITY) L += fast_exp2(sk - M);
  const float inv = 1.0f / L;
  float* dst = p.out + (static_cast<size_t>(b) * p.n_heads + h) * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = o[e] * inv;
}

template <int D, int G>
hipError_t launch_shape(const AttnParams& p, bool any_split, hipStream_t s, hipEvent_t mark) {
  const uint32_t blocks = (p.n_waves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((decode_attn_kernel<D, G>), dim3(blocks), dim3(kWave * kWavesPerBlock), 0, s,
                     p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && mark) e = hipEventRecord(mark, s);
  if (e != hipSuccess || !any_split) return e;
  const uint32_t mwaves = p.B * p.n_heads;
  const uint32_t mblocks = (mwaves + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((merge_kernel<D>), dim3(mblocks), dim3(kWave * kWavesPerBlock), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, uint32_t G, bool any_split, hipStream_t s,
                    hipEvent_t mark) {
  switch (G) {
    case 1: return launch_shape<D, 1>(p, any_split, s, mark);
    case 2: return launch_shape<D, 2>(p, any_split, s, mark);
    case 4: return launch_shape<D, 4>(p, any_split, s, mark);
    case 8: return launch_shape<D, 8>(p, any_split, s, mark);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_shape_supported(uint32_t head_dim, uint32_t group) {
  const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
  return d_ok && g_ok;
}

int launch_decode(const AttnParams& p, uint32_t head_dim, uint32_t group, bool any_split,
                  void* stream, void* after_attn) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t mark = static_cast<hipEvent_t>(after_attn);
  switch (head_dim) {
    case 64: return launch_d<64>(p, group, any_split, s, mark);
    case 128: return launch_d<128>(p, group, any_split, s, mark);
    case 256: return launch_d<256>(p, group, any_split, s, mark);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace slotkv
