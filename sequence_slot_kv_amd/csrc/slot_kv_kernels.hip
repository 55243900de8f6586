// slot_kv_kernels.hip -- gfx950 kernel of the batched decode step over a
// slot-indexed KV cache ("Forward Cuda Gemma", decodeBatch: per-head Q/K
// norm, RoPE, KV write and causal softmax attention of every row against its
// own slot; "Forward Cuda", init: inv_freq and sinks).
//
// One persistent launch does the whole step.  The work is cut into units
// (row b, chunk c of C keys, kv head j); the NW waves of a workgroup split a
// unit's keys evenly (whole pipeline stages each; C/NW keys per wave in a
// full chunk).  Workgroups pull units from an agent-scope queue (full
// chunks first, then partial chunks longest first), asking for the next one
// when the current unit's second pass starts, so that:
//   - the next unit's query heads (and new key) are normalised, rotated and
//     staged in LDS before the current unit ends; the unit that holds a
//     row's last chunk also writes the row's KV entry -- rotated key and
//     v_new at (slot*slot_ctx + pos)*kv_dim -- from that staging step;
//   - the next unit's first K stage is in flight while the current unit's
//     epilogue (the wave merge, its partial's stores, the merge of a row
//     whose counter the previous partial completed) runs.
// Per unit and wave, two passes stream the history rows once each with
// 128-bit non-temporal loads, double-buffered: pass 1 reads K, computes the
// scores (LPK lanes per key row, DPP reductions) into LDS and the running
// max; pass 2 reads V and accumulates exp2(score - max) * v.  No accumulator
// is ever rescaled inside a wave.  Key groups, then the NW waves (through
// LDS), merge; a row of one chunk is finished with its sink; a longer row's
// chunk leaves an unnormalised partial (acc, max, sum) through agent-coherent
// stores and the last workgroup of that (row, kv head) -- an agent-scope
// counter, bumped one unit later when the stores are long complete, decides
// -- merges the row's partials in chunk order.
// Chunk boundaries depend only on the row's position, every merge runs in a
// fixed order and no result depends on which workgroup ran a unit, so a
// row's result does not depend on the rest of the batch.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "slot_kv_device.h"
#include "slot_kv_internal.h"

namespace slotkv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWave = kWaveLanes;
constexpr float kLog2e = 1.4426950408889634f;
#ifndef SLOT_KV_WAVES_PER_EU
#define SLOT_KV_WAVES_PER_EU 2  // occupancy the register budget is fitted to
#endif

// Lanes per key row (LPK) and keys per key group per stage come from
// decode_lpk / decode_unroll.  The lane's elements of a head vector are
// d = i*4*LPK + 4*r + c (slice i, lane r of the key group, component c);
// queries reach that layout from their LDS staging, where they were rotated.

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
  v += dpp_mov<0xB1>(v);                            // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);                            // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPK >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror: i <-> 7-i
  if constexpr (LPK >= 16) v += dpp_mov<0x140>(v);  // row_mirror: i <-> 15-i
  return v;
}

__device__ __forceinline__ float dot4(f4 a, f4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
#ifndef SLOT_KV_NT_LOADS
#define SLOT_KV_NT_LOADS 1  // stream history rows past the caches
#endif
__device__ __forceinline__ f4 ld4_stream(const float* p) {
#if SLOT_KV_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
#else
  return *reinterpret_cast<const f4*>(p);
#endif
}
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// max without the NaN canonicalisation of fmaxf (inputs are never NaN here).
__device__ __forceinline__ float max_nc(float a, float b) { return a > b ? a : b; }

// Weight exp2(m - m_new) of a state with max m; an empty state (m = -inf)
// weighs 0.
__device__ __forceinline__ float rescale(float m, float m_new) {
  return m == -INFINITY ? 0.f : fast_exp2(m - m_new);
}

constexpr uint32_t kNoUnit = 0xffffffffu;  // mailbox empty

// Wait for another wave of the workgroup to post a value in LDS.
__device__ __forceinline__ uint32_t mbox_wait(const uint32_t* slot) {
  uint32_t v;
  while ((v = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) == kNoUnit)
    __builtin_amdgcn_s_sleep(1);
  return __builtin_amdgcn_readfirstlane(v);
}

template <int D, int G>
constexpr int wg_waves() {
  return decode_waves(D, G);
}

template <int D, int G>
struct alignas(16) Lds {
  static constexpr int NW = wg_waves<D, G>();
  // Wave w's (acc, max, sum) per head for the workgroup's merge.  In the
  // matrix-core form acc[w] is 16 rows long and is also the wave's K tile
  // during pass 1: the wave stores its accumulators there only after its
  // pass 2, and the next unit's pass 1 starts after the merge.
  static constexpr int ROWS = decode_mfma(D, G) ? 16 : G;
  float acc[NW][ROWS][D];
  float m[NW][G];
  float l[NW][G];
  uint32_t last;
};

// Occupancy the register allocation targets: shapes whose lanes hold more
// than 64 floats of query (and as many of accumulator) get the whole
// register file.
template <int D, int G>
constexpr int waves_per_eu() {
  return G * D / decode_lpk(D, G) > 64 ? 1 : SLOT_KV_WAVES_PER_EU;
}

// The most stages per pass that any wave of a unit takes, over every count
// of history keys a chunk can hold.
constexpr uint32_t max_wave_stages(int D, int G, int chunk) {
  uint32_t most = 0;
  for (uint32_t n = 0; n <= static_cast<uint32_t>(chunk); ++n)
    for (uint32_t w = 0; w < static_cast<uint32_t>(decode_waves(D, G)); ++w) {
      const uint32_t st = wave_keys(n, decode_step(D, G), decode_waves(D, G), w).n_st;
      most = st > most ? st : most;
    }
  return most;
}

template <int D, int G>
struct Shape {
  static constexpr int NW = decode_waves(D, G);                 // waves per workgroup
  static constexpr int LPK = decode_lpk(D, G);
  static constexpr int U = decode_unroll(D, G);
  static constexpr int NV4 = D / (4 * LPK);                  // float4 per lane per head vector
  static constexpr int NG = kWave / LPK;                     // key groups per wave
  static constexpr int SL = 4 * LPK;                         // floats per slice
  static constexpr bool MFMA = decode_mfma(D, G);            // the matrix-core form
  static constexpr int STEP = decode_step(D, G);             // keys per wave per stage
  // stages per pass the wave's LDS score buffer holds
  static constexpr int NST = decode_stage_bound(D, G, SLOT_KV_CHUNK);
  // score slots per wave: per stage [key group][G][U] (vector form) or
  // [lane group][G][4] (matrix form)
  static constexpr int SCORES = MFMA ? NST * STEP * G : NST * NG * G * U;
  static_assert(MFMA ? STEP % 16 == 0 : STEP == NG * U, "one stage size");
  static_assert(NV4 >= 1 && D % (4 * LPK) == 0, "whole float4 slices per lane");
  static_assert(SLOT_KV_CHUNK % NW == 0, "a chunk splits evenly over the waves");
  static_assert(max_wave_stages(D, G, SLOT_KV_CHUNK) <= static_cast<uint32_t>(NST),
                "no wave's stages outgrow its LDS score buffer");
};

// One work unit as one wave sees it: chunk `chunk` of row b against kv head
// j; the wave owns history keys [k_begin, k_begin + len) of that chunk.
struct UnitPlan {
  uint32_t b, j, chunk, pos, slot, n_chunks;
  uint32_t k_begin, len, n_full, n_st;  // n_st = stages per pass, even; those past n_full masked
  bool new_key;                         // this wave also owns the row's new key
};

// Row, kv head and chunk of a unit (the row lookup is done once per unit).
struct UnitId {
  uint32_t b, j, chunk;
};

__device__ __forceinline__ UnitId locate_unit(const AttnArgs& a, uint32_t unit) {
  const AttnParams& p = a.p;
  UnitId id;
  id.j = unit % p.n_kv_heads;
  locate_item(a.rows, p.n_rows, p.n_full, p.chunk, unit / p.n_kv_heads, &id.b, &id.chunk);
  return id;
}

template <int D, int G>
__device__ __forceinline__ UnitPlan plan_unit(const AttnArgs& a, const UnitId& id, uint32_t w) {
  using S = Shape<D, G>;
  constexpr int NW = S::NW;
  const AttnParams& p = a.p;
  UnitPlan u;
  u.b = id.b;
  u.j = id.j;
  u.chunk = id.chunk;
  u.pos = a.rows.pos[u.b];
  u.slot = a.rows.slot[u.b];
  u.n_chunks = u.pos / p.chunk + 1;
  const uint32_t c0 = u.chunk * p.chunk;
  const uint32_t t_end = min(c0 + p.chunk, u.pos);
  const WaveKeys wk = wave_keys(t_end - c0, S::STEP, NW, w);
  u.k_begin = c0 + wk.begin;
  u.len = wk.len;
  u.n_full = wk.n_full;
  u.n_st = wk.n_st;
  u.new_key = (w == 0) && (u.chunk == u.n_chunks - 1);
  return u;
}

// The next unit's query heads (and its new key) are normalised and rotated
// while the current unit streams, and staged in LDS in two parity buffers.
// Vector v < G is query head j*G + v; v == G is the new key, present only
// for the unit that holds the row's last chunk.  Wave w takes vectors
// w, w + NW, ...; lane l holds elements l*EPL .. l*EPL + EPL-1, so the RoPE
// partner of element d (d +- D/2) sits in lane l ^ 32.
template <int D, int G>
struct alignas(16) PrepLds {
  float q[2][G][D];  // normalised, rotated, times scale*log2(e)
  float kn[2][D];    // normalised, rotated new key
  float vn[2][D];    // its value row (v_new)
};
template <int D, int G>
struct PrepRaw {
  static constexpr int NW = wg_waves<D, G>();
  static constexpr int EPL = D / kWave;
  static constexpr int SLOTS = (G + 1 + NW - 1) / NW;
  float x[SLOTS][EPL];
  float vn[EPL];  // v_new of the row, for the wave that holds the new key
};
// The lane's norm weights (1 + w under SLOT_KV_FLAG_NORM_ONE_PLUS_W) and the
// RoPE frequencies of its elements, the same for every unit.  Element d of a
// head vector uses frequency d mod D/2 for rotate-half pairs and d / 2 for
// interleaved pairs.
template <int D>
struct PrepConst {
  static constexpr int EPL = D / kWave;
  float wq[EPL], wk[EPL], freq[EPL];
};
template <int D>
__device__ __forceinline__ PrepConst<D> prep_const(const AttnParams& p, uint32_t lane) {
  constexpr int EPL = PrepConst<D>::EPL;
  const float one = (p.flags & SLOT_KV_FLAG_NORM_ONE_PLUS_W) ? 1.f : 0.f;
  const bool inter = p.flags & SLOT_KV_FLAG_ROPE_INTERLEAVED;
  PrepConst<D> c;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    c.wq[e] = one + p.q_norm_w[lane * EPL + e];
    c.wk[e] = one + p.k_norm_w[lane * EPL + e];
    c.freq[e] = p.inv_freq[inter ? (lane * EPL + e) / 2 : (lane & 31) * EPL + e];
  }
  return c;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <int D, int G>
__device__ __forceinline__ bool prep_has(const AttnArgs& a, const UnitId& id, uint32_t v) {
  return v < G || (v == G && id.chunk == a.rows.pos[id.b] / a.p.chunk);
}

template <int D, int G>
__device__ __forceinline__ void prep_issue(const AttnArgs& a, const UnitId& id, uint32_t w,
                                           uint32_t lane, PrepRaw<D, G>& raw) {
  using R = PrepRaw<D, G>;
  const AttnParams& p = a.p;
#pragma unroll
  for (int s = 0; s < R::SLOTS; ++s) {
    const uint32_t v = w + s * R::NW;
    if (!prep_has<D, G>(a, id, v)) continue;  // wave-uniform
    const float* src = v < G ? p.q + (static_cast<size_t>(id.b) * p.n_heads + id.j * G + v) * D
                             : p.k_new + static_cast<size_t>(id.b) * p.kv_dim + id.j * D;
#pragma unroll
    for (int e = 0; e < R::EPL; ++e) raw.x[s][e] = src[lane * R::EPL + e];
    if (v == G) {
      const float* vsrc = p.v_new + static_cast<size_t>(id.b) * p.kv_dim + id.j * D;
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) raw.vn[e] = vsrc[lane * R::EPL + e];
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void prep_finish(const AttnArgs& a, const UnitId& id, uint32_t w,
                                            uint32_t lane, const PrepRaw<D, G>& raw,
                                            const PrepConst<D>& pc, PrepLds<D, G>& prep,
                                            uint32_t par) {
  using R = PrepRaw<D, G>;
  const AttnParams& p = a.p;
  const uint32_t pos = a.rows.pos[id.b];
  const float fpos = static_cast<float>(pos);
#pragma unroll
  for (int s = 0; s < R::SLOTS; ++s) {
    const uint32_t v = w + s * R::NW;
    if (!prep_has<D, G>(a, id, v)) continue;  // wave-uniform
    // norm with weights wts, then RoPE at pos (two inlined copies, so that
    // each reads its weights straight from registers)
    // RoPE partners: element d pairs with d +- D/2 (lane ^ 32, same slot) or,
    // interleaved, with d ^ 1 (the neighbouring slot of the lane, or lane ^ 1
    // when a lane holds one element).
    const bool inter = p.flags & SLOT_KV_FLAG_ROPE_INTERLEAVED;  // uniform
    auto norm_rope = [&](const float (&wts)[R::EPL], float (&y)[R::EPL]) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) ss += raw.x[s][e] * raw.x[s][e];
      ss = wave_sum(ss);
      const float rn = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
      float xs[R::EPL];
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) xs[e] = raw.x[s][e] * rn * wts[e];
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) {
        float partner;
        bool first;
        if (inter) {
          if constexpr (R::EPL >= 2) partner = xs[e ^ 1];
          else partner = __shfl_xor(xs[e], 1);
          first = ((lane * R::EPL + e) & 1u) == 0;
        } else {
          partner = __shfl_xor(xs[e], 32);
          first = lane < 32;
        }
        const float ang = fpos * pc.freq[e];  // one f32 multiply
        float sn, cs;
        sincosf(ang, &sn, &cs);
        y[e] = first ? xs[e] * cs - partner * sn : xs[e] * cs + partner * sn;
      }
    };
    float y[R::EPL];
    if (v < G) norm_rope(pc.wq, y); else norm_rope(pc.wk, y);
    if (v < G) {
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) prep.q[par][v][lane * R::EPL + e] = y[e] * p.qk_scale_log2;
    } else {
      // the step's KV write: rotated key and v_new (or its weightless RMSNorm
      // under SLOT_KV_FLAG_V_NORM) at (slot*slot_ctx + pos)*kv_dim
      const uint64_t at = static_cast<uint64_t>(a.rows.slot[id.b]) * p.slot_stride +
                          static_cast<uint64_t>(pos) * p.kv_dim + id.j * D + lane * R::EPL;
      float vw[R::EPL];
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) vw[e] = raw.vn[e];
      if (p.flags & SLOT_KV_FLAG_V_NORM) {  // uniform
        float sv = 0.f;
#pragma unroll
        for (int e = 0; e < R::EPL; ++e) sv += vw[e] * vw[e];
        const float rv = 1.0f / sqrtf(wave_sum(sv) * (1.0f / D) + p.eps);
#pragma unroll
        for (int e = 0; e < R::EPL; ++e) vw[e] *= rv;
      }
#pragma unroll
      for (int e = 0; e < R::EPL; ++e) {
        prep.kn[par][lane * R::EPL + e] = y[e];
        prep.vn[par][lane * R::EPL + e] = vw[e];
        p.k_cache[at + e] = y[e];
        p.v_cache[at + e] = vw[e];
      }
    }
  }
}

// ---------------------------------------------------------------- per-unit compute
// A unit's work for one wave, in two forms with one interface: `load` issues
// stage qi (K stage qi < n_st, else V stage qi - n_st) into a register
// stage; `begin` takes the unit's query heads (and new key) from LDS;
// `score` turns a K stage into scores (log2 units) in the wave's LDS score
// buffer and a running max; `finish_max` makes the wave's max per head;
// `weights` may turn the stored scores into exp2(score - max) in place;
// `accumulate` adds a V stage weighted by them; `add_new_key` adds the row's
// new key (the unit's wave that owns it); `store` leaves the wave's (acc,
// max, sum) per head in LDS for the workgroup's merge.
//
// Every `load` issues the same loads whatever the stage: a key past the
// wave's range re-reads the wave's last key row (pass 1 masks its score to
// -inf, so pass 2 gives it weight 0).  The count of loads in flight therefore
// never depends on the data, and the compiler can leave one stage in flight
// while the other is consumed.

// Vector-ALU form.  LPK lanes own one key row, each holding 4 floats of
// every 4*LPK-float slice; a stage holds U keys per key group of LPK lanes
// (key k_begin + s*STEP + gi + NG*u).  A score is the key group's DPP sum;
// stored scores become weights in a pass of their own between the passes,
// once per (key, head) rather than in every lane of a key group.
template <int D, int G>
struct ValuCore {
  using S = Shape<D, G>;
  static constexpr int LPK = S::LPK, U = S::U, NV4 = S::NV4, NG = S::NG, SL = S::SL;
  struct Stage {
    f4 x[U][NV4];
  };
  uint32_t lane, gi, lo;  // lo: the lane's float offset inside a slice
  f4 q[G][NV4];
  float mx[G];     // running max of this lane's key group, per head
  float s_new[G];  // the new key's scores
  float m[G];      // wave max per head: all key groups (and the new key) share it
  float l[G];
  f4 acc[G][NV4];

  __device__ __forceinline__ void init(uint32_t lane_) {
    lane = lane_;
    gi = lane / LPK;
    lo = 4 * (lane % LPK);
  }
  __device__ __forceinline__ void load(const AttnParams& p, const UnitPlan& u, Stage& sg,
                                       uint32_t qi) const {
    const bool is_v = qi >= u.n_st;
    const uint32_t st = is_v ? qi - u.n_st : qi;
    const float* base = (is_v ? p.v_cache : p.k_cache) +
                        static_cast<uint64_t>(u.slot) * p.slot_stride + u.j * D + lo;
    const uint32_t first = u.k_begin + st * S::STEP + gi;
    const uint32_t last = u.k_begin + u.len - 1;
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const uint32_t row = min(first + NG * uu, last);
      const float* r = base + static_cast<uint64_t>(row) * p.kv_dim;
#pragma unroll
      for (int i = 0; i < NV4; ++i) sg.x[uu][i] = ld4_stream(r + i * SL);
    }
    // keep the loads ahead of the work on the other buffer
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void begin(const PrepLds<D, G>& prep, uint32_t par, bool new_key) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NV4; ++i) q[g][i] = ld4(&prep.q[par][g][i * SL + lo]);
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = -INFINITY;
    if (new_key) {  // wave 0 of the row's last chunk scores the new key
      f4 kn[NV4];
#pragma unroll
      for (int i = 0; i < NV4; ++i) kn[i] = ld4(&prep.kn[par][i * SL + lo]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sdot = dot4(q[g][0], kn[0]);
#pragma unroll
        for (int i = 1; i < NV4; ++i) sdot += dot4(q[g][i], kn[i]);
        s_new[g] = group_sum<LPK>(sdot);
        mx[g] = s_new[g];
      }
    }
  }
  __device__ __forceinline__ void score(const Stage& sg, uint32_t st, const UnitPlan& u,
                                        float* sc_w, float*) {
    const bool tail = st >= u.n_full;
    float sc[G * U];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        float d = dot4(q[g][0], sg.x[uu][0]);
#pragma unroll
        for (int i = 1; i < NV4; ++i) d += dot4(q[g][i], sg.x[uu][i]);
        d = group_sum<LPK>(d);
        if (tail && st * S::STEP + gi + NG * uu >= u.len) d = -INFINITY;
        sc[g * U + uu] = d;
        mx[g] = max_nc(mx[g], d);
      }
    }
    if (lane % LPK == 0) {
      float* dst = sc_w + (st * NG + gi) * (G * U);
      if constexpr ((G * U) % 4 == 0) {
#pragma unroll
        for (int e = 0; e < G * U; e += 4) st4(dst + e, f4{sc[e], sc[e + 1], sc[e + 2], sc[e + 3]});
      } else {
#pragma unroll
        for (int e = 0; e < G * U; ++e) dst[e] = sc[e];
      }
    }
  }
  __device__ __forceinline__ void finish_max() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float v = mx[g];
#pragma unroll
      for (int off = LPK; off < kWave; off <<= 1) v = max_nc(v, __shfl_xor(v, off));
      m[g] = v;
      l[g] = 0.f;  // pass 2's state starts here, so it holds no registers in pass 1
#pragma unroll
      for (int i = 0; i < NV4; ++i) acc[g][i] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // Each stored score becomes its weight exp2(s - max), the wave's lanes
  // taking four entries at a time.  An entry's head is fixed by its place in a
  // stage's [key group][G][U] block, and a block's G*U entries divide 256, so
  // each lane's four heads stay the same from one step of the loop to the next.
  __device__ __forceinline__ void weights(float* sc_w, uint32_t n_st) const {
    constexpr uint32_t GU = G * U;
    static_assert(256 % GU == 0 && (NG * GU) % 4 == 0, "weight pass lane layout");
    float mc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t g_c = ((4 * lane + c) % GU) / U;
      mc[c] = m[0];
#pragma unroll
      for (int g = 1; g < G; ++g) mc[c] = g_c == static_cast<uint32_t>(g) ? m[g] : mc[c];
    }
    const uint32_t n_ent = n_st * NG * GU;  // a multiple of 4
    for (uint32_t e = 4 * lane; e < n_ent; e += 4 * kWave) {
      f4 v = ld4(sc_w + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = fast_exp2(v[c] - mc[c]);  // masked keys: exp2(-inf) = 0
      st4(sc_w + e, v);
    }
  }
  __device__ __forceinline__ void accumulate(const Stage& sg, uint32_t st, const float* sc_w) {
    const float* src = sc_w + (st * NG + gi) * (G * U);
    float sc[G * U];
    if constexpr ((G * U) % 4 == 0) {
#pragma unroll
      for (int e = 0; e < G * U; e += 4) {
        const f4 v = ld4(src + e);
        sc[e] = v[0];
        sc[e + 1] = v[1];
        sc[e + 2] = v[2];
        sc[e + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < G * U; ++e) sc[e] = src[e];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const float pu = sc[g * U + uu];  // exp2(score - max), from the weight pass
        l[g] += pu;
#pragma unroll
        for (int i = 0; i < NV4; ++i) acc[g][i] += pu * sg.x[uu][i];
      }
    }
  }
  __device__ __forceinline__ void add_new_key(const PrepLds<D, G>& prep, uint32_t par) {
    if (gi != 0) return;  // one key group adds it (the groups are summed next)
    f4 vn[NV4];
#pragma unroll
    for (int i = 0; i < NV4; ++i) vn[i] = ld4(&prep.vn[par][i * SL + lo]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pn = fast_exp2(s_new[g] - m[g]);
      l[g] += pn;
#pragma unroll
      for (int i = 0; i < NV4; ++i) acc[g][i] += pn * vn[i];
    }
  }
  __device__ __forceinline__ void store(Lds<D, G>& sh, uint32_t w) {
    // sum the wave's key groups (they share m)
#pragma unroll
    for (int off = LPK; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        l[g] += __shfl_xor(l[g], off);
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
          f4 other;
#pragma unroll
          for (int c = 0; c < 4; ++c) other[c] = __shfl_xor(acc[g][i][c], off);
          acc[g][i] += other;
        }
      }
    }
    if (gi == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int i = 0; i < NV4; ++i) st4(&sh.acc[w][g][i * SL + lo], acc[g][i]);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sh.m[w][g] = m[g];
        sh.l[w][g] = l[g];
      }
    }
  }
};

// Matrix-core form, on v_mfma_f32_16x16x4f32 with the kv head's G query
// heads as the 16 columns of the tile (columns G..15 hold zero queries and
// are dropped).  A stage is TPS tiles of 16 keys (tile t: keys 16t ..
// 16t + 15 of the stage).  Lane l works on column c = l % 16 and lane group
// g = l / 16:
//   S^T = K Q^T, summed over head_dim in MFMA steps (v, e), v < D/16, e < 4:
//     A = K[key c][d], B = Q[head c][d], d = 16v + 4g + e;
//     result register r: S[key 4g + r][head c].
//     Loading A straight from memory would make each load instruction read
//     64 bytes from each of 16 key rows, which streams about 10% slower than
//     the V pattern below; so K rows are loaded as V rows are (each lane group
//     reading 256 contiguous bytes of one row) and pass through a per-wave LDS
//     tile, 16 rows of D floats whose 16-byte segments are XOR-swizzled by row
//     (segment s of row r at s ^ (r % 16)), so that both the writes and the A
//     reads of sixteen lanes fall in distinct banks.
//   O^T += V^T P^T, MFMA steps (m, u), m < 4, u < D/16:
//     A = V[key 4g + m][d(c, u)], B = P[key 4g + m][head c] = the weight of
//     score register m, so the scores never move between lanes;
//     d(x, u) = 4x + 64(u/4) + u%4 (a V load of the sixteen lanes of a lane
//     group reads 256 contiguous bytes of one row);
//     result register r of tile u: O[head c][d(4g + r, u)].
// A lane keeps the scores of its own column, so the weights are taken in
// pass 2 (four per lane per stage) and the lane's maximum and sum need only
// the two exchanges across its lane groups.
template <int D, int G>
struct MfmaCore {
  using S = Shape<D, G>;
  static constexpr int TPS = S::STEP / 16;  // tiles per stage
  static constexpr int NK = D / 16;  // float4 loads per lane per tile (K, and V)
  static constexpr int TD = D / 16;  // output tiles of 16 head_dim values
  static constexpr int NV = TD / 4;  // V float4 per lane per key of its lane group
  static_assert(TPS * 16 == S::STEP && NK == 4 * NV && NV >= 1, "16-key tiles, head_dim >= 64");
  static_assert(Lds<D, G>::ROWS == 16, "the K tile shares the wave's accumulator slot");
  struct Stage {
    // tile t, K or V: x[t][m*NV + i] = row 16t + 4g + m, floats 4c + 64i ..
    f4 x[TPS][NK];
  };
  // float offset of 16-byte segment s of row r in the LDS K tile
  static __device__ __forceinline__ uint32_t kt_at(uint32_t r, uint32_t s) {
    return r * D + 4 * (s ^ (r % 16));
  }
  uint32_t lane, g, c;
  bool col;  // c < G: a real query head
  float qv[D / 4];
  float mx, s_new, m, l;  // this lane's head c
  f4 o[TD];

  __device__ __forceinline__ void init(uint32_t lane_) {
    lane = lane_;
    g = lane / 16;
    c = lane % 16;
    col = c < G;
  }
  __device__ __forceinline__ void load(const AttnParams& p, const UnitPlan& u, Stage& sg,
                                       uint32_t qi) const {
    const bool is_v = qi >= u.n_st;
    const uint32_t st = is_v ? qi - u.n_st : qi;
    const uint32_t last = u.k_begin + u.len - 1;
    const float* base = (is_v ? p.v_cache : p.k_cache) +
                        static_cast<uint64_t>(u.slot) * p.slot_stride + u.j * D;
#pragma unroll
    for (int t = 0; t < TPS; ++t) {
      const uint32_t kb = u.k_begin + st * S::STEP + 16 * t;
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const float* r =
            base + static_cast<uint64_t>(min(kb + 4 * g + mm, last)) * p.kv_dim + 4 * c;
#pragma unroll
        for (int i = 0; i < NV; ++i) sg.x[t][mm * NV + i] = ld4_stream(r + 64 * i);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void begin(const PrepLds<D, G>& prep, uint32_t par, bool new_key) {
    const float* qh = &prep.q[par][col ? c : 0][4 * g];
#pragma unroll
    for (int v = 0; v < NK; ++v) {
      const f4 x = ld4(qh + 16 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[4 * v + e] = col ? x[e] : 0.f;
    }
    mx = -INFINITY;
    if (new_key) {  // wave 0 of the row's last chunk scores the new key
      float sdot = 0.f;
#pragma unroll
      for (int v = 0; v < NK; ++v) {
        const f4 k = ld4(&prep.kn[par][16 * v + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sdot += qv[4 * v + e] * k[e];
      }
      sdot += __shfl_xor(sdot, 16);
      sdot += __shfl_xor(sdot, 32);
      s_new = sdot;
      mx = sdot;
    }
  }
  __device__ __forceinline__ void score(const Stage& sg, uint32_t st, const UnitPlan& u,
                                        float* sc_w, float* kt) {
#pragma unroll
    for (int t = 0; t < TPS; ++t) {
      // the tile's K rows into the LDS tile, then back as the A operand
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
#pragma unroll
        for (int i = 0; i < NV; ++i) st4(kt + kt_at(4 * g + mm, c + 16 * i), sg.x[t][mm * NV + i]);
      f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < NK; ++v) {
        const f4 a = ld4(kt + kt_at(c, 4 * v + g));
#pragma unroll
        for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], qv[4 * v + e], s, 0, 0, 0);
      }
      if (st >= u.n_full) {  // the wave's last partial stage, or a padding one
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (st * S::STEP + 16 * t + 4 * g + r >= u.len) s[r] = -INFINITY;
      }
      mx = max_nc(mx, max_nc(max_nc(s[0], s[1]), max_nc(s[2], s[3])));
      if (col) st4(sc_w + (((st * TPS + t) * 4 + g) * G + c) * 4, s);
    }
  }
  __device__ __forceinline__ void finish_max() {
    float v = mx;
    v = max_nc(v, __shfl_xor(v, 16));
    v = max_nc(v, __shfl_xor(v, 32));
    m = v;
    l = 0.f;
#pragma unroll
    for (int t = 0; t < TD; ++t) o[t] = f4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void weights(float*, uint32_t) const {}  // taken in accumulate
  __device__ __forceinline__ void accumulate(const Stage& sg, uint32_t st, const float* sc_w) {
#pragma unroll
    for (int t = 0; t < TPS; ++t) {
      const f4 sv = ld4(sc_w + (((st * TPS + t) * 4 + g) * G + (col ? c : 0)) * 4);
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = col ? fast_exp2(sv[r] - m) : 0.f;  // masked keys: exp2(-inf) = 0
        l += pr[r];
      }
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[4 * i + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(sg.x[t][mm * NV + i][e], pr[mm],
                                                                 o[4 * i + e], 0, 0, 0);
    }
  }
  __device__ __forceinline__ void add_new_key(const PrepLds<D, G>& prep, uint32_t par) {
    if (!col) return;
    const float pn = fast_exp2(s_new - m);
    if (g == 0) l += pn;  // once per head (the lane groups are summed next)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const f4 vn = ld4(&prep.vn[par][16 * g + 4 * r + 64 * i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * i + e][r] += pn * vn[e];
      }
  }
  __device__ __forceinline__ void store(Lds<D, G>& sh, uint32_t w) {
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (col) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < NV; ++i)
          st4(&sh.acc[w][c][16 * g + 4 * r + 64 * i],
              f4{o[4 * i][r], o[4 * i + 1][r], o[4 * i + 2][r], o[4 * i + 3][r]});
      if (g == 0) {
        sh.m[w][c] = m;
        sh.l[w][c] = l;
      }
    }
  }
};

template <int D, int G>
using DecodeCore = typename std::conditional<Shape<D, G>::MFMA, MfmaCore<D, G>, ValuCore<D, G>>::type;

template <int D, int G>
__device__ __forceinline__ void merge_row(const AttnParams& p, uint32_t b, uint32_t j,
                                          uint32_t n_chunks, uint32_t tid, uint32_t n_threads);

// Persistent decode kernel: as many workgroups as are resident at once.
// Workgroup g starts with unit g, then takes units from an agent-scope queue.
// Each unit asks the queue for the one after it when its second pass starts;
// wave 0 posts the answer in an LDS mailbox before its last V stage and the
// other waves read it there, so every workgroup holds at most one unit it has
// not begun, and only while its second pass runs.  Units are ordered full chunks
// first, then partial chunks longest first, so the work left at the end is
// short.  The queue word and the split rows' counters carry the launch's
// epoch, so no launch has to leave them cleared for the next.  No workgroup
// ever waits for another.  A row of one chunk is finished here; a longer row
// leaves one unnormalised partial per chunk, merged by the row's last
// workgroup.
template <int D, int G>
__global__ void __launch_bounds__((kWave * wg_waves<D, G>()))
    __attribute__((amdgpu_waves_per_eu(waves_per_eu<D, G>()))) decode_attn_kernel(const AttnArgs a) {
  using S = Shape<D, G>;
  using Core = DecodeCore<D, G>;
  constexpr int NW = S::NW, kThreads = kWave * NW;
  __shared__ Lds<D, G> sh;
  __shared__ __attribute__((aligned(16))) float sc_lds[NW][S::SCORES];
  __shared__ uint32_t mbox[2];  // next unit, by unit parity; kNoUnit until posted
  __shared__ PrepLds<D, G> prep;
  if (a.magic != kArgsMagic) return;  // argument block not delivered whole
  const AttnParams& p = a.p;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid % kWave;
  const uint32_t w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const uint32_t n_blocks = gridDim.x;
  Core cc;
  cc.init(lane);

  if (tid == 0) {
    mbox[0] = kNoUnit;
    mbox[1] = kNoUnit;
  }
  const UnitId first = locate_unit(a, blockIdx.x);  // blocks <= n_units
  UnitPlan u = plan_unit<D, G>(a, first, w);
  typename Core::Stage A, B;
  if (u.n_st > 0) cc.load(p, u, A, 0);  // A always holds the next stage
  const PrepConst<D> pconst = prep_const<D>(p, lane);
  PrepRaw<D, G> praw;
  prep_issue<D, G>(a, first, w, lane, praw);
  prep_finish<D, G>(a, first, w, lane, praw, pconst, prep, 0);
  __syncthreads();
  // The split-row partial this workgroup stored last, whose counter increment
  // is still due (workgroup-uniform).  It is made one unit later, when the
  // stores have long completed, so no unit waits for its own stores.
  bool pending = false;
  uint32_t pend_b = 0, pend_j = 0, pend_n = 0;

  for (uint32_t it = 0;; ++it) {  // workgroup-uniform
    const uint32_t par = it & 1;
    // The unit after this one is asked for when pass 2 starts and read before
    // the last V stage is consumed: the atomic's round trip hides behind the
    // V stages, and a workgroup holds a unit it has not begun only for the
    // end of the current one, so that few units sit reserved when the queue
    // runs dry.
    uint64_t ticket = 0;  // the queue word before the ask (lane 0 of wave 0)
    // (The workgroup's first ask lifts the queue word to this launch's epoch;
    // its later asks find it there.)
    auto ask_next = [&]() {
      if (tid == 0) ticket = epoch_increment(p.sched, p.epoch_tag, it == 0);
    };
    uint32_t nxt = kNoUnit;
    bool has_next = false;
    UnitId un{};
    // Wave 0 posts the next unit in the mailbox (every wave of it reads the
    // ticket register, so that no write to it is outstanding when the next
    // unit sets it again); the other waves wait for the post, which wave 0
    // makes before it waits for any other wave.  The raw next queries go out.
    auto take_next = [&]() {
      if (w == 0) {
        nxt = __builtin_amdgcn_readfirstlane(epoch_count(ticket)) + n_blocks;
        if (lane == 0) __hip_atomic_store(&mbox[par], nxt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        nxt = mbox_wait(&mbox[par]);
      }
      has_next = nxt < p.n_units;
      if (has_next) {
        un = locate_unit(a, nxt);
        prep_issue<D, G>(a, un, w, lane, praw);  // consumed after the wave merge
      }
    };

    // ---- prologue: queries and new key from LDS ------------------------------
    cc.begin(prep, par, u.new_key);

    // ---- two passes over this wave's history keys ------------------------
    // Pass 1 streams the K rows, keeps each key's scores (log2 units) in LDS
    // and the running max per head; pass 2 streams the V rows and
    // accumulates exp2(score - max) * v against the wave's final max, so no
    // accumulator is ever rescaled.  Both passes form one double-buffered
    // sequence of 2 * n_st stages.  Stage loads run one ahead of use in two
    // buffers: K stages, then V stages; stage index qi < n_st is K stage qi,
    // qi >= n_st is V stage qi - n_st.  n_st is even, so each pass starts in
    // A.  The last V stage is consumed with nothing behind it; the next unit's
    // first K stage goes out once this unit's results are stored.
    float* sc_w = &sc_lds[w][0];
    float* kt_w = &sh.acc[w][0][0];  // the K tile of the matrix-core form
    const uint32_t n_st = u.n_st;
    if (n_st > 0) {  // wave-uniform
      // pass 1
      cc.load(p, u, B, 1);
      cc.score(A, 0, u, sc_w, kt_w);
      cc.load(p, u, A, 2);  // V stage 0 when n_st == 2
      cc.score(B, 1, u, sc_w, kt_w);
      for (uint32_t st = 2; st < n_st; st += 2) {
        cc.load(p, u, B, st + 1);
        cc.score(A, st, u, sc_w, kt_w);
        cc.load(p, u, A, st + 2);  // the last trip loads V stage 0
        cc.score(B, st + 1, u, sc_w, kt_w);
      }
      cc.finish_max();
      ask_next();
      cc.weights(sc_w, n_st);
      uint32_t st = 0;
      for (; st + 2 < n_st; st += 2) {  // pass 2 while two more stages follow
        cc.load(p, u, B, n_st + st + 1);
        cc.accumulate(A, st, sc_w);
        cc.load(p, u, A, n_st + st + 2);
        cc.accumulate(B, st + 1, sc_w);
      }
      cc.load(p, u, B, n_st + st + 1);  // the last stage
      cc.accumulate(A, st, sc_w);
      take_next();
      cc.accumulate(B, st + 1, sc_w);
    } else {
      ask_next();
      take_next();
      cc.finish_max();
    }
    if (u.new_key) cc.add_new_key(prep, par);

    // ---- the wave's (acc, max, sum) per head into LDS; merge the NW waves ----
    cc.store(sh, w);
    // Publication of the previous unit's partial.  Its stores are agent-scope
    // atomic stores, written through to the level all XCDs share, and were
    // issued a whole unit ago; every wave waits for them to be acknowledged
    // (nothing else of note is in flight here), the barrier then orders all
    // waves' completed stores before the counter increment that one lane
    // issues after it.  The merging workgroup reads the partials only after
    // the increment that completes the count has returned, with agent-scope
    // atomic loads, which read that shared level.  This is the lowering of an
    // agent-scope release / acquire pair without the L2 writeback and
    // invalidate, which only non-atomic data would need.  The increment's
    // result is read at the end of this unit.
    if (pending) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    uint64_t done_prev = 0;  // the previous partial's counter word before its increment
    if (pending && tid == 0)
      done_prev = epoch_increment(&p.counters[pend_b * p.n_kv_heads + pend_j], p.epoch_tag, true);
    const uint32_t h0 = u.j * G;
    const bool split = u.n_chunks > 1;
    for (uint32_t e = tid; e < G * D; e += kThreads) {
      const uint32_t g = e / D, d = e % D;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < NW; ++v) M = fmaxf(M, sh.m[v][g]);
      float L = 0.f, Acc = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float wv = rescale(sh.m[v][g], M);
        L += sh.l[v][g] * wv;
        Acc += sh.acc[v][g][d] * wv;
      }
      if (!split) {
        // the whole row lives in this unit: add the sink and normalise
        float sa = 1.f;
        if (p.sinks) {
          const float sk = p.sinks[h0 + g] * kLog2e;
          const float mn = fmaxf(M, sk);
          sa = fast_exp2(M - mn);
          L = L * sa + (sk == -INFINITY ? 0.f : fast_exp2(sk - mn));
        }
        p.out[(static_cast<size_t>(u.b) * p.n_heads + h0 + g) * D + d] = Acc * (sa / L);
      } else {
        const size_t ph = (static_cast<size_t>(u.b) * p.max_chunks + u.chunk) * p.n_heads + h0 + g;
        store_agent(&p.part_acc[ph * D + d], Acc);
        if (d == 0) {
          store_agent(&p.part_ml[ph * 2 + 0], M);
          store_agent(&p.part_ml[ph * 2 + 1], L);
        }
      }
    }
    // the next unit's queries: their raw loads went out with take_next
    if (has_next) prep_finish<D, G>(a, un, w, lane, praw, pconst, prep, par ^ 1u);
    // the next unit's first K stage into A
    auto prefetch_next = [&]() {
      if (has_next) {
        const UnitPlan nu = plan_unit<D, G>(a, un, w);
        if (nu.n_st > 0) cc.load(p, nu, A, 0);
      }
    };
    prefetch_next();
    if (pending) {  // workgroup-uniform
      // the last workgroup of the previous partial's (row, kv head) merges
      // the row's chunks in order
      // (read through readfirstlane here, so that the wait for the atomic's
      // return stays at this use instead of right after the atomic)
      const uint32_t done_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(done_prev));
      if (tid == 0) sh.last = (epoch_count(done_lo) == pend_n - 1) ? 1u : 0u;
      __syncthreads();
      if (sh.last) merge_row<D, G>(p, pend_b, pend_j, pend_n, tid, kThreads);
    }
    pending = split;
    pend_b = u.b;
    pend_j = u.j;
    pend_n = u.n_chunks;
    if (tid == 0)  // every wave read it before the merge barrier
      __hip_atomic_store(&mbox[par], kNoUnit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();  // LDS free for the next unit
    if (!has_next) break;
    u = plan_unit<D, G>(a, un, w);
  }
  if (pending) {  // the last unit's partial: publish it now (as above)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const uint64_t done =
          epoch_increment(&p.counters[pend_b * p.n_kv_heads + pend_j], p.epoch_tag, true);
      sh.last = (epoch_count(done) == pend_n - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (sh.last) merge_row<D, G>(p, pend_b, pend_j, pend_n, tid, kThreads);
  }
}

// Merge of the partials of a row cut into several chunks, for the G query
// heads of kv head j: chunks combined in index order (one online pass, eight
// chunks' loads in flight at a time); the sink joins the denominator.
template <int D, int G>
__device__ __forceinline__ void merge_row(const AttnParams& p, uint32_t b, uint32_t j,
                                          uint32_t n_chunks, uint32_t tid, uint32_t n_threads) {
  const size_t first = static_cast<size_t>(b) * p.max_chunks;
  for (uint32_t e = tid; e < G * D; e += n_threads) {
    const uint32_t g = e / D, d = e % D;
    const uint32_t h = j * G + g;
    float M = -INFINITY, L = 0.f, Acc = 0.f;
#pragma unroll 8
    for (uint32_t c = 0; c < n_chunks; ++c) {
      const size_t ph = (first + c) * p.n_heads + h;
      const float mc = load_agent(&p.part_ml[ph * 2]);
      const float lc = load_agent(&p.part_ml[ph * 2 + 1]);
      const float ac = load_agent(&p.part_acc[ph * D + d]);
      const float mn = fmaxf(M, mc);
      const float s_old = rescale(M, mn), s_new = fast_exp2(mc - mn);
      L = L * s_old + lc * s_new;
      Acc = Acc * s_old + ac * s_new;
      M = mn;
    }
    if (p.sinks) {
      const float sk = p.sinks[h] * kLog2e;
      if (sk != -INFINITY) {
        const float mn = fmaxf(M, sk);
        const float s_old = fast_exp2(M - mn);
        L = L * s_old + fast_exp2(sk - mn);
        Acc *= s_old;
      }
    }
    p.out[(static_cast<size_t>(b) * p.n_heads + h) * D + d] = Acc / L;
  }
}

template <int D, int G>
hipError_t launch_shape(const AttnArgs& a, uint32_t blocks, hipStream_t s, hipEvent_t mark) {
  hipLaunchKernelGGL((decode_attn_kernel<D, G>), dim3(blocks), dim3(kWave * wg_waves<D, G>()), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && mark) e = hipEventRecord(mark, s);
  return e;
}

template <int D, int G>
uint32_t resident_shape() {
  static uint32_t cached = 0;  // one device per process is the supported setup
  if (!cached) {
    int per_cu = 0, cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_attn_kernel<D, G>,
                                                     kWave * wg_waves<D, G>(), 0) != hipSuccess)
      return 0;
    cached = static_cast<uint32_t>(per_cu > 0 ? per_cu : 1) * static_cast<uint32_t>(cus);
  }
  return cached;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, uint32_t G, uint32_t blocks, hipStream_t s,
                    hipEvent_t mark) {
  switch (G) {
    case 1: return launch_shape<D, 1>(a, blocks, s, mark);
    case 2: return launch_shape<D, 2>(a, blocks, s, mark);
    case 4: return launch_shape<D, 4>(a, blocks, s, mark);
    case 8: return launch_shape<D, 8>(a, blocks, s, mark);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
uint32_t resident_d(uint32_t G) {
  switch (G) {
    case 1: return resident_shape<D, 1>();
    case 2: return resident_shape<D, 2>();
    case 4: return resident_shape<D, 4>();
    case 8: return resident_shape<D, 8>();
    default: return 0;
  }
}

}  // namespace

bool decode_shape_supported(uint32_t head_dim, uint32_t group) {
  const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
  return d_ok && g_ok;
}

int launch_decode(const AttnArgs& a, uint32_t head_dim, uint32_t group, uint32_t blocks,
                  void* stream, void* after_decode) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t mark = static_cast<hipEvent_t>(after_decode);
  switch (head_dim) {
    case 64: return launch_d<64>(a, group, blocks, s, mark);
    case 128: return launch_d<128>(a, group, blocks, s, mark);
    case 256: return launch_d<256>(a, group, blocks, s, mark);
    default: return hipErrorInvalidValue;
  }
}

uint32_t resident_blocks(uint32_t head_dim, uint32_t group) {
  switch (head_dim) {
    case 64: return resident_d<64>(group);
    case 128: return resident_d<128>(group);
    case 256: return resident_d<256>(group);
    default: return 0;
  }
}

}  // namespace slotkv
