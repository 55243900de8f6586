// slot_kv_state.hip -- zeroing of per-slot SSM state on admit (gfx950).
//
// "Forward Cuda": a reused slot's conv ring and recurrent state are zeroed
// in every ssm layer before a new request prefills into it, because that
// state accumulates over a sequence instead of being indexed by position.
// Each layer keeps two buffers laid out [slot][len]; slot s's region starts
// s*len floats in (the page's slot*conv_state_len*4 and slot*ssm_state_len*4
// byte offsets).
//
// The work is pure HBM writes.  One workgroup zeroes one 16 KiB tile of one
// slot's region of one segment: 256 threads, each storing four 16-byte
// units 4 KiB apart, so every store instruction of a wave covers 1 KiB of
// consecutive bytes.  Units are aligned to 16 bytes in absolute address; a
// region that starts or ends inside a unit (len not a multiple of 4) has its
// edge units written float by float.
#include <hip/hip_runtime.h>

#include "slot_kv_internal.h"

namespace slotkv {
namespace {

__global__ __launch_bounds__(kResetThreads) void state_reset_kernel(ResetArgs a) {
  const uint32_t b = blockIdx.x;
  const uint32_t i = b / a.tiles_per_slot;
  const uint32_t t = b - i * a.tiles_per_slot;
  // the segment holding tile t: the last k with segs[k].tile0 <= t
  uint32_t lo = 0, hi = a.n_seg;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (a.segs[mid].tile0 <= t) lo = mid; else hi = mid;
  }
  const StateSeg seg = a.segs[lo];
  const uint64_t slot = a.slots[i];
  float* const start = seg.base + slot * seg.len;
  float* const end = start + seg.len;
  const uint64_t u_begin = reinterpret_cast<uintptr_t>(start) / 16;
  const uint64_t u_end = (reinterpret_cast<uintptr_t>(end) + 15) / 16;
  const uint64_t u0 = u_begin + uint64_t(t - seg.tile0) * kResetTileUnits + threadIdx.x;
#pragma unroll
  for (uint32_t j = 0; j < kResetUnitsPerThread; ++j) {
    const uint64_t u = u0 + j * kResetThreads;
    if (u >= u_end) break;
    float* p = reinterpret_cast<float*>(u * 16);
    if (p >= start && p + 4 <= end) {
      *reinterpret_cast<float4*>(p) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      for (int e = 0; e < 4; ++e)
        if (p + e >= start && p + e < end) p[e] = 0.f;
    }
  }
}

}  // namespace

int launch_state_reset(const ResetArgs& a, void* stream, void* before, void* after) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (before) {
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(before), s);
    if (e != hipSuccess) return e;
  }
  const uint32_t blocks = a.n * a.tiles_per_slot;
  hipLaunchKernelGGL(state_reset_kernel, dim3(blocks), dim3(kResetThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (after) e = hipEventRecord(static_cast<hipEvent_t>(after), s);
  return e;
}

}  // namespace slotkv
