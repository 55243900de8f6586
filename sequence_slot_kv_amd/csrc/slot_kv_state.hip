// slot_kv_state.hip -- zeroing of per-slot SSM state on admit (gfx950).
//
// "Forward Cuda": a reused slot's conv ring and recurrent state are zeroed
// in every ssm layer before a new request prefills into it, because that
// state accumulates over a sequence instead of being indexed by position.
// Each layer keeps two buffers laid out [slot][len]; slot s's region starts
// s*len floats in (the page's slot*conv_state_len*4 and slot*ssm_state_len*4
// byte offsets).
//
// The work is pure HBM writes.  One workgroup zeroes one 8 KiB tile of one
// slot's region of one segment: 256 threads, each storing two 16-byte units
// 4 KiB apart, so every store instruction of a wave covers 1 KiB of
// consecutive bytes.  Consecutive workgroups take the same tile of the
// listed slots in turn, so the writes in flight at any time are spread over
// as many regions as there are slots in the call.  Units are aligned to 16
// bytes in absolute address; a tile lying wholly inside its region is
// written without checks, and a region that starts or ends inside a unit
// (len not a multiple of 4) has its edge units written float by float.
#include <hip/hip_runtime.h>

#include "slot_kv_internal.h"

namespace slotkv {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) v4f global_v4f;
typedef __attribute__((address_space(1))) float global_f;

__global__ __launch_bounds__(kResetThreads) void state_reset_kernel(ResetArgs a) {
  // block b: tile t of the slot's tiles, for listed slot i (slot-minor order)
  const uint32_t t = blockIdx.x / a.n;
  const uint32_t i = blockIdx.x - t * a.n;
  // the segment holding tile t: the last k with segs[k].tile0 <= t
  const uint32_t lo = last_le(a.n_seg, t, [&](uint32_t k) { return a.segs[k].tile0; });
  const StateSeg seg = a.segs[lo];
  // byte addresses of the slot's region [r0, r1) and of the tile's first unit
  const uint64_t r0 = reinterpret_cast<uintptr_t>(seg.base) + uint64_t(a.slots[i]) * seg.len * 4;
  const uint64_t r1 = r0 + seg.len * 4;
  const uint64_t tile = (r0 / 16 + uint64_t(t - seg.tile0) * kResetTileUnits) * 16;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if (tile >= r0 && tile + kResetTileUnits * 16ull <= r1) {
#pragma unroll
    for (uint32_t j = 0; j < kResetUnitsPerThread; ++j)
      *reinterpret_cast<global_v4f*>(tile + (j * kResetThreads + threadIdx.x) * 16ull) = zero;
    return;
  }
  for (uint32_t j = 0; j < kResetUnitsPerThread; ++j) {
    const uint64_t p = tile + (j * kResetThreads + threadIdx.x) * 16ull;
    if (p >= r1) break;
    if (p >= r0 && p + 16 <= r1) {
      *reinterpret_cast<global_v4f*>(p) = zero;
    } else {
      for (uint32_t e = 0; e < 4; ++e)
        if (p + 4 * e >= r0 && p + 4 * e < r1) *reinterpret_cast<global_f*>(p + 4 * e) = 0.f;
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
