// slot_kv_internal.h -- types shared by the host runtime and the kernels of
// the slot-KV decode step.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef SLOT_KV_CHUNK
#define SLOT_KV_CHUNK 256  // keys per split-K chunk (multiple of 64)
#endif

namespace slotkv {

// One batch row as the kernels see it (16 bytes, one vector load).
struct RowInfo {
  uint32_t pos;        // position written and attended up to (inclusive)
  uint32_t slot;       // slot index
  uint32_t part_base;  // first partial-result index of this row (split rows)
  uint32_t n_chunks;   // ceil((pos + 1) / chunk)
};

// One split-K work item: keys [chunk*C, min((chunk+1)*C, pos+1)) of one row.
struct WorkItem {
  uint32_t row;
  uint32_t chunk;
};

// Host-side plan of one decode call.
struct Plan {
  uint32_t n_items = 0;       // work items (per kv head)
  uint32_t n_split_rows = 0;  // rows with more than one chunk
  uint32_t n_parts = 0;       // partial results per head (sum of chunks of split rows)
};

// Validation of one batch (no device access).  Returns a SLOT_KV_* status.
int check_batch(uint32_t n_slots, uint32_t slot_ctx, const uint32_t* positions,
                const uint32_t* slots, uint32_t B);

// Build the row table and the work list (full chunks first, then the partial
// last chunks, longest first).  rows must hold B entries and items at least
// count_items(...) entries.
Plan build_plan(const uint32_t* positions, const uint32_t* slots, uint32_t B,
                uint32_t chunk, RowInfo* rows, WorkItem* items);
uint32_t count_items(const uint32_t* positions, uint32_t B, uint32_t chunk);

// Kernel-side parameters of one decode launch.
struct AttnParams {
  float* k_cache;          // layer K buffer [n_slots][slot_ctx][kv_dim]
  float* v_cache;          // layer V buffer
  const float* q;          // [B][n_heads*D]
  const float* k_new;      // [B][kv_dim]
  const float* v_new;      // [B][kv_dim]
  float* out;              // [B][n_heads*D]
  float* part_acc;         // [n_parts][n_heads][D]   unnormalised partial outputs
  float* part_ml;          // [n_parts][n_heads][2]   running max (log2 units), sum
  const RowInfo* rows;     // [B]
  const WorkItem* items;   // [n_items]
  const float* q_norm_w;   // [D]
  const float* k_norm_w;   // [D]
  const float* inv_freq;   // [D/2]
  const float* sinks;      // [n_heads] or nullptr
  uint64_t slot_stride;    // slot_ctx * kv_dim (floats)
  uint32_t kv_dim;
  uint32_t n_kv_heads;
  uint32_t n_heads;
  uint32_t n_waves;        // n_items * n_kv_heads
  uint32_t chunk;
  uint32_t B;
  float eps;
  float qk_scale_log2;     // scale * log2(e)
};

// Launches (defined with the kernels).  Return a hipError_t value.
// `after_attn` (may be null) is a hipEvent_t recorded right after the fused
// kernel, before the merge kernel.
int launch_decode(const AttnParams& p, uint32_t head_dim, uint32_t group,
                  bool any_split, void* stream, void* after_attn);
bool decode_shape_supported(uint32_t head_dim, uint32_t group);

}  // namespace slotkv
