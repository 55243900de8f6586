// slot_kv_plan.cpp -- host-side validation and split-K planning of one
// decode call.  Plain C++ (no HIP), so it also runs where no GPU is present.
//
// Preconditions follow "Forward Cuda Gemma", decodeBatch: n_slots >
// max(slots), slot_ctx > max(positions); each row owns its slot, so a slot
// named twice in one batch is rejected (two rows would race on its rows).
#include <algorithm>
#include <vector>

#include "slot_kv.h"
#include "slot_kv_internal.h"

namespace slotkv {

int check_batch(uint32_t n_slots, uint32_t slot_ctx, const uint32_t* positions,
                const uint32_t* slots, uint32_t B) {
  if (B == 0) return SLOT_KV_OK;
  if (!positions || !slots) return SLOT_KV_EINVAL;
  for (uint32_t b = 0; b < B; ++b)
    if (slots[b] >= n_slots || positions[b] >= slot_ctx) return SLOT_KV_ERANGE;
  // duplicate detection: one bit per slot
  std::vector<uint64_t> seen((static_cast<size_t>(n_slots) + 63) / 64, 0);
  for (uint32_t b = 0; b < B; ++b) {
    uint64_t bit = uint64_t(1) << (slots[b] & 63);
    uint64_t& word = seen[slots[b] >> 6];
    if (word & bit) return SLOT_KV_EDUP;
    word |= bit;
  }
  return SLOT_KV_OK;
}

uint32_t count_items(const uint32_t* positions, uint32_t B, uint32_t chunk) {
  uint64_t n = 0;
  for (uint32_t b = 0; b < B; ++b) n += (uint64_t(positions[b]) + chunk) / chunk;
  return static_cast<uint32_t>(n);
}

Plan build_plan(const uint32_t* positions, const uint32_t* slots, uint32_t B,
                uint32_t chunk, RowInfo* rows, WorkItem* items) {
  Plan plan;
  uint32_t part = 0;
  for (uint32_t b = 0; b < B; ++b) {
    const uint32_t nc = (positions[b] + chunk) / chunk;  // ceil((pos+1)/chunk)
    rows[b] = RowInfo{positions[b], slots[b], nc > 1 ? part : 0u, nc};
    if (nc > 1) {
      part += nc;
      ++plan.n_split_rows;
    }
  }
  plan.n_parts = part;
  // Full chunks first (row order), then each row's shorter last chunk, the
  // longest first: equal-cost items fill the machine, short ones close the tail.
  uint32_t n = 0;
  std::vector<std::pair<uint32_t, uint32_t>> tails;  // (keys, row)
  for (uint32_t b = 0; b < B; ++b) {
    const uint32_t keys = positions[b] + 1;
    const uint32_t full = keys / chunk;
    for (uint32_t c = 0; c < full; ++c) items[n++] = WorkItem{b, c};
    if (keys % chunk) tails.emplace_back(keys % chunk, b);
  }
  std::stable_sort(tails.begin(), tails.end(),
                   [](const auto& a, const auto& b) { return a.first > b.first; });
  for (const auto& t : tails) items[n++] = WorkItem{t.second, rows[t.second].n_chunks - 1};
  plan.n_items = n;
  return plan;
}

}  // namespace slotkv
