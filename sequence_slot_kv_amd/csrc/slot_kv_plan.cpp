// slot_kv_plan.cpp -- host-side validation and split-K row tables of one
// decode call.  Plain C++ (no HIP), so it also runs where no GPU is present.
//
// Preconditions follow "Forward Cuda Gemma", decodeBatch: n_slots >
// max(slots), slot_ctx > max(positions); each row owns its slot, so a slot
// named twice in one batch is rejected (two rows would race on its rows).
#include <algorithm>
#include <atomic>
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

LaunchWork fill_rows(LaunchRows& rows, const uint32_t* positions, const uint32_t* slots,
                     uint32_t n, uint32_t chunk) {
  LaunchWork work;
  uint32_t tails[kMaxRowsPerLaunch];
  uint32_t n_tails = 0;
  for (uint32_t b = 0; b < n; ++b) {
    const uint32_t keys = positions[b] + 1;
    rows.pos[b] = positions[b];
    rows.slot[b] = slots[b];
    rows.full_prefix[b] = work.n_full;
    work.n_full += keys / chunk;
    if (keys % chunk) tails[n_tails++] = b;
    work.max_chunks = std::max(work.max_chunks, (keys + chunk - 1) / chunk);
  }
  rows.full_prefix[n] = work.n_full;
  // longest partial chunk first; ties keep row order
  std::stable_sort(tails, tails + n_tails, [&](uint32_t x, uint32_t y) {
    return (positions[x] + 1) % chunk > (positions[y] + 1) % chunk;
  });
  for (uint32_t t = 0; t < n_tails; ++t) rows.tail_row[t] = static_cast<uint8_t>(tails[t]);
  work.n_items = work.n_full + n_tails;
  return work;
}

uint64_t next_epoch() {
  static std::atomic<uint64_t> last{0};
  uint64_t e = last.load(std::memory_order_relaxed);
  do {
    if (e >= kMaxEpoch) return 0;
  } while (!last.compare_exchange_weak(e, e + 1, std::memory_order_relaxed));
  return e + 1;
}

}  // namespace slotkv
