// slot_kv_plan.cpp -- host-side validation and split-K row tables of one
// decode call.  Plain C++ (no HIP), so it also runs where no GPU is present.
//
// Preconditions follow "Forward Cuda Gemma", decodeBatch: n_slots >
// max(slots), slot_ctx > max(positions); each row owns its slot, so a slot
// named twice in one batch is rejected (two rows would race on its rows).
#include <algorithm>
#include <atomic>
#include <cstring>

#include "slot_kv.h"
#include "slot_kv_internal.h"

namespace slotkv {

bool has_duplicate(const uint32_t* slots, uint32_t n) {
  if (n < 2) return false;
  // One bit per slot, over windows of kWindow slots between the smallest and
  // the largest slot named: a fixed stack bitmap, so the check allocates
  // nothing (slot counts up to kWindow take a single pass).
  constexpr uint32_t kWindow = 1u << 16;
  uint64_t bits[kWindow / 64];
  uint32_t lo = slots[0], hi = slots[0];
  for (uint32_t i = 1; i < n; ++i) {
    lo = std::min(lo, slots[i]);
    hi = std::max(hi, slots[i]);
  }
  for (uint64_t base = lo; base <= hi; base += kWindow) {
    std::memset(bits, 0, sizeof(bits));
    for (uint32_t i = 0; i < n; ++i) {
      const uint64_t off = slots[i] - base;
      if (slots[i] < base || off >= kWindow) continue;
      uint64_t& word = bits[off >> 6];
      const uint64_t bit = uint64_t(1) << (off & 63);
      if (word & bit) return true;
      word |= bit;
    }
  }
  return false;
}

int check_batch(uint32_t n_slots, uint32_t slot_ctx, const uint32_t* positions,
                const uint32_t* slots, uint32_t B) {
  if (B == 0) return SLOT_KV_OK;
  if (!positions || !slots) return SLOT_KV_EINVAL;
  for (uint32_t b = 0; b < B; ++b)
    if (slots[b] >= n_slots || positions[b] >= slot_ctx) return SLOT_KV_ERANGE;
  return has_duplicate(slots, B) ? SLOT_KV_EDUP : SLOT_KV_OK;
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
    for (uint32_t i = work.n_full; i < std::min(work.n_full + keys / chunk, kFirstItems); ++i)
      rows.first_row[i] = static_cast<uint8_t>(b);
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
