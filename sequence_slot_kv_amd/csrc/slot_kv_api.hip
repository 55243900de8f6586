// slot_kv_api.hip -- the C ABI of include/slot_kv.h: handle, slot-KV
// allocator, 64-bit offsets, host validation, and the decode launches (the
// row table of each launch travels in the kernel arguments, so a decode
// call enqueues exactly one kernel per 256 rows and no copies).
//
// "Forward Cuda Gemma": allocSlotKv (idempotent, frees first), slotKvOffsetBytes
// ((slot*slot_ctx + pos)*kv_dim*4), decodeBatch (preconditions, per-row
// slot and position); "Forward Cuda": init (zeroed cache, inv_freq and sinks
// uploaded), allocation of the per-sequence slot state (attention KV, and a
// conv ring and recurrent state per ssm layer), their byte offsets, and the
// reset of a reused slot (nothing to clear for attention KV; the SSM state
// is zeroed).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "slot_kv.h"
#include "slot_kv_internal.h"

using slotkv::AttnArgs;
using slotkv::AttnParams;

namespace {

struct LayerState {
  uint32_t kv_dim = 0;
  float* k = nullptr;
  float* v = nullptr;
  bool configured = false;
  uint32_t n_heads = 0, n_kv_heads = 0, head_dim = 0;
  float* params = nullptr;  // q_norm_w[D] | k_norm_w[D] | inv_freq[D/2] | sinks[n_heads]
  bool has_sinks = false;
  float eps = 0.f, scale = 0.f;
  uint32_t flags = 0;  // SLOT_KV_FLAG_*
};

struct SsmLayer {
  uint32_t conv_len = 0, ssm_len = 0;  // floats per slot
  float* conv = nullptr;               // [n_slots][conv_len]
  float* ssm = nullptr;                // [n_slots][ssm_len]
};

}  // namespace

struct slot_kv {
  int device = -1;
  uint32_t n_cu = 0;  // compute units of the device
  uint32_t n_slots = 0, slot_ctx = 0;
  std::vector<LayerState> layers;
  std::vector<SsmLayer> ssm;                  // per-slot SSM state, one entry per ssm layer
  slotkv::StateSeg* state_segs = nullptr;     // device table of the reset kernel
  uint32_t state_tiles_per_slot = 0;
  float* part = nullptr;         // partial results of split rows (acc, then max/sum)
  size_t part_cap = 0;           // floats
  uint64_t* counters = nullptr;  // work queue [1], then per (row, kv head) chunk counters;
                                 // epoch-tagged words, zeroed when allocated
  size_t counters_cap = 0;       // entries
  AttnArgs args;                 // kernel arguments of the decode launch being built
  slotkv::PrefillArgs pargs;     // kernel arguments of the prefill launch being built
  slotkv::ResetArgs rargs;       // kernel arguments of the state-reset launch being built
  bool profiling = false;
  std::vector<hipEvent_t> prof_events;  // start/end pairs
  size_t prof_used = 0;                 // pairs recorded since profile_begin
  bool allocated() const { return n_slots != 0; }
};

namespace {

void free_layers(slot_kv* h) {
  for (auto& L : h->layers) {
    if (L.k) (void)hipFree(L.k);
    if (L.v) (void)hipFree(L.v);
    if (L.params) (void)hipFree(L.params);
  }
  h->layers.clear();
  for (auto& S : h->ssm) {
    if (S.conv) (void)hipFree(S.conv);
    if (S.ssm) (void)hipFree(S.ssm);
  }
  h->ssm.clear();
  if (h->state_segs) (void)hipFree(h->state_segs);
  h->state_segs = nullptr;
  h->state_tiles_per_slot = 0;
}

void free_scratch(slot_kv* h) {
  if (h->part) (void)hipFree(h->part);
  h->part = nullptr;
  h->part_cap = 0;
  if (h->counters) (void)hipFree(h->counters);
  h->counters = nullptr;
  h->counters_cap = 0;
  for (hipEvent_t e : h->prof_events) (void)hipEventDestroy(e);
  h->prof_events.clear();
  h->prof_used = 0;
  h->profiling = false;
}

// Bytes of an f32 buffer of a * b * c floats; false when the product passes
// 2^64 - 1 (nothing is written to *bytes then).
bool buffer_bytes(uint64_t a, uint64_t b, uint64_t c, uint64_t* bytes) {
  uint64_t n = 0;
  if (__builtin_mul_overflow(a, b, &n) || __builtin_mul_overflow(n, c, &n) ||
      __builtin_mul_overflow(n, uint64_t(sizeof(float)), &n))
    return false;
  if (bytes) *bytes = n;
  return true;
}

int check_layer(const slot_kv* h, uint32_t layer) {
  if (!h) return SLOT_KV_EINVAL;
  if (!h->allocated()) return SLOT_KV_ENOTALLOC;
  if (layer >= h->layers.size()) return SLOT_KV_EINVAL;
  return SLOT_KV_OK;
}

int ensure_partials(slot_kv* h, size_t floats) {
  if (h->part_cap >= floats) return SLOT_KV_OK;
  // Kernels of earlier calls may still read the old buffer.
  if (hipDeviceSynchronize() != hipSuccess) return SLOT_KV_EDEVICE;
  if (h->part) (void)hipFree(h->part);
  h->part = nullptr;
  h->part_cap = 0;
  size_t cap = 1 << 20;
  while (cap < floats) cap *= 2;
  if (hipMalloc(&h->part, cap * sizeof(float)) != hipSuccess) {
    h->part = nullptr;
    return SLOT_KV_ENOMEM;
  }
  h->part_cap = cap;
  return SLOT_KV_OK;
}

// When profiling, the next HIP event pair of the handle (created on first
// use); *e0 = *e1 = nullptr otherwise.
int prof_pair(slot_kv* h, hipEvent_t* e0, hipEvent_t* e1) {
  *e0 = *e1 = nullptr;
  if (!h->profiling) return SLOT_KV_OK;
  if (h->prof_events.size() < 2 * (h->prof_used + 1)) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess) return SLOT_KV_EDEVICE;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return SLOT_KV_EDEVICE;
    }
    h->prof_events.push_back(a);
    h->prof_events.push_back(b);
  }
  *e0 = h->prof_events[2 * h->prof_used];
  *e1 = h->prof_events[2 * h->prof_used + 1];
  ++h->prof_used;
  return SLOT_KV_OK;
}

// The work-queue and split-row counter words carry a launch epoch (see
// kEpochShift), so they are cleared only when (re)allocated: zero is epoch 0,
// older than every launch's.
int ensure_counters(slot_kv* h, size_t entries) {
  if (h->counters_cap >= entries) return SLOT_KV_OK;
  if (hipDeviceSynchronize() != hipSuccess) return SLOT_KV_EDEVICE;
  if (h->counters) (void)hipFree(h->counters);
  h->counters = nullptr;
  h->counters_cap = 0;
  void* c = nullptr;
  if (hipMalloc(&c, entries * sizeof(uint64_t)) != hipSuccess) return SLOT_KV_ENOMEM;
  if (hipMemset(c, 0, entries * sizeof(uint64_t)) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(c);
    return SLOT_KV_EDEVICE;
  }
  h->counters = static_cast<uint64_t*>(c);
  h->counters_cap = entries;
  return SLOT_KV_OK;
}

// ---------------------------------------------------------------- fixed scratch
// The scratch of slot_decode_attn_noalloc: one array per device, held until
// the process ends, shared by every call on that device.  Its first
// kScratchCounterBytes hold the queue word and the split-row counters
// (epoch-tagged, so they start valid at zero and are never cleared), the rest
// the partials.  Host code never uses the array's name as an address: the
// address comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr size_t kScratchCounterBytes = size_t(256) << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // per device; null until looked up

// Looks up this device's scratch address (the device is current); once per
// device.
void scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev]) return;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr)
    g_scratch_ptr[dev] = ptr;
  else
    (void)hipGetLastError();  // the allocation-free decode then returns EDEVICE
}

void* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int slot_kv_create(slot_kv** out) {
  if (!out) return SLOT_KV_EINVAL;
  *out = new (std::nothrow) slot_kv();
  return *out ? SLOT_KV_OK : SLOT_KV_ENOMEM;
}

void slot_kv_destroy(slot_kv* h) {
  if (!h) return;
  if (h->device >= 0) (void)hipDeviceSynchronize();
  free_layers(h);
  free_scratch(h);
  delete h;
}

int slot_state_alloc(slot_kv* h, uint32_t n_slots, uint32_t slot_ctx, const uint32_t* kv_dims,
                     uint32_t n_attn_layers, const uint32_t* conv_state_len,
                     const uint32_t* ssm_state_len, uint32_t n_ssm_layers) {
  if (!h || n_slots == 0 || slot_ctx == 0 || n_attn_layers + uint64_t(n_ssm_layers) == 0)
    return SLOT_KV_EINVAL;
  if (n_attn_layers && !kv_dims) return SLOT_KV_EINVAL;
  if (n_ssm_layers && (!conv_state_len || !ssm_state_len)) return SLOT_KV_EINVAL;
  // Every buffer's byte size is checked here, before any HIP call: a K/V
  // buffer is n_slots * slot_ctx * kv_dim * 4 bytes, three 32-bit factors
  // whose product can pass 2^64 (and would wrap to a small allocation that
  // the offsets then overrun); a state buffer is n_slots * len * 4.
  for (uint32_t L = 0; L < n_attn_layers; ++L)
    if (kv_dims[L] == 0 || !buffer_bytes(n_slots, slot_ctx, kv_dims[L], nullptr))
      return SLOT_KV_EINVAL;
  uint64_t tiles = 0;
  for (uint32_t L = 0; L < n_ssm_layers; ++L) {
    if (conv_state_len[L] == 0 || ssm_state_len[L] == 0) return SLOT_KV_EINVAL;
    if (!buffer_bytes(n_slots, 1, conv_state_len[L], nullptr) ||
        !buffer_bytes(n_slots, 1, ssm_state_len[L], nullptr))
      return SLOT_KV_EINVAL;
    tiles += slotkv::reset_tiles(conv_state_len[L]) + slotkv::reset_tiles(ssm_state_len[L]);
  }
  // one slot's reset must fit one grid (and tile0 must fit 32 bits)
  if (tiles > 0x7fffffffu) return SLOT_KV_EINVAL;
  // Idempotent: drop any earlier allocation (and its layer configurations).
  if (h->device >= 0) (void)hipDeviceSynchronize();
  free_layers(h);
  free_scratch(h);
  h->n_slots = h->slot_ctx = 0;
  int dev = 0;
  int cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SLOT_KV_EDEVICE;
  h->device = dev;
  h->n_cu = static_cast<uint32_t>(std::max(cus, 1));
  scratch_setup(dev);  // the allocation-free decode's scratch on this device
  // Everything is allocated into h's vectors as it goes, so a failure part
  // way frees exactly what was made.
  auto fail = [h](int rc) {
    (void)hipGetLastError();
    free_layers(h);
    return rc;
  };
  // "Forward Cuda", init: the KV cache and the SSM state start zeroed.
  auto zeroed = [](size_t bytes, float** out) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return SLOT_KV_ENOMEM;
    *out = static_cast<float*>(p);
    return hipMemset(p, 0, bytes) == hipSuccess ? SLOT_KV_OK : SLOT_KV_EDEVICE;
  };
  h->layers.resize(n_attn_layers);
  for (uint32_t L = 0; L < n_attn_layers; ++L) {
    uint64_t bytes = 0;
    (void)buffer_bytes(n_slots, slot_ctx, kv_dims[L], &bytes);  // checked above
    h->layers[L].kv_dim = kv_dims[L];
    int rc = zeroed(bytes, &h->layers[L].k);
    if (!rc) rc = zeroed(bytes, &h->layers[L].v);
    if (rc) return fail(rc);
  }
  h->ssm.resize(n_ssm_layers);
  std::vector<slotkv::StateSeg> segs;
  uint32_t tile0 = 0;
  for (uint32_t L = 0; L < n_ssm_layers; ++L) {
    SsmLayer& S = h->ssm[L];
    S.conv_len = conv_state_len[L];
    S.ssm_len = ssm_state_len[L];
    uint64_t conv_bytes = 0, ssm_bytes = 0;  // checked above
    (void)buffer_bytes(n_slots, 1, S.conv_len, &conv_bytes);
    (void)buffer_bytes(n_slots, 1, S.ssm_len, &ssm_bytes);
    int rc = zeroed(conv_bytes, &S.conv);
    if (!rc) rc = zeroed(ssm_bytes, &S.ssm);
    if (rc) return fail(rc);
    segs.push_back({S.conv, S.conv_len, tile0, 0});
    tile0 += static_cast<uint32_t>(slotkv::reset_tiles(S.conv_len));
    segs.push_back({S.ssm, S.ssm_len, tile0, 0});
    tile0 += static_cast<uint32_t>(slotkv::reset_tiles(S.ssm_len));
  }
  if (!segs.empty()) {
    const size_t bytes = segs.size() * sizeof(slotkv::StateSeg);
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return fail(SLOT_KV_ENOMEM);
    h->state_segs = static_cast<slotkv::StateSeg*>(p);
    if (hipMemcpy(p, segs.data(), bytes, hipMemcpyHostToDevice) != hipSuccess)
      return fail(SLOT_KV_EDEVICE);
    h->state_tiles_per_slot = tile0;
  }
  if (hipDeviceSynchronize() != hipSuccess) return fail(SLOT_KV_EDEVICE);
  h->n_slots = n_slots;
  h->slot_ctx = slot_ctx;
  return SLOT_KV_OK;
}

int slot_kv_alloc(slot_kv* h, uint32_t n_slots, uint32_t slot_ctx, const uint32_t* kv_dims,
                  uint32_t n_layers) {
  if (!h || !kv_dims || n_layers == 0) return SLOT_KV_EINVAL;
  return slot_state_alloc(h, n_slots, slot_ctx, kv_dims, n_layers, nullptr, nullptr, 0);
}

int slot_kv_set_layer(slot_kv* h, uint32_t layer, uint32_t n_heads, uint32_t n_kv_heads,
                      uint32_t head_dim, const float* q_norm_w, const float* k_norm_w,
                      const float* inv_freq, const float* sinks, float eps, float scale) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  LayerState& L = h->layers[layer];
  if (!q_norm_w || !k_norm_w || !inv_freq) return SLOT_KV_EINVAL;
  if (n_heads == 0 || n_kv_heads == 0 || head_dim == 0 || n_heads % n_kv_heads != 0)
    return SLOT_KV_EINVAL;
  if (static_cast<uint64_t>(n_kv_heads) * head_dim != L.kv_dim) return SLOT_KV_EINVAL;
  if (!slotkv::decode_shape_supported(head_dim, n_heads / n_kv_heads)) return SLOT_KV_EINVAL;
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(scale)) return SLOT_KV_EINVAL;
  const size_t D = head_dim;
  const size_t n = 2 * D + D / 2 + n_heads;
  std::vector<float> host(n, 0.f);
  std::memcpy(host.data(), q_norm_w, D * sizeof(float));
  std::memcpy(host.data() + D, k_norm_w, D * sizeof(float));
  std::memcpy(host.data() + 2 * D, inv_freq, D / 2 * sizeof(float));
  if (sinks) std::memcpy(host.data() + 2 * D + D / 2, sinks, n_heads * sizeof(float));
  float* dev = nullptr;
  if (L.params) {
    if (hipDeviceSynchronize() != hipSuccess) return SLOT_KV_EDEVICE;
    (void)hipFree(L.params);
    L.params = nullptr;
    L.configured = false;
  }
  if (hipMalloc(&dev, n * sizeof(float)) != hipSuccess) return SLOT_KV_ENOMEM;
  if (hipMemcpy(dev, host.data(), n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dev);
    return SLOT_KV_EDEVICE;
  }
  L.params = dev;
  L.n_heads = n_heads;
  L.n_kv_heads = n_kv_heads;
  L.head_dim = head_dim;
  L.has_sinks = sinks != nullptr;
  L.eps = eps;
  L.scale = scale;
  L.flags = 0;
  L.configured = true;
  return SLOT_KV_OK;
}

int slot_kv_set_layer_flags(slot_kv* h, uint32_t layer, uint32_t flags) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  LayerState& L = h->layers[layer];
  const uint32_t known =
      SLOT_KV_FLAG_V_NORM | SLOT_KV_FLAG_ROPE_INTERLEAVED | SLOT_KV_FLAG_NORM_ONE_PLUS_W;
  if (!L.configured || (flags & ~known)) return SLOT_KV_EINVAL;
  L.flags = flags;
  return SLOT_KV_OK;
}

int slot_kv_offset_bytes(const slot_kv* h, uint32_t layer, uint32_t slot, uint32_t pos,
                         uint64_t* out_bytes) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (!out_bytes) return SLOT_KV_EINVAL;
  if (slot >= h->n_slots || pos >= h->slot_ctx) return SLOT_KV_ERANGE;
  *out_bytes = (static_cast<uint64_t>(slot) * h->slot_ctx + pos) *
               static_cast<uint64_t>(h->layers[layer].kv_dim) * sizeof(float);
  return SLOT_KV_OK;
}

int slot_reset_batch(slot_kv* h, const uint32_t* slots, uint32_t n, void* stream) {
  if (!h) return SLOT_KV_EINVAL;
  if (!h->allocated()) return SLOT_KV_OK;  // no-op when nothing is allocated
  if (n && !slots) return SLOT_KV_EINVAL;
  for (uint32_t i = 0; i < n; ++i)
    if (slots[i] >= h->n_slots) return SLOT_KV_ERANGE;
  // Attention KV needs no clearing; only ssm layers have state to zero.
  if (h->ssm.empty() || n == 0) return SLOT_KV_OK;
  slotkv::ResetArgs& a = h->rargs;
  a.segs = h->state_segs;
  a.n_seg = static_cast<uint32_t>(2 * h->ssm.size());
  a.tiles_per_slot = h->state_tiles_per_slot;
  // slots per launch: at most kMaxResetPerLaunch, and a grid below 2^31
  const uint32_t per = static_cast<uint32_t>(std::min<uint64_t>(
      slotkv::kMaxResetPerLaunch, std::max<uint64_t>(1, 0x7fffffffu / a.tiles_per_slot)));
  for (uint32_t i0 = 0; i0 < n; i0 += per) {
    a.n = std::min(per, n - i0);
    std::memcpy(a.slots, slots + i0, a.n * sizeof(uint32_t));
    hipEvent_t e0, e1;
    int rc = prof_pair(h, &e0, &e1);
    if (rc) return rc;
    if (slotkv::launch_state_reset(a, stream, e0, e1) != hipSuccess) return SLOT_KV_EDEVICE;
  }
  return SLOT_KV_OK;
}

int slot_reset(slot_kv* h, uint32_t slot, void* stream) {
  return slot_reset_batch(h, &slot, 1, stream);
}

// Offset of `slot` in ssm layer `ssm_layer`'s conv buffer (which = 0) or
// recurrent-state buffer (which = 1).
static int state_offset(const slot_kv* h, uint32_t ssm_layer, uint32_t slot, uint32_t which,
                        uint64_t* out_bytes) {
  if (!h) return SLOT_KV_EINVAL;
  if (!h->allocated()) return SLOT_KV_ENOTALLOC;
  if (ssm_layer >= h->ssm.size() || which > 1 || !out_bytes) return SLOT_KV_EINVAL;
  if (slot >= h->n_slots) return SLOT_KV_ERANGE;
  const SsmLayer& S = h->ssm[ssm_layer];
  *out_bytes = static_cast<uint64_t>(slot) * (which ? S.ssm_len : S.conv_len) * sizeof(float);
  return SLOT_KV_OK;
}

int slot_conv_offset_bytes(const slot_kv* h, uint32_t ssm_layer, uint32_t slot,
                           uint64_t* out_bytes) {
  return state_offset(h, ssm_layer, slot, 0, out_bytes);
}

int slot_ssm_offset_bytes(const slot_kv* h, uint32_t ssm_layer, uint32_t slot,
                          uint64_t* out_bytes) {
  return state_offset(h, ssm_layer, slot, 1, out_bytes);
}

int slot_state_ptrs(const slot_kv* h, uint32_t ssm_layer, float** conv, float** ssm) {
  if (!h) return SLOT_KV_EINVAL;
  if (!h->allocated()) return SLOT_KV_ENOTALLOC;
  if (ssm_layer >= h->ssm.size()) return SLOT_KV_EINVAL;
  if (conv) *conv = h->ssm[ssm_layer].conv;
  if (ssm) *ssm = h->ssm[ssm_layer].ssm;
  return SLOT_KV_OK;
}

int slot_kv_check_batch(uint32_t n_slots, uint32_t slot_ctx, const uint32_t* positions,
                        const uint32_t* slots, uint32_t B, uint32_t chunk_keys,
                        uint32_t* n_items, uint32_t* n_split_rows) {
  if (chunk_keys == 0) return SLOT_KV_EINVAL;
  int rc = slotkv::check_batch(n_slots, slot_ctx, positions, slots, B);
  if (rc) return rc;
  uint32_t items = 0, split = 0;
  for (uint32_t b = 0; b < B; ++b) {
    const uint32_t nc = static_cast<uint32_t>((uint64_t(positions[b]) + chunk_keys) / chunk_keys);
    items += nc;
    split += nc > 1;
  }
  if (n_items) *n_items = items;
  if (n_split_rows) *n_split_rows = split;
  return SLOT_KV_OK;
}

uint32_t slot_kv_chunk_keys(void) { return SLOT_KV_CHUNK; }

}  // extern "C"

namespace {

// Scratch a decode call needs: the partials of its largest launch (floats)
// and the queue word plus the per-(row, kv head) counters (64-bit words).
struct DecodeNeeds {
  size_t part_floats = 0;
  size_t counter_words = 0;
};

// Validates a decode call (nothing is enqueued) and sizes its scratch.
int plan_decode(const slot_kv* h, uint32_t layer, const float* q, const float* k_new,
                const float* v_new, const uint32_t* positions, const uint32_t* slots,
                uint32_t B, const float* out, DecodeNeeds* needs) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  const LayerState& L = h->layers[layer];
  if (!L.configured) return SLOT_KV_EINVAL;
  if (B == 0) return SLOT_KV_OK;
  if (!q || !k_new || !v_new || !out) return SLOT_KV_EINVAL;
  rc = slotkv::check_batch(h->n_slots, h->slot_ctx, positions, slots, B);
  if (rc) return rc;
  const uint32_t C = SLOT_KV_CHUNK;
  const uint32_t R = slotkv::kMaxRowsPerLaunch;
  size_t part_floats = 0;
  for (uint32_t r0 = 0; r0 < B; r0 += R) {
    const uint32_t n = std::min(B - r0, R);
    uint64_t items = 0, max_chunks = 0;
    for (uint32_t b = r0; b < r0 + n; ++b) {
      const uint64_t nc = (uint64_t(positions[b]) + C) / C;
      items += nc;
      max_chunks = std::max(max_chunks, nc);
    }
    // a launch's units are counted below the epoch bits of the queue word
    // (no cache that fits a GPU's memory comes near this)
    if (items * L.n_kv_heads > slotkv::kCountMask) return SLOT_KV_EINVAL;
    part_floats = std::max(part_floats,
                           static_cast<size_t>(n * max_chunks) * L.n_heads * (L.head_dim + 2));
  }
  needs->part_floats = part_floats;
  needs->counter_words = 1 + static_cast<size_t>(R) * L.n_kv_heads;
  return SLOT_KV_OK;
}

// Enqueues a validated decode call (B > 0): one launch of the fused kernel
// per kMaxRowsPerLaunch rows, its partials in `part` and its queue word and
// counters in `counters` (scratch sized by plan_decode).  With `profile`, the
// handle's event pairs are recorded around each launch.
int run_decode(slot_kv* h, uint32_t layer, const float* q, const float* k_new,
               const float* v_new, const uint32_t* positions, const uint32_t* slots, uint32_t B,
               float* out, void* stream, float* part, uint64_t* counters, bool profile) {
  const LayerState& L = h->layers[layer];
  const uint32_t C = SLOT_KV_CHUNK;
  const size_t D = L.head_dim;
  const uint32_t R = slotkv::kMaxRowsPerLaunch;
  const uint32_t G = L.n_heads / L.n_kv_heads;
  const uint32_t resident = slotkv::resident_blocks(L.head_dim, G);
  if (resident == 0) return SLOT_KV_EDEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnArgs& a = h->args;
  a.magic = slotkv::kArgsMagic;
  AttnParams& p = a.p;
  p.k_cache = L.k;
  p.v_cache = L.v;
  p.sched = counters;
  p.counters = counters + 1;
  p.q_norm_w = L.params;
  p.k_norm_w = L.params + D;
  p.inv_freq = L.params + 2 * D;
  p.sinks = L.has_sinks ? L.params + 2 * D + D / 2 : nullptr;
  p.slot_stride = static_cast<uint64_t>(h->slot_ctx) * L.kv_dim;
  p.kv_dim = L.kv_dim;
  p.n_kv_heads = L.n_kv_heads;
  p.n_heads = L.n_heads;
  p.chunk = C;
  p.eps = L.eps;
  p.qk_scale_log2 = L.scale * 1.4426950408889634f;
  p.flags = L.flags;
  const size_t qd = static_cast<size_t>(L.n_heads) * D;
  for (uint32_t r0 = 0; r0 < B; r0 += R) {  // rows are independent: launch in slices
    const uint32_t n = std::min(B - r0, R);
    const slotkv::LaunchWork work = slotkv::fill_rows(a.rows, positions + r0, slots + r0, n, C);
    p.n_rows = n;
    p.n_full = work.n_full;
    p.n_units = work.n_items * L.n_kv_heads;
    p.max_chunks = work.max_chunks;
    p.q = q + r0 * qd;
    p.k_new = k_new + static_cast<size_t>(r0) * L.kv_dim;
    p.v_new = v_new + static_cast<size_t>(r0) * L.kv_dim;
    p.out = out + r0 * qd;
    p.part_acc = part;
    p.part_ml = part + static_cast<size_t>(n) * work.max_chunks * L.n_heads * D;
    const uint64_t epoch = slotkv::next_epoch();
    if (epoch == 0) return SLOT_KV_EDEVICE;  // 2^40 launches in one process
    p.epoch_tag = epoch << slotkv::kEpochShift;

    hipEvent_t ev_start = nullptr, ev_end = nullptr;
    if (profile) {
      const int rc = prof_pair(h, &ev_start, &ev_end);
      if (rc) return rc;
    }
    if (ev_start && hipEventRecord(ev_start, s) != hipSuccess) return SLOT_KV_EDEVICE;
    const uint32_t blocks = std::min(p.n_units, resident);
    if (slotkv::launch_decode(a, L.head_dim, G, blocks, stream, ev_end) != hipSuccess)
      return SLOT_KV_EDEVICE;
  }
  return SLOT_KV_OK;
}

}  // namespace

extern "C" {

int slot_decode_attn(slot_kv* h, uint32_t layer, const float* q, const float* k_new,
                     const float* v_new, const uint32_t* positions, const uint32_t* slots,
                     uint32_t B, float* out, void* stream) {
  DecodeNeeds needs;
  int rc = plan_decode(h, layer, q, k_new, v_new, positions, slots, B, out, &needs);
  if (rc || B == 0) return rc;
  // Size the scratch for the largest launch before enqueueing anything.
  rc = ensure_partials(h, needs.part_floats);
  if (rc) return rc;
  rc = ensure_counters(h, needs.counter_words);
  if (rc) return rc;
  return run_decode(h, layer, q, k_new, v_new, positions, slots, B, out, stream, h->part,
                    h->counters, h->profiling);
}

int slot_decode_attn_noalloc(slot_kv* h, uint32_t layer, const float* q, const float* k_new,
                             const float* v_new, const uint32_t* positions,
                             const uint32_t* slots, uint32_t B, float* out, void* stream) {
  DecodeNeeds needs;
  int rc = plan_decode(h, layer, q, k_new, v_new, positions, slots, B, out, &needs);
  if (rc || B == 0) return rc;
  if (needs.counter_words * sizeof(uint64_t) > kScratchCounterBytes ||
      needs.part_floats * sizeof(float) > kScratchBytes - kScratchCounterBytes)
    return SLOT_KV_ESCRATCH;
  unsigned char* base = static_cast<unsigned char*>(scratch_of(h->device));
  if (!base) return SLOT_KV_EDEVICE;  // the look-up at allocation failed
  return run_decode(h, layer, q, k_new, v_new, positions, slots, B, out, stream,
                    reinterpret_cast<float*>(base + kScratchCounterBytes),
                    reinterpret_cast<uint64_t*>(base), false);
}

namespace {

// One sequence of a prefill / verify call: `len` rows starting at row `row`
// of the call's q / k_new / v_new / out, at positions pos0 .. pos0+len-1.
struct SeqRows {
  uint32_t slot, pos0, len, row;
};

// Validated sequences of a call (no zero-length ones) -> launches of at most
// kMaxSeqPerLaunch sequences, each sequence-major in the caller's buffers.
// One launch of a prefill / verify: sequences [s0, s0 + n) of the call.
struct PrefillLaunch {
  size_t s0 = 0;
  uint32_t n = 0, rows = 0;
  uint32_t split_keys = 0;  // keys per chunk; 0: whole key ranges (tiled only)
  uint32_t n_items = 0;     // partial items
};

// Tiled workgroups of a launch (per kv head), and its partial items when cut
// into chunks of ck keys.
void tiled_counts(const std::vector<SeqRows>& seqs, size_t s0, uint32_t n, uint32_t G,
                  uint32_t ck, uint64_t* groups, uint64_t* items_per_head) {
  *groups = *items_per_head = 0;
  const uint64_t rpg = slotkv::kPrefillRowsPerGroup;
  for (size_t i = s0; i < s0 + n; ++i) {
    const uint64_t tiles = (uint64_t(seqs[i].len) * G + 15) / 16;
    const uint64_t n_ck = ck ? (uint64_t(seqs[i].pos0) + seqs[i].len + ck - 1) / ck : 1;
    *groups += (tiles * 16 + rpg - 1) / rpg * n_ck;
    *items_per_head += tiles * n_ck;
  }
}

// Keys per chunk of a tiled launch whose workgroups are too few to fill the
// chip: about kChunkTargetGroups workgroups, chunks a multiple of 64 keys
// (0: no cut).
uint32_t plan_tiled_chunks(const std::vector<SeqRows>& seqs, size_t s0, uint32_t n, uint32_t G,
                           uint32_t n_kv_heads, uint32_t* n_items) {
  uint64_t groups, items;
  tiled_counts(seqs, s0, n, G, 0, &groups, &items);
  groups *= n_kv_heads;
  if (groups == 0 || groups >= slotkv::kChunkBelowGroups) return 0;
  uint64_t max_keys = 0;
  for (size_t i = s0; i < s0 + n; ++i)
    max_keys = std::max<uint64_t>(max_keys, uint64_t(seqs[i].pos0) + seqs[i].len);
  const uint64_t want = (slotkv::kChunkTargetGroups + groups - 1) / groups;
  const uint64_t ck = ((max_keys + want - 1) / want + 63) / 64 * 64;
  if (ck >= max_keys) return 0;
  tiled_counts(seqs, s0, n, G, static_cast<uint32_t>(ck), &groups, &items);
  items *= n_kv_heads;
  if (items > slotkv::kMaxSplitItems) return 0;
  *n_items = static_cast<uint32_t>(items);
  return static_cast<uint32_t>(ck);
}

// Keys per chunk of a split-K launch: the smallest power-of-two multiple of
// kSplitMinKeys that keeps its work items within kMaxSplitItems (0 if none).
uint32_t plan_split(const std::vector<SeqRows>& seqs, size_t s0, uint32_t n, uint32_t G,
                    uint32_t n_kv_heads, uint32_t* n_items) {
  uint64_t max_keys = 0;
  for (size_t i = s0; i < s0 + n; ++i)
    max_keys = std::max<uint64_t>(max_keys, uint64_t(seqs[i].pos0) + seqs[i].len);
  for (uint64_t ck = slotkv::kSplitMinKeys;; ck *= 2) {
    uint64_t items = 0;  // one per workgroup of kSplitChunksPerGroup chunks
    for (size_t i = s0; i < s0 + n; ++i) {
      const uint64_t tiles = (uint64_t(seqs[i].len) * G + 15) / 16;
      items += tiles * slotkv::split_groups(seqs[i].pos0 + seqs[i].len, static_cast<uint32_t>(ck)) *
               n_kv_heads;
    }
    if (items <= slotkv::kMaxSplitItems) {
      *n_items = static_cast<uint32_t>(items);
      return static_cast<uint32_t>(ck);
    }
    if (ck >= max_keys) return 0;
  }
}


int run_prefill(slot_kv* h, uint32_t layer, const float* q, const float* k_new,
                const float* v_new, float* out, const std::vector<SeqRows>& seqs, void* stream) {
  LayerState& L = h->layers[layer];
  const uint32_t G = L.n_heads / L.n_kv_heads;
  if (!slotkv::decode_shape_supported(L.head_dim, G)) return SLOT_KV_EINVAL;
  const size_t D = L.head_dim;
  const uint32_t M = slotkv::kMaxSeqPerLaunch;
  // Sequences with few query rows per kv head (a verify of k rows, a short
  // prefill) run the split-K attention; others the tiled one, whose
  // workgroups share each K/V block between four tiles.
  bool split = true;
  for (const SeqRows& r : seqs) split = split && uint64_t(r.len) * G <= slotkv::kSplitMaxRows;
  // plan every launch, then size the scratch (the rows' query table, then
  // the key-chunked partials) for the largest one, before any enqueue
  std::vector<PrefillLaunch> plan;
  size_t scratch = 0;
  for (size_t s0 = 0; s0 < seqs.size(); s0 += M) {
    PrefillLaunch pl;
    pl.s0 = s0;
    pl.n = static_cast<uint32_t>(std::min<size_t>(seqs.size() - s0, M));
    for (size_t i = s0; i < s0 + pl.n; ++i) pl.rows += seqs[i].len;
    if (split) pl.split_keys = plan_split(seqs, s0, pl.n, G, L.n_kv_heads, &pl.n_items);
    plan.push_back(pl);
  }
  // one call takes one kernel: split-K only if every launch can
  for (const PrefillLaunch& pl : plan) split = split && pl.split_keys != 0;
  for (PrefillLaunch& pl : plan) {
    if (!split)
      pl.split_keys = plan_tiled_chunks(seqs, pl.s0, pl.n, G, L.n_kv_heads, &pl.n_items);
    if (!pl.split_keys) pl.n_items = 0;
    scratch = std::max(scratch, size_t(pl.rows) * 2 * D + size_t(pl.n_items) * 16 * (D + 2));
  }
  int rc = ensure_partials(h, scratch);
  if (rc) return rc;

  slotkv::PrefillArgs& a = h->pargs;
  a.magic = slotkv::kArgsMagic;
  slotkv::PrefillParams& p = a.p;
  p.k_cache = L.k;
  p.v_cache = L.v;
  p.rope = h->part;
  p.q_norm_w = L.params;
  p.k_norm_w = L.params + D;
  p.inv_freq = L.params + 2 * D;
  p.sinks = L.has_sinks ? L.params + 2 * D + D / 2 : nullptr;
  p.slot_stride = static_cast<uint64_t>(h->slot_ctx) * L.kv_dim;
  p.kv_dim = L.kv_dim;
  p.n_heads = L.n_heads;
  p.n_kv_heads = L.n_kv_heads;
  p.eps = L.eps;
  p.qk_scale_log2 = L.scale * 1.4426950408889634f;
  p.flags = L.flags;
  const size_t qd = static_cast<size_t>(L.n_heads) * D;
  for (const PrefillLaunch& pl : plan) {
    const uint32_t n = pl.n;
    const uint32_t first_row = seqs[pl.s0].row;
    uint32_t rows = 0;
    for (uint32_t i = 0; i < n; ++i) {
      const SeqRows& r = seqs[pl.s0 + i];
      a.s.slot[i] = r.slot;
      a.s.pos0[i] = r.pos0;
      a.s.len[i] = r.len;
      a.s.row_off[i] = rows;
      rows += r.len;
    }
    a.s.row_off[n] = rows;
    // partial items (key-chunked launches)
    const uint32_t ck = pl.split_keys;
    uint32_t items = 0;
    for (uint32_t i = 0; i < n; ++i) {
      a.s.item_off[i] = items;
      const uint32_t keys = a.s.pos0[i] + a.s.len[i];
      if (ck)  // split-K: per group of chunks; chunked tiled: per chunk
        items += (a.s.len[i] * G + 15) / 16 *
                 (split ? slotkv::split_groups(keys, ck) : (keys + ck - 1) / ck) * L.n_kv_heads;
    }
    a.s.item_off[n] = items;
    if (split) slotkv::order_split_groups(a.s, n, G, L.n_kv_heads, ck);
    p.part = ck ? h->part + size_t(pl.rows) * 2 * D : nullptr;
    p.n_items = items;
    p.split_keys = ck;
    p.n_groups = 0;
    p.band = 0;
    if (!split) {  // tiled workgroups, heaviest sequence first
      std::vector<uint64_t> work(n);
      for (uint32_t i = 0; i < n; ++i) {
        a.s.by_work[i] = static_cast<uint8_t>(i);
        work[i] = static_cast<uint64_t>(a.s.len[i]) * (2ull * a.s.pos0[i] + a.s.len[i]);
      }
      std::stable_sort(a.s.by_work, a.s.by_work + n,
                       [&](uint32_t x, uint32_t y) { return work[x] > work[y]; });
      uint32_t groups = 0;
      for (uint32_t k = 0; k < n; ++k) {
        const uint32_t i = a.s.by_work[k];
        a.s.grp_off[k] = groups;
        const uint32_t tiles = (a.s.len[i] * G + 15) / 16;
        const uint32_t n_ck = ck ? (a.s.pos0[i] + a.s.len[i] + ck - 1) / ck : 1;
        groups += (tiles * 16 + slotkv::kPrefillRowsPerGroup - 1) /
                  slotkv::kPrefillRowsPerGroup * n_ck;
      }
      a.s.grp_off[n] = groups;
      p.n_groups = groups;
      // Launch bands of one workgroup per CU: the kv heads of a group rank
      // are launched together, so a band is n_cu / n_kv_heads ranks.
      p.band = std::max<uint32_t>(1, h->n_cu / L.n_kv_heads);
    }
    p.n_seq = n;
    p.n_rows = rows;
    // prep: one key head per wave while that keeps the workgroups few (up
    // to about 2048, 8 per CU); more per wave for long calls
    {
      const uint32_t n_vec4 = (L.n_kv_heads + 3) / 4;
      p.prep_vpw = std::max<uint32_t>(1, std::min<uint32_t>(n_vec4, rows * n_vec4 / 2048));
    }
    p.q = q + first_row * qd;
    p.k_new = k_new + static_cast<size_t>(first_row) * L.kv_dim;
    p.v_new = v_new + static_cast<size_t>(first_row) * L.kv_dim;
    p.out = out + first_row * qd;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    rc = prof_pair(h, &e0, &e1);
    if (rc) return rc;
    if (slotkv::launch_prefill(a, L.head_dim, G, split, stream, e0, e1) != hipSuccess)
      return SLOT_KV_EDEVICE;
  }
  return SLOT_KV_OK;
}

}  // namespace

int slot_prefill_attn(slot_kv* h, uint32_t layer, const float* q, const float* k_new,
                      const float* v_new, uint32_t slot, uint32_t pos0, uint32_t T,
                      float* out, void* stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  LayerState& L = h->layers[layer];
  if (!L.configured) return SLOT_KV_EINVAL;
  if (T == 0) return SLOT_KV_OK;
  if (!q || !k_new || !v_new || !out) return SLOT_KV_EINVAL;
  if (slot >= h->n_slots || static_cast<uint64_t>(pos0) + T > h->slot_ctx) return SLOT_KV_ERANGE;
  if (static_cast<uint64_t>(T) * (L.n_heads + L.n_kv_heads) >= (uint64_t(1) << 31))
    return SLOT_KV_EINVAL;  // keeps the kernels' 32-bit row and tile counts exact
  return run_prefill(h, layer, q, k_new, v_new, out, {SeqRows{slot, pos0, T, 0}}, stream);
}

int slot_verify_attn(slot_kv* h, uint32_t layer, const float* q, const float* k_new,
                     const float* v_new, const uint32_t* slots, const uint32_t* pos0,
                     const uint32_t* ks, uint32_t n_seq, float* out, void* stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  LayerState& L = h->layers[layer];
  if (!L.configured) return SLOT_KV_EINVAL;
  if (n_seq == 0) return SLOT_KV_OK;
  if (!slots || !pos0 || !ks) return SLOT_KV_EINVAL;
  std::vector<SeqRows> seqs;
  seqs.reserve(n_seq);
  std::vector<uint64_t> seen((static_cast<size_t>(h->n_slots) + 63) / 64, 0);
  uint64_t rows = 0;
  for (uint32_t i = 0; i < n_seq; ++i) {
    if (slots[i] >= h->n_slots || pos0[i] >= h->slot_ctx ||
        static_cast<uint64_t>(pos0[i]) + ks[i] > h->slot_ctx)
      return SLOT_KV_ERANGE;
    uint64_t& word = seen[slots[i] >> 6];
    const uint64_t bit = uint64_t(1) << (slots[i] & 63);
    if (word & bit) return SLOT_KV_EDUP;
    word |= bit;
    if (ks[i]) seqs.push_back(SeqRows{slots[i], pos0[i], ks[i], static_cast<uint32_t>(rows)});
    rows += ks[i];
    if (rows * (L.n_heads + L.n_kv_heads) >= (uint64_t(1) << 31)) return SLOT_KV_EINVAL;
  }
  if (seqs.empty()) return SLOT_KV_OK;
  if (!q || !k_new || !v_new || !out) return SLOT_KV_EINVAL;
  return run_prefill(h, layer, q, k_new, v_new, out, seqs, stream);
}

int slot_kv_layer_ptrs(const slot_kv* h, uint32_t layer, float** k, float** v) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (k) *k = h->layers[layer].k;
  if (v) *v = h->layers[layer].v;
  return SLOT_KV_OK;
}

static int copy_rows(const slot_kv* h, uint32_t layer, uint32_t slot, uint32_t pos0,
                     uint32_t n_rows, float* dst_k, const float* src_k, float* dst_v,
                     const float* src_v, bool into_cache, void* stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (slot >= h->n_slots || pos0 >= h->slot_ctx ||
      static_cast<uint64_t>(pos0) + n_rows > h->slot_ctx)
    return SLOT_KV_ERANGE;
  if (n_rows == 0) return SLOT_KV_OK;
  const LayerState& L = h->layers[layer];
  const uint64_t off = (static_cast<uint64_t>(slot) * h->slot_ctx + pos0) * L.kv_dim;
  const size_t bytes = static_cast<size_t>(n_rows) * L.kv_dim * sizeof(float);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int which = 0; which < 2; ++which) {
    float* cache = which == 0 ? L.k : L.v;
    const void* src = into_cache ? (which == 0 ? static_cast<const void*>(src_k)
                                               : static_cast<const void*>(src_v))
                                 : cache + off;
    void* dst = into_cache ? static_cast<void*>(cache + off)
                           : (which == 0 ? static_cast<void*>(dst_k) : static_cast<void*>(dst_v));
    if (!(into_cache ? src : dst)) continue;  // that side skipped
    if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return SLOT_KV_EDEVICE;
  }
  return SLOT_KV_OK;
}

int slot_kv_write_rows(slot_kv* h, uint32_t layer, uint32_t slot, uint32_t pos0, uint32_t n_rows,
                       const float* k_src, const float* v_src, void* stream) {
  return copy_rows(h, layer, slot, pos0, n_rows, nullptr, k_src, nullptr, v_src, true, stream);
}

int slot_kv_read_rows(const slot_kv* h, uint32_t layer, uint32_t slot, uint32_t pos0,
                      uint32_t n_rows, float* k_dst, float* v_dst, void* stream) {
  return copy_rows(h, layer, slot, pos0, n_rows, k_dst, nullptr, v_dst, nullptr, false, stream);
}

int slot_kv_profile_begin(slot_kv* h) {
  if (!h) return SLOT_KV_EINVAL;
  h->profiling = true;
  h->prof_used = 0;
  return SLOT_KV_OK;
}

int slot_kv_profile_end(slot_kv* h, double* kernel_ms, uint32_t* launches) {
  if (!h) return SLOT_KV_EINVAL;
  double total = 0.0;
  int rc = SLOT_KV_OK;
  for (size_t i = 0; i < h->prof_used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(h->prof_events[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, h->prof_events[2 * i], h->prof_events[2 * i + 1]) != hipSuccess) {
      rc = SLOT_KV_EDEVICE;
      break;
    }
    total += ms;
  }
  if (kernel_ms) *kernel_ms = total;
  if (launches) *launches = static_cast<uint32_t>(h->prof_used);
  h->profiling = false;
  h->prof_used = 0;
  return rc;
}

const char* slot_kv_strerror(int status) {
  switch (status) {
    case SLOT_KV_OK: return "ok";
    case SLOT_KV_EINVAL: return "invalid argument or unconfigured layer";
    case SLOT_KV_ERANGE: return "slot or position out of range";
    case SLOT_KV_ENOTALLOC: return "slot KV not allocated";
    case SLOT_KV_ENOMEM: return "out of memory";
    case SLOT_KV_EDUP: return "slot used by two rows of one batch";
    case SLOT_KV_EDEVICE: return "HIP device error";
    case SLOT_KV_ESCRATCH: return "call needs more scratch than the fixed array holds";
    default: return "unknown status";
  }
}

}  // extern "C"
