/*
 * slot_kv.h -- C ABI of the slot-indexed KV cache and its batched decode step
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations follow two pages of the ZINC engine documentation:
 *   "Forward Cuda Gemma" (Zig API of ForwardGemma): sections decodeBatch,
 *       allocSlotKv, slotKvOffsetBytes, slotKvSmoke;
 *   "Forward Cuda" (Zig API of ForwardCuda): sections on init (upload of the
 *       inv_freq table and the sinks, zeroed KV cache and SSM state), the
 *       allocation of per-sequence slot state, the slot K/V, conv-ring and
 *       recurrent-state byte offsets, and the reset of a reused slot on admit.
 *
 * Conventions shared by every entry point
 *   - Status codes: 0 on success, a negative SLOT_KV_E* value on failure;
 *     slot_kv_strerror() names them.  Every argument is validated before any
 *     device work is enqueued: a call that fails writes nothing.
 *   - "device" pointers are HIP device allocations (for example the data
 *     pointer of a torch tensor on the GPU); "host" pointers are ordinary
 *     process memory, read before the call returns.
 *   - All floating-point data is IEEE float32, C-contiguous, row-major.
 *   - A handle is not thread-safe.  Calls that enqueue work (decode, row
 *     copies) are asynchronous on the stream passed in; a handle keeps one
 *     set of device scratch buffers, so two calls on one handle that run
 *     concurrently on different streams race.  Serialise them on one stream
 *     (or synchronise between them).
 *   - The handle binds to the HIP device that is current when
 *     slot_kv_alloc() is called.
 */
#ifndef SLOT_KV_H
#define SLOT_KV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLOT_KV_OK 0
#define SLOT_KV_EINVAL (-1)    /* bad argument, unconfigured layer, shape mismatch  */
#define SLOT_KV_ERANGE (-2)    /* slot >= n_slots or pos >= slot_ctx                 */
#define SLOT_KV_ENOTALLOC (-3) /* the slot KV has not been allocated                 */
#define SLOT_KV_ENOMEM (-4)    /* a device or pinned-host allocation failed          */
#define SLOT_KV_EDUP (-5)      /* one slot named by two rows of a batch              */
#define SLOT_KV_EDEVICE (-6)   /* HIP runtime or launch error                        */
#define SLOT_KV_ESCRATCH (-7)  /* more scratch than slot_decode_attn_noalloc's array  */

typedef struct slot_kv slot_kv; /* opaque; owns all slot KV device memory */

/* Create an empty handle (no device memory yet).  *out receives it.
 * Makes no HIP call.  Returns SLOT_KV_EINVAL if out is NULL. */
int slot_kv_create(slot_kv **out);

/* Free every device and host allocation of the handle, then the handle.
 * NULL is accepted.  Synchronises the device first. */
void slot_kv_destroy(slot_kv *h);

/* "Forward Cuda Gemma", allocSlotKv; "Forward Cuda", allocation of the
 * per-sequence slot state.
 * Allocates, per layer L < n_layers, one K and one V buffer of
 * n_slots * slot_ctx * kv_dims[L] floats each, laid out [slot][pos][kv_dim],
 * and fills them with zeros.  kv_dims is a host array of n_layers counts of
 * floats per KV row.  Idempotent: any previous allocation of this handle is
 * freed first (layer configurations are dropped with it).
 * Errors: EINVAL (zero sizes, NULL kv_dims, a buffer of more than 2^64 - 1
 * bytes; checked before any HIP call), ENOMEM, EDEVICE.
 * The same as slot_state_alloc with no ssm layers. */
int slot_kv_alloc(slot_kv *h, uint32_t n_slots, uint32_t slot_ctx,
                  const uint32_t *kv_dims, uint32_t n_layers);

/* "Forward Cuda", allocation of the per-sequence slot state for a hybrid
 * attention + SSM model: attention layers get slot KV (as slot_kv_alloc),
 * ssm layers get per slot a conv ring and a recurrent state, all zeroed.
 * Attention layers are numbered 0 .. n_attn_layers-1 and ssm layers,
 * separately, 0 .. n_ssm_layers-1.  Ssm layer l owns two device buffers:
 *   conv  [n_slots][conv_state_len[l]] floats,
 *   state [n_slots][ssm_state_len[l]]  floats.
 * kv_dims (host, n_attn_layers entries) may be NULL when n_attn_layers is 0;
 * conv_state_len and ssm_state_len (host, n_ssm_layers entries, each > 0)
 * may be NULL when n_ssm_layers is 0.  At least one layer is required.
 * What the SSM kernels keep in the buffers is theirs to define; this library
 * lays them out, addresses them and zeroes them.  Idempotent: any previous
 * allocation of the handle (KV and state, and the layer configurations) is
 * freed first.  Errors: EINVAL (zero sizes, NULL arrays, a buffer of more
 * than 2^64 - 1 bytes, one slot's state above 2^31 tiles of 8 KiB; all
 * checked before any HIP call), ENOMEM, EDEVICE. */
int slot_state_alloc(slot_kv *h, uint32_t n_slots, uint32_t slot_ctx,
                     const uint32_t *kv_dims, uint32_t n_attn_layers,
                     const uint32_t *conv_state_len, const uint32_t *ssm_state_len,
                     uint32_t n_ssm_layers);

/* "Forward Cuda", init: upload of inv_freq and sinks.
 * Configures attention layer `layer`: n_heads query heads and n_kv_heads KV
 * heads of head_dim floats (n_kv_heads * head_dim must equal kv_dims[layer];
 * n_heads must be a multiple of n_kv_heads; head_dim one of 64, 128, 256;
 * n_heads / n_kv_heads one of 1, 2, 4, 8).
 * Host arrays, copied to the device: q_norm_w[head_dim] and k_norm_w[head_dim]
 * (RMSNorm weights shared by all query heads, resp. all key heads),
 * inv_freq[head_dim/2] (RoPE frequencies), sinks[n_heads] (one extra softmax
 * logit per query head; NULL for none).  eps is the RMSNorm epsilon and
 * scale multiplies q.k (not the sink).  The layer's convention flags are
 * reset to 0 (see slot_kv_set_layer_flags).
 * Errors: ENOTALLOC, EINVAL, EDEVICE. */
int slot_kv_set_layer(slot_kv *h, uint32_t layer, uint32_t n_heads,
                      uint32_t n_kv_heads, uint32_t head_dim,
                      const float *q_norm_w, const float *k_norm_w,
                      const float *inv_freq, const float *sinks, float eps,
                      float scale);

/* Convention flags of a layer ("Forward Cuda Gemma", decodeBatch: "per-head
 * V/Q/K norm"; variants a model may use).  Default 0:
 *   SLOT_KV_FLAG_V_NORM            each value head is replaced by its
 *                                  weightless RMSNorm, v / sqrt(mean(v^2) +
 *                                  eps), before it is written and attended;
 *   SLOT_KV_FLAG_ROPE_INTERLEAVED  RoPE rotates the pairs (x[2i], x[2i+1]) by
 *                                  angle float(pos)*inv_freq[i] instead of the
 *                                  pairs (x[i], x[i + head_dim/2]);
 *   SLOT_KV_FLAG_NORM_ONE_PLUS_W   the query and key norms multiply by
 *                                  (1 + w) instead of w. */
#define SLOT_KV_FLAG_V_NORM 1u
#define SLOT_KV_FLAG_ROPE_INTERLEAVED 2u
#define SLOT_KV_FLAG_NORM_ONE_PLUS_W 4u

/* Sets the convention flags of configured layer `layer` for every later call
 * (slot_kv_set_layer resets them to 0).  Errors: ENOTALLOC, EINVAL (layer
 * unconfigured, unknown flag bits). */
int slot_kv_set_layer_flags(slot_kv *h, uint32_t layer, uint32_t flags);

/* "Forward Cuda Gemma", slotKvOffsetBytes; "Forward Cuda", slot K/V offset.
 * *out_bytes = (slot * slot_ctx + pos) * kv_dims[layer] * 4, in 64 bits: the
 * byte offset of the row (slot, pos) inside layer `layer`'s K buffer (the V
 * buffer uses the same offset).  Errors: ENOTALLOC, EINVAL (layer or
 * out_bytes), ERANGE (slot or pos out of range). */
int slot_kv_offset_bytes(const slot_kv *h, uint32_t layer, uint32_t slot,
                         uint32_t pos, uint64_t *out_bytes);

/* "Forward Cuda", byte offsets of slot `slot`'s conv ring and recurrent state
 * in ssm layer `ssm_layer`'s buffers: slot * conv_state_len * 4 and
 * slot * ssm_state_len * 4, in 64 bits.  Errors: ENOTALLOC, EINVAL (ssm_layer
 * or out_bytes), ERANGE (slot >= n_slots). */
int slot_conv_offset_bytes(const slot_kv *h, uint32_t ssm_layer, uint32_t slot,
                           uint64_t *out_bytes);
int slot_ssm_offset_bytes(const slot_kv *h, uint32_t ssm_layer, uint32_t slot,
                          uint64_t *out_bytes);

/* Device pointers of ssm layer `ssm_layer`'s conv and recurrent-state buffers
 * (owned by the handle, valid until the next allocation or slot_kv_destroy;
 * either output may be NULL).  Errors: ENOTALLOC, EINVAL. */
int slot_state_ptrs(const slot_kv *h, uint32_t ssm_layer, float **conv, float **ssm);

/* "Forward Cuda", reset of a reused slot on admit, before the new request's
 * prefill.  The SSM state accumulates over a sequence, so the slot's conv
 * ring and recurrent state are zeroed in every ssm layer (one kernel launch
 * on `stream`, hipStream_t, NULL = the null stream).  The attention slot KV
 * needs no clearing: it is indexed by position, each sequence overwrites from
 * position 0 and reads only what it wrote, so it is left as it is; with no
 * ssm layers the call only validates.  Returns OK without doing anything when
 * nothing is allocated, ERANGE when slot >= n_slots. */
int slot_reset(slot_kv *h, uint32_t slot, void *stream);

/* slot_reset for n slots at once (host array, copied before the call
 * returns; a slot may appear twice).  Every slot is checked before anything
 * is enqueued; one launch per 256 slots.  n == 0 is a no-op.  Errors: EINVAL
 * (NULL slots with n > 0), ERANGE, EDEVICE. */
int slot_reset_batch(slot_kv *h, const uint32_t *slots, uint32_t n, void *stream);

/* "Forward Cuda Gemma", decodeBatch (its attention part).
 * Advances B independent sequences by one token each.  Row b uses its own
 * slot slots[b] at its own position positions[b]:
 *   1. RMSNorm each query head of q[b] (weights q_norm_w) and each key head
 *      of k_new[b] (weights k_norm_w), then rotate both with RoPE at
 *      positions[b] (pairs (i, i + head_dim/2), angle float(pos)*inv_freq[i]);
 *   2. store the rotated key row and v_new[b] unchanged at byte offset
 *      (slots[b]*slot_ctx + positions[b]) * kv_dim * 4 of the layer's K / V;
 *   3. out[b] = causal softmax attention of each query head h over keys
 *      0..positions[b] (inclusive) of that slot, against kv head
 *      h / (n_heads / n_kv_heads), scores scale*q.k, plus the head's sink
 *      logit in the denominator when sinks are set.
 * Requires history rows 0..positions[b]-1 of the slot to hold that sequence's
 * keys and values (written by earlier calls or slot_kv_write_rows).
 *   q      device [B][n_heads*head_dim]        k_new, v_new  device [B][kv_dim]
 *   out    device [B][n_heads*head_dim]; must not overlap q, k_new or v_new
 *   positions, slots  host [B]; copied before the call returns
 *   stream hipStream_t (NULL = the null stream)
 * B == 0 is a no-op.  Errors: ENOTALLOC, EINVAL (layer unconfigured, NULL
 * pointer), ERANGE (slots[b] >= n_slots or positions[b] >= slot_ctx), EDUP
 * (a slot repeated in the batch), ENOMEM, EDEVICE (launch failure).  Faults
 * inside the kernels surface at the caller's next synchronisation. */
int slot_decode_attn(slot_kv *h, uint32_t layer, const float *q,
                     const float *k_new, const float *v_new,
                     const uint32_t *positions, const uint32_t *slots,
                     uint32_t B, float *out, void *stream);

/* For callers that cannot allocate device memory during the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same step as slot_decode_attn, with the same arguments, kernels,
 * results (bit for bit) and errors, but the call makes no allocation of any
 * kind and no synchronisation: its scratch (the split rows' partial results
 * and the work queue's counters) lives in one fixed array per GPU, 64 MiB,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends.  The array's address is looked up when slot_kv_alloc (or
 * slot_state_alloc) runs on the device.  Limit: the partials of a launch
 * (256 rows; rows * (largest chunk count of those rows) * n_heads *
 * (head_dim + 2) floats, a row at position p counting p / slot_kv_chunk_keys()
 * + 1 chunks) must fit 64 MiB - 256 KiB, and n_kv_heads * 256 + 1 counter
 * words 256 KiB (n_kv_heads <= 127); a larger call returns SLOT_KV_ESCRATCH
 * before anything is enqueued.  The counters carry a per-launch epoch, so
 * nothing in the array needs clearing between calls.  Every call on one GPU,
 * from any handle, shares the array: calls that can run at the same time on
 * one GPU (different streams) race and give wrong results; calls on one
 * stream are ordered.  Launches are not recorded by slot_kv_profile_*.
 * Errors: those of slot_decode_attn, SLOT_KV_ESCRATCH, and EDEVICE when the
 * array's address could not be looked up. */
int slot_decode_attn_noalloc(slot_kv *h, uint32_t layer, const float *q,
                             const float *k_new, const float *v_new,
                             const uint32_t *positions, const uint32_t *slots,
                             uint32_t B, float *out, void *stream);

/* "Forward Cuda", batched prefill that writes the KV cache into a slot's
 * per-sequence region; "Forward Cuda Gemma", prefillBatched, defined there as
 * equal to running the one-token step on every prompt token in order.
 * T tokens of one sequence, at positions pos0 .. pos0+T-1 of slot `slot`: for
 * token t the same per-head RMSNorm and RoPE (at pos0+t), KV write and
 * attention as slot_decode_attn gives a row at that position, with the tokens
 * taken in order, so token t attends over positions 0 .. pos0+t (the slot's
 * earlier history and tokens 0..t of this call).
 *   q      device [T][n_heads*head_dim]        k_new, v_new  device [T][kv_dim]
 *   out    device [T][n_heads*head_dim]; must not overlap q, k_new or v_new
 *   stream hipStream_t (NULL = the null stream)
 * Requires history rows 0..pos0-1 of the slot to hold the sequence's keys and
 * values.  The handle keeps a scratch buffer (grown on demand, freed with
 * the handle) for a per-row table of the query heads' norm, rotation and
 * scale factors, 2*T*head_dim floats, and, when the keys are cut into
 * chunks, the chunks' partial results: at most 16,384
 * items of 16*(head_dim+2) floats per launch.  Calls with at most 64 query
 * rows per kv head (T * n_heads / n_kv_heads <= 64) run the split-K kernel;
 * longer ones the tiled kernel, cut into key chunks when it would have
 * fewer than 512 workgroups.  Results do not depend on which is taken
 * beyond f32 rounding.  T == 0 is a no-op.  Errors:
 * ENOTALLOC, EINVAL (layer unconfigured or head shape unsupported, NULL
 * pointer), ERANGE (slot >= n_slots or pos0 + T > slot_ctx), ENOMEM, EDEVICE.
 * Nothing is written when an error is returned. */
int slot_prefill_attn(slot_kv *h, uint32_t layer, const float *q,
                      const float *k_new, const float *v_new, uint32_t slot,
                      uint32_t pos0, uint32_t T, float *out, void *stream);

/* Several rows per sequence for a batch of sequences (the other system's
 * batched verify, decode_verify_multi: ks[i] consecutive rows for each of
 * n_seq sequences, sequence-major).  Sequence i has ks[i] rows at positions
 * pos0[i] .. pos0[i]+ks[i]-1 of slot slots[i]; its rows follow those of
 * sequences 0..i-1 in q / k_new / v_new / out.  Every row is processed as
 * slot_prefill_attn processes the tokens of one sequence: row r of sequence i
 * attends over positions 0 .. pos0[i]+r of its slot.
 *   slots, pos0, ks  host [n_seq]; copied before the call returns
 *   q, out  device [sum ks][n_heads*head_dim]   k_new, v_new  device [sum ks][kv_dim]
 * Sequences with ks[i] == 0 contribute no rows (their slot and position are
 * still checked).  Scratch and kernel choice are those of slot_prefill_attn,
 * with the split-K kernel taken when every sequence has at most 64 query rows
 * per kv head; one launch per 128 sequences.  n_seq == 0 is a no-op.
 * Errors: ENOTALLOC, EINVAL (layer unconfigured or head shape unsupported,
 * NULL pointer), ERANGE (a slot >= n_slots or pos0[i] + ks[i] > slot_ctx),
 * EDUP (a slot repeated), ENOMEM, EDEVICE.  Nothing is written when an error
 * is returned. */
int slot_verify_attn(slot_kv *h, uint32_t layer, const float *q,
                     const float *k_new, const float *v_new, const uint32_t *slots,
                     const uint32_t *pos0, const uint32_t *ks, uint32_t n_seq,
                     float *out, void *stream);

/* Device pointers of layer `layer`'s K and V buffers ([n_slots][slot_ctx]
 * [kv_dim] floats each; owned by the handle, valid until the next
 * slot_kv_alloc / slot_state_alloc or slot_kv_destroy).  Errors: ENOTALLOC,
 * EINVAL. */
int slot_kv_layer_ptrs(const slot_kv *h, uint32_t layer, float **k, float **v);

/* Copy n_rows consecutive K and V rows (kv_dim floats each) from device
 * buffers k_src / v_src into slot `slot` at positions pos0 .. pos0+n_rows-1
 * of layer `layer` (a prefill by copy; either source may be NULL to skip
 * it).  Asynchronous on `stream`.  Errors: ENOTALLOC, EINVAL, ERANGE, EDEVICE. */
int slot_kv_write_rows(slot_kv *h, uint32_t layer, uint32_t slot, uint32_t pos0,
                       uint32_t n_rows, const float *k_src, const float *v_src,
                       void *stream);

/* The reverse copy: rows pos0 .. pos0+n_rows-1 of slot `slot` into device
 * buffers k_dst / v_dst (either may be NULL).  Same errors. */
int slot_kv_read_rows(const slot_kv *h, uint32_t layer, uint32_t slot,
                      uint32_t pos0, uint32_t n_rows, float *k_dst, float *v_dst,
                      void *stream);

/* "Forward Cuda Gemma", decodeBatch preconditions, checked on the host only
 * (no device access, usable without a GPU): every slots[b] < n_slots, every
 * positions[b] < slot_ctx, no slot twice.  On success, when the pointers are
 * non-NULL, *n_items receives the number of split-K work items the decode
 * step launches per kv head (a row at position p is cut into
 * ceil((p+1)/chunk_keys) chunks of chunk_keys keys) and *n_split_rows the
 * number of rows cut into more than one chunk.  Errors: EINVAL, ERANGE, EDUP. */
int slot_kv_check_batch(uint32_t n_slots, uint32_t slot_ctx,
                        const uint32_t *positions, const uint32_t *slots,
                        uint32_t B, uint32_t chunk_keys, uint32_t *n_items,
                        uint32_t *n_split_rows);

/* Keys per split-K chunk used by slot_decode_attn (a build constant; chunk
 * boundaries depend only on each row's position, never on the batch). */
uint32_t slot_kv_chunk_keys(void);

/* Profiling of the attention kernels.  Between slot_kv_profile_begin and
 * slot_kv_profile_end the handle records a HIP event pair on the call's
 * stream immediately around each launch of the fused decode kernel (one
 * launch per 256 rows of a slot_decode_attn call; it does the whole step), of
 * the prefill attention kernel (one per slot_prefill_attn call, one per 128
 * sequences of a slot_verify_attn call) and of the state-reset kernel (one per
 * 256 slots of a slot_reset / slot_reset_batch call).
 * slot_kv_profile_end waits for the recorded launches and returns their
 * summed duration in milliseconds and their count (either pointer may be
 * NULL), then stops recording.  Errors: EINVAL, EDEVICE. */
int slot_kv_profile_begin(slot_kv *h);
int slot_kv_profile_end(slot_kv *h, double *kernel_ms, uint32_t *launches);

/* Static text for a status code. */
const char *slot_kv_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SLOT_KV_H */
