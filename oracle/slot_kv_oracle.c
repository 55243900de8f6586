/*
 * slot_kv_oracle.c -- CPU oracle for the slot-indexed batched decode-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library.
 *
 * Arithmetic: every floating-point reduction is carried in double precision;
 * values that the step stores (the K row written into the cache, the output
 * row) are rounded to float exactly once, at the end.
 *
 * Source of the definitions (web pages, cited by title and section):
 *   [FG]  "Forward Cuda Gemma" (ZINC Zig API), sections decodeBatch,
 *         allocSlotKv, slotKvOffsetBytes, slotKvSmoke.
 *   [FC]  "Forward Cuda" (ZINC Zig API), sections on init (upload of
 *         inv_freq and sinks), per-slot offsets and slot reset on admit.
 *
 * Readings taken where the pages are silent (conventions the pages do not
 * fix by value; the pins in the test suite fix the oracle to each of them):
 *   - attention covers keys 0..pos inclusive; key pos is the row this step
 *     writes ([FG] decodeBatch: the slot already holds 0..pos-1 and the
 *     step writes the new K/V, then attends over the history up to pos);
 *   - RMSNorm is x * (mean(x^2) + eps)^(-1/2) * w, per head, one weight
 *     vector of length head_dim shared by all Q heads (and one by all K heads);
 *   - RoPE pairs element i with element i + head_dim/2 ("rotate half"),
 *     angle = float32(float(pos) * inv_freq[i]), sin/cos of that value;
 *   - norm first, then RoPE; the cache stores rotated K and V verbatim;
 *   - scores are scale * q.k; a per-q-head sink adds exp(sink - m) to the
 *     softmax denominator and contributes no value vector;
 *   - q head h reads kv head h / (n_heads / n_kv_heads);
 *   - a kv row is laid out head-major: [n_kv_heads][head_dim].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ERANGE (-2)
#define ORACLE_EDUP (-5)

/* Convention flags (the pages' "per-head V/Q/K norm" and the variants a model
 * may use; default 0 = the conventions described above):
 *   V_NORM            weightless RMSNorm of each value head before it is
 *                     written (the "V" of "per-head V/Q/K norm");
 *   ROPE_INTERLEAVED  RoPE pairs (x[2i], x[2i+1]) instead of (x[i], x[i+D/2]);
 *   NORM_ONE_PLUS_W   the Q and K norms multiply by (1 + w) instead of w. */
#define ORACLE_V_NORM 1u
#define ORACLE_ROPE_INTERLEAVED 2u
#define ORACLE_NORM_ONE_PLUS_W 4u

/* [FG] slotKvOffsetBytes; [FC] slot K/V byte offset:
 * byte offset of (slot, pos) in one layer's slot KV buffer,
 * (slot * slot_ctx + pos) * kv_dim * sizeof(f32), computed in 64 bits. */
uint64_t oracle_slot_kv_offset_bytes(uint32_t slot, uint32_t pos,
                                     uint32_t slot_ctx, uint32_t kv_dim) {
    uint64_t row = (uint64_t)slot * (uint64_t)slot_ctx + (uint64_t)pos;
    return row * (uint64_t)kv_dim * (uint64_t)sizeof(float);
}

/* [FG] decodeBatch, "per-head ... norm": RMSNorm of one head vector.
 * y[i] = x[i] / sqrt(mean(x^2) + eps) * w[i], all in double. */
void oracle_rms_norm(const float *x, const float *w, uint32_t n, double eps,
                     double *y) {
    double ss = 0.0;
    for (uint32_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (uint32_t i = 0; i < n; ++i) y[i] = (double)x[i] * r * (double)w[i];
}

/* [FG] decodeBatch "+ RoPE"; [FC] init uploads the inv_freq table.
 * Rotate-half RoPE of one head vector at position pos, in place.
 * For i < D/2 the pair (x[i], x[i + D/2]) is rotated by the angle
 * theta_i = float32(float(pos) * inv_freq[i]). */
void oracle_rope(double *x, const float *inv_freq, uint32_t pos, uint32_t D) {
    uint32_t half = D / 2;
    for (uint32_t i = 0; i < half; ++i) {
        volatile float ang_f = (float)pos * inv_freq[i]; /* one f32 multiply */
        double th = (double)ang_f;
        double c = cos(th), s = sin(th);
        double a = x[i], b = x[i + half];
        x[i] = a * c - b * s;
        x[i + half] = b * c + a * s;
    }
}

/* NORM_ONE_PLUS_W variant of oracle_rms_norm: y[i] = x[i] / sqrt(mean(x^2) +
 * eps) * (1 + w[i]), all in double. */
void oracle_rms_norm_1pw(const float *x, const float *w, uint32_t n, double eps, double *y) {
    double ss = 0.0;
    for (uint32_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (uint32_t i = 0; i < n; ++i) y[i] = (double)x[i] * r * (1.0 + (double)w[i]);
}

/* V_NORM: the weightless RMSNorm y[i] = x[i] / sqrt(mean(x^2) + eps). */
void oracle_rms_norm_plain(const float *x, uint32_t n, double eps, double *y) {
    double ss = 0.0;
    for (uint32_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (uint32_t i = 0; i < n; ++i) y[i] = (double)x[i] * r;
}

/* ROPE_INTERLEAVED: the pair (x[2i], x[2i+1]) is rotated by
 * theta_i = float32(float(pos) * inv_freq[i]), for i < D/2. */
void oracle_rope_interleaved(double *x, const float *inv_freq, uint32_t pos, uint32_t D) {
    for (uint32_t i = 0; i < D / 2; ++i) {
        volatile float ang_f = (float)pos * inv_freq[i]; /* one f32 multiply */
        double th = (double)ang_f;
        double c = cos(th), s = sin(th);
        double a = x[2 * i], b = x[2 * i + 1];
        x[2 * i] = a * c - b * s;
        x[2 * i + 1] = b * c + a * s;
    }
}

/* [FG] decodeBatch: the whole step for one row b.
 *
 *   q_row      [n_heads * head_dim]      this row's query
 *   k_new_row  [kv_dim]                  this row's new key (before norm/RoPE)
 *   v_new_row  [kv_dim]                  this row's new value
 *   hist_k/v   pos rows of kv_dim floats, row t at hist + t * hist_stride:
 *              the slot's history 0..pos-1 (may be NULL when pos == 0)
 *   k_written  [kv_dim]  the K row this step stores at (slot, pos)
 *   v_written  [kv_dim]  the V row this step stores at (slot, pos)
 *   out_row    [n_heads * head_dim]      attention output
 *   sinks      [n_heads] or NULL
 *   flags      ORACLE_V_NORM | ORACLE_ROPE_INTERLEAVED | ORACLE_NORM_ONE_PLUS_W
 *
 * Returns ORACLE_OK, or ORACLE_EINVAL for an inconsistent head shape. */
int oracle_decode_row(uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                      const float *q_norm_w, const float *k_norm_w,
                      const float *inv_freq, const float *sinks,
                      float eps, float scale, uint32_t pos,
                      const float *q_row, const float *k_new_row,
                      const float *v_new_row,
                      const float *hist_k, const float *hist_v,
                      uint64_t hist_stride,
                      float *k_written, float *v_written, float *out_row,
                      uint32_t flags) {
    if (n_heads == 0 || n_kv_heads == 0 || head_dim == 0 || head_dim % 2 != 0 ||
        n_heads % n_kv_heads != 0)
        return ORACLE_EINVAL;
    const uint32_t D = head_dim;
    const uint32_t kv_dim = n_kv_heads * D;
    const uint32_t G = n_heads / n_kv_heads;
    if (pos > 0 && hist_stride < kv_dim) return ORACLE_EINVAL;

    double *tmp = (double *)malloc(sizeof(double) * D);
    double *qh = (double *)malloc(sizeof(double) * D);
    double *sc = (double *)malloc(sizeof(double) * ((size_t)pos + 1));
    double *acc = (double *)malloc(sizeof(double) * D);
    if (!tmp || !qh || !sc || !acc) {
        free(tmp); free(qh); free(sc); free(acc);
        return ORACLE_EINVAL;
    }

    /* New K row: norm, then RoPE at pos, rounded once to f32.  V verbatim
     * (or, with V_NORM, its weightless RMSNorm rounded once to f32). */
    for (uint32_t j = 0; j < n_kv_heads; ++j) {
        if (flags & ORACLE_NORM_ONE_PLUS_W)
            oracle_rms_norm_1pw(k_new_row + (size_t)j * D, k_norm_w, D, (double)eps, tmp);
        else
            oracle_rms_norm(k_new_row + (size_t)j * D, k_norm_w, D, (double)eps, tmp);
        if (flags & ORACLE_ROPE_INTERLEAVED)
            oracle_rope_interleaved(tmp, inv_freq, pos, D);
        else
            oracle_rope(tmp, inv_freq, pos, D);
        for (uint32_t d = 0; d < D; ++d) {
            k_written[(size_t)j * D + d] = (float)tmp[d];
            v_written[(size_t)j * D + d] = v_new_row[(size_t)j * D + d];
        }
        if (flags & ORACLE_V_NORM) {
            oracle_rms_norm_plain(v_new_row + (size_t)j * D, D, (double)eps, tmp);
            for (uint32_t d = 0; d < D; ++d) v_written[(size_t)j * D + d] = (float)tmp[d];
        }
    }

    for (uint32_t h = 0; h < n_heads; ++h) {
        const uint32_t j = h / G;
        if (flags & ORACLE_NORM_ONE_PLUS_W)
            oracle_rms_norm_1pw(q_row + (size_t)h * D, q_norm_w, D, (double)eps, qh);
        else
            oracle_rms_norm(q_row + (size_t)h * D, q_norm_w, D, (double)eps, qh);
        if (flags & ORACLE_ROPE_INTERLEAVED)
            oracle_rope_interleaved(qh, inv_freq, pos, D);
        else
            oracle_rope(qh, inv_freq, pos, D);

        /* scores over keys 0..pos; key pos is the row written above */
        double m = -INFINITY;
        for (uint32_t t = 0; t <= pos; ++t) {
            const float *krow = (t < pos)
                ? hist_k + (size_t)t * hist_stride + (size_t)j * D
                : k_written + (size_t)j * D;
            double dot = 0.0;
            for (uint32_t d = 0; d < D; ++d) dot += qh[d] * (double)krow[d];
            sc[t] = (double)scale * dot;
            if (sc[t] > m) m = sc[t];
        }
        const int has_sink = (sinks != NULL);
        const double sink = has_sink ? (double)sinks[h] : -INFINITY;
        if (has_sink && sink > m) m = sink;

        double den = 0.0;
        for (uint32_t d = 0; d < D; ++d) acc[d] = 0.0;
        for (uint32_t t = 0; t <= pos; ++t) {
            const float *vrow = (t < pos)
                ? hist_v + (size_t)t * hist_stride + (size_t)j * D
                : v_written + (size_t)j * D;
            double e = exp(sc[t] - m);
            den += e;
            for (uint32_t d = 0; d < D; ++d) acc[d] += e * (double)vrow[d];
        }
        if (has_sink && sink != -INFINITY) den += exp(sink - m);
        for (uint32_t d = 0; d < D; ++d)
            out_row[(size_t)h * D + d] = (float)(acc[d] / den);
    }
    free(tmp); free(qh); free(sc); free(acc);
    return ORACLE_OK;
}

/* [FG] decodeBatch preconditions: n_slots > max(slots), slot_ctx >
 * max(positions); each row owns its slot (a repeated slot is rejected). */
int oracle_check_batch(uint32_t n_slots, uint32_t slot_ctx,
                       const uint32_t *positions, const uint32_t *slots,
                       uint32_t B) {
    for (uint32_t b = 0; b < B; ++b) {
        if (slots[b] >= n_slots || positions[b] >= slot_ctx) return ORACLE_ERANGE;
        for (uint32_t c = 0; c < b; ++c)
            if (slots[c] == slots[b]) return ORACLE_EDUP;
    }
    return ORACLE_OK;
}

/* [FG] decodeBatch over a host mirror of one layer's slot KV
 * ([n_slots][slot_ctx][kv_dim] f32 for K and for V).  Each row b writes its
 * K/V row at (slots[b], positions[b]) and attends over its own slot's
 * positions 0..positions[b].  Rows are independent; they run in index order. */
int oracle_decode_batch(uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                        const float *q_norm_w, const float *k_norm_w,
                        const float *inv_freq, const float *sinks,
                        float eps, float scale,
                        float *cache_k, float *cache_v,
                        uint32_t n_slots, uint32_t slot_ctx,
                        const float *q, const float *k_new, const float *v_new,
                        const uint32_t *positions, const uint32_t *slots,
                        uint32_t B, float *out, uint32_t flags) {
    if (n_kv_heads == 0 || head_dim == 0) return ORACLE_EINVAL;
    const uint32_t kv_dim = n_kv_heads * head_dim;
    const size_t qd = (size_t)n_heads * head_dim;
    int rc = oracle_check_batch(n_slots, slot_ctx, positions, slots, B);
    if (rc != ORACLE_OK) return rc;
    for (uint32_t b = 0; b < B; ++b) {
        const uint32_t p = positions[b], s = slots[b];
        const uint64_t base = oracle_slot_kv_offset_bytes(s, 0, slot_ctx, kv_dim) / sizeof(float);
        const uint64_t at = oracle_slot_kv_offset_bytes(s, p, slot_ctx, kv_dim) / sizeof(float);
        rc = oracle_decode_row(n_heads, n_kv_heads, head_dim, q_norm_w, k_norm_w,
                               inv_freq, sinks, eps, scale, p,
                               q + (size_t)b * qd, k_new + (size_t)b * kv_dim,
                               v_new + (size_t)b * kv_dim,
                               cache_k + base, cache_v + base, kv_dim,
                               cache_k + at, cache_v + at, out + (size_t)b * qd, flags);
        if (rc != ORACLE_OK) return rc;
    }
    return ORACLE_OK;
}

/* Slot prefill ("Forward Cuda", batched prefill that writes the KV cache into
 * the given slot's per-sequence region; "Forward Cuda Gemma", prefillBatched,
 * which the pages define as equal to running the one-token step on every
 * prompt token in order): the T tokens of one sequence, at positions
 * pos0 .. pos0+T-1 of slot `slot`, each written and attended exactly as a
 * one-row decode step at its position would be, in token order.  Token t
 * therefore attends over positions 0 .. pos0+t: the slot's earlier history
 * and the rows of tokens 0..t of this call. */
int oracle_prefill(uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                   const float *q_norm_w, const float *k_norm_w,
                   const float *inv_freq, const float *sinks,
                   float eps, float scale,
                   float *cache_k, float *cache_v,
                   uint32_t n_slots, uint32_t slot_ctx,
                   const float *q, const float *k_new, const float *v_new,
                   uint32_t slot, uint32_t pos0, uint32_t T, float *out, uint32_t flags) {
    if (n_kv_heads == 0 || head_dim == 0) return ORACLE_EINVAL;
    if (slot >= n_slots || pos0 >= slot_ctx || T > slot_ctx - pos0) return ORACLE_ERANGE;
    const uint32_t kv_dim = n_kv_heads * head_dim;
    const size_t qd = (size_t)n_heads * head_dim;
    for (uint32_t t = 0; t < T; ++t) {
        const uint32_t p = pos0 + t;
        int rc = oracle_decode_batch(n_heads, n_kv_heads, head_dim, q_norm_w, k_norm_w,
                                     inv_freq, sinks, eps, scale, cache_k, cache_v,
                                     n_slots, slot_ctx, q + (size_t)t * qd,
                                     k_new + (size_t)t * kv_dim, v_new + (size_t)t * kv_dim,
                                     &p, &slot, 1, out + (size_t)t * qd, flags);
        if (rc != ORACLE_OK) return rc;
    }
    return ORACLE_OK;
}

/* Several rows for each of n_seq sequences (the other system's batched
 * verify, decode_verify_multi: ks[i] consecutive rows per sequence, rows
 * sequence-major): sequence i's rows are a slot prefill of slot slots[i] at
 * positions pos0[i] .. pos0[i]+ks[i]-1, and sequences do not interact (each
 * owns its slot, so a slot named twice is rejected).  Every check runs before
 * anything is written. */
int oracle_verify(uint32_t n_heads, uint32_t n_kv_heads, uint32_t head_dim,
                  const float *q_norm_w, const float *k_norm_w,
                  const float *inv_freq, const float *sinks,
                  float eps, float scale,
                  float *cache_k, float *cache_v,
                  uint32_t n_slots, uint32_t slot_ctx,
                  const float *q, const float *k_new, const float *v_new,
                  const uint32_t *slots, const uint32_t *pos0, const uint32_t *ks,
                  uint32_t n_seq, float *out, uint32_t flags) {
    if (n_kv_heads == 0 || head_dim == 0) return ORACLE_EINVAL;
    for (uint32_t i = 0; i < n_seq; ++i) {
        if (slots[i] >= n_slots || pos0[i] >= slot_ctx || ks[i] > slot_ctx - pos0[i])
            return ORACLE_ERANGE;
        for (uint32_t c = 0; c < i; ++c)
            if (slots[c] == slots[i]) return ORACLE_EDUP;
    }
    const uint32_t kv_dim = n_kv_heads * head_dim;
    const size_t qd = (size_t)n_heads * head_dim;
    size_t row = 0;
    for (uint32_t i = 0; i < n_seq; ++i) {
        if (ks[i] > 0) {
            int rc = oracle_prefill(n_heads, n_kv_heads, head_dim, q_norm_w, k_norm_w,
                                    inv_freq, sinks, eps, scale, cache_k, cache_v,
                                    n_slots, slot_ctx, q + row * qd, k_new + row * kv_dim,
                                    v_new + row * kv_dim, slots[i], pos0[i], ks[i],
                                    out + row * qd, flags);
            if (rc != ORACLE_OK) return rc;
        }
        row += ks[i];
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- per-slot SSM state
 * [FC] allocation of the per-sequence slot state: every ssm layer gets, per
 * slot, a conv ring of conv_state_len floats and a recurrent state of
 * ssm_state_len floats, each layer's buffers laid out [slot][state_len] and
 * zero-initialised.  ssm layers are numbered on their own (0 .. n_layers-1).
 *
 * [FC] per-slot offsets: slot `slot`'s conv ring starts slot*conv_state_len*4
 * bytes into its layer's conv buffer, and its recurrent state
 * slot*ssm_state_len*4 bytes into its layer's state buffer.  One function
 * serves both: the byte offset of slot `slot` in a [slot][state_len] f32
 * buffer, in 64 bits. */
uint64_t oracle_slot_state_offset_bytes(uint32_t slot, uint32_t state_len) {
    return (uint64_t)slot * (uint64_t)state_len * (uint64_t)sizeof(float);
}

/* [FC] reset of a reused slot on admit: the SSM state accumulates over a
 * sequence rather than being indexed by position, so a slot handed to a new
 * request has its conv ring and its recurrent state zeroed in every ssm
 * layer; the attention KV of the slot is left alone (nothing reads it past
 * the new sequence's own positions).  A call names n slots (a slot may
 * appear more than once: zeroing twice is zeroing once).  Every slot is
 * checked before anything is written; with no state allocated (n_slots == 0)
 * the call does nothing and succeeds.
 * conv[l] / ssm[l] are layer l's buffers of n_slots*conv_len[l] and
 * n_slots*ssm_len[l] floats. */
int oracle_slot_reset(float **conv, float **ssm, const uint32_t *conv_len,
                      const uint32_t *ssm_len, uint32_t n_layers, uint32_t n_slots,
                      const uint32_t *slots, uint32_t n) {
    if (n_slots == 0) return ORACLE_OK;
    for (uint32_t i = 0; i < n; ++i)
        if (slots[i] >= n_slots) return ORACLE_ERANGE;
    for (uint32_t i = 0; i < n; ++i) {
        for (uint32_t l = 0; l < n_layers; ++l) {
            float *c = conv[l] + oracle_slot_state_offset_bytes(slots[i], conv_len[l]) / sizeof(float);
            for (uint32_t e = 0; e < conv_len[l]; ++e) c[e] = 0.0f;
            float *s = ssm[l] + oracle_slot_state_offset_bytes(slots[i], ssm_len[l]) / sizeof(float);
            for (uint32_t e = 0; e < ssm_len[l]; ++e) s[e] = 0.0f;
        }
    }
    return ORACLE_OK;
}
