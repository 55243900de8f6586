"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them.  CPU only: each mutant is compiled with gcc into a
temporary directory and the pin suite runs against it in a subprocess."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "slot_kv_oracle.c")

MUTANTS = {
    "offset_uses_32bit": ("return row * (uint64_t)kv_dim * (uint64_t)sizeof(float);",
                          "return (uint32_t)(row * kv_dim * sizeof(float));"),
    "norm_sum_not_mean": ("sqrt(ss / (double)n + eps)", "sqrt(ss + eps)"),
    "norm_drops_eps": ("sqrt(ss / (double)n + eps)", "sqrt(ss / (double)n)"),
    "norm_drops_weight": ("y[i] = (double)x[i] * r * (double)w[i];", "y[i] = (double)x[i] * r;"),
    "rope_minus_theta": ("x[i] = a * c - b * s;", "x[i] = a * c + b * s;"),
    "rope_second_sign": ("x[i + half] = b * c + a * s;", "x[i + half] = b * c - a * s;"),
    "rope_f64_angle": ("double th = (double)ang_f;", "double th = (double)pos * (double)inv_freq[i];"),
    "rope_pos_plus_one": ("volatile float ang_f = (float)pos * inv_freq[i];",
                          "volatile float ang_f = (float)(pos + 1) * inv_freq[i];"),
    "range_exclusive": ("for (uint32_t t = 0; t <= pos; ++t) {\n            const float *vrow",
                        "for (uint32_t t = 0; t < pos + (pos == 0); ++t) {\n            const float *vrow"),
    "gqa_modulo": ("const uint32_t j = h / G;", "const uint32_t j = h % n_kv_heads;"),
    "no_scale": ("sc[t] = (double)scale * dot;", "sc[t] = dot;"),
    "sink_dropped": ("if (has_sink && sink != -INFINITY) den += exp(sink - m);", ";"),
    "sink_scaled": ("den += exp(sink - m);", "den += exp((double)scale * sink - m);"),
    "no_max_subtraction": ("double e = exp(sc[t] - m);", "double e = exp(sc[t]);"),
    "v_not_verbatim": ("v_written[(size_t)j * D + d] = v_new_row[(size_t)j * D + d];",
                       "v_written[(size_t)j * D + d] = (float)tmp[d];"),
    "new_key_unrotated": ("oracle_rope(tmp, inv_freq, pos, D);\n        for",
                          "for"),
    "dup_slots_allowed": ("if (slots[c] == slots[b]) return ORACLE_EDUP;", "continue;"),
    "pos_bound_off_by_one": ("positions[b] >= slot_ctx", "positions[b] > slot_ctx"),
    # slot prefill
    "prefill_ignores_pos0": ("const uint32_t p = pos0 + t;", "const uint32_t p = t;"),
    "prefill_reverse_order": ("const uint32_t p = pos0 + t;", "const uint32_t p = pos0 + (T - 1 - t);"),
    "prefill_range_off_by_one": ("T > slot_ctx - pos0", "T > slot_ctx - pos0 + 1"),
    # multi-row verify
    "verify_dup_allowed": ("if (slots[c] == slots[i]) return ORACLE_EDUP;", "continue;"),
    "verify_rows_not_advanced": ("        row += ks[i];\n", "        row += (ks[i] > 0);\n"),
    "verify_range_off_by_one": ("ks[i] > slot_ctx - pos0[i]", "ks[i] > slot_ctx - pos0[i] + 1"),
    # convention flags
    "interleaved_minus_theta": ("x[2 * i] = a * c - b * s;", "x[2 * i] = a * c + b * s;"),
    "interleaved_angle_index": ("double a = x[2 * i], b = x[2 * i + 1];",
                                "double a = x[2 * i], b = x[2 * i + 1]; th = th * 2.0; c = cos(th); s = sin(th);"),
    "one_plus_w_dropped": ("y[i] = (double)x[i] * r * (1.0 + (double)w[i]);",
                           "y[i] = (double)x[i] * r * (double)w[i];"),
    "vnorm_skipped": ("if (flags & ORACLE_V_NORM) {", "if (0) {"),
    "interleaved_not_on_queries": ("if (flags & ORACLE_ROPE_INTERLEAVED)\n            oracle_rope_interleaved(qh",
                                   "if (0)\n            oracle_rope_interleaved(qh"),
    # per-slot SSM state
    "state_offset_32bit": (
        "return (uint64_t)slot * (uint64_t)state_len * (uint64_t)sizeof(float);",
        "return (uint64_t)(uint32_t)(slot * state_len * 4u);"),
    "reset_conv_only": (
        "for (uint32_t e = 0; e < ssm_len[l]; ++e) s[e] = 0.0f;", "(void)s;"),
    "reset_first_layer_only": (
        "for (uint32_t l = 0; l < n_layers; ++l) {\n            float *c",
        "for (uint32_t l = 0; l < n_layers && l < 1; ++l) {\n            float *c"),
    "reset_short_by_one": (
        "e < conv_len[l]; ++e) c[e]", "e + 1 < conv_len[l]; ++e) c[e]"),
    "reset_ssm_stride_from_conv": (
        "oracle_slot_state_offset_bytes(slots[i], ssm_len[l])",
        "oracle_slot_state_offset_bytes(slots[i], conv_len[l])"),
    "reset_partial_write_on_error": (
        "for (uint32_t i = 0; i < n; ++i)\n        if (slots[i] >= n_slots) return ORACLE_ERANGE;\n"
        "    for (uint32_t i = 0; i < n; ++i) {\n",
        "for (uint32_t i = 0; i < n; ++i) {\n        if (slots[i] >= n_slots) return ORACLE_ERANGE;\n"),
    "reset_unallocated_not_noop": (
        "if (n_slots == 0) return ORACLE_OK;\n    for (uint32_t i = 0; i < n; ++i)\n        if (slots",
        "for (uint32_t i = 0; i < n; ++i)\n        if (slots"),
}
PIN_FILES = ["test_oracle_pins.py", "test_oracle_prefill_pins.py", "test_oracle_conventions.py",
             "test_oracle_state_pins.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(old, new, 1))
    lib = oracle.build(force=True, src=str(mut_src), out=str(tmp_path / "libmutant.so"))
    env = dict(os.environ, SLOT_KV_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
