"""Plants plausible mistakes in a copy of the oracle source (CPU only) and
checks that the pins catch each one.

Each mutant is a one-line textual change of ``oracle/dit_oracle.c`` built
into a temporary library; the named pin tests run against it and at least
one must fail.  This shows the pins constrain the oracle's arithmetic rather
than merely re-running it.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
import test_oracle_pins as pins

MUTANTS = {
    "variance divisor D-1": (
        "float var = orc_sum_wave(t, D) / (float)D;",
        "float var = orc_sum_wave(t, D) / (float)(D - 1);",
        ["test_ln_row_vs_double"]),
    "LayerNorm eps dropped": (
        "float rho = 1.0f / sqrtf(var + eps);",
        "float rho = 1.0f / sqrtf(var);",
        ["test_ln_row_vs_double"]),
    "1 + scale not rounded": (
        "float s1 = orc_bf16_value(orc_one_plus(sc[i]));",
        "float s1 = 1.0f + orc_bf16_value(sc[i]);",
        ["test_ln_modulate_composition_and_mod_rows"]),
    "modulation row index": (
        "const uint16_t *sc = scale + (r / per_mod) * mod_rs;\n    const uint16_t *sh",
        "const uint16_t *sc = scale + (r % mod_rows) * mod_rs;\n    const uint16_t *sh",
        ["test_ln_modulate_composition_and_mod_rows"]),
    "shift and product swapped": (
        "out[r * out_rs + i] = orc_bf16_round(p + orc_bf16_value(sh[i]));",
        "out[r * out_rs + i] = orc_bf16_round(p + orc_bf16_value(sc[i]));",
        ["test_ln_constant_row_gives_shift"]),
    "RMSNorm eps dropped": (
        "uint16_t v = orc_bf16_round(orc_bf16_value(ms) + eps);",
        "uint16_t v = orc_bf16_round(orc_bf16_value(ms));",
        ["test_rms_chain_near_ideal_and_unit_rms"]),
    "RMSNorm squares not rounded": (
        "t[i] = bfv(xv * xv);",
        "t[i] = xv * xv;",
        ["test_rms_rounded_squares_closed_form"]),
    "RMSNorm mean square not rounded": (
        "uint16_t ms = orc_bf16_round(orc_sum_wave(t, D) / (float)D);\n"
        "  uint16_t v = orc_bf16_round(orc_bf16_value(ms) + eps);",
        "float msf = orc_sum_wave(t, D) / (float)D;\n"
        "  uint16_t ms = orc_bf16_round(msf);\n"
        "  uint16_t v = orc_bf16_round(msf + eps);",
        ["test_rms_rounded_squares_closed_form"]),
    "RMSNorm weight skipped": (
        "y2[i] = orc_bf16_round(y1 * orc_bf16_value(w[i]));",
        "y2[i] = orc_bf16_round(y1);",
        ["test_rms_constant_power_of_two_rows"]),
    "tanh sign lost": (
        "return orc_bf16_round_f64(tanh((double)v));",
        "return orc_bf16_round_f64(tanh(fabs((double)v)));",
        ["test_tanh_properties"]),
    "gate product not rounded": (
        "float gy = bfv(orc_bf16_value(g[i]) * orc_bf16_value(y[r * y_rs + i]));",
        "float gy = orc_bf16_value(g[i]) * orc_bf16_value(y[r * y_rs + i]);",
        ["test_residual_gate_add_exact"]),
    "fused LN reads the residual instead of r'": (
        "orc_ln_modulate(out + r * out_rs, out_rs, rp, dim,",
        "orc_ln_modulate(out + r * out_rs, out_rs, residual + r * res_rs, dim,",
        ["test_gate_add_ln_cancellation_gives_shift", "test_gate_add_ln_vs_exact_and_double"]),
    "fused gate from modulation row 0": (
        "gate + m * mod_rs, mod_rs, 1, 1, dim);",
        "gate, mod_rs, 1, 1, dim);",
        ["test_gate_add_ln_vs_exact_and_double"]),
    "fused shift taken from scale": (
        "scale + m * mod_rs, shift + m * mod_rs,",
        "scale + m * mod_rs, scale + m * mod_rs,",
        ["test_gate_add_ln_zero_gate_constant_residual"]),
    "E4M3 ties away from zero": (
        "if (dh < dl || (dh == dl && (hi & 1) == 0)) c = hi;",
        "if (dh <= dl) c = hi;",
        ["test_e4m3_midpoints_tie_to_even_and_saturate"]),
    "E4M3 overflow to NaN": (
        "if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
        "if (a > 464.0) return (uint8_t)(sign | 0x7F);",
        ["test_e4m3_midpoints_tie_to_even_and_saturate"]),
    "FP8 scale by reciprocal": (
        "return orc_e4m3(orc_bf16_value(h) / scale);",
        "return orc_e4m3(orc_bf16_value(h) * (1.0f / scale));",
        ["test_fp8_quantization_divides_by_the_scale"]),
    "modulation table written token-major": (
        "out[((k * batch + b) * tokens + s) * dim + i] = table[k * dim + i] + e;",
        "out[((b * tokens + s) * n_mod + k) * dim + i] = table[k * dim + i] + e;",
        ["test_wan_mod_table_layout_with_tagged_values"]),
    "modulation table reads chunk 0": (
        "const float e = orc_bf16_value(temb[((b * tokens + s) * n_mod + k) * dim + i]);",
        "const float e = orc_bf16_value(temb[((b * tokens + s) * n_mod) * dim + i]);",
        ["test_wan_mod_table_layout_with_tagged_values"]),
    "modulate product not rounded": (
        "float p = bfv(orc_bf16_value(x[r * x_rs + i]) * one_plus);",
        "float p = orc_bf16_value(x[r * x_rs + i]) * one_plus;",
        ["test_modulate_scale_shift_exact_steps"]),
    "heads dealt to destinations round-robin": (
        "int64_t ho = dst + (h / hpd) * dest_stride + (h % hpd) * Dh;",
        "int64_t ho = dst + (h % (heads / hpd)) * dest_stride + (h / (heads / hpd)) * Dh;",
        ["test_qk_norm_rope_destination_major_layout"]),
    "RoPE sign": (
        "o[2 * i] = orc_bf16_round(a * c[i] - b * z[i]);",
        "o[2 * i] = orc_bf16_round(a * c[i] + b * z[i]);",
        ["test_qk_head_quarter_and_half_turns"]),
    "RoPE cos/sin transposed": (
        "o[2 * i + 1] = orc_bf16_round(a * z[i] + b * c[i]);",
        "o[2 * i + 1] = orc_bf16_round(a * c[i] + b * z[i]);",
        ["test_qk_head_quarter_and_half_turns"]),
    "QK eps dropped": (
        "float rho = 1.0f / sqrtf(ms + eps);",
        "float rho = 1.0f / sqrtf(ms);",
        ["test_qk_head_identity_rotation_is_rmsnorm"]),
    "image stream written at text rows": (
        "qkv_stream(q_out, k_out, v_out, out_tok_stride, out_batch_stride, img,\n"
        "               txt ? txt->tokens : 0,",
        "qkv_stream(q_out, k_out, v_out, out_tok_stride, out_batch_stride, img,\n"
        "               0,",
        ["test_qk_norm_rope_joint_placement_and_v_copy"]),
    "head tree half-width": (
        "for (int m = 1; m < lanes; m <<= 1) {",
        "for (int m = 1; m < lanes / 2; m <<= 1) {",
        ["test_sum_head", "test_qk_head_identity_rotation_is_rmsnorm"]),
    "wave lane stride": (
        "int64_t e = 512 * c + 8 * l + j;",
        "int64_t e = 512 * c + 64 * j + l;",
        ["test_sum_wave_order_sensitive_case"]),
    "rounding ties away": (
        "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
        "return (uint16_t)((u + 0x8000u) >> 16);",
        ["test_bf16_round_edges_vs_fractions"]),
    "RMSNorm y1 not rounded": (
        "float y1 = bfv(orc_bf16_value(x[i]) * rv);",
        "float y1 = orc_bf16_value(x[i]) * rv;",
        ["test_rms_y1_rounded_before_the_weight"]),
    "RMSNorm rstd from the unrounded ms + eps": (
        "uint16_t rstd = orc_rms_rstd(v);",
        "uint16_t rstd = orc_bf16_round(1.0f / sqrtf(orc_bf16_value(ms) + eps));",
        ["test_rms_rstd_taken_from_the_rounded_mean_square_plus_eps"]),
    "QK head x * rho not rounded": (
        "float n = bfv(orc_bf16_value(x[i]) * rho);",
        "float n = orc_bf16_value(x[i]) * rho;",
        ["test_qk_head_normalized_value_rounded_before_the_weight"]),
    "RoPE first output fused": (
        "o[2 * i] = orc_bf16_round(a * c[i] - b * z[i]);",
        "o[2 * i] = orc_bf16_round(fmaf(a, c[i], -(b * z[i])));",
        ["test_qk_head_rope_products_rounded_separately"]),
    "RoPE second output fused": (
        "o[2 * i + 1] = orc_bf16_round(a * z[i] + b * c[i]);",
        "o[2 * i + 1] = orc_bf16_round(fmaf(a, z[i], b * c[i]));",
        ["test_qk_head_rope_products_rounded_separately"]),
    "LayerNorm divides by sigma": (
        "for (int64_t i = 0; i < D; ++i) n[i] = orc_bf16_round(d[i] * rho);",
        "for (int64_t i = 0; i < D; ++i) n[i] = orc_bf16_round(d[i] / sqrtf(var + eps));",
        ["test_ln_normalizes_by_multiplying_with_rho"]),
}


def _run_param(fn):
    """Runs a pin test function, expanding the parametrize marks it carries."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        fn()
        return
    name, values = marks[0].args
    for v in values:
        fn(**{name: v})


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path):
    before, after, tests = MUTANTS[mutant]
    src = open(obuild.SRC).read()
    assert src.count(before) == 1, "mutation anchor not found: " + before
    mpath = tmp_path / "dit_oracle.c"
    mpath.write_text(src.replace(before, after))
    lib = str(tmp_path / "libmutant.so")
    obuild.build(src=str(mpath), lib=lib)
    caught = []
    with oracle.using_library(lib):
        for t in tests:
            try:
                _run_param(getattr(pins, t))
            except AssertionError:
                caught.append(t)
    assert caught, f"no pin caught mutant {mutant!r} (ran {tests})"
