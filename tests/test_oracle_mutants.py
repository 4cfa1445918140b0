"""Plant plausible mistakes in copies of the oracle and check the pins catch them.

Each mutant is a one-line textual change to oracle/oracle.c (a dropped term,
a wrong sign, index, rounding rule or operand order), compiled with gcc into
a temporary library.  The pins of tests/test_oracle_pins.py are then run
against that build; at least one of them must fail.  This is CPU-only: the
mistakes live in throwaway copies of the oracle, never in the GPU path.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
HDR = os.path.join(os.path.dirname(oracle.__file__), "oracle.h")

ALL_PINS = [
    pins.pin_quantize_golden, pins.pin_quantize_invariants, pins.pin_block_dots, pins.pin_matvec,
    pins.pin_rmsnorm, pins.pin_rope, pins.pin_silu, pins.pin_attention, pins.pin_moe_route,
    pins.pin_moe_block, lambda: pins.pin_layer(0, 1), lambda: pins.pin_layer(1, 1),
    lambda: pins.pin_layer(0, 0), pins.pin_f16, pins.pin_bf16, pins.pin_lm_head, pins.pin_gelu,
    pins.pin_attention_softcap, pins.pin_rope_freqs, pins.pin_matmul, pins.pin_q4_0, pins.pin_q6_k,
    lambda: pins.test_layer_zero_projections_is_identity(0, 1),
    lambda: pins.test_layer_zero_projections_is_identity(1, 1),
    lambda: pins.test_layer_one_position_closed_form(0, 1),
    lambda: pins.test_layer_one_position_closed_form(1, 1),
]

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("q4_high_nibble_dropped", "q[j + 16] = (int8_t)((blk[2 + j] >> 4) - 8);",
     "q[j + 16] = (int8_t)((blk[2 + j] & 0x0F) - 8);"),
    ("q4_offset", "q[j] = (int8_t)((blk[2 + j] & 0x0F) - 8);", "q[j] = (int8_t)((blk[2 + j] & 0x0F) - 7);"),
    ("q6_qh_shift", "const int hi = (qh[32 * h + l] >> (2 * g)) & 3;", "const int hi = (qh[32 * h + l] >> g) & 3;"),
    ("q6_ql_half", "const uint8_t lb = ql[64 * h + 32 * (g % 2) + l];",
     "const uint8_t lb = ql[64 * h + 32 * (g / 2) + l];"),
    ("q6_offset", "q[i] = (int8_t)((lo | (hi << 4)) - 32);", "q[i] = (int8_t)((lo | (hi << 4)) - 31);"),
    ("q6_scale_by_32", "w[256 * b + i] = d * (double)sc[i / 16] * (double)q[i];",
     "w[256 * b + i] = d * (double)sc[i / 32] * (double)q[i];"),
    ("q6_matvec_scale", "acc += d * (double)sc[k] * (double)orc_f16_to_f32(xd[c0 / 32]) * (double)dot;",
     "acc += d * (double)sc[k / 2] * (double)orc_f16_to_f32(xd[c0 / 32]) * (double)dot;"),
    ("q6_matvec_act_block", "acc += d * (double)sc[k] * (double)orc_f16_to_f32(xd[c0 / 32]) * (double)dot;",
     "acc += d * (double)sc[k] * (double)orc_f16_to_f32(xd[(256 * b) / 32]) * (double)dot;"),
    ("matmul_token_stride", "orc_q8_matvec(wq, wd, rows, cols, xq + t * cols, xd + t * (cols / 32),",
     "orc_q8_matvec(wq, wd, rows, cols, xq + t, xd + t * (cols / 32),"),
    ("rope_factor_multiplies", "if (factors) inv_freq = inv_freq / (double)factors[i];",
     "if (factors) inv_freq = inv_freq * (double)factors[i];"),
    ("moe_scale_ignored", "if (m->expert_scale) ws *= (double)m->expert_scale[e];", "(void)e;"),
    ("moe_scale_by_slot", "if (m->expert_scale) ws *= (double)m->expert_scale[e];",
     "if (m->expert_scale) ws *= (double)m->expert_scale[s];"),
    ("gelu_coefficient", "0.044715 * z * z * z", "0.44715 * z * z * z"),
    ("gelu_no_half", "double gz = 0.5 * z *", "double gz = 1.0 * z *"),
    ("attn_cap_missing", "if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);", "(void)softcap;"),
    ("attn_cap_no_divide", "if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);",
     "if (softcap > 0.0) s[j] = softcap * tanh(s[j]);"),
    ("head_no_norm", "        orc_rmsnorm(x, hidden, gamma, eps, n);", "        for (int64_t c = 0; c < hidden; ++c) n[c] = x[c];"),
    ("head_transposed", "acc += (double)orc_f16_to_f32(row[c]) * (double)n[c];",
     "acc += (double)orc_f16_to_f32(w[c * vocab + r < vocab * hidden ? c * vocab + r : 0]) * (double)n[c];"),
    ("head_cap_no_divide", "if (cap > 0.0) acc = cap * tanh(acc / cap);", "if (cap > 0.0) acc = cap * tanh(acc);"),
    ("round_half_even", "float r = roundf(v);", "float r = rintf(v);"),
    ("scale_over_128", "float db = amax / 127.0f;", "float db = amax / 128.0f;"),
    ("no_clamp_and_trunc", "float r = roundf(v);", "float r = truncf(v);"),
    ("f16_truncates", "double m = nearbyint(ldexp(v, 10 - E));", "double m = floor(ldexp(v, 10 - E));"),
    ("f16_subnormal_floor", "double m = nearbyint(ldexp(v, 24));", "double m = floor(ldexp(v, 24));"),
    ("bf16_truncates", "double m = nearbyint(ldexp(v, 7 - E));", "double m = floor(ldexp(v, 7 - E));"),
    ("block_dot_index", "acc += (int32_t)wq[r * cols + 32 * b + i] * (int32_t)xq[32 * b + i];",
     "acc += (int32_t)wq[r * cols + 32 * b + i] * (int32_t)xq[i];"),
    ("matvec_drops_dx", "(double)orc_f16_to_f32(xd[b]) * (double)dot;", "(double)dot;"),
    ("matvec_transposed_scale", "acc += (double)orc_f16_to_f32(wd[r * nb + b]) *",
     "acc += (double)orc_f16_to_f32(wd[b * rows + r < rows * nb ? b * rows + r : 0]) *"),
    ("matvec_no_residual", "if (residual) acc += (double)residual[r];", "(void)residual;"),
    ("rmsnorm_no_mean", "double rinv = 1.0 / sqrt(ss / (double)n + eps);", "double rinv = 1.0 / sqrt(ss + eps);"),
    ("rmsnorm_no_gamma", "double g = gamma ? (double)gamma[i] : 1.0;", "double g = 1.0;"),
    ("rmsnorm_one_plus_gamma", "double g = gamma ? (double)gamma[i] : 1.0;",
     "double g = gamma ? 1.0 + (double)gamma[i] : 1.0;"),
    ("rope_sign", "x[i] = (float)(a * c - b * s);", "x[i] = (float)(a * c + b * s);"),
    ("rope_freq", "double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);",
     "double inv_freq = pow(theta, -1.0 * (double)i / (double)hd);"),
    ("rope_interleaved", "double a = (double)x[i], b = (double)x[i + half];",
     "double a = (double)x[i], b = (double)x[i + 1 < hd ? i + 1 : i];"),
    ("silu_sign", "h[i] = (float)((z / (1.0 + exp(-z))) * (double)u[i]);",
     "h[i] = (float)((z / (1.0 + exp(z))) * (double)u[i]);"),
    ("attn_head_map", "int64_t g = h / G;", "int64_t g = h % n_kv;"),
    ("attn_no_scale", "s[j] = scale * acc;", "s[j] = acc;"),
    ("attn_unnormalised", "double p = s[j] / z;", "double p = s[j];"),
    ("attn_start_ignored", "int64_t base = g * head_stride + (start + j) * pos_stride;\n            double acc",
     "int64_t base = g * head_stride + j * pos_stride;\n            double acc"),
    ("route_tie_high_id", "if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("moe_unweighted", "double ws = (double)w[slot];", "double ws = 1.0;"),
    ("layer_gate_up_swapped", "orc_silu_mul(gu, gu + I, I, tmp);", "orc_silu_mul(gu + I, gu, I, tmp);"),
    ("layer_window_off_by_one", "if (L->window > 0 && pos - L->window + 1 > 0) start = pos - L->window + 1;",
     "if (L->window > 0 && pos - L->window > 0) start = pos - L->window;"),
    ("layer_no_v_norm", "if (L->v_unit_norm) {", "if (0) {"),
    ("layer_no_k_rope", "orc_rope_neox(k + g * hd, hd, c_row, s_row);", "(void)0;"),
    ("layer_post_norm_weight", "orc_rmsnorm(tmp, H, L->g_post, L->eps, n);", "orc_rmsnorm(tmp, H, L->g_in, L->eps, n);"),
    ("layer_o_no_residual", "orc_q8_matvec(L->o_qs, L->o_d, H, qd, q8, d8, x, x1);",
     "orc_q8_matvec(L->o_qs, L->o_d, H, qd, q8, d8, NULL, x1);"),
    ("layer_down_residual_x", "orc_q8_matvec(L->dn_qs, L->dn_d, H, I, q8, d8, x1, x);",
     "orc_q8_matvec(L->dn_qs, L->dn_d, H, I, q8, d8, x, x);"),
    ("layer_postnorm_residual_doubled", "x1[i] = (float)((double)x[i] + (double)n[i]);",
     "x1[i] = (float)(2.0 * (double)x[i] + (double)n[i]);"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: target text not found"
    mutated = src.replace(old, new, 1)
    d = tmp_path / name
    d.mkdir()
    (d / "oracle.c").write_text(mutated)
    shutil.copy(HDR, d / "oracle.h")
    so = d / "liboracle.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-w",
                    "-o", str(so), str(d / "oracle.c"), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    so = _build_mutant(tmp_path, name, old, new)
    caught = None
    with oracle.using(so):
        for pin in ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError, IndexError) as e:
                caught = (getattr(pin, "__name__", "pin"), type(e).__name__)
                break
    assert caught is not None, f"planted mistake {name} survived every pin"
