"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (CPU only; the real oracle is untouched).

Each mutant is moe_oracle.c with one textual substitution, compiled with the
same flags into a temporary library and run through the pin that should fail.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
import pins
import workloads as W
from oracle import build as obuild

MUTANTS = {
    # layout: slot counted after the increment (off by one)
    "slot_off_by_one": (
        "send_token_idx[t * k + j] = token_per_expert[e];\n      token_per_expert[e] += 1;",
        "token_per_expert[e] += 1;\n      send_token_idx[t * k + j] = token_per_expert[e];",
        "layout"),
    # layout: per-rank count over the wrong experts
    "rank_sum_window": (
        "for (int64_t e = r * epr; e < (r + 1) * epr; ++e) sum += token_per_expert[e];",
        "for (int64_t e = r; e < num_experts; e += ranks) sum += token_per_expert[e];",
        "layout"),
    # notify: inclusive instead of exclusive scan
    "inclusive_scan": (
        "      put_offset[e] = acc;\n      acc += token_per_expert[e];",
        "      acc += token_per_expert[e];\n      put_offset[e] = acc;",
        "notify"),
    # multi-source notify: sources in descending order inside an expert
    "multi_source_descending": (
        "for (int64_t src = 0; src < num_src; ++src) {",
        "for (int64_t src = num_src - 1; src >= 0; --src) {",
        "notify_multi"),
    # multi-source notify: count matrix read transposed
    "multi_count_transposed": (
        "token_per_expert[src * num_experts + e]",
        "token_per_expert[e * num_src + src]",
        "notify_multi"),
    # multi-source notify: offsets stored source-major
    "multi_put_source_major": (
        "put_offset[e * num_src + src] = acc;",
        "put_offset[src * num_experts + e] = acc;",
        "notify_multi"),
    # dispatch: destination rank taken modulo instead of divided
    "dest_rank_modulo": (
        "return (int64_t)recv_base[e / epr] + put_offset[e] + slot;",
        "return (int64_t)recv_base[e % ranks_of(epr, num_experts)] + put_offset[e] + slot;",
        "dispatch"),
    # quant: round half away from zero
    "round_half_away": ("float r = nearbyintf(y);", "float r = roundf(y);", "quant"),
    # quant: the 1e-12 term dropped
    "no_epsilon": ("float denom = amax + 1e-12f;", "float denom = amax;", "quant_zero"),
    # quant: the scale stored instead of its inverse
    "store_scale": ("*inv = 1.0f / s;", "*inv = s;", "quant"),
    # quant: max over signed values instead of magnitudes
    "signed_max": ("float a = fabsf(to_f32(x[i], x_kind));", "float a = to_f32(x[i], x_kind);",
                   "quant"),
    # combine: fused multiply-add
    "fused_fma": ("float p = v * w;\n        acc[i] = acc[i] + p;", "acc[i] = fmaf(v, w, acc[i]);",
                  "combine_golden"),
    # combine: weights read in reverse order
    "weights_reversed": ("float w = topk_w[t * k + j];", "float w = topk_w[t * k + (k - 1 - j)];",
                         "combine_random"),
    # combine: last entry dropped
    "drop_last_term": ("for (int64_t j = 0; j < k; ++j) {\n      int64_t dst = dest_row(topk_idx, send_token_idx, put_offset, recv_base, k, epr,\n                             num_experts, t, j);\n      if (dst < 0) continue;\n      if (dst >= rows) return ORACLE_INTERNAL;\n      float w",
                       "for (int64_t j = 0; j + 1 < k; ++j) {\n      int64_t dst = dest_row(topk_idx, send_token_idx, put_offset, recv_base, k, epr,\n                             num_experts, t, j);\n      if (dst < 0) continue;\n      if (dst >= rows) return ORACLE_INTERNAL;\n      float w",
                       "combine_bound"),
    # combine: dequantise after the weight (q * (inv * w))
    "dequant_reassociated": ("v = (float)codes[dst * h + i] * inv[dst];\n        } else {\n          v = to_f32(recv_rows[dst * h + i], recv_kind);\n        }\n        float p = v * w;",
                             "v = (float)codes[dst * h + i];\n          v = v * (inv[dst] * w);\n        } else {\n          v = to_f32(recv_rows[dst * h + i], recv_kind) * w;\n        }\n        float p = v;",
                             "combine_int8_exact"),
    # epilogue: gate and up halves swapped
    "swiglu_halves_swapped": (
        "float g = (float)acc[i] * weight_scale[i];\n  g = g * token_scale;\n  float u = (float)acc[n + i] * weight_scale[n + i];",
        "float g = (float)acc[n + i] * weight_scale[n + i];\n  g = g * token_scale;\n  float u = (float)acc[i] * weight_scale[i];",
        "swiglu"),
    # epilogue: sigmoid instead of x * sigmoid(x)
    "sigmoid_not_silu": ("float y = g / d;", "float y = 1.0f / d;", "swiglu"),
    # epilogue: e^g instead of e^-g
    "exp_sign": ("float e = exp_cw(-g);", "float e = exp_cw(g);", "swiglu"),
    # epilogue: the +1 of the denominator dropped
    "no_plus_one": ("float d = e + 1.0f;", "float d = e;", "swiglu"),
    # epilogue: the token scale not applied to the gate
    "no_token_scale": ("  g = g * token_scale;", "  (void)0;", "swiglu"),
    # epilogue: the up half dequantised with the gate column's scale
    "up_scale_column": ("float u = (float)acc[n + i] * weight_scale[n + i];",
                        "float u = (float)acc[n + i] * weight_scale[i];", "swiglu"),
    # epilogue: the two scales multiplied together first
    "dequant_scales_first": ("float g = (float)acc[i] * weight_scale[i];\n  g = g * token_scale;",
                             "float g = (float)acc[i] * (weight_scale[i] * token_scale);",
                             "swiglu_dequant"),
    # epilogue: the scale stored instead of its inverse
    "swiglu_store_scale": ("inv[0] = 1.0f / s;", "inv[0] = s;", "swiglu"),
    # first expert matmul: weights read as [groups][k][n]
    "gemm_weights_transposed": ("(int64_t)w[(owner * n + j) * k + i]",
                                "(int64_t)w[(owner * k + i) * n + j]", "gemm"),
    # first expert matmul: a row past an expert's end still counted as its
    "gemm_group_end_inclusive": ("if (m >= start && m < start + c) {",
                                 "if (m >= start && m <= start + c) {", "gemm"),
    # first expert matmul: negative counts not clamped
    "gemm_negative_count": ("int64_t c = group_count[g] > 0 ? group_count[g] : 0;",
                            "int64_t c = group_count[g];", "gemm"),
    # first expert matmul: the last product dropped
    "gemm_drop_last_k": ("for (int64_t i = 0; i < k; ++i)\n        acc += (int64_t)a",
                         "for (int64_t i = 0; i + 1 < k; ++i)\n        acc += (int64_t)a", "gemm"),
    # first expert matmul: rows read densely instead of at the row stride
    "gemm_dense_rows": ("(int64_t)a[m * a_stride + i]", "(int64_t)a[m * k + i]", "gemm"),
    # exp: Taylor series cut at degree 6
    "exp_degree6": ("float p = 1.0f / 5040.0f;\n  p = p * r + 1.0f / 720.0f;",
                    "float p = 1.0f / 720.0f;", "exp"),
    # exp: the low part of ln 2 dropped from the reduction
    "exp_no_c2": ("r = r - kf * c2;", "(void)c2;", "exp"),
    # exp: k truncated instead of rounded (|r| up to ln 2)
    "exp_trunc_k": ("float kf = nearbyintf(x * log2e);", "float kf = truncf(x * log2e);", "exp"),
    # exp: subnormal results flushed to zero
    "exp_flush_subnormal": ("if (k < -126) return (p * pow2i(k + 64)) * pow2i(-64);",
                            "if (k < -126) return 0.0f;", "exp"),
    # conversions: bf16 narrowing by truncation
    "bf16_truncate": ("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
                      "(void)lower;", "conversions"),
    # conversions: fp16 subnormal scale off by one binade
    "f16_subnormal": ("mag = ldexpf((float)man, -24);", "mag = ldexpf((float)man, -25);",
                      "conversions"),
}

_HELPER = "static int64_t ranks_of(int64_t epr, int64_t ne) { return ne / epr; }\n"


def _build_mutant(tmp_path, name):
    old, new, _ = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique / not found"
    src = src.replace(old, new)
    if "ranks_of" in new:
        src = src.replace("/* Destination row of entry", _HELPER + "/* Destination row of entry")
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *obuild.CFLAGS, "-Wno-error", "-o", str(so), str(c), "-lm"], check=True)
    return oracle.Oracle(str(so))


def _combine_int8_exact(orc):
    """int8 combine against the exact stepwise definition: v = R(q * inv),
    p = R(v * w), acc = R(acc + p), computed in rationals."""
    from fractions import Fraction

    w = W.random_case(71, 6, 16, 3, 6, 3, routing="uniform")
    lay = orc.layout(w.topk_idx, 2, 3)
    no = orc.notify(lay["token_per_expert"], 2, 3)
    d = orc.dispatch(w.x, "bf16", w.topk_idx, lay["send_token_idx"], no["put_offset"],
                     no["recv_base"], 2, 3, True)
    out = orc.combine(d, "int8", w.topk_idx, w.topk_w, lay["send_token_idx"], no["put_offset"],
                      no["recv_base"], 2, 3, "fp32")
    for t in range(w.bs):
        for i in range(16):
            acc = Fraction(0)
            for j in range(w.topk):
                e = int(w.topk_idx[t, j])
                row = int(no["recv_base"][e // 2] + no["put_offset"][e] + lay["send_token_idx"][t, j])
                v = pins.round_f32(Fraction(int(d["codes"][row, i])) * pins.frac(d["inv"][row]))
                p = pins.round_f32(v * pins.frac(w.topk_w[t, j]))
                acc = pins.round_f32(acc + p)
            assert pins.f32_bits(out[t, i]) == pins.f32_bits(np.float32(float(acc))), (t, i)


def _run_pin(orc, which):
    if which == "layout":
        pins.check_layout_bruteforce(orc)
    elif which == "notify":
        w = W.make_workload("small")
        lay = orc.layout(w.topk_idx, w.expert_num_per_rank, w.rank_size)
        pins.check_notify(orc, lay["token_per_expert"], w.expert_num_per_rank, w.rank_size)
    elif which == "notify_multi":
        pins.check_notify_multi_golden(orc)
        idxs = [W.random_case(450 + i, bs, 8, 4, 12, 3, routing="dup").topk_idx
                for i, bs in enumerate((20, 7, 13))]
        pins.check_multi_receive_order(orc, idxs, 4, 3)
    elif which == "dispatch":
        w = W.make_workload("small")
        pins.check_dispatch_passthrough(orc, w.x, "bf16", w.topk_idx, w.expert_num_per_rank,
                                        w.rank_size)
    elif which == "quant":
        pins.check_quant_golden(orc)
    elif which == "quant_zero":
        pins.check_quant_golden(orc)
    elif which == "combine_golden":
        pins.check_combine_golden(orc)
    elif which == "combine_bound":
        w = W.random_case(42, 33, 40, 8, 16, 4, routing="dup")
        lay = orc.layout(w.topk_idx, 4, 4)
        no = orc.notify(lay["token_per_expert"], 4, 4)
        d = orc.dispatch(w.x, "bf16", w.topk_idx, lay["send_token_idx"], no["put_offset"],
                         no["recv_base"], 4, 4, False)
        pins.check_combine_bound(orc, d, "bf16", w.topk_idx, w.topk_w, lay["send_token_idx"],
                                 no["put_offset"], no["recv_base"], 4, 4)
    elif which == "combine_random":
        pins.check_combine_random_rows(orc)
    elif which == "combine_int8_exact":
        _combine_int8_exact(orc)
    elif which == "swiglu":
        pins.check_swiglu_golden(orc)
        pins.check_swiglu_bound(orc)
    elif which == "swiglu_dequant":
        pins.check_swiglu_dequant_exact(orc)
    elif which == "exp":
        pins.check_exp(orc)
    elif which == "gemm":
        pins.check_gemm_per_expert_matmul(orc)
        pins.check_gemm_closed_forms(orc)
        pins.check_gemm_permutation(orc)
        pins.check_gemm_ownership(orc)
    elif which == "conversions":
        pins.check_conversions(orc)
    else:
        raise ValueError(which)


def test_pins_pass_on_real_oracle(orc):
    for which in sorted({m[2] for m in MUTANTS.values()}):
        _run_pin(orc, which)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    mut = _build_mutant(tmp_path, name)
    with pytest.raises((AssertionError, oracle.OracleError)):
        _run_pin(mut, MUTANTS[name][2])
