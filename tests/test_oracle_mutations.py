"""The pins reject plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU, in a
temporary directory), builds it, loads it in place of the real oracle and runs the
pin tests; at least one pin must fail. The real oracle is restored afterwards.
"""
import os

import pytest

import oracle
import test_oracle_backward_pins as bpins
import test_oracle_loss_pins as lpins
import test_oracle_pins as pins

# (name, text in the source, planted replacement)
MUTATIONS = [
    ("router bias dropped", "acc += (double)bias[e];", "acc += 0.0;"),
    ("router weight transposed", "const float *we = w_r + e * d_h;",
     "const float *we = w_r + e;"),
    ("relu lets negatives through", "double r = lt[e] > 0.0 ? lt[e] : 0.0;",
     "double r = lt[e] > -0.5 ? lt[e] : 0.0;"),
    ("rms without the mean", "double mean_sq = sumsq / (double)E;",
     "double mean_sq = sumsq;"),
    ("rms norm without sqrt", "double denom = sqrt(mean_sq + eps);",
     "double denom = (mean_sq + eps);"),
    ("gain ignored", "double g = gain ? (double)gain[e] : 1.0;", "double g = 1.0;"),
    ("chunk skips its first token", "for (int64_t t = c * n; t < t_end; ++t)",
     "for (int64_t t = c * n + 1; t < t_end; ++t)"),
    ("union bit in the wrong word", "mc[e / 64] |= (uint64_t)1 << (e % 64);",
     "mc[0] |= (uint64_t)1 << (e % 64);"),
    ("swish sign flipped", "h[k] = a / (1.0 + exp(-a));", "h[k] = a / (1.0 + exp(a));"),
    ("relu instead of swish", "h[k] = a / (1.0 + exp(-a));", "h[k] = a > 0 ? a : 0;"),
    ("fc1 transposed", "a += (double)w1e[k * d_h + j] * (double)xt[j];",
     "a += (double)w1e[j * d_e + k] * (double)xt[j];"),
    ("fc2 transposed", "z += (double)w2e[j * d_e + k] * h[k];",
     "z += (double)w2e[k * d_h + j] * h[k];"),
    ("no masking by the score", "yt[j] += s * z;", "yt[j] += z;"),
    ("score applied twice", "yt[j] += s * z;", "yt[j] += s * s * z;"),
    ("score inside the activation",
     "add_expert_output(x + t * d_h, w1 + e * d_e * d_h, w2 + e * d_h * d_e,\n"
     "                              (double)scores[t * E + e], d_h, d_e, h, yt);",
     "add_expert_output(x + t * d_h, w1 + e * d_e * d_h, w2 + e * d_h * d_e,\n"
     "                              (double)scores[t * E + e] + 1.0, d_h, d_e, h, yt);"),
    ("wrong expert slab for fc2",
     "add_expert_output(x + t * d_h, w1 + e * d_e * d_h, w2 + e * d_h * d_e,\n"
     "                              (double)scores[t * E + e], d_h, d_e, h, yt);",
     "add_expert_output(x + t * d_h, w1 + e * d_e * d_h, w2,\n"
     "                              (double)scores[t * E + e], d_h, d_e, h, yt);"),
    ("probs ignore sharpness", "probs[i] = 1.0 / (1.0 + exp(-sharpness * scores[i]));",
     "probs[i] = 1.0 / (1.0 + exp(-scores[i]));"),
    ("layernorm unbiased variance", "var /= (double)d;", "var /= (double)(d - 1);"),
    ("layernorm eps outside sqrt", "double inv = 1.0 / sqrt(var + eps);",
     "double inv = 1.0 / (sqrt(var) + eps);"),
    ("layernorm beta dropped", "(beta ? (double)beta[j] : 0.0);", "0.0;"),
    ("layernorm residual dropped",
     "mean += (double)y[t * d + j] + (double)x[t * d + j];", "mean += (double)y[t * d + j];"),
    ("sharpening without the 2p - 1", "return 1.0 / (1.0 + exp(-alpha * (2.0 * p - 1.0)));",
     "return 1.0 / (1.0 + exp(-alpha * p));"),
    ("locality bce target and input swapped",
     "sum += -(c * log(nx + LOSS_LOG_EPS) + (1.0 - c) * log(1.0 - nx + LOSS_LOG_EPS));",
     "sum += -(nx * log(c + LOSS_LOG_EPS) + (1.0 - nx) * log(1.0 - c + LOSS_LOG_EPS));"),
    ("locality divided by S", "return loss / (double)(S - 1 > 1 ? S - 1 : 1);",
     "return loss / (double)S;"),
    ("chunk one token short", "const int64_t t0 = c * L, t1 = t0 + L < S ? t0 + L : S;\n"
     "        double sum", "const int64_t t0 = c * L, t1 = t0 + L - 1 < S ? t0 + L - 1 : S;\n"
     "        double sum"),
    ("chunk count floored", "const int64_t nc = (S + L - 1) / L;\n    double loss",
     "const int64_t nc = S / L > 0 ? S / L : 1;\n    double loss"),
    ("locality grad without the sharpening slope",
     "grad[a0] += scale * dc * 2.0 * alpha * c * (1.0 - c);", "grad[a0] += scale * dc;"),
    ("locality grad next-row sign",
     "double dn = -(c / (nx + LOSS_LOG_EPS) - (1.0 - c) / (1.0 - nx + LOSS_LOG_EPS));",
     "double dn = (c / (nx + LOSS_LOG_EPS) - (1.0 - c) / (1.0 - nx + LOSS_LOG_EPS));"),
    ("sparsification grad includes its own factor", "if (j != k)", "if (1)"),
    ("backward: swish slope without its second term",
     "dat[k] = dh * (sg[k] * (1.0 + a[k] * (1.0 - sg[k])));", "dat[k] = dh * sg[k];"),
    ("backward: dW2 without the score", "g2[j * d_e + k] += s * (double)dyt[j] * h[k];",
     "g2[j * d_e + k] += (double)dyt[j] * h[k];"),
    ("backward: hidden gradient without the score",
     "dh += (double)w2e[j * d_e + k] * s * (double)dyt[j];",
     "dh += (double)w2e[j * d_e + k] * (double)dyt[j];"),
    ("backward: rmsnorm coupling sign",
     "const double dr = g * inv * dst[e] - inv * inv * inv * r / (double)E * coup;",
     "const double dr = g * inv * dst[e] + inv * inv * inv * r / (double)E * coup;"),
    ("backward: rmsnorm coupling without 1/E",
     "const double dr = g * inv * dst[e] - inv * inv * inv * r / (double)E * coup;",
     "const double dr = g * inv * dst[e] - inv * inv * inv * r * coup;"),
    ("backward: relu gate dropped", "dst[e] = active ? dr : 0.0;", "dst[e] = dr;"),
    ("backward: probability slope without sharpness",
     "dst[e] += (double)dprobs[t * E + e] * sharpness * p * (1.0 - p);",
     "dst[e] += (double)dprobs[t * E + e] * p * (1.0 - p);"),
    ("backward: gain gradient without the norm", "logits[t * E + e] = dst[e] * r * inv;",
     "logits[t * E + e] = dst[e] * r;"),
    ("backward: router term of dx dropped",
     "dxt[j] += (double)w_r[e * d_h + j] * dst[e];", "dxt[j] += 0.0 * dst[e];"),
    ("backward: dW_r from the wrong token row",
     "dw_r[e * d_h + j] += dl * (double)x[t * d_h + j];",
     "dw_r[e * d_h + j] += dl * (double)x[(T - 1 - t) * d_h + j];"),
]

PIN_TESTS = [
    pins.test_router_worked_example,
    pins.test_ffn_worked_example,
    lambda: pins.test_router_matches_torch_modules(True),
    pins.test_rmsnorm_closed_form,
    pins.test_router_scale_invariance_and_gain,
    lambda: pins.test_union_matches_numpy(70, 8),
    lambda: pins.test_union_then_mask_equals_bruteforce("hand"),
    pins.test_dense_special_case_matches_torch_layer,
    pins.test_score_homogeneity_and_additivity,
    pins.test_single_token_single_expert_closed_form,
    lpins.test_probs_half_at_zero_and_library_sigmoid,
    lpins.test_layernorm_worked_example,
    lpins.test_layernorm_matches_library,
    lpins.test_layernorm_residual_is_added_not_replaced,
    lambda: lpins.test_locality_equals_library_bce(2.0),
    lpins.test_locality_single_token_and_scale,
    lpins.test_sparsification_closed_forms,
    lambda: lpins.test_sparsification_brute_force(13, 4),
    lambda: lpins.test_locality_grad_finite_differences(2.0),
    lambda: lpins.test_sparsification_grad_finite_differences(9, 4),
    lpins.test_sparsification_grad_closed_forms,
    lambda: bpins.test_backward_matches_torch_autograd(bpins.CASES[0]),
    lambda: bpins.test_backward_matches_torch_autograd(bpins.CASES[1]),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(tmp_path, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.build(src=path, out=os.path.join(tmp_path, "libmutant.so"))
    failures = 0
    oracle.use_library(lib)
    try:
        for pin in PIN_TESTS:
            try:
                pin()
            except AssertionError:
                failures += 1
    finally:
        oracle.use_library(None)
    assert failures > 0, f"no pin caught the planted mistake: {name}"
