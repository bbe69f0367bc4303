"""The pins reject plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU, in a
temporary directory), builds it, loads it in place of the real oracle and runs the
pin tests; at least one pin must fail. The real oracle is restored afterwards.
"""
import os

import pytest

import oracle
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
