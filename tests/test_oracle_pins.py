"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compare the oracle with itself: each check is a closed form, a
hand-derived worked example, a special case that reduces to a library routine
(torch's nn.Linear / SiLU / RMSNorm in float64), brute force, or an exact
invariant of the definition (bitwise equalities).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunk_level_activation_amd import inputs
from golden_io import load


def _markov_inputs(seed, T, d_h, E, d_e, tls, cls, L=8):
    rng = np.random.default_rng(seed)
    x = inputs.gaussian(rng, (T, d_h), 1.0, False)
    w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, False)
    scores = inputs.scores_for_mask(rng, inputs.markov_active(rng, T, E, tls, cls, L))
    return x, scores, w1, w2


def _hand_masks(T, E, n, seed=0):
    """Hand-built activity masks: an empty chunk, a full chunk, one expert only,
    an alternating pattern and a partial last chunk."""
    rng = np.random.default_rng(seed)
    act = np.zeros((T, E), bool)
    # chunk 0 empty; chunk 1 full; chunk 2 one expert on one token
    act[n:2 * n, :] = True
    act[2 * n + 1, E - 1] = True
    # chunk 3: alternating tokens and experts
    for t in range(3 * n, 4 * n):
        act[t, (t % 2)::2] = True
    # the rest: sparse random
    act[4 * n:] = rng.random((T - 4 * n, E)) < 0.1
    return act


# ----------------------------------------------------------------- worked examples

def test_router_worked_example():
    g = load("router_worked_example.txt")
    logits, scores = oracle.router(g["x"], g["W_r"], gain=g["gain"][0], eps=0.0)
    np.testing.assert_array_equal(logits, g["logits"])
    np.testing.assert_allclose(scores, g["scores_over_sqrt3_div5"] * math.sqrt(3) / 5,
                               rtol=1e-15, atol=0)


def test_ffn_worked_example():
    g = load("ffn_worked_example.txt")
    L = math.log(3.0)
    w1 = g["W1"].reshape(2, 2, 3)
    w2 = g["W2"].reshape(2, 3, 2)
    x = (g["x_over_L"] * L).astype(np.float32)
    s = g["scores"].astype(np.float32)
    # x reaches the oracle rounded to fp32 (relative change <= 2^-24); through Swish
    # and the linear maps that moves y by a few 1e-8 relative, far below any
    # formula mistake, which would move it by O(1).
    y_ref = g["y_over_L"] * L
    for fn in (lambda: oracle.chunk_ffn(x, s, w1, w2, n=2),
               lambda: oracle.token_ffn(x, s, w1, w2)):
        np.testing.assert_allclose(fn(), y_ref, rtol=5e-7, atol=1e-12)
    masks, lists, counts = oracle.chunk_union(s, n=2)
    assert counts.tolist() == [2, 2]
    assert lists[0, :2].tolist() == g["union_chunk0"][0].astype(int).tolist()
    assert lists[1, :2].tolist() == g["union_chunk1"][0].astype(int).tolist()
    assert masks[:, 0].tolist() == [3, 3]


# ----------------------------------------------------------------- router

def _torch_router(x, w_r, gain, bias, eps):
    """The router assembled from torch's own modules in float64."""
    T, d_h = x.shape
    E = w_r.shape[0]
    lin = torch.nn.Linear(d_h, E, bias=bias is not None, dtype=torch.float64)
    norm = torch.nn.RMSNorm(E, eps=eps, dtype=torch.float64)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(w_r.astype(np.float64)))
        if bias is not None:
            lin.bias.copy_(torch.from_numpy(bias.astype(np.float64)))
        norm.weight.copy_(torch.from_numpy(gain.astype(np.float64)))
        logits = lin(torch.from_numpy(x.astype(np.float64)))
        scores = norm(torch.nn.functional.relu(logits))
    return logits.numpy(), scores.numpy()


@pytest.mark.parametrize("use_bias", [False, True])
def test_router_matches_torch_modules(use_bias):
    inp = inputs.make_workload("tiny", seed=3)
    rng = np.random.default_rng(7)
    gain = (rng.random(inp.E) + 0.5).astype(np.float32)
    bias = inputs.router_shift(inp.w_r, 0.8) if use_bias else None
    l_o, s_o = oracle.router(inp.x, inp.w_r, gain=gain, bias=bias)
    l_t, s_t = _torch_router(inp.x, inp.w_r, gain, bias, oracle.FP32_EPS)
    np.testing.assert_allclose(l_o, l_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s_o, s_t, rtol=1e-12, atol=1e-12)


def test_rmsnorm_closed_form():
    inp = inputs.make_workload("tiny", seed=1)
    l, s = oracle.router(inp.x, inp.w_r)
    r = np.maximum(l, 0.0)
    ms = (r ** 2).mean(axis=1)
    lhs = (s ** 2).sum(axis=1)
    rhs = inp.E * ms / (ms + oracle.FP32_EPS)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)
    # with eps = 0 every row with an active expert has sum of squares exactly E
    _, s0 = oracle.router(inp.x, inp.w_r, eps=0.0)
    rows = (l > 0).any(axis=1)
    np.testing.assert_allclose((s0[rows] ** 2).sum(axis=1), inp.E, rtol=1e-12)


def test_router_all_inactive_row_is_zero():
    x = np.ones((2, 8), np.float32)
    w_r = -np.ones((4, 8), np.float32)
    _, s = oracle.router(x, w_r)
    assert np.all(s == 0.0)


def test_router_scale_invariance_and_gain():
    inp = inputs.make_workload("tiny", seed=2)
    _, s1 = oracle.router(inp.x, inp.w_r, eps=0.0)
    _, s4 = oracle.router(inp.x, inp.w_r * np.float32(4.0), eps=0.0)
    np.testing.assert_array_equal(s1, s4)          # powers of two scale exactly
    g = np.where(np.arange(inp.E) % 2 == 0, 2.0, 0.5).astype(np.float32)
    _, sg = oracle.router(inp.x, inp.w_r, gain=g, eps=0.0)
    np.testing.assert_array_equal(sg, s1 * g)


# ----------------------------------------------------------------- union

@pytest.mark.parametrize("T,n", [(64, 8), (70, 8), (96, 32), (5, 8), (33, 32)])
def test_union_matches_numpy(T, n):
    E = 80                                        # two mask words, second partial
    act = np.random.default_rng(T).random((T, E)) < 0.05
    s = np.where(act, 1.0, 0.0).astype(np.float32)
    s[0, 3] = -0.0                                # negative zero is inactive
    masks, lists, counts = oracle.chunk_union(s, n)
    C = -(-T // n)
    assert masks.shape == (C, 2)
    for c in range(C):
        u = (s[c * n:c * n + n] != 0).any(axis=0)
        ids = np.nonzero(u)[0]
        assert counts[c] == len(ids)
        assert lists[c, :len(ids)].tolist() == ids.tolist()
        assert np.all(lists[c, len(ids):] == -1)
        bits = [int(masks[c, w]) for w in range(2)]
        for e in range(E):
            assert bool((bits[e // 64] >> (e % 64)) & 1) == bool(u[e])


# ----------------------------------------------------------------- FFN

@pytest.mark.parametrize("case", ["router", "markov", "hand"])
def test_union_then_mask_equals_bruteforce(case):
    """P-1: extra union experts carry score 0 and add exactly nothing (bitwise)."""
    T, d_h, E, d_e, n = 64, 64, 16, 32, 8
    if case == "router":
        inp = inputs.make_workload("tiny", seed=4)
        _, sc = oracle.router(inp.x, inp.w_r)
        x, w1, w2, n = inp.x, inp.w1, inp.w2, inp.n
        s = sc.astype(np.float32)
    elif case == "markov":
        x, s, w1, w2 = _markov_inputs(5, T, d_h, E, d_e, 0.8, 0.5)
    else:
        rng = np.random.default_rng(6)
        x = inputs.gaussian(rng, (T + 3, d_h), 1.0, False)
        w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, False)
        s = inputs.scores_for_mask(rng, _hand_masks(T + 3, E, n))
    y_union = oracle.chunk_ffn(x, s, w1, w2, n)
    y_token = oracle.token_ffn(x, s, w1, w2)
    assert np.array_equal(y_union, y_token)
    # and the union is really wider than the tokens' own sets somewhere
    _, _, counts = oracle.chunk_union(s, n)
    assert counts.sum() * n > (s != 0).sum()


def _torch_dense_layer(x, s, w1, w2):
    """The pages' dense special case: every expert as torch nn.Linear/SiLU modules in
    float64, gated by the scores and summed over experts."""
    E, d_e, d_h = w1.shape
    xt = torch.from_numpy(x.astype(np.float64))
    out = torch.zeros_like(xt)
    with torch.no_grad():
        for e in range(E):
            fc1 = torch.nn.Linear(d_h, d_e, bias=False, dtype=torch.float64)
            fc2 = torch.nn.Linear(d_e, d_h, bias=False, dtype=torch.float64)
            fc1.weight.copy_(torch.from_numpy(w1[e].astype(np.float64)))
            fc2.weight.copy_(torch.from_numpy(w2[e].astype(np.float64)))
            out += torch.from_numpy(s[:, e:e + 1].astype(np.float64)) * \
                fc2(torch.nn.SiLU()(fc1(xt)))
    return out.numpy()


def test_dense_special_case_matches_torch_layer():
    """P-3: with every expert active the layer is the dense sum of all expert MLPs."""
    inp = inputs.make_workload("tiny", seed=8, T=24)
    rng = np.random.default_rng(9)
    s = (np.abs(rng.standard_normal((inp.T, inp.E))) + 0.1).astype(np.float32)
    y = oracle.chunk_ffn(inp.x, s, inp.w1, inp.w2, inp.n)
    y_ref = _torch_dense_layer(inp.x, s, inp.w1, inp.w2)
    np.testing.assert_allclose(y, y_ref, rtol=0, atol=1e-12 * np.abs(y_ref).max())
    # with unit scores it is exactly the dense FFN of equal parameters
    ones = np.ones_like(s)
    y1 = oracle.chunk_ffn(inp.x, ones, inp.w1, inp.w2, inp.n)
    w1cat = inp.w1.reshape(inp.E * inp.d_e, inp.d_h).astype(np.float64)
    w2cat = inp.w2.transpose(1, 0, 2).reshape(inp.d_h, inp.E * inp.d_e).astype(np.float64)
    fc1 = torch.nn.functional.linear(torch.from_numpy(inp.x.astype(np.float64)),
                                     torch.from_numpy(w1cat))
    dense = torch.nn.functional.linear(torch.nn.functional.silu(fc1),
                                       torch.from_numpy(w2cat)).numpy()
    np.testing.assert_allclose(y1, dense, rtol=0, atol=1e-12 * np.abs(dense).max())


def test_experts_outside_union_are_never_read():
    """P-2: NaN weights on experts outside every union leave y unchanged."""
    T, d_h, E, d_e, n = 32, 64, 16, 32, 8
    x, s, w1, w2 = _markov_inputs(10, T, d_h, E, d_e, 0.9, 0.85)
    masks, _, _ = oracle.chunk_union(s, n)
    used = np.zeros(E, bool)
    for c in range(masks.shape[0]):
        used |= [(int(masks[c, 0]) >> e) & 1 == 1 for e in range(E)]
    assert not used.all(), "draw must leave some expert unused"
    w1n, w2n = w1.copy(), w2.copy()
    w1n[~used] = np.nan
    w2n[~used] = np.nan
    y = oracle.chunk_ffn(x, s, w1, w2, n)
    yn = oracle.chunk_ffn(x, s, w1n, w2n, n)
    assert np.all(np.isfinite(yn))
    assert np.array_equal(y, yn)


def test_chunk_size_invariance():
    """P-6: y does not depend on n (bitwise), partial last chunks included."""
    T, d_h, E, d_e = 40, 64, 16, 32
    x, s, w1, w2 = _markov_inputs(11, T, d_h, E, d_e, 0.8, 0.7)
    ys = [oracle.chunk_ffn(x, s, w1, w2, n) for n in (1, 5, 8, 32, T, 1000)]
    for y in ys[1:]:
        assert np.array_equal(ys[0], y)


def test_score_homogeneity_and_additivity():
    """P-7: y is linear in the scores: y(2s) == 2 y(s) bitwise, and scores split over
    two disjoint expert sets add up."""
    T, d_h, E, d_e, n = 32, 64, 16, 32, 8
    x, s, w1, w2 = _markov_inputs(12, T, d_h, E, d_e, 0.6, 0.4)
    y = oracle.chunk_ffn(x, s, w1, w2, n)
    assert np.array_equal(oracle.chunk_ffn(x, 2 * s, w1, w2, n), 2 * y)
    a = s.copy()
    a[:, E // 2:] = 0
    b = s - a
    ya = oracle.chunk_ffn(x, a, w1, w2, n)
    yb = oracle.chunk_ffn(x, b, w1, w2, n)
    np.testing.assert_allclose(ya + yb, y, rtol=0, atol=1e-13 * np.abs(y).max())


def test_expert_permutation():
    """P-9: renaming experts permutes the union list and leaves y unchanged."""
    T, d_h, E, d_e, n = 32, 64, 16, 32, 8
    x, s, w1, w2 = _markov_inputs(13, T, d_h, E, d_e, 0.8, 0.7)
    perm = np.random.default_rng(0).permutation(E)
    y = oracle.chunk_ffn(x, s, w1, w2, n)
    yp = oracle.chunk_ffn(x, s[:, perm], w1[perm], w2[perm], n)
    np.testing.assert_allclose(yp, y, rtol=0, atol=1e-13 * np.abs(y).max())
    _, l0, c0 = oracle.chunk_union(s, n)
    _, l1, c1 = oracle.chunk_union(s[:, perm], n)
    assert np.array_equal(c0, c1)
    inv = np.argsort(perm)
    for c in range(len(c0)):
        assert sorted(perm[l1[c, :c1[c]]].tolist()) == l0[c, :c0[c]].tolist()
        assert sorted(inv[l0[c, :c0[c]]].tolist()) == l1[c, :c1[c]].tolist()


def test_single_token_single_expert_closed_form():
    """One token, one active expert: y = s * W2 swish(W1 x), with swish from its
    definition evaluated through torch's sigmoid in float64."""
    rng = np.random.default_rng(14)
    d_h, E, d_e = 16, 4, 8
    x = rng.standard_normal((1, d_h)).astype(np.float32)
    w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, False)
    s = np.zeros((1, E), np.float32)
    s[0, 2] = 1.5
    a = w1[2].astype(np.float64) @ x[0].astype(np.float64)
    h = a * torch.sigmoid(torch.from_numpy(a)).numpy()
    y_ref = 1.5 * (w2[2].astype(np.float64) @ h)
    np.testing.assert_allclose(oracle.chunk_ffn(x, s, w1, w2, 32)[0], y_ref,
                               rtol=1e-13, atol=1e-13)
