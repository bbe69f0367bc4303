"""Pins of the oracle's layer epilogue and training losses.

Pages: skill page "Router Architecture Setup" (probabilities are the sigmoid of the
sharpened scores), "Full BlockFFN Layer with Combined Losses" (LayerNorm of the
expert output plus the residual), "Activation Locality Loss" and "Chunk
Sparsification Loss". Each check is a library routine in float64 (torch's sigmoid,
layer_norm, binary_cross_entropy), a closed form, brute force over activation
patterns, or central finite differences for the gradients; none compares the oracle
with itself.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _probs(seed, B, S, E):
    """float32 probabilities whose float32 values are exact multiples of 2^-16, so
    finite-difference steps of 2^-12 stay exact."""
    rng = np.random.default_rng(seed)
    return (np.round(rng.uniform(0.02, 0.98, (B, S, E)) * 65536) / 65536).astype(np.float32)


# --- router probabilities --------------------------------------------------------

def test_probs_half_at_zero_and_library_sigmoid():
    assert np.all(oracle.router_probs(np.zeros(5)) == 0.5)
    s = np.random.default_rng(1).uniform(0, 3, (7, 9))
    for sharp in (1.0, 2.0, 0.5):
        ref = torch.sigmoid(sharp * torch.from_numpy(s)).numpy()
        np.testing.assert_allclose(oracle.router_probs(s, sharp), ref, rtol=1e-15, atol=0)


def test_probs_symmetry_and_sharpness_scaling():
    s = np.random.default_rng(2).uniform(-3, 3, 50)
    np.testing.assert_allclose(oracle.router_probs(s) + oracle.router_probs(-s), 1.0,
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.router_probs(s, 3.0), oracle.router_probs(3.0 * s),
                               rtol=1e-15, atol=0)


# --- residual + LayerNorm --------------------------------------------------------

def test_layernorm_worked_example():
    """y = (1, 2, 3, 4), x = 0: mean 2.5, biased variance 1.25."""
    y = np.array([[1, 2, 3, 4]], np.float32)
    out = oracle.add_layernorm(y, np.zeros_like(y))
    ref = (np.array([1, 2, 3, 4]) - 2.5) / math.sqrt(1.25 + 1e-5)
    np.testing.assert_allclose(out[0], ref, rtol=1e-15, atol=0)


def test_layernorm_closed_form_moments():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((6, 64)).astype(np.float32)
    x = (3 + 2 * rng.standard_normal((6, 64))).astype(np.float32)
    out = oracle.add_layernorm(y, x, eps=0.0)
    np.testing.assert_allclose(out.mean(1), 0.0, atol=1e-14)
    np.testing.assert_allclose((out ** 2).mean(1), 1.0, rtol=1e-13)


def test_layernorm_matches_library():
    rng = np.random.default_rng(4)
    T, d = 9, 48
    y = rng.standard_normal((T, d)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, d).astype(np.float32)
    b = rng.standard_normal(d).astype(np.float32)
    v = torch.from_numpy(y).double() + torch.from_numpy(x).double()
    for eps in (1e-5, 1e-2):
        ref = F.layer_norm(v, (d,), torch.from_numpy(g).double(), torch.from_numpy(b).double(),
                           eps).numpy()
        np.testing.assert_allclose(oracle.add_layernorm(y, x, g, b, eps), ref,
                                   rtol=1e-12, atol=1e-12)


def test_layernorm_residual_is_added_not_replaced():
    """LN(y + x) depends on y and x only through their sum."""
    rng = np.random.default_rng(5)
    y = rng.standard_normal((3, 32)).astype(np.float32)
    x = rng.standard_normal((3, 32)).astype(np.float32)
    a = oracle.add_layernorm(y, x)
    b = oracle.add_layernorm(np.zeros_like(y), (y.astype(np.float64) + x).astype(np.float32))
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)
    assert not np.allclose(a, oracle.add_layernorm(y, np.zeros_like(x)), atol=1e-2)


# --- activation locality loss ----------------------------------------------------

def _sharp(p, alpha):
    return torch.sigmoid(alpha * (2 * torch.from_numpy(p).double() - 1))


@pytest.mark.parametrize("alpha", [2.0, 5.0])
def test_locality_equals_library_bce(alpha):
    """Each adjacent pair is a binary cross entropy with the earlier sharpened row as
    the target; torch's BCE omits the +1e-8 inside the logs, whose effect on values in
    [sigmoid(-alpha), sigmoid(alpha)] is below 1e-7 relative."""
    p = _probs(6, 3, 11, 5)
    q = _sharp(p, alpha)
    ref = sum(F.binary_cross_entropy(q[:, i + 1], q[:, i]).item() for i in range(10)) / 10
    assert oracle.locality_loss(p, alpha) == pytest.approx(ref, rel=1e-6)


def test_locality_entropy_floor_for_identical_rows():
    """Identical adjacent rows: every pair term is the binary entropy of q."""
    rng = np.random.default_rng(7)
    row = rng.uniform(0.05, 0.95, (2, 1, 6)).astype(np.float32)
    p = np.repeat(row, 9, axis=1)
    q = _sharp(row[:, 0], 2.0).numpy()
    ent = (-(q * np.log(q) + (1 - q) * np.log(1 - q))).mean()
    assert oracle.locality_loss(p) == pytest.approx(ent, rel=1e-6)
    # Gibbs: each pair term is at least the entropy of its target (earlier) row, with
    # equality only when the two rows agree.
    p2 = rng.uniform(0.05, 0.95, (2, 9, 6)).astype(np.float32)
    q2 = _sharp(p2, 2.0).numpy()
    h2 = -(q2 * np.log(q2) + (1 - q2) * np.log(1 - q2))
    floor = h2[:, :-1].mean(axis=(0, 2)).mean()
    assert oracle.locality_loss(p2) > floor + 1e-4


def test_locality_single_token_and_scale():
    assert oracle.locality_loss(_probs(8, 2, 1, 4)) == 0.0
    # Two tokens: the loss is one BCE mean; three tokens: the mean of two.
    p = _probs(9, 1, 3, 4)
    q = _sharp(p, 2.0)
    b01 = F.binary_cross_entropy(q[:, 1], q[:, 0]).item()
    b12 = F.binary_cross_entropy(q[:, 2], q[:, 1]).item()
    assert oracle.locality_loss(p[:, :2]) == pytest.approx(b01, rel=1e-6)
    assert oracle.locality_loss(p) == pytest.approx((b01 + b12) / 2, rel=1e-6)


# --- chunk sparsification loss ---------------------------------------------------

def test_sparsification_closed_forms():
    z = np.zeros((2, 13, 5), np.float32)
    assert oracle.chunk_sparsification_loss(z, 8) == 0.0
    assert oracle.chunk_sparsification_loss(np.ones_like(z), 8) == 1.0
    p = _probs(10, 2, 13, 5)
    assert oracle.chunk_sparsification_loss(p, 1) == pytest.approx(p.astype(np.float64).mean(),
                                                                   rel=1e-14)


def _brute_chunk_activation(col):
    """P(at least one of the tokens is active), enumerating every activation pattern
    of independent Bernoulli(p_k) tokens."""
    total = 0.0
    for pat in itertools.product((0, 1), repeat=len(col)):
        if any(pat):
            pr = 1.0
            for a, pk in zip(pat, col):
                pr *= pk if a else 1.0 - pk
            total += pr
    return total


@pytest.mark.parametrize("S,L", [(13, 4), (8, 8), (5, 8), (9, 3)])
def test_sparsification_brute_force(S, L):
    """Aligned chunks, ceil(S/L) of them, the last possibly partial; each term is the
    probability that the expert fires somewhere in the chunk."""
    p = _probs(11, 2, S, 3).astype(np.float64)
    nc = -(-S // L)
    acc = 0.0
    for c in range(nc):
        terms = [_brute_chunk_activation(p[b, c * L:min(c * L + L, S), e])
                 for b in range(2) for e in range(3)]
        acc += np.mean(terms)
    assert oracle.chunk_sparsification_loss(p.astype(np.float32), L) == pytest.approx(
        acc / nc, rel=1e-12)


# --- gradients -------------------------------------------------------------------

_H = 2.0 ** -12


def _fd_grad(fn, p):
    g = np.empty(p.shape, np.float64)
    for idx in np.ndindex(p.shape):
        hi, lo = p.copy(), p.copy()
        hi[idx] += np.float32(_H)
        lo[idx] -= np.float32(_H)
        g[idx] = (fn(hi) - fn(lo)) / (2 * _H)
    return g


@pytest.mark.parametrize("alpha", [2.0, 4.0])
def test_locality_grad_finite_differences(alpha):
    p = _probs(12, 2, 7, 3)
    g = oracle.locality_loss_grad(p, alpha)
    fd = _fd_grad(lambda q: oracle.locality_loss(q, alpha), p)
    np.testing.assert_allclose(g, fd, rtol=1e-5, atol=1e-7 * np.abs(fd).max())


@pytest.mark.parametrize("S,L", [(9, 4), (8, 8), (5, 8), (7, 1)])
def test_sparsification_grad_finite_differences(S, L):
    p = _probs(13, 2, S, 3)
    g = oracle.chunk_sparsification_loss_grad(p, L)
    fd = _fd_grad(lambda q: oracle.chunk_sparsification_loss(q, L), p)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-9 * np.abs(fd).max())


def test_sparsification_grad_closed_forms():
    B, S, E = 2, 10, 3
    z = np.zeros((B, S, E), np.float32)
    np.testing.assert_allclose(oracle.chunk_sparsification_loss_grad(z, 4),
                               1.0 / (B * E * 3), rtol=1e-15)
    p = _probs(14, B, S, E)
    np.testing.assert_allclose(oracle.chunk_sparsification_loss_grad(p, 1),
                               1.0 / (B * E * S), rtol=1e-15)
    # A chunk in which some other token has p = 1 passes no gradient to the rest.
    p[0, 0:4, 0] = [1.0, 0.3, 0.2, 0.5]
    g = oracle.chunk_sparsification_loss_grad(p, 4)
    assert np.all(g[0, 1:4, 0] == 0.0) and g[0, 0, 0] > 0.0
