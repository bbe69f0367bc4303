"""Pins of the oracle's layer backward.

The layer (skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
Deployment", "Architecture Overview", "Router Architecture Setup", "Core Concept",
"Full BlockFFN Layer with Combined Losses") is rebuilt from torch's library routines
in float64: F.linear, F.relu, F.rms_norm over the experts, F.silu, torch.sigmoid.
Outside a chunk's union the scores are zero, so the dense sum over all experts equals
the union-then-mask output; torch's autograd of
    L = sum(dy * y) + sum(dprobs * sigmoid(sharpness * scores))
is then the reference gradient. ReLU's derivative at 0 is 0 in both.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _case(seed, T, d_h, E, d_e, gain=True, bias=True, dprobs=True, zero_expert=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d_h)).astype(np.float32)
    w_r = (rng.standard_normal((E, d_h)) / np.sqrt(d_h)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3 - 0.3).astype(np.float32) if bias else None
    if zero_expert:
        # expert 0 never active: a large negative logit shift
        w_r[0] *= 0.01
        if b is not None:
            b[0] = -5.0
    g = rng.uniform(0.5, 1.5, E).astype(np.float32) if gain else None
    w1 = (rng.standard_normal((E, d_e, d_h)) / np.sqrt(d_h)).astype(np.float32)
    w2 = (rng.standard_normal((E, d_h, d_e)) / np.sqrt(d_e)).astype(np.float32)
    dy = rng.standard_normal((T, d_h)).astype(np.float32)
    dp = rng.standard_normal((T, E)).astype(np.float32) if dprobs else None
    return x, w_r, g, b, w1, w2, dy, dp


def _torch_grads(x, w_r, g, b, w1, w2, dy, dp, eps, sharpness):
    d = lambda a: None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X, WR, G, B, W1, W2 = d(x), d(w_r), d(g), d(b), d(w1), d(w2)
    E = w_r.shape[0]
    logits = F.linear(X, WR, B)
    s = F.rms_norm(F.relu(logits), (E,), G, eps)
    y = torch.zeros_like(X)
    for e in range(E):
        y = y + s[:, e:e + 1] * F.linear(F.silu(F.linear(X, W1[e])), W2[e])
    loss = (torch.tensor(dy, dtype=torch.float64) * y).sum()
    if dp is not None:
        loss = loss + (torch.tensor(dp, dtype=torch.float64) * torch.sigmoid(sharpness * s)).sum()
    loss.backward()
    out = dict(dx=X.grad, dw_r=WR.grad, dw1=W1.grad, dw2=W2.grad,
               dgain=G.grad if G is not None else None, dbias=B.grad if B is not None else None)
    return {k: (None if v is None else v.numpy()) for k, v in out.items()}, logits.detach().numpy()


CASES = [
    # (seed, T, d_h, E, d_e, n, gain, bias, dprobs, zero_expert, sharpness)
    (1, 6, 16, 4, 8, 4, True, True, True, False, 1.0),      # partial last chunk
    (2, 9, 24, 6, 8, 1, True, True, True, True, 2.0),       # one-token chunks, idle expert
    (3, 8, 16, 5, 4, 8, False, True, False, True, 1.0),     # one chunk, no gain
    (4, 12, 32, 8, 16, 5, True, False, True, False, 0.5),   # no bias
]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_backward_matches_torch_autograd(case):
    seed, T, d_h, E, d_e, n, gain, bias, dprobs, zero_expert, sharp = case
    x, w_r, g, b, w1, w2, dy, dp = _case(seed, T, d_h, E, d_e, gain, bias, dprobs, zero_expert)
    eps = oracle.FP32_EPS
    ref, logits = _torch_grads(x, w_r, g, b, w1, w2, dy, dp, eps, sharp)
    # the ReLU kink is not exercised: no logit near 0
    assert np.abs(logits).min() > 1e-4
    got = oracle.layer_backward(x, w_r, w1, w2, dy, n, gain=g, bias=b, eps=eps, dprobs=dp,
                                sharpness=sharp)
    for k in ("dx", "dw_r", "dw1", "dw2", "dgain", "dbias"):
        if ref[k] is None:
            continue
        scale = max(np.abs(ref[k]).max(), 1e-30)
        assert np.abs(got[k] - ref[k]).max() <= 1e-11 * scale, k
    if zero_expert:
        assert np.all(got["dw1"][0] == 0) and np.all(got["dw2"][0] == 0)


def test_backward_linear_in_upstream_gradients():
    """The gradients are linear in (dy, dprobs): g(dy1 + 2 dy2) = g(dy1) + 2 g(dy2)."""
    x, w_r, g, b, w1, w2, dy, dp = _case(5, 7, 16, 4, 8)
    # multiples of 2^-10, so dy + 2 dy2 is exact in float32
    dy = (np.round(dy * 1024) / 1024).astype(np.float32)
    dy2 = (np.round(np.random.default_rng(9).standard_normal(dy.shape) * 1024) / 1024
           ).astype(np.float32)
    ga = oracle.layer_backward(x, w_r, w1, w2, dy, 4, gain=g, bias=b)
    gb = oracle.layer_backward(x, w_r, w1, w2, dy2, 4, gain=g, bias=b)
    gc = oracle.layer_backward(x, w_r, w1, w2, (dy.astype(np.float64) + 2 * dy2).astype(np.float32),
                               4, gain=g, bias=b)
    for k in ga:
        np.testing.assert_allclose(gc[k], ga[k] + 2 * gb[k], rtol=1e-9,
                                   atol=1e-9 * np.abs(gc[k]).max())


def test_backward_zero_upstream_and_all_inactive():
    x, w_r, g, b, w1, w2, dy, dp = _case(6, 5, 16, 4, 8)
    z = oracle.layer_backward(x, w_r, w1, w2, np.zeros_like(dy), 4, gain=g, bias=b)
    assert all(np.all(v == 0) for v in z.values())
    # every logit negative: no expert active, nothing flows anywhere
    neg = oracle.layer_backward(x, w_r, w1, w2, dy, 4, gain=g,
                                bias=np.full(4, -100.0, np.float32), dprobs=dp)
    assert all(np.all(v == 0) for v in neg.values())
