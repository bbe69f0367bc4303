"""Parity of the layer epilogue (router probabilities, residual + LayerNorm) and of
the sparsity losses with their gradient (HIP path through the C ABI) against the
CPU oracle.

Bars:
  * probs: |p - sigmoid(a s_ref)| <= a/4 * max|s - s_ref| + 2e-7 (the sigmoid's
    slope is at most a/4, plus fp32 rounding of the sigmoid); inactive experts give
    exactly 0.5.
  * LayerNorm: max|out - ref| / max|ref| <= 1e-2 (bf16 output) or 1e-5 (fp32).
  * losses: |loss - ref| <= 1e-5 |ref|; gradient max|g - ref| <= 1e-5 max|ref|.
    fp32 per-element arithmetic with a handful of roundings and correctly rounded
    log/exp to a few ulps (about 1e-6 relative), products over at most L <= 64
    factors (64 ulps ~ 4e-6); the loss sums are fp64.
  * repeated calls give identical bits (fixed reduction order).
"""
import numpy as np
import pytest
import torch

import chunk_level_activation_amd as bf
import oracle
from chunk_level_activation_amd import inputs
from gpu_helpers import DEV, TOL_BF16, TOL_F32, dev, host, rel_err

pytestmark = pytest.mark.gpu

LOSS_TOL = 1e-5


# ------------------------------------------------------------------ router probabilities

@pytest.mark.parametrize("T,sharp", [(4096, 1.0), (32, 2.0), (1, 0.5), (100, 1.0)])
def test_router_probs(T, sharp):
    inp = inputs.make_workload("e2e", seed=21, T=T)
    ws = bf.blockffn_router_workspace(T, inp.d_h, inp.E, bf.BLOCKFFN_BF16, DEV)
    probs = torch.empty((T, inp.E), dtype=torch.float32, device=DEV)
    s = bf.blockffn_router(dev(inp.x, torch.bfloat16), dev(inp.w_r, torch.bfloat16),
                           dev(inp.gain), dev(inp.bias), probs=probs, sharpness=sharp,
                           workspace=ws)
    torch.cuda.synchronize()
    s, p = s.cpu().numpy(), probs.cpu().numpy()
    _, s_ref = oracle.router(inp.x, inp.w_r, gain=inp.gain, bias=inp.bias)
    p_ref = oracle.router_probs(s_ref, sharp)
    bound = sharp / 4 * np.abs(s - s_ref).max() + 2e-7
    assert np.abs(p - p_ref).max() <= bound
    assert np.all(p[s == 0] == 0.5)
    assert np.all(p[s > 0] > 0.5)


def test_router_probs_f32():
    inp = inputs.make_workload("tiny", seed=3)
    probs = torch.empty((inp.T, inp.w_r.shape[0]), dtype=torch.float32, device=DEV)
    s = bf.blockffn_router(dev(inp.x), dev(inp.w_r), dev(inp.gain), probs=probs,
                           sharpness=2.0)
    torch.cuda.synchronize()
    s, p = s.cpu().numpy(), probs.cpu().numpy()
    _, s_ref = oracle.router(inp.x, inp.w_r, gain=inp.gain)
    assert np.abs(p - oracle.router_probs(s_ref, 2.0)).max() <= \
        0.5 * np.abs(s - s_ref).max() + 2e-7


# ------------------------------------------------------------------ residual + LayerNorm

LN_CASES = [
    # (T, d_h, dtype): register windows of 1/2/4/8 vectors per lane, the three-pass path
    # beyond 4096 (bf16) / 2048 (fp32), ragged rows per workgroup, short rows
    (32, 2048, "bf16"), (4096, 2048, "bf16"), (5, 4096, "bf16"), (7, 8192, "bf16"),
    (3, 4104, "bf16"), (1, 8, "bf16"), (9, 520, "bf16"), (33, 1024, "bf16"),
    (6, 2048, "f32"), (5, 4, "f32"), (3, 100, "f32"), (4, 2052, "f32"), (2, 4096, "f32"),
]


def run_ln(y, x, gamma, beta, dt, eps=1e-5, inplace=None):
    yd, xd = dev(y, dt), dev(x, dt)
    out = {"y": yd, "x": xd}.get(inplace)
    o = bf.blockffn_add_layernorm(yd, xd, None if gamma is None else dev(gamma),
                                  None if beta is None else dev(beta), eps, out=out)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("T,d_h,dt", LN_CASES, ids=[f"{c[0]}x{c[1]}-{c[2]}" for c in LN_CASES])
def test_add_layernorm(T, d_h, dt):
    bf16 = dt == "bf16"
    y, x, g, b = inputs.layernorm_inputs(T * 7 + d_h, T, d_h, bf16)
    tdt = torch.bfloat16 if bf16 else torch.float32
    out = run_ln(y, x, g, b, tdt)
    ref = oracle.add_layernorm(y, x, g, b)
    assert rel_err(out, ref) <= (TOL_BF16 if bf16 else TOL_F32)


@pytest.mark.parametrize("inplace", ["y", "x"])
@pytest.mark.parametrize("d_h", [2048, 8192])
def test_add_layernorm_in_place_and_defaults(inplace, d_h):
    y, x, _, _ = inputs.layernorm_inputs(5, 9, d_h, True)
    out = run_ln(y, x, None, None, torch.bfloat16, eps=1e-3, inplace=inplace)
    ref = oracle.add_layernorm(y, x, None, None, 1e-3)
    assert rel_err(out, ref) <= TOL_BF16


def test_add_layernorm_constant_row():
    """A row whose residual sum is constant has zero variance: the output is beta."""
    T, d_h = 4, 256
    y = np.full((T, d_h), 1.5, np.float32)
    x = np.full((T, d_h), -0.25, np.float32)
    _, _, g, b = inputs.layernorm_inputs(1, T, d_h, False)
    out = run_ln(y, x, g, b, torch.float32)
    assert np.allclose(out, np.broadcast_to(b, (T, d_h)), rtol=0, atol=1e-6)
    assert rel_err(out, oracle.add_layernorm(y, x, g, b)) <= TOL_F32


def test_layer_epilogue_chain_decode():
    """Router scores of the decode workload -> chunk FFN -> residual + LayerNorm on the
    GPU, against the oracle's chain in float64."""
    inp = inputs.make_workload("decode", seed=4)
    dt = torch.bfloat16
    xd = dev(inp.x, dt)
    y = bf.blockffn_chunk_ffn(xd, dev(inp.scores), dev(inp.w1, dt), dev(inp.w2, dt), inp.n)
    _, _, g, b = inputs.layernorm_inputs(9, inp.T, inp.d_h, True)
    out = bf.blockffn_add_layernorm(y, xd, dev(g), dev(b))
    torch.cuda.synchronize()
    y_ref = oracle.chunk_ffn(inp.x, inp.scores, inp.w1, inp.w2, inp.n)
    ref = oracle.add_layernorm(y_ref.astype(np.float32), inp.x, g, b)
    assert rel_err(host(out), ref) <= TOL_BF16


# ------------------------------------------------------------------ sparsity losses

def run_losses(p, alpha=2.0, L=8, lal=1.0, lcs=1.0, want_grad=True, ws=None):
    pd = dev(p)
    losses, grad = bf.blockffn_sparsity_losses(pd, alpha, L, lal, lcs, want_grad=want_grad,
                                               workspace=ws)
    torch.cuda.synchronize()
    return losses.cpu().numpy(), None if grad is None else grad.cpu().numpy()


def check_losses(p, alpha, L, lal, lcs, losses, grad):
    al = oracle.locality_loss(p, alpha)
    cs = oracle.chunk_sparsification_loss(p, L)
    assert abs(losses[0] - al) <= LOSS_TOL * abs(al), (losses[0], al)
    assert abs(losses[1] - cs) <= LOSS_TOL * abs(cs), (losses[1], cs)
    if grad is not None:
        ref = (lal * oracle.locality_loss_grad(p, alpha) +
               lcs * oracle.chunk_sparsification_loss_grad(p, L)).reshape(grad.shape)
        assert rel_err(grad, ref) <= LOSS_TOL


LOSS_CASES = [
    # (B, S, E, L, alpha, lambda_al, lambda_cs)
    (1, 4096, 64, 8, 2.0, 1.0, 1.0),       # the e2e token count, the pages' L and alpha
    (8, 512, 64, 8, 2.0, 0.1, 0.3),        # the pages' weight ranges
    (3, 37, 40, 8, 2.0, 1.0, 1.0),         # ragged last chunk, E = 40
    (2, 100, 64, 32, 5.0, 1.0, 0.5),       # 32-token window
    (2, 100, 64, 33, 2.0, 1.0, 1.0),       # any-L path
    (1, 300, 16, 64, 2.0, 0.0, 1.0),       # any-L path, CS only
    (4, 70, 8, 1, 2.0, 1.0, 0.0),          # L = 1, AL only
    (2, 9, 5, 16, 2.0, 1.0, 1.0),          # one partial chunk, L > S
    (1, 1, 64, 8, 2.0, 1.0, 1.0),          # one token: AL = 0
    (5, 33, 1, 8, 2.0, 1.0, 1.0),          # one expert
    (1, 2048, 256, 8, 2.0, 1.0, 1.0),      # E = 256
]


@pytest.mark.parametrize("case", LOSS_CASES, ids=[
    "B{}-S{}-E{}-L{}-a{}".format(*c[:5]) for c in LOSS_CASES])
def test_sparsity_losses(case):
    B, S, E, L, alpha, lal, lcs = case
    p = inputs.activation_probs(B * 1000 + S + E, B, S, E, L=8)
    losses, grad = run_losses(p, alpha, L, lal, lcs)
    check_losses(p, alpha, L, lal, lcs, losses, grad)


def test_sparsity_losses_deterministic_and_workspace_reset():
    B, S, E, L = 2, 4096, 64, 8
    p = inputs.activation_probs(77, B, S, E)
    ws = bf.blockffn_sparsity_losses_workspace(B, S, E, L, DEV)
    l1, g1 = run_losses(p, ws=ws)
    assert not ws[:65 * 128].cpu().numpy().any()
    l2, g2 = run_losses(p, ws=ws)
    assert np.array_equal(l1, l2) and np.array_equal(g1, g2)
    check_losses(p, 2.0, L, 1.0, 1.0, l1, g1)
    # a smaller problem on the same workspace
    p3 = inputs.activation_probs(78, 1, 100, 64)
    l3, g3 = run_losses(p3, ws=ws)
    check_losses(p3, 2.0, L, 1.0, 1.0, l3, g3)


def test_sparsity_losses_without_gradient():
    p = inputs.activation_probs(5, 2, 257, 64)
    losses, grad = run_losses(p, want_grad=False)
    assert grad is None
    check_losses(p, 2.0, 8, 1.0, 1.0, losses, None)


@pytest.mark.parametrize("L", [8, 33])
def test_sparsity_losses_exact_zeros_and_ones(L):
    """p = 0 everywhere gives CS = 0 and a CS gradient of 1/(B E nc); a token with
    p = 1 zeroes the CS gradient of the other tokens of its chunk."""
    B, S, E = 2, 80, 16
    z = np.zeros((B, S, E), np.float32)
    losses, grad = run_losses(z, L=L, lal=0.0)
    nc = -(-S // L)
    assert losses[1] == 0.0
    assert np.allclose(grad, 1.0 / (B * E * nc), rtol=1e-6, atol=0)
    p = inputs.activation_probs(6, B, S, E)
    p[0, 3, 2] = 1.0
    p[1, S - 1, 0] = 1.0
    p[1, 10:20, 5] = 0.0
    losses, grad = run_losses(p, L=L)
    check_losses(p, 2.0, L, 1.0, 1.0, losses, grad)
    _, g_cs = run_losses(p, L=L, lal=0.0)
    c0 = (3 // L) * L
    others = [t for t in range(c0, min(c0 + L, S)) if t != 3]
    assert np.all(g_cs[0, others, 2] == 0.0)


def _offset_copy(a):
    """A device copy of `a` that starts 4 bytes into its allocation: not 16-byte
    aligned, so the kernel takes one expert per thread."""
    n = a.size
    buf = torch.zeros(n + 4, dtype=torch.float32, device=DEV)
    view = buf[1:1 + n].view(a.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return view


@pytest.mark.parametrize("B,S,E,offset", [
    (16, 4096, 64, False),     # the benchmarked batch: four experts per thread
    (16, 4096, 64, True),      # same, one expert per thread, 2048 workgroups
    (320, 100, 64, False),     # four experts per thread with a ragged last chunk
    (512, 100, 40, False),     # E = 40, four experts per thread
])
def test_sparsity_losses_large(B, S, E, offset):
    p = inputs.activation_probs(B + S + E, B, S, E)
    pd = _offset_copy(p) if offset else dev(p)
    gd = _offset_copy(np.zeros_like(p)) if offset else None
    ws = bf.blockffn_sparsity_losses_workspace(B, S, E, 8, DEV)
    l1, g1 = bf.blockffn_sparsity_losses(pd, 2.0, 8, 0.1, 0.3, grad=gd, workspace=ws)
    torch.cuda.synchronize()
    l1, g1 = l1.cpu().numpy(), g1.cpu().numpy()
    check_losses(p, 2.0, 8, 0.1, 0.3, l1, g1)
    l2, g2 = bf.blockffn_sparsity_losses(pd, 2.0, 8, 0.1, 0.3, grad=gd, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(l1, l2.cpu().numpy()) and np.array_equal(g1, g2.cpu().numpy())
    assert not ws[:65 * 128].cpu().numpy().any()
