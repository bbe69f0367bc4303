"""Parity of blockffn_layer_forward (router + chunk FFN in one call; for a single
chunk of <= 32 bf16 tokens with E <= 64 the router runs inside the FFN launch) with
the oracle's router feeding the oracle's chunk FFN.

Bars: y within max|dy| / max|y_ref| <= 1e-2 (bf16); the scores within 1e-4 of
max|s_ref| with the same activity wherever the oracle's logit has |l| >= 1e-3; the
inputs are drawn so that no oracle logit comes within 1e-5 of zero (the two sides
then take the same ReLU branches everywhere). Repeated calls and graph replays give
identical bits.
"""
import numpy as np
import pytest
import torch

import chunk_level_activation_amd as bf
import oracle
from chunk_level_activation_amd import inputs
from gpu_helpers import DEV, TOL_BF16, dev, host, rel_err

pytestmark = pytest.mark.gpu
b16 = torch.bfloat16


def _draw(seed, T, d_h, E, d_e, n, gain=True, bias=True):
    inp = inputs.make_workload("e2e", seed=seed, T=T, d_h=d_h, E=E, d_e=d_e, n=n)
    g = np.random.default_rng(seed + 7).uniform(0.5, 1.5, E).astype(np.float32) if gain else None
    b = inp.bias if bias else None
    return inp, g, b


def _run(inp, g, b, n, workspace=None, scores=True):
    sc = torch.empty((inp.T, inp.E), dtype=torch.float32, device=DEV) if scores else None
    y = bf.blockffn_layer_forward(dev(inp.x, b16), dev(inp.w_r, b16), dev(inp.w1, b16),
                                  dev(inp.w2, b16), n, gain=None if g is None else dev(g),
                                  bias=None if b is None else dev(b), scores=sc,
                                  workspace=workspace)
    torch.cuda.synchronize()
    return host(y), (sc.cpu().numpy() if scores else None)


def _check(inp, g, b, n, y, s):
    logits, s_ref = oracle.router(inp.x, inp.w_r, gain=g, bias=b)
    assert np.abs(logits).min() > 1e-5
    y_ref = oracle.chunk_ffn(inp.x, s_ref.astype(np.float32), inp.w1, inp.w2, n)
    assert rel_err(y, y_ref) <= TOL_BF16
    if s is not None:
        decided = np.abs(logits) >= 1e-3
        assert np.array_equal((s != 0)[decided], (logits > 0)[decided])
        assert rel_err(s, s_ref) <= 1e-4


CASES = [
    # (label, seed, T, d_h, E, d_e, n, gain, bias): the first NFUSED run fused
    ("decode chunk", 1, 32, 2048, 64, 128, 32, True, True),
    ("5 tokens", 2, 5, 2048, 64, 128, 32, True, True),
    ("one token", 3, 1, 2048, 64, 128, 32, True, True),
    ("E=40", 4, 32, 2048, 40, 128, 32, True, True),
    ("E=16 d_h=1024 d_e=64", 5, 32, 1024, 16, 64, 32, True, True),
    ("no gain, no bias", 6, 32, 2048, 64, 128, 32, False, False),
    ("d_h=768", 10, 32, 768, 64, 128, 32, True, True),
    ("d_e=256 (recommended E=40)", 9, 32, 2048, 40, 256, 32, True, True),
    ("d_e=512 (recommended E=40)", 12, 32, 2048, 40, 512, 32, True, True),
    # router + chunk FFN launches
    ("E=128", 7, 32, 2048, 128, 128, 32, True, True),
    ("multi-chunk T=256", 8, 256, 1024, 64, 128, 32, True, True),
    ("E=64 d_e=512", 13, 32, 2048, 64, 512, 32, True, True),
]
NFUSED = 9


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_layer_forward(idx):
    label, seed, T, d_h, E, d_e, n, gain, bias = CASES[idx]
    assert bf.blockffn_layer_forward_fused(T, d_h, E, d_e, n, bf.BLOCKFFN_BF16) == (idx < NFUSED)
    inp, g, b = _draw(seed, T, d_h, E, d_e, n, gain, bias)
    y, s = _run(inp, g, b, n)
    _check(inp, g, b, n, y, s)


def test_layer_forward_matches_separate_calls():
    """The fused launch and blockffn_router + blockffn_chunk_ffn agree to rounding."""
    inp, g, b = _draw(11, 32, 2048, 64, 128, 32)
    y_f, s_f = _run(inp, g, b, 32)
    x = dev(inp.x, b16)
    s = bf.blockffn_router(x, dev(inp.w_r, b16), dev(g), dev(b))
    y = bf.blockffn_chunk_ffn(x, s, dev(inp.w1, b16), dev(inp.w2, b16), 32)
    torch.cuda.synchronize()
    assert rel_err(y_f, host(y)) <= 1e-2
    assert rel_err(s_f, s.cpu().numpy()) <= 1e-5


def test_layer_forward_deterministic_and_graph_replays():
    draws = [_draw(20 + i, 32, 2048, 64, 128, 32) for i in range(3)]
    ws = bf.blockffn_layer_forward_workspace(32, 2048, 64, 128, 32, bf.BLOCKFFN_BF16, DEV)
    eager = [_run(inp, g, b, 32, workspace=ws, scores=False)[0] for inp, g, b in draws]
    again = [_run(inp, g, b, 32, workspace=ws, scores=False)[0] for inp, g, b in draws]
    assert all(np.array_equal(a, c) for a, c in zip(eager, again))
    args = [(dev(i.x, b16), dev(i.w_r, b16), dev(i.w1, b16), dev(i.w2, b16), dev(g), dev(b))
            for i, g, b in draws]
    ys = [torch.empty((32, 2048), dtype=b16, device=DEV) for _ in draws]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (x, w_r, w1, w2, g, b), y in zip(args, ys):
            bf.blockffn_layer_forward(x, w_r, w1, w2, 32, gain=g, bias=b, y=y, workspace=ws)
    for rep in range(3):
        for y in ys:
            y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for y, ref in zip(ys, eager):
            assert np.array_equal(host(y), ref), rep


# ---------------------------------------------------------------- packed weights

def _tiles(m):
    """numpy reference of the tiled layout: [..., R, C] -> [..., R/16, C/32, 16, 32], flat."""
    *lead, R, C = m.shape
    t = m.reshape(*lead, R // 16, 16, C // 32, 32)
    t = np.swapaxes(t, -3, -2)
    return t.reshape(-1)


@pytest.mark.parametrize("E,d_h,d_e", [(64, 2048, 128), (3, 96, 64), (1, 32, 32)])
def test_pack_weights_layout(E, d_h, d_e):
    rng = np.random.default_rng(40 + E)
    w1 = (rng.standard_normal((E, d_e, d_h)) * 8).astype(np.float32)
    w2 = (rng.standard_normal((E, d_h, d_e)) * 8).astype(np.float32)
    w1_16, w2_16 = dev(w1, b16), dev(w2, b16)
    packed = bf.blockffn_pack_weights(w1_16, w2_16)
    torch.cuda.synchronize()
    got = packed.view(torch.int16).cpu().numpy()
    ref = np.concatenate([_tiles(w1_16.view(torch.int16).cpu().numpy()),
                          _tiles(w2_16.view(torch.int16).cpu().numpy())])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("idx", range(7), ids=[c[0] for c in CASES[:7]])
def test_layer_forward_packed(idx):
    """Packed weights: the same bits as row-major weights, and the oracle's bar."""
    label, seed, T, d_h, E, d_e, n, gain, bias = CASES[idx]
    inp, g, b = _draw(seed, T, d_h, E, d_e, n, gain, bias)
    y_ref, s_ref = _run(inp, g, b, n)
    w1, w2 = dev(inp.w1, b16), dev(inp.w2, b16)
    packed = bf.blockffn_pack_weights(w1, w2)
    sc = torch.empty((T, E), dtype=torch.float32, device=DEV)
    y = bf.blockffn_layer_forward_packed(dev(inp.x, b16), dev(inp.w_r, b16), packed, E, d_e, n,
                                         gain=None if g is None else dev(g),
                                         bias=None if b is None else dev(b), scores=sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), y_ref)
    assert np.array_equal(sc.cpu().numpy(), s_ref)
    _check(inp, g, b, n, host(y), sc.cpu().numpy())


def test_layer_forward_packed_rejects_unfused_sizes():
    inp, g, b = _draw(7, 32, 2048, 128, 128, 32)
    packed = bf.blockffn_pack_weights(dev(inp.w1, b16), dev(inp.w2, b16))
    with pytest.raises(bf.BlockFFNError):
        bf.blockffn_layer_forward_packed(dev(inp.x, b16), dev(inp.w_r, b16), packed, 128, 128, 32)
