"""The allocation-free layer entry point (blockffn_layer_forward_noalloc) against the
entry point it varies (blockffn_layer_forward with a zero-filled workspace), through
the C ABI: two calls in a row, the second with a smaller input, each compared element by
element (the same kernels in the same order, so the bits agree; the oracle's bar is
checked as well). Also: sizes beyond the library's scratch array are rejected on the
host, and a bounded-wait time-out forced from the host is cleared by the next call.
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


def _draw(seed, T, d_h, E, d_e):
    inp = inputs.make_workload("e2e", seed=seed, T=T, d_h=d_h, E=E, d_e=d_e, n=32)
    g = np.random.default_rng(seed + 3).uniform(0.5, 1.5, E).astype(np.float32)
    return inp, g


def _both(inp, g, n=32):
    args = (dev(inp.x, b16), dev(inp.w_r, b16), dev(inp.w1, b16), dev(inp.w2, b16))
    s_ref = torch.empty((inp.T, inp.E), dtype=torch.float32, device=DEV)
    y_ref = bf.blockffn_layer_forward(*args, n, gain=dev(g), bias=dev(inp.bias), scores=s_ref)
    s_na = torch.empty((inp.T, inp.E), dtype=torch.float32, device=DEV)
    y_na = torch.empty_like(y_ref)
    print(f"noalloc call T={inp.T} d_h={inp.d_h} E={inp.E} d_e={inp.d_e}", flush=True)
    bf.blockffn_layer_forward_noalloc(*args, n, gain=dev(g), bias=dev(inp.bias), y=y_na,
                                      scores=s_na)
    torch.cuda.synchronize()
    return y_ref, s_ref, y_na, s_na


def _oracle_bar(inp, g, y, n=32):
    logits, s_ref = oracle.router(inp.x, inp.w_r, gain=g, bias=inp.bias)
    y_ref = oracle.chunk_ffn(inp.x, s_ref.astype(np.float32), inp.w1, inp.w2, n)
    if np.abs(logits).min() > 1e-5:
        assert rel_err(host(y), y_ref) <= TOL_BF16


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # first the decode chunk (the one-launch schedule), then a smaller layer
    for seed, T, d_h, E, d_e in [(31, 32, 2048, 64, 128), (32, 7, 1024, 16, 64)]:
        inp, g = _draw(seed, T, d_h, E, d_e)
        y_ref, s_ref, y_na, s_na = _both(inp, g)
        assert torch.equal(y_na, y_ref), (T, d_h)
        assert torch.equal(s_na, s_ref), (T, d_h)
        _oracle_bar(inp, g, y_na)


def test_noalloc_repeated_calls_keep_giving_equal_bits():
    inp, g = _draw(33, 32, 2048, 64, 128)
    outs = [_both(inp, g)[2] for _ in range(3)]
    assert all(torch.equal(o, outs[0]) for o in outs)


def test_noalloc_rejects_sizes_beyond_its_array():
    inp, g = _draw(34, 4, 256, 8, 64)
    x = torch.zeros((4096, 2048), dtype=b16, device=DEV)
    w_r = torch.zeros((64, 2048), dtype=b16, device=DEV)
    w1 = torch.zeros((64, 128, 2048), dtype=b16, device=DEV)
    w2 = torch.zeros((64, 2048, 128), dtype=b16, device=DEV)
    with pytest.raises(bf.BlockFFNError) as err:
        bf.blockffn_layer_forward_noalloc(x, w_r, w1, w2, 32)
    assert err.value.status == 2 and "scratch" in str(err.value)
