"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: union masks, expert lists and counts bit-exact; y within
max|dy| / max|y_ref| <= 1e-2 for bf16 inputs and <= 1e-5 for fp32; router masks
equal wherever the oracle's pre-ReLU logit has |l| >= 1e-3.
"""
import numpy as np
import pytest
import torch

import chunk_level_activation_amd as bf
import oracle
from chunk_level_activation_amd import inputs
from gpu_helpers import DEV, TOL_BF16, TOL_F32, dev, host, rel_err, tol, wdtype

pytestmark = pytest.mark.gpu


def run_ffn(inp, scores=None, workspace=None, n=None):
    """GPU chunk FFN for a workload; returns (y, masks, lists, counts) on the host."""
    n = inp.n if n is None else n
    s = inp.scores if scores is None else scores
    T, E = s.shape
    C = -(-T // n)
    masks = torch.empty((C, -(-E // 64)), dtype=torch.int64, device=DEV)
    lists = torch.empty((C, E), dtype=torch.int32, device=DEV)
    counts = torch.empty((C,), dtype=torch.int32, device=DEV)
    dt = wdtype(inp)
    y = bf.blockffn_chunk_ffn(dev(inp.x, dt), dev(s), dev(inp.w1, dt), dev(inp.w2, dt), n,
                              workspace=workspace, union_masks=masks, expert_lists=lists,
                              union_counts=counts)
    torch.cuda.synchronize()
    return (host(y), masks.cpu().numpy().view(np.uint64), lists.cpu().numpy(),
            counts.cpu().numpy())


def check_union(scores, n, masks, lists, counts):
    m_ref, l_ref, c_ref = oracle.chunk_union(scores, n)
    assert np.array_equal(counts, c_ref)
    assert np.array_equal(masks, m_ref)
    assert np.array_equal(lists, l_ref)


# ------------------------------------------------------------------ union

@pytest.mark.parametrize("T,E,n,kind", [
    (32, 64, 32, "markov"), (2048, 64, 32, "markov"), (512, 128, 32, "markov"),
    (70, 80, 8, "markov"), (1, 16, 32, "markov"), (100, 256, 32, "markov"),
    (33, 64, 32, "hand"), (96, 200, 32, "hand"), (64, 1, 8, "markov"),
])
def test_union_bit_exact(T, E, n, kind):
    rng = np.random.default_rng(T + E)
    if kind == "markov":
        act = inputs.markov_active(rng, T, E, 0.8, 0.7, 8)
    else:
        act = rng.random((T, E)) < 0.02
        act[:min(n, T)] = False                      # empty first chunk
        if T > 2 * n:
            act[n:2 * n] = True                      # full second chunk
    s = inputs.scores_for_mask(rng, act)
    s[act == 0] = np.where(rng.random(int((~act).sum())) < 0.5, 0.0, -0.0)
    x = inputs.gaussian(rng, (T, 32), 1.0, True)
    w1, w2 = inputs.expert_weights(rng, E, 16, 32, True)
    inp = inputs.LayerInputs("union", "bf16", T, 32, E, 16, n, x, w1, w2, scores=s)
    _, masks, lists, counts = run_ffn(inp)
    check_union(s, n, masks, lists, counts)


# ------------------------------------------------------------------ chunk FFN, bf16

@pytest.fixture(scope="module")
def decode_draws():
    return [inputs.make_workload("decode", seed=s) for s in range(3)]


@pytest.mark.parametrize("i", range(3))
def test_decode_chunk_full(decode_draws, i):
    """d_h=2048, E=64, d_e=128, one 32-token chunk, Markov 80% TLS / 70% CLS_8."""
    inp = decode_draws[i]
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, inp.n, masks, lists, counts)
    y_ref = oracle.chunk_ffn(inp.x, inp.scores, inp.w1, inp.w2, inp.n)
    assert rel_err(y, y_ref) <= TOL_BF16
    assert 16 < counts[0] < 60     # a sparse but non-trivial union


def test_prefill_full():
    """T=2048 = 64 chunks: unions and every row of y (the oracle's per-token form, which
    equals its union-then-mask form bit for bit)."""
    inp = inputs.make_workload("prefill", seed=5)
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, inp.n, masks, lists, counts)
    y_ref = oracle.token_ffn(inp.x, inp.scores, inp.w1, inp.w2)
    assert rel_err(y, y_ref) <= TOL_BF16


def test_rec256_prefill_full():
    """The recommended shape at 2048 tokens (E=40, d_e=256: two 128-unit passes in the
    up-projection, four k steps per expert in the down-projection): unions and every
    row of y."""
    inp = inputs.make_workload("rec256_prefill", seed=6)
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, inp.n, masks, lists, counts)
    y_ref = oracle.token_ffn(inp.x, inp.scores, inp.w1, inp.w2)
    assert rel_err(y, y_ref) <= TOL_BF16


@pytest.mark.parametrize("tls,cls,dense", [(0.5, 0.3, False), (0.8, 0.7, False),
                                           (0.9, 0.85, False), (0.8, 0.7, True)])
def test_large_layer_sweep_full(tls, cls, dense):
    """d_h=4096, E=128 (two mask words), T=512: the sparsity sweep and all-active, every
    row of y."""
    inp = inputs.make_workload("large", seed=7, tls=tls, cls=cls, dense=dense)
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, inp.n, masks, lists, counts)
    if dense:
        assert np.all(counts == 128)
    y_ref = oracle.token_ffn(inp.x, inp.scores, inp.w1, inp.w2)
    assert rel_err(y, y_ref) <= TOL_BF16


# ------------------------------------------------------------------ decode schedule

DECODE = [
    # (label, T, E, d_h, d_e, tls, cls, dense): single chunks of <= 32 tokens
    ("T=32 E=64", 32, 64, 2048, 128, 0.8, 0.7, False),
    ("one token", 1, 64, 2048, 128, 0.8, 0.7, False),
    ("T=5", 5, 64, 2048, 128, 0.8, 0.7, False),
    ("T=31", 31, 64, 2048, 128, 0.8, 0.7, False),
    ("all experts active", 32, 64, 2048, 128, 0.8, 0.7, True),
    ("d_e=64", 32, 64, 2048, 64, 0.8, 0.7, False),
    ("d_h=1024", 32, 64, 1024, 128, 0.8, 0.7, False),
    ("d_h=128", 32, 64, 128, 128, 0.8, 0.7, False),
    ("E=8", 32, 8, 2048, 128, 0.5, 0.3, False),
    ("E=1", 32, 1, 2048, 128, 0.5, 0.3, False),
    ("E=40", 32, 40, 2048, 128, 0.8, 0.7, False),
    # wide experts: pieces of more than 32 rows take a second pass (all active: 40 rows
    # per member at E=40, 64 at E=64, whose group ranges fill the hidden block)
    ("d_e=256", 32, 32, 2048, 256, 0.8, 0.7, False),
    ("recommended E=40 d_e=256", 32, 40, 2048, 256, 0.8, 0.7, False),
    ("recommended E=40 d_e=256 T=5", 5, 40, 2048, 256, 0.8, 0.7, False),
    ("recommended E=40 d_e=256 all active", 32, 40, 2048, 256, 0.8, 0.7, True),
    ("E=64 d_e=256 all active", 32, 64, 2048, 256, 0.8, 0.7, True),
    ("d_e=256 d_h=1024 all active", 32, 64, 1024, 256, 0.8, 0.7, True),
    # d_e=512: pieces of up to 96 rows (three passes) and group ranges of up to 2560
    # units (the hidden block in two LDS chunks when all 40 experts are active)
    ("recommended E=40 d_e=512", 32, 40, 2048, 512, 0.8, 0.7, False),
    ("recommended d_e=512 T=7", 7, 40, 2048, 512, 0.8, 0.7, False),
    ("recommended E=40 d_e=512 all active", 32, 40, 2048, 512, 0.8, 0.7, True),
    ("E=24 d_e=512 d_h=1024 all active", 32, 24, 1024, 512, 0.5, 0.3, True),
    # sizes outside the one-workgroup-per-CU schedule (other single-chunk paths)
    ("d_h=4096", 32, 64, 4096, 128, 0.8, 0.7, False),
    ("E=128", 32, 128, 2048, 128, 0.8, 0.7, False),
    ("E=64 d_e=512", 32, 64, 2048, 512, 0.8, 0.7, False),
]


@pytest.mark.parametrize("label,T,E,d_h,d_e,tls,cls,dense", DECODE,
                         ids=[d[0] for d in DECODE])
def test_decode_shapes(label, T, E, d_h, d_e, tls, cls, dense):
    inp = inputs.make_workload("decode", seed=21, T=T, E=E, d_h=d_h, d_e=d_e, tls=tls,
                               cls=cls, dense=dense)
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, inp.n, masks, lists, counts)
    y_ref = oracle.chunk_ffn(inp.x, inp.scores, inp.w1, inp.w2, inp.n)
    assert rel_err(y, y_ref) <= TOL_BF16, label


def test_decode_all_zero_scores_give_zero():
    inp = inputs.make_workload("decode", seed=22)
    s = np.zeros_like(inp.scores)
    s[3, 9] = -0.0
    y, masks, lists, counts = run_ffn(inp, scores=s)
    assert counts.tolist() == [0] and np.all(masks == 0) and np.all(lists == -1)
    assert np.all(y == 0)


def test_decode_single_active_entry():
    inp = inputs.make_workload("decode", seed=23)
    s = np.zeros_like(inp.scores)
    s[17, 42] = 0.75
    y, _, lists, counts = run_ffn(inp, scores=s)
    assert counts.tolist() == [1] and lists[0, 0] == 42
    assert np.all(y[np.arange(32) != 17] == 0)
    y_ref = oracle.chunk_ffn(inp.x, s, inp.w1, inp.w2, 32)
    assert rel_err(y, y_ref) <= TOL_BF16


def test_decode_experts_outside_union_are_never_read():
    inp = inputs.make_workload("decode", seed=24, tls=0.9, cls=0.85)
    _, _, c_ref = oracle.chunk_union(inp.scores, 32)
    used = np.any(inp.scores != 0, axis=0)
    assert 0 < c_ref[0] < 64
    y, *_ = run_ffn(inp)
    inp.w1 = inp.w1.copy()
    inp.w2 = inp.w2.copy()
    inp.w1[~used] = np.nan
    inp.w2[~used] = np.nan
    yn, *_ = run_ffn(inp)
    assert np.all(np.isfinite(yn))
    assert np.array_equal(y, yn)


# ------------------------------------------------------------------ multi-chunk schedule

GROUPED = [
    # (label, T, n, E, d_h, d_e, dense): several chunk tiles, full check against the oracle
    ("T=256 n=32", 256, 32, 64, 2048, 128, False),
    ("T=100 n=48 partial tiles", 100, 48, 64, 2048, 128, False),
    ("n=64 two tiles per chunk", 256, 64, 64, 2048, 128, False),
    ("n=128", 256, 128, 64, 1024, 128, False),
    ("n=8", 128, 8, 64, 1024, 128, False),
    ("d_e=256", 96, 32, 40, 1024, 256, False),
    ("E=40", 160, 32, 40, 2048, 128, False),
    ("E=128", 96, 32, 128, 512, 128, False),
    # four mask words, four tiles per down workgroup
    ("E=256", 128, 32, 256, 256, 128, False),
    ("d_h=256", 64, 32, 16, 256, 128, False),
    ("all experts active", 64, 32, 64, 1024, 128, True),
    ("recommended E=40 d_e=256", 128, 32, 40, 2048, 256, False),
    ("recommended E=40 d_e=512", 96, 32, 40, 2048, 512, False),
]


@pytest.mark.parametrize("label,T,n,E,d_h,d_e,dense", GROUPED, ids=[g[0] for g in GROUPED])
def test_multichunk_shapes(label, T, n, E, d_h, d_e, dense):
    inp = inputs.make_workload("prefill", seed=31, T=T, n=n, E=E, d_h=d_h, d_e=d_e,
                               dense=dense)
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, n, masks, lists, counts)
    y_ref = oracle.chunk_ffn(inp.x, inp.scores, inp.w1, inp.w2, n)
    assert rel_err(y, y_ref) <= TOL_BF16, label


def test_multichunk_zero_single_and_outside_union():
    """All-zero scores give y = 0; one active entry touches only its token; NaN weights
    on experts outside every union are never read."""
    inp = inputs.make_workload("prefill", seed=32, T=192, d_h=1024, tls=0.9, cls=0.85)
    s = np.zeros_like(inp.scores)
    s[7, 3] = -0.0
    y, _, lists, counts = run_ffn(inp, scores=s)
    assert np.all(counts == 0) and np.all(lists == -1) and np.all(y == 0)
    s[100, 11] = 2.5
    y, _, lists, counts = run_ffn(inp, scores=s)
    assert counts.tolist() == [0, 0, 0, 1, 0, 0] and lists[3, 0] == 11
    assert np.all(y[np.arange(192) != 100] == 0)
    assert rel_err(y, oracle.chunk_ffn(inp.x, s, inp.w1, inp.w2, 32)) <= TOL_BF16
    used = np.any(inp.scores != 0, axis=0)
    assert not used.all()
    y, *_ = run_ffn(inp)
    inp.w1 = inp.w1.copy()
    inp.w2 = inp.w2.copy()
    inp.w1[~used] = np.nan
    inp.w2[~used] = np.nan
    yn, *_ = run_ffn(inp)
    assert np.all(np.isfinite(yn)) and np.array_equal(y, yn)


# ------------------------------------------------------------------ edge cases

def small(dtype, T, n, E=16, d_h=64, d_e=32, tls=0.8, cls=0.6, seed=0):
    return inputs.make_workload("decode", seed=seed, T=T, n=n, E=E, d_h=d_h, d_e=d_e,
                                dtype=dtype, tls=tls, cls=cls)


EDGE = [
    # (label, T, n, E, d_h, d_e)
    ("one token", 1, 32, 16, 64, 32),
    ("ragged tail of one token", 33, 32, 16, 64, 32),
    ("n=1", 40, 1, 16, 64, 32),
    ("n=48 spans two tiles", 100, 48, 16, 64, 32),
    ("n larger than T", 40, 64, 16, 64, 32),
    ("n=8", 64, 8, 16, 256, 64),
    ("one expert", 64, 32, 1, 64, 32),
    ("E=80 partial mask word", 96, 32, 80, 64, 32),
    ("E=256 four mask words", 64, 32, 256, 64, 16),
    ("minimum bf16 sizes", 32, 32, 4, 32, 16),
    ("many chunks", 1000, 32, 16, 64, 32),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("label,T,n,E,d_h,d_e", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(dtype, label, T, n, E, d_h, d_e):
    inp = small(dtype, T, n, E=E, d_h=d_h, d_e=d_e, tls=0.8, cls=0.6)
    y, masks, lists, counts = run_ffn(inp)
    check_union(inp.scores, n, masks, lists, counts)
    y_ref = oracle.chunk_ffn(inp.x, inp.scores, inp.w1, inp.w2, n)
    assert rel_err(y, y_ref) <= tol(inp), label


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_zero_scores_give_zero(dtype):
    inp = small(dtype, 70, 32)
    s = np.zeros_like(inp.scores)
    s[5, 3] = -0.0
    y, masks, lists, counts = run_ffn(inp, scores=s)
    assert np.all(counts == 0) and np.all(masks == 0) and np.all(lists == -1)
    assert np.all(y == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_active_entry(dtype):
    inp = small(dtype, 64, 32)
    s = np.zeros_like(inp.scores)
    s[40, 7] = 1.25
    y, _, lists, counts = run_ffn(inp, scores=s)
    assert counts.tolist() == [0, 1] and lists[1, 0] == 7
    assert np.all(y[np.arange(64) != 40] == 0)
    y_ref = oracle.chunk_ffn(inp.x, s, inp.w1, inp.w2, 32)
    assert rel_err(y, y_ref) <= tol(inp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_experts_outside_union_are_never_read(dtype):
    """NaN weights on experts outside every union leave y finite and unchanged."""
    inp = small(dtype, 64, 32, E=32, tls=0.9, cls=0.85, seed=3)
    m_ref, _, _ = oracle.chunk_union(inp.scores, 32)
    used = np.zeros(32, bool)
    for c in range(m_ref.shape[0]):
        used |= [(int(m_ref[c, 0]) >> e) & 1 == 1 for e in range(32)]
    assert not used.all()
    y, *_ = run_ffn(inp)
    inp.w1 = inp.w1.copy()
    inp.w2 = inp.w2.copy()
    inp.w1[~used] = np.nan
    inp.w2[~used] = np.nan
    yn, *_ = run_ffn(inp)
    assert np.all(np.isfinite(yn))
    assert np.array_equal(y, yn)


def test_deterministic_and_workspace_reuse():
    """Calls agree bitwise (the split-sum path included), and one zeroed workspace
    stays valid across many calls of different shapes: every call returns its
    arrival counters to zero."""
    inp = inputs.make_workload("decode", seed=11)
    shapes = [(32, 32), (256, 32), (77, 48)]
    nbytes = max(bf.blockffn_chunk_ffn_workspace_bytes(T, 2048, 64, 128, n, bf.BLOCKFFN_BF16)
                 for T, n in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    y1, *_ = run_ffn(inp, workspace=ws)
    y2, *_ = run_ffn(inp, workspace=ws)
    assert np.array_equal(y1, y2)
    big = inputs.make_workload("prefill", seed=12, T=256)
    yb1, *_ = run_ffn(big, workspace=ws)
    odd = inputs.make_workload("decode", seed=13, T=77, n=48)
    yo, *_ = run_ffn(odd, workspace=ws)
    y3, *_ = run_ffn(inp, workspace=ws)
    assert np.array_equal(y1, y3)
    yb2, *_ = run_ffn(big, workspace=ws)
    assert np.array_equal(yb1, yb2)
    y_ref = oracle.chunk_ffn(odd.x, odd.scores, odd.w1, odd.w2, 48)
    assert rel_err(yo, y_ref) <= TOL_BF16
    fresh = bf.blockffn_chunk_ffn_workspace(2048, 2048, 64, 128, 32, bf.BLOCKFFN_BF16, DEV)
    y4, *_ = run_ffn(inp, workspace=fresh)
    assert np.array_equal(y1, y4)


def test_score_scaling_by_two_is_exact():
    """y(2s) == 2 y(s) bitwise: powers of two commute with every rounding step."""
    inp = inputs.make_workload("decode", seed=13)
    y1, *_ = run_ffn(inp)
    y2, *_ = run_ffn(inp, scores=inp.scores * np.float32(2.0))
    assert np.array_equal(y2, 2 * y1)


def test_chunk_length_changes_only_unions():
    """y does not depend on n beyond rounding; the unions do."""
    inp = inputs.make_workload("prefill", seed=14, T=256)
    y32, *_ = run_ffn(inp, n=32)
    y8, m8, l8, c8 = run_ffn(inp, n=8)
    check_union(inp.scores, 8, m8, l8, c8)
    assert rel_err(y8, y32) <= TOL_BF16


def test_small_workspace_rejected():
    inp = small("bf16", 64, 32)
    ws = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(bf.BlockFFNError) as ei:
        run_ffn(inp, workspace=ws)
    assert ei.value.status == 3


# ------------------------------------------------------------------ router

def router_ws(inp):
    code = bf.BLOCKFFN_BF16 if inp.dtype == "bf16" else bf.BLOCKFFN_F32
    return bf.blockffn_router_workspace(inp.T, inp.d_h, inp.w_r.shape[0], code, DEV)


def run_router(inp, use_gain=True, use_bias=True, logits=True, workspace=None):
    dt = wdtype(inp)
    T, E = inp.T, inp.w_r.shape[0]
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV) if logits else None
    s = bf.blockffn_router(dev(inp.x, dt), dev(inp.w_r, dt),
                           dev(inp.gain) if (use_gain and inp.gain is not None) else None,
                           dev(inp.bias) if (use_bias and inp.bias is not None) else None,
                           logits=lg, workspace=workspace)
    torch.cuda.synchronize()
    return s.cpu().numpy(), (lg.cpu().numpy() if logits else None)


def check_router(inp, s, lg, use_gain=True, use_bias=True, score_tol=1e-4):
    gain = inp.gain if use_gain else None
    bias = inp.bias if use_bias else None
    l_ref, s_ref = oracle.router(inp.x, inp.w_r, gain=gain, bias=bias)
    # forward error bound of an fp32 sum of d_h products (bf16 x bf16 products are
    # exact in fp32; fp32 products add one rounding each): (d_h + 2) u sum|x_j w_j|
    u = 2.0 ** -24
    absdot = np.abs(inp.x.astype(np.float64)) @ np.abs(inp.w_r.astype(np.float64)).T
    if bias is not None:
        absdot += np.abs(bias)
    bound = (inp.d_h + 2) * u * absdot
    if lg is not None:
        assert np.all(np.abs(lg - l_ref) <= bound)
    decided = np.abs(l_ref) >= 1e-3
    assert np.array_equal((s != 0)[decided], (l_ref > 0)[decided])
    assert rel_err(s, s_ref) <= score_tol


def test_router_e2e_full():
    """T=4096, d_h=2048, E=64, bf16, logit shift for ~80% zeros after ReLU."""
    inp = inputs.make_workload("e2e", seed=0)
    s, lg = run_router(inp)
    check_router(inp, s, lg)
    assert abs((s == 0).mean() - 0.8) < 0.02
    s2, lg2 = run_router(inp, workspace=router_ws(inp))
    check_router(inp, s2, lg2)


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1, 32, 100, 2048])
def test_router_split_sum(T):
    """Few tokens: the d_h sum is split over workgroups (with a workspace); the
    result matches the oracle and, bit for bit, a second call on the same
    workspace (the counters returned to zero, the split order is fixed)."""
    inp = inputs.make_workload("e2e", seed=11, T=T)
    ws = router_ws(inp)
    s, lg = run_router(inp, workspace=ws)
    check_router(inp, s, lg)
    ctrl = ws[:4096].cpu().numpy()
    assert not ctrl.any()
    s2, lg2 = run_router(inp, workspace=ws)
    assert np.array_equal(s, s2) and np.array_equal(lg, lg2)


def test_router_tiny_f32():
    inp = inputs.make_workload("tiny", seed=0)
    s, lg = run_router(inp)
    check_router(inp, s, lg, score_tol=TOL_F32)


ROUTER_EDGE = [
    # (label, dtype, T, d_h, E, gain, bias)
    ("one expert", "bf16", 64, 256, 1, True, False),
    ("E=40", "bf16", 96, 512, 40, True, True),
    ("E=256", "bf16", 64, 256, 256, True, True),
    ("ragged T", "bf16", 33, 256, 64, False, False),
    ("one token", "bf16", 1, 256, 16, True, False),
    ("f32 E=40", "f32", 50, 100, 40, True, True),
    ("f32 E=256", "f32", 20, 64, 256, False, True),
]


@pytest.mark.parametrize("label,dtype,T,d_h,E,g,b", ROUTER_EDGE, ids=[r[0] for r in ROUTER_EDGE])
def test_router_edge_cases(label, dtype, T, d_h, E, g, b):
    rng = np.random.default_rng(T * 7 + E)
    bfl = dtype == "bf16"
    x = inputs.gaussian(rng, (T, d_h), 1.0, bfl)
    w_r = inputs.gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), bfl)
    inp = inputs.LayerInputs("router", dtype, T, d_h, E, 16, 32, x, None, None, w_r=w_r)
    inp.gain = (rng.random(E) + 0.5).astype(np.float32) if g else None
    inp.bias = inputs.router_shift(w_r, 0.6) if b else None
    s, lg = run_router(inp, use_gain=g, use_bias=b, logits=(T % 2 == 0))
    check_router(inp, s, lg, use_gain=g, use_bias=b,
                 score_tol=1e-4 if bfl else TOL_F32)


def test_router_all_negative_row():
    x = np.ones((4, 64), np.float32)
    w_r = -np.ones((8, 64), np.float32) / 64
    inp = inputs.LayerInputs("router", "bf16", 4, 64, 8, 16, 32, x, None, None, w_r=w_r)
    s, _ = run_router(inp, use_gain=False, use_bias=False)
    assert np.all(s == 0)


# ------------------------------------------------------------------ end to end

def test_end_to_end_router_then_ffn_full():
    """Router on the GPU feeds the GPU chunk FFN; every row compared with the oracle's
    router feeding the oracle's FFN. (Where a logit is within rounding of zero the two
    routers may decide its activity differently; such a score is itself that small, so
    its term stays far inside the tolerance.)"""
    inp = inputs.make_workload("e2e", seed=1)
    dt = torch.bfloat16
    x = dev(inp.x, dt)
    s = bf.blockffn_router(x, dev(inp.w_r, dt), dev(inp.gain), dev(inp.bias))
    y = bf.blockffn_chunk_ffn(x, s, dev(inp.w1, dt), dev(inp.w2, dt), inp.n)
    torch.cuda.synchronize()
    _, s_ref = oracle.router(inp.x, inp.w_r, gain=inp.gain, bias=inp.bias)
    y_ref = oracle.token_ffn(inp.x, s_ref.astype(np.float32), inp.w1, inp.w2)
    assert rel_err(host(y), y_ref) <= TOL_BF16


def test_tiny_fp32_end_to_end():
    """The tiny fp32 workload: router from x, ~50% active, n=8."""
    inp = inputs.make_workload("tiny", seed=2)
    x = dev(inp.x)
    s = bf.blockffn_router(x, dev(inp.w_r), dev(inp.gain))
    y = bf.blockffn_chunk_ffn(x, s, dev(inp.w1), dev(inp.w2), inp.n)
    torch.cuda.synchronize()
    _, s_ref = oracle.router(inp.x, inp.w_r, gain=inp.gain)
    y_ref = oracle.chunk_ffn(inp.x, s_ref.astype(np.float32), inp.w1, inp.w2, inp.n)
    assert rel_err(host(y), y_ref) <= TOL_F32
    assert 0.3 < (host(s) == 0).mean() < 0.7


# ------------------------------------------------------------------ graph capture

def test_graph_replays_match_eager():
    """The calls captured in a HIP graph (as the benchmark runs them) give the eager
    results on every replay, with eager work and synchronisations in between."""
    draws = [inputs.make_workload("decode", seed=20 + i) for i in range(3)]
    dt = torch.bfloat16
    w1 = dev(draws[0].w1, dt)
    w2 = dev(draws[0].w2, dt)
    xs = [dev(d.x, dt) for d in draws]
    ss = [dev(d.scores) for d in draws]
    ws = bf.blockffn_chunk_ffn_workspace(32, 2048, 64, 128, 32, bf.BLOCKFFN_BF16, DEV)
    ys = [torch.empty((32, 2048), dtype=dt, device=DEV) for _ in draws]
    eager = []
    for x, s in zip(xs, ss):
        eager.append(host(bf.blockffn_chunk_ffn(x, s, w1, w2, 32, workspace=ws)))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, s, y in zip(xs, ss, ys):
            bf.blockffn_chunk_ffn(x, s, w1, w2, 32, y=y, workspace=ws)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, ref in zip(ys, eager):
            assert np.array_equal(host(y), ref), f"replay {rep}"
        # eager work on the same workspace between replays
        bf.blockffn_chunk_ffn(xs[rep % 3], ss[(rep + 1) % 3], w1, w2, 32, workspace=ws)
        torch.cuda.synchronize()
