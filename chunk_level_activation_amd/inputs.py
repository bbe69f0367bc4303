"""Seeded synthetic inputs for the BlockFFN layer forward.

This module is shared by the tests and the benchmark; it is the only code the test
reference and the GPU path have in common. It holds
none of the layer's arithmetic. It only draws numbers:

* Gaussian activations and weights (``np.random.default_rng(seed)``), rounded to bf16
  by round-to-nearest-even where a workload is bf16;
* per-expert on/off activity masks from independent two-state Markov chains over the
  tokens, whose two transition probabilities are solved in closed form so that the
  masks hit a target token-level sparsity (TLS) and L-token chunk-level sparsity
  (CLS). The pages report trained models at over 80% TLS and 70% 8-token CLS
  (paper-card Abstract; skill page, "Key Hyperparameters"), and no trained router is
  available here, so these masks stand in for a trained router's output;
* router scores for a mask: |N(0,1)| + 0.1 where active, exactly 0 where inactive.

Markov chain per expert: q = P(off -> on), p = P(on -> off), the first token drawn
from the stationary law P(on) = q / (p + q). Then
    TLS   = P(off)               = p / (p + q)
    CLS_L = P(off for L tokens)  = TLS * (1 - q)^(L - 1)
so  q = 1 - (CLS / TLS)^(1 / (L - 1)),  p = q * TLS / (1 - TLS),  feasible when
CLS <= TLS; the expected union fraction of an n-token chunk is
1 - TLS * (1 - q)^(n - 1). The chunk probability is the product form that the skill
page's "Chunk Sparsification Loss" writes for an expert staying off in a chunk,
specialised to a Markov chain.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.special import ndtri


# ------------------------------------------------------------------ bf16 encoding

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(a)] = 0x7FC0
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ------------------------------------------------------------------ masks and scores

def markov_params(tls: float, cls: float, L: int) -> tuple[float, float]:
    """Transition probabilities (q = off->on, p = on->off) for target TLS and CLS_L."""
    if not (0.0 < cls <= tls < 1.0):
        raise ValueError(f"need 0 < CLS <= TLS < 1, got TLS={tls}, CLS={cls}")
    if L < 2:
        raise ValueError("chunk length L must be >= 2")
    q = 1.0 - (cls / tls) ** (1.0 / (L - 1))
    p = q * tls / (1.0 - tls)
    if p > 1.0:
        raise ValueError("target infeasible for a two-state chain (p > 1)")
    return q, p


def expected_union_fraction(tls: float, cls: float, L: int, n: int) -> float:
    q, _ = markov_params(tls, cls, L)
    return 1.0 - tls * (1.0 - q) ** (n - 1)


def markov_active(rng: np.random.Generator, T: int, E: int, tls: float, cls: float,
                  L: int = 8) -> np.ndarray:
    """[T, E] bool activity mask, one independent stationary chain per expert."""
    q, p = markov_params(tls, cls, L)
    u = rng.random((T, E))
    out = np.empty((T, E), dtype=bool)
    on = u[0] < (1.0 - tls)
    out[0] = on
    for t in range(1, T):
        on = np.where(on, u[t] >= p, u[t] < q)
        out[t] = on
    return out


def iid_active(rng: np.random.Generator, T: int, E: int, tls: float) -> np.ndarray:
    return rng.random((T, E)) >= tls


def scores_for_mask(rng: np.random.Generator, active: np.ndarray) -> np.ndarray:
    """float32 scores: |N(0,1)| + 0.1 where active, exactly 0 elsewhere."""
    mag = (np.abs(rng.standard_normal(active.shape)) + 0.1).astype(np.float32)
    return np.where(active, mag, np.float32(0.0)).astype(np.float32)


# ------------------------------------------------------------------ layers

def gaussian(rng: np.random.Generator, shape, std: float, bf16: bool) -> np.ndarray:
    a = (rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    return round_bf16(a) if bf16 else a.astype(np.float32)


@dataclass
class LayerInputs:
    """One workload: float32 arrays (bf16-exact values when dtype == 'bf16')."""
    name: str
    dtype: str                      # 'f32' or 'bf16': the type the layer computes in
    T: int
    d_h: int
    E: int
    d_e: int
    n: int
    x: np.ndarray                   # [T, d_h]
    w1: np.ndarray                  # [E, d_e, d_h]  fc1 weights (nn.Linear layout)
    w2: np.ndarray                  # [E, d_h, d_e]  fc2 weights
    scores: np.ndarray | None = None    # [T, E] float32 when given directly
    w_r: np.ndarray | None = None       # [E, d_h] router weight when scores come from it
    gain: np.ndarray | None = None      # [E] RMSNorm gain
    bias: np.ndarray | None = None      # [E] router logit shift (end-to-end workload)
    extra: dict = field(default_factory=dict)


def expert_weights(rng, E, d_e, d_h, bf16):
    """W1 ~ N(0, 1/d_h), W2 ~ N(0, 1/d_e): unit-variance pre-activations and outputs."""
    w1 = gaussian(rng, (E, d_e, d_h), 1.0 / np.sqrt(d_h), bf16)
    w2 = gaussian(rng, (E, d_h, d_e), 1.0 / np.sqrt(d_e), bf16)
    return w1, w2


# Workloads, named by what they are.
#   tiny     d_h=256,  E=16,  d_e=64,  T=64,   n=8,  f32, scores from the router
#   decode   d_h=2048, E=64,  d_e=128, T=32,   n=32, bf16, Markov 80% TLS / 70% CLS_8
#   prefill  d_h=2048, E=64,  d_e=128, T=2048, n=32, bf16, Markov 80/70
#   large    d_h=4096, E=128, d_e=128, T=512,  n=32, bf16, Markov at (tls, cls) or dense
#   e2e      d_h=2048, E=64,  d_e=128, T=4096, n=32, bf16, router with a logit shift
#            giving ~80% zeros after ReLU
#   rec256, rec512          d_h=2048, E=40, d_e=256 / 512, T=32, n=32, bf16, Markov
#            80/70: the expert count and widths the skill page recommends ("Key
#            Hyperparameters"), one decode chunk
#   rec256_prefill          the same with d_e=256 and T=2048
WORKLOADS = {
    "tiny": dict(d_h=256, E=16, d_e=64, T=64, n=8, dtype="f32"),
    "decode": dict(d_h=2048, E=64, d_e=128, T=32, n=32, dtype="bf16"),
    "prefill": dict(d_h=2048, E=64, d_e=128, T=2048, n=32, dtype="bf16"),
    "large": dict(d_h=4096, E=128, d_e=128, T=512, n=32, dtype="bf16"),
    "e2e": dict(d_h=2048, E=64, d_e=128, T=4096, n=32, dtype="bf16"),
    "rec256": dict(d_h=2048, E=40, d_e=256, T=32, n=32, dtype="bf16"),
    "rec512": dict(d_h=2048, E=40, d_e=512, T=32, n=32, dtype="bf16"),
    "rec256_prefill": dict(d_h=2048, E=40, d_e=256, T=2048, n=32, dtype="bf16"),
}

# z such that P(N(0,1) > z) = 0.2: a logit shift of -z * ||W_r[e]|| leaves each
# expert active for 20% of N(0, I) tokens.
Z_80 = float(ndtri(0.8))


def router_shift(w_r: np.ndarray, zero_fraction: float) -> np.ndarray:
    z = float(ndtri(zero_fraction))
    norms = np.sqrt((w_r.astype(np.float64) ** 2).sum(axis=1))
    return (-z * norms).astype(np.float32)


def make_workload(name: str, seed: int = 0, *, tls: float = 0.8, cls: float = 0.7,
                  L: int = 8, dense: bool = False, T: int | None = None,
                  **overrides) -> LayerInputs:
    """Draw one workload. Markov workloads take (tls, cls) at chunk length L;
    ``dense`` makes every score active (the all-experts special case)."""
    cfg = dict(WORKLOADS[name])
    if T is not None:
        cfg["T"] = T
    cfg.update(overrides)
    d_h, E, d_e, n, dtype = cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"], cfg["dtype"]
    T = cfg["T"]
    bf16 = dtype == "bf16"
    rng = np.random.default_rng(seed)
    x = gaussian(rng, (T, d_h), 1.0, bf16)
    w1, w2 = expert_weights(rng, E, d_e, d_h, bf16)
    inp = LayerInputs(name=name, dtype=dtype, T=T, d_h=d_h, E=E, d_e=d_e, n=n,
                      x=x, w1=w1, w2=w2)
    if name == "tiny":
        inp.w_r = gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), bf16)
        inp.gain = np.ones(E, np.float32)
    elif name == "e2e":
        inp.w_r = gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), bf16)
        inp.gain = np.ones(E, np.float32)
        inp.bias = router_shift(inp.w_r, 0.8)
    else:
        if dense:
            active = np.ones((T, E), bool)
        else:
            active = markov_active(rng, T, E, tls, cls, L)
        inp.scores = scores_for_mask(rng, active)
        inp.extra.update(tls=tls, cls=cls, L=L, dense=dense)
    return inp


def markov_scores(seed: int, T: int, E: int, tls: float = 0.8, cls: float = 0.7,
                  L: int = 8) -> np.ndarray:
    """A fresh mask draw with scores, for rotating masks across benchmark steps."""
    rng = np.random.default_rng(seed)
    return scores_for_mask(rng, markov_active(rng, T, E, tls, cls, L))


# ------------------------------------------------------------------ epilogue and losses

def activation_probs(seed: int, B: int, S: int, E: int, tls: float = 0.8, cls: float = 0.7,
                     L: int = 8) -> np.ndarray:
    """float32 [B, S, E] activation probabilities for the sparsity losses: per sequence
    a Markov on/off mask at (tls, cls), then U(0.5, 1) where on and U(0, 0.5) where
    off, a stand-in for a trained router's probabilities (on/off structure with
    locality, values spread over the whole open interval)."""
    rng = np.random.default_rng(seed)
    out = np.empty((B, S, E), np.float32)
    for b in range(B):
        act = markov_active(rng, S, E, tls, cls, L)
        u = rng.random((S, E))
        out[b] = np.where(act, 0.5 + 0.5 * u, 0.5 * u).astype(np.float32)
    return out


def layernorm_inputs(seed: int, T: int, d_h: int, bf16: bool):
    """(y, x, gamma, beta) for the residual + LayerNorm epilogue: y ~ N(0, 1) standing
    in for the expert output (unit-variance by the weight scaling of expert_weights),
    x ~ N(0, 1), gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1^2); y and x bf16-exact when bf16."""
    rng = np.random.default_rng(seed)
    y = gaussian(rng, (T, d_h), 1.0, bf16)
    x = gaussian(rng, (T, d_h), 1.0, bf16)
    gamma = rng.uniform(0.5, 1.5, d_h).astype(np.float32)
    beta = (0.1 * rng.standard_normal(d_h)).astype(np.float32)
    return y, x, gamma, beta


# ------------------------------------------------------------------ router inputs with a prescribed activity

def router_weight_orthonormal(rng: np.random.Generator, E: int, d_h: int, bf16: bool) -> np.ndarray:
    """W_r [E, d_h] with orthonormal rows (from the QR factor of a Gaussian matrix): the
    same scale as W_r ~ N(0, 1/d_h), and W_r W_r^T = I (up to bf16 rounding)."""
    q, _ = np.linalg.qr(rng.standard_normal((d_h, E)))
    w = q.T.astype(np.float32)
    return round_bf16(w) if bf16 else w


def tokens_for_mask(rng: np.random.Generator, w_r: np.ndarray, active: np.ndarray,
                    bf16: bool) -> np.ndarray:
    """x [T, d_h] whose router logits W_r x_t equal a prescribed c_t: c[t,e] =
    |N(0,1)| + 0.1 where active[t,e], -(|N(0,1)| + 0.1) elsewhere, so a router with
    these orthonormal W_r rows (and no logit shift) is active exactly on the mask.
    x_t = W_r^T c_t + the component of z_t ~ N(0, I) orthogonal to W_r's rows, so x
    keeps unit-variance coordinates. With bf16 rounding of x and W_r the logits move
    by ~1e-3 at d_h = 2048, far below the 0.1 margin, so the mask is exact."""
    T, E = active.shape
    w = w_r.astype(np.float64)
    mag = np.abs(rng.standard_normal((T, E))) + 0.1
    c = np.where(active, mag, -mag)
    z = rng.standard_normal((T, w.shape[1]))
    x = c @ w + z - (z @ w.T) @ w
    x = x.astype(np.float32)
    return round_bf16(x) if bf16 else x
