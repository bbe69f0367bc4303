"""CPU oracle for the BlockFFN layer (router + chunk-union expert FFN, forward and
backward), its residual + LayerNorm epilogue and the two sparsity training losses
with gradients.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this package; the GPU library never imports, links or calls it,
and shares no code with it. The arithmetic lives in ``blockffn_oracle.c`` (plain
loops, double accumulation); this module builds it with gcc, loads it with ctypes
and adds the sparsity meter used to check the synthetic masks.

Pages followed (BlockFFN, arXiv 2507.08771):
  * skill page "BlockFFN: Sparse Mixture-of-Experts Optimized for End-Device
    Deployment": "Core Concept" (union of active experts over n tokens, masking after
    the computation), "Architecture Overview" (ReLU + RMSNorm router, non-gated Swish
    experts), "Router Architecture Setup" (no router bias, RMSNorm over experts),
    "Chunk Sparsification Loss" (aligned chunks, ceil(S/L) of them), "Activation
    Locality Loss" (BCE of adjacent sharpened patterns), "Full BlockFFN Layer with
    Combined Losses" (LayerNorm of expert output plus residual).
  * paper card, Abstract: TLS and 8-token CLS as the sparsity measures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "blockffn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# torch.nn.RMSNorm's default eps for fp32 inputs (torch.finfo(torch.float32).eps):
# the pages construct the norm without an eps, so the module default applies.
FP32_EPS = float(np.finfo(np.float32).eps)


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction, OpenMP)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


# A build with the address and undefined-behaviour sanitizers (clang, so that one
# sanitizer runtime serves this library and the HIP library's host code in the same
# process). Selected by BLOCKFFN_SANITIZE=1; see chunk_level_activation_amd.build_lib.
_SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")
_CLANG = "/opt/rocm/lib/llvm/bin/clang"


def build_sanitized(verbose: bool = False, src: str = _SRC, out: str = _SAN_LIB_PATH) -> str:
    """The same C file with -fsanitize=address,undefined (no recovery), for host-side
    checking of the oracle's memory accesses and arithmetic."""
    cmd = [_CLANG, "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared-libasan",
           "-shared", "-fPIC", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


_lib = None


def use_library(path: str | None):
    """Load the oracle from another build of the C file (the mutation tests use this
    to check that the pins reject planted mistakes); None restores the default."""
    global _lib
    _lib = None
    if path is not None:
        _bind(ctypes.CDLL(path))


def _load():
    if _lib is not None:
        return _lib
    if os.environ.get("BLOCKFFN_SANITIZE") == "1":
        if not os.path.exists(_SAN_LIB_PATH) or (
                os.path.getmtime(_SAN_LIB_PATH) < os.path.getmtime(_SRC)):
            build_sanitized()
        return _bind(ctypes.CDLL(_SAN_LIB_PATH))
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    return _bind(ctypes.CDLL(_LIB_PATH))


def _bind(lib):
    global _lib
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_router.argtypes = [P, P, P, P, ctypes.c_double, I64, I64, I64, P, P]
    lib.oracle_router.restype = None
    lib.oracle_chunk_union.argtypes = [P, I64, I64, I64, P, P, P]
    lib.oracle_chunk_union.restype = None
    lib.oracle_chunk_ffn.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, P, P, P, P, P]
    lib.oracle_chunk_ffn.restype = None
    lib.oracle_token_ffn.argtypes = [P, P, P, P, I64, I64, I64, I64, P, P]
    lib.oracle_token_ffn.restype = None
    D = ctypes.c_double
    lib.oracle_router_probs.argtypes = [P, I64, D, P]
    lib.oracle_router_probs.restype = None
    lib.oracle_add_layernorm.argtypes = [P, P, P, P, D, I64, I64, P]
    lib.oracle_add_layernorm.restype = None
    lib.oracle_locality_loss.argtypes = [P, I64, I64, I64, D]
    lib.oracle_locality_loss.restype = D
    lib.oracle_chunk_sparsification_loss.argtypes = [P, I64, I64, I64, I64]
    lib.oracle_chunk_sparsification_loss.restype = D
    lib.oracle_locality_loss_grad.argtypes = [P, I64, I64, I64, D, P]
    lib.oracle_locality_loss_grad.restype = None
    lib.oracle_chunk_sparsification_loss_grad.argtypes = [P, I64, I64, I64, I64, P]
    lib.oracle_chunk_sparsification_loss_grad.restype = None
    lib.oracle_layer_backward.argtypes = [P, P, P, P, D, P, P, I64, I64, I64, I64, I64, P, P,
                                          D, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_layer_backward.restype = None
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def router(x, w_r, gain=None, bias=None, eps: float = FP32_EPS):
    """Return (logits, scores), both float64 [T, E]. See oracle_router in the C file."""
    lib = _load()
    x = _f32(x)
    w_r = _f32(w_r)
    T, d_h = x.shape
    E = w_r.shape[0]
    assert w_r.shape == (E, d_h)
    gain = None if gain is None else _f32(gain)
    bias = None if bias is None else _f32(bias)
    logits = np.empty((T, E), np.float64)
    scores = np.empty((T, E), np.float64)
    lib.oracle_router(_ptr(x), _ptr(w_r), _ptr(gain), _ptr(bias), float(eps),
                      T, d_h, E, _ptr(logits), _ptr(scores))
    return logits, scores


def chunk_union(scores, n: int):
    """Return (masks uint64 [C, W], lists int32 [C, E], counts int32 [C])."""
    lib = _load()
    scores = _f32(scores)
    T, E = scores.shape
    C = -(-T // n)
    W = -(-E // 64)
    masks = np.empty((C, W), np.uint64)
    lists = np.empty((C, E), np.int32)
    counts = np.empty((C,), np.int32)
    lib.oracle_chunk_union(_ptr(scores), T, E, n, _ptr(masks), _ptr(lists), _ptr(counts))
    return masks, lists, counts


def _check_ffn_shapes(x, scores, w1, w2):
    T, d_h = x.shape
    E, d_e, d_h1 = w1.shape
    assert d_h1 == d_h and w2.shape == (E, d_h, d_e) and scores.shape == (T, E)
    return T, d_h, E, d_e


def chunk_ffn(x, scores, w1, w2, n: int) -> np.ndarray:
    """Union-then-mask FFN, float64 [T, d_h]."""
    lib = _load()
    x, scores, w1, w2 = _f32(x), _f32(scores), _f32(w1), _f32(w2)
    T, d_h, E, d_e = _check_ffn_shapes(x, scores, w1, w2)
    C = -(-T // n)
    y = np.empty((T, d_h), np.float64)
    masks = np.empty((C, -(-E // 64)), np.uint64)
    lists = np.empty((C, E), np.int32)
    counts = np.empty((C,), np.int32)
    h = np.empty((lib.oracle_num_threads(), d_e), np.float64)
    lib.oracle_chunk_ffn(_ptr(x), _ptr(scores), _ptr(w1), _ptr(w2), T, d_h, E, d_e, n,
                         _ptr(y), _ptr(masks), _ptr(lists), _ptr(counts), _ptr(h))
    return y


def token_ffn(x, scores, w1, w2) -> np.ndarray:
    """Per-token brute force over each token's own active experts, float64 [T, d_h]."""
    lib = _load()
    x, scores, w1, w2 = _f32(x), _f32(scores), _f32(w1), _f32(w2)
    T, d_h, E, d_e = _check_ffn_shapes(x, scores, w1, w2)
    y = np.empty((T, d_h), np.float64)
    h = np.empty((lib.oracle_num_threads(), d_e), np.float64)
    lib.oracle_token_ffn(_ptr(x), _ptr(scores), _ptr(w1), _ptr(w2), T, d_h, E, d_e,
                         _ptr(y), _ptr(h))
    return y


# Layer epilogue and the training losses (skill page: "Router Architecture Setup",
# "Full BlockFFN Layer with Combined Losses", "Activation Locality Loss", "Chunk
# Sparsification Loss"). Probabilities are [B, S, E] (a [S, E] array is one batch).

def router_probs(scores, sharpness: float = 1.0) -> np.ndarray:
    """float64 sigmoid(sharpness * scores), same shape."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    out = np.empty_like(s)
    _load().oracle_router_probs(_ptr(s), s.size, float(sharpness), _ptr(out))
    return out


def add_layernorm(y, x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """float64 LayerNorm(y + x) over the last axis; y, x [T, d]; gamma/beta [d]."""
    y, x = _f32(y), _f32(x)
    T, d = x.shape
    assert y.shape == (T, d)
    gamma = None if gamma is None else _f32(gamma)
    beta = None if beta is None else _f32(beta)
    out = np.empty((T, d), np.float64)
    _load().oracle_add_layernorm(_ptr(y), _ptr(x), _ptr(gamma), _ptr(beta), float(eps),
                                 T, d, _ptr(out))
    return out


def _bse(p):
    p = _f32(p)
    if p.ndim == 2:
        p = p[None]
    return p, p.shape


def locality_loss(p, alpha: float = 2.0) -> float:
    p, (B, S, E) = _bse(p)
    return float(_load().oracle_locality_loss(_ptr(p), B, S, E, float(alpha)))


def chunk_sparsification_loss(p, L: int = 8) -> float:
    p, (B, S, E) = _bse(p)
    return float(_load().oracle_chunk_sparsification_loss(_ptr(p), B, S, E, int(L)))


def locality_loss_grad(p, alpha: float = 2.0) -> np.ndarray:
    p, (B, S, E) = _bse(p)
    g = np.empty((B, S, E), np.float64)
    _load().oracle_locality_loss_grad(_ptr(p), B, S, E, float(alpha), _ptr(g))
    return g


def chunk_sparsification_loss_grad(p, L: int = 8) -> np.ndarray:
    p, (B, S, E) = _bse(p)
    g = np.empty((B, S, E), np.float64)
    _load().oracle_chunk_sparsification_loss_grad(_ptr(p), B, S, E, int(L), _ptr(g))
    return g


def layer_backward(x, w_r, w1, w2, dy, n: int, gain=None, bias=None, eps: float = FP32_EPS,
                   dprobs=None, sharpness: float = 1.0) -> dict:
    """Gradients (float64) of sum(dy * y) + sum(dprobs * probs) for the layer
    y = chunk_ffn(x, router(x)), probs = sigmoid(sharpness * scores): a dict with dx,
    dw_r, dgain, dbias, dw1, dw2 (see oracle_layer_backward in the C file)."""
    lib = _load()
    x, w_r, w1, w2, dy = _f32(x), _f32(w_r), _f32(w1), _f32(w2), _f32(dy)
    T, d_h = x.shape
    E, d_e, _ = w1.shape
    assert w_r.shape == (E, d_h) and w2.shape == (E, d_h, d_e) and dy.shape == (T, d_h)
    assert d_e <= 4096
    gain = None if gain is None else _f32(gain)
    bias = None if bias is None else _f32(bias)
    dprobs = None if dprobs is None else _f32(dprobs)
    out = dict(dx=np.empty((T, d_h)), dw_r=np.empty((E, d_h)), dgain=np.empty(E),
               dbias=np.empty(E), dw1=np.empty((E, d_e, d_h)), dw2=np.empty((E, d_h, d_e)))
    logits, scores, ds = np.empty((T, E)), np.empty((T, E)), np.empty((T, E))
    da = np.empty((T, E, d_e))
    lib.oracle_layer_backward(_ptr(x), _ptr(w_r), _ptr(gain), _ptr(bias), float(eps),
                              _ptr(w1), _ptr(w2), T, d_h, E, d_e, int(n), _ptr(dy),
                              _ptr(dprobs), float(sharpness), _ptr(out["dx"]),
                              _ptr(out["dw_r"]), _ptr(out["dgain"]), _ptr(out["dbias"]),
                              _ptr(out["dw1"]), _ptr(out["dw2"]), _ptr(logits), _ptr(scores),
                              _ptr(ds), _ptr(da))
    return out


# --------------------------------------------------------------------------------
# Sparsity meter. The pages name token-level sparsity (TLS) and L-token chunk-level
# sparsity (CLS) without defining them in formulas; the readings used here are:
#   TLS   = fraction of (token, expert) pairs that are inactive;
#   CLS_L = 1 - mean over aligned, non-overlapping L-token chunks of |U|/E,
#           i.e. the fraction of experts left out of a chunk's union (paper-card
#           Abstract: the union of consecutive tokens is what CLS measures; chunks as
#           in "Chunk Sparsification Loss"). A partial last chunk counts as a chunk.
# --------------------------------------------------------------------------------

def tls(active: np.ndarray) -> float:
    active = np.asarray(active, dtype=bool)
    return 1.0 - float(active.sum()) / active.size


def union_fraction(active: np.ndarray, L: int) -> np.ndarray:
    """|U_c| / E for every aligned L-token chunk c."""
    active = np.asarray(active, dtype=bool)
    T, E = active.shape
    C = -(-T // L)
    out = np.empty(C)
    for c in range(C):
        out[c] = active[c * L:min(c * L + L, T)].any(axis=0).sum() / E
    return out


def cls(active: np.ndarray, L: int) -> float:
    return 1.0 - float(union_fraction(active, L).mean())
