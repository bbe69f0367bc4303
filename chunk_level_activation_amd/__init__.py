"""MI355X (gfx950) BlockFFN layer forward: Python binding of libblockffn.so.

The functions here carry the names of the C ABI in include/blockffn.h and only
marshal arguments: they check tensor placement/dtype/contiguity, allocate outputs
with torch when the caller gives none, and pass raw device pointers and torch's
current HIP stream. Every step of the layer runs in the library's HIP kernels; there
is no fallback. If the library is missing the calls raise.

Layer (BlockFFN, arXiv 2507.08771; skill page "BlockFFN: Sparse Mixture-of-Experts
Optimized for End-Device Deployment", "Core Concept" and "Architecture Overview"):
    scores = RMSNorm_E(ReLU(x W_r^T)) * g
    y_t    = sum_{e in U_c(t)} scores[t,e] * W2_e swish(W1_e x_t)
with U_c the union of experts active in the n-token chunk c holding t.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "BLOCKFFN_F32", "BLOCKFFN_BF16", "BlockFFNError", "FP32_EPS", "library_path",
    "blockffn_router", "blockffn_router_workspace_bytes", "blockffn_router_workspace",
    "blockffn_chunk_ffn", "blockffn_chunk_ffn_workspace_bytes",
    "blockffn_chunk_ffn_workspace", "blockffn_add_layernorm", "blockffn_sparsity_losses",
    "blockffn_sparsity_losses_workspace_bytes", "blockffn_sparsity_losses_workspace",
    "blockffn_layer_backward", "blockffn_layer_backward_workspace_bytes",
    "blockffn_layer_forward", "blockffn_layer_forward_workspace_bytes",
    "blockffn_layer_forward_workspace", "blockffn_layer_forward_fused",
    "blockffn_pack_weights_bytes", "blockffn_pack_weights", "blockffn_layer_forward_packed",
    "blockffn_layer_forward_full", "blockffn_layer_forward_full_workspace_bytes",
    "blockffn_layer_forward_full_workspace", "blockffn_layer_forward_noalloc", "blockffn_init", "blockffn_workspace_check", "blockffn_last_error", "blockffn_version",
    "load_library",
]

BLOCKFFN_F32 = 0
BLOCKFFN_BF16 = 1
# torch.nn.RMSNorm's default eps for fp32 (torch.finfo(torch.float32).eps).
FP32_EPS = 1.1920928955078125e-07

STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "EWORKSPACE", 4: "EHIP",
                5: "ETIMEOUT"}

_HERE = os.path.dirname(os.path.abspath(__file__))
# BLOCKFFN_SANITIZE=1 selects the build whose host code runs under the address and
# undefined-behaviour sanitizers (build_lib.py --sanitize); the kernels are the same.
library_path = os.path.join(_HERE, "libblockffn_san.so" if os.environ.get("BLOCKFFN_SANITIZE") == "1"
                            else "libblockffn.so")
_lib = None


class BlockFFNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"blockffn status {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library():
    """Load libblockffn.so (built in-tree by build_lib.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m chunk_level_activation_amd.build_lib` (or __graft_entry__.build())")
    lib = ctypes.CDLL(library_path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    F = ctypes.c_float
    lib.blockffn_router.argtypes = [P, P, P, P, F, I64, I64, I64, I, P, P, F, P, P,
                                    ctypes.c_size_t, P]
    lib.blockffn_router.restype = I
    lib.blockffn_router_workspace_bytes.argtypes = [I64, I64, I64, I]
    lib.blockffn_router_workspace_bytes.restype = ctypes.c_size_t
    lib.blockffn_chunk_ffn_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
    lib.blockffn_chunk_ffn_workspace_bytes.restype = ctypes.c_size_t
    lib.blockffn_chunk_ffn.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, P, P,
                                       ctypes.c_size_t, P, P, P, P]
    lib.blockffn_chunk_ffn.restype = I
    lib.blockffn_add_layernorm.argtypes = [P, P, P, P, F, I64, I64, I, P, P]
    lib.blockffn_add_layernorm.restype = I
    lib.blockffn_sparsity_losses_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.blockffn_sparsity_losses_workspace_bytes.restype = ctypes.c_size_t
    lib.blockffn_sparsity_losses.argtypes = [P, I64, I64, I64, F, I64, F, F, P, P, P,
                                             ctypes.c_size_t, P]
    lib.blockffn_sparsity_losses.restype = I
    lib.blockffn_layer_backward_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
    lib.blockffn_layer_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.blockffn_layer_backward.argtypes = [P, P, P, P, F, P, P, I64, I64, I64, I64, I64, I, P,
                                            P, F, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.blockffn_layer_backward.restype = I
    lib.blockffn_layer_forward_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
    lib.blockffn_layer_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.blockffn_layer_forward.argtypes = [P, P, P, P, F, P, P, I64, I64, I64, I64, I64, I, P, P,
                                           P, ctypes.c_size_t, P]
    lib.blockffn_layer_forward.restype = I
    lib.blockffn_layer_forward_fused.argtypes = [I64, I64, I64, I64, I64, I, P]
    lib.blockffn_layer_forward_fused.restype = I
    lib.blockffn_pack_weights_bytes.argtypes = [I64, I64, I64, I]
    lib.blockffn_pack_weights_bytes.restype = ctypes.c_size_t
    lib.blockffn_pack_weights.argtypes = [P, P, I64, I64, I64, I, P, P]
    lib.blockffn_pack_weights.restype = I
    lib.blockffn_layer_forward_packed.argtypes = [P, P, P, P, F, P, I64, I64, I64, I64, I64, I, P,
                                                  P, P, ctypes.c_size_t, P]
    lib.blockffn_layer_forward_packed.restype = I
    lib.blockffn_layer_forward_full_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
    lib.blockffn_layer_forward_full_workspace_bytes.restype = ctypes.c_size_t
    lib.blockffn_layer_forward_full.argtypes = [P, P, P, P, F, P, P, P, I64, I64, I64, I64, I64, I,
                                                P, P, F, P, F, P, P, P, P, ctypes.c_size_t, P]
    lib.blockffn_layer_forward_full.restype = I
    lib.blockffn_layer_forward_noalloc.argtypes = [P, P, P, P, F, P, P, I64, I64, I64, I64, I64,
                                                   I, P, P, P]
    lib.blockffn_layer_forward_noalloc.restype = I
    lib.blockffn_init.argtypes = [P]
    lib.blockffn_init.restype = I
    lib.blockffn_workspace_check.argtypes = [P, ctypes.c_size_t, P]
    lib.blockffn_workspace_check.restype = I
    lib.blockffn_last_error.argtypes = []
    lib.blockffn_last_error.restype = ctypes.c_char_p
    lib.blockffn_version.argtypes = []
    lib.blockffn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def blockffn_init(stream=None) -> None:
    """Probe the current device for the one-launch schedules (see blockffn.h); optional,
    and to be called outside graph capture."""
    _check(load_library().blockffn_init(_stream(stream)))


def blockffn_workspace_check(workspace, stream=None) -> None:
    """Raise BlockFFNError (status ETIMEOUT) if a kernel that used this workspace timed
    out in one of its bounded waits; synchronises the stream (see blockffn.h)."""
    _check(load_library().blockffn_workspace_check(
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def blockffn_last_error() -> str:
    return load_library().blockffn_last_error().decode()


def blockffn_version() -> str:
    return load_library().blockffn_version().decode()


def _check(status: int):
    if status != 0:
        raise BlockFFNError(status, blockffn_last_error())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return BLOCKFFN_F32
    if t.dtype == torch.bfloat16:
        return BLOCKFFN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def blockffn_router_workspace_bytes(T: int, d_h: int, E: int, dtype: int) -> int:
    nbytes = load_library().blockffn_router_workspace_bytes(T, d_h, E, dtype)
    if nbytes == 0:
        raise BlockFFNError(1, blockffn_last_error())
    return int(nbytes)


def blockffn_router_workspace(T: int, d_h: int, E: int, dtype: int, device="cuda"):
    """A zero-filled router workspace (see blockffn.h): it must start zeroed and is
    returned to that state by every call."""
    import torch
    nbytes = blockffn_router_workspace_bytes(T, d_h, E, dtype)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def blockffn_router(x, w_r, gain=None, bias=None, eps: float = FP32_EPS, *, scores=None,
                    logits=None, probs=None, sharpness: float = 1.0, workspace=None,
                    stream=None):
    """scores [T, E] fp32 = RMSNorm_E(ReLU(x W_r^T + bias)) * gain. x [T, d_h] and
    w_r [E, d_h] are both float32 or both bfloat16; gain/bias are [E] float32.
    `probs` ([T, E] fp32), when given, receives sigmoid(sharpness * scores).
    `workspace` (from blockffn_router_workspace) lets few-token calls split the d_h
    sum over several workgroups; without one the call runs unsplit."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    E = w_r.shape[0]
    if tuple(w_r.shape) != (E, d_h) or w_r.dtype != x.dtype:
        raise ValueError("w_r must be [E, d_h] with the dtype of x")
    if scores is None:
        scores = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_dev(x, "x"), _dev(w_r, "w_r"), _dev(gain, "gain", torch.float32),
            _dev(bias, "bias", torch.float32), float(eps), T, d_h, E, _dtype_code(x),
            _dev(scores, "scores", torch.float32), _dev(logits, "logits", torch.float32),
            float(sharpness), _dev(probs, "probs", torch.float32),
            _dev(workspace, "workspace"), ws_bytes, _stream(stream)]
    _check(lib.blockffn_router(*args))
    return scores


def blockffn_chunk_ffn_workspace_bytes(T: int, d_h: int, E: int, d_e: int, n: int,
                                       dtype: int) -> int:
    nbytes = load_library().blockffn_chunk_ffn_workspace_bytes(T, d_h, E, d_e, n, dtype)
    if nbytes == 0:
        raise BlockFFNError(1, blockffn_last_error())
    return int(nbytes)


def blockffn_chunk_ffn_workspace(T: int, d_h: int, E: int, d_e: int, n: int, dtype: int,
                                 device="cuda"):
    """A zero-filled workspace of the size the C ABI asks for (see blockffn.h): it
    must start zeroed and is returned to that state by every call."""
    import torch
    nbytes = blockffn_chunk_ffn_workspace_bytes(T, d_h, E, d_e, n, dtype)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def blockffn_chunk_ffn(x, scores, w1, w2, n: int, *, y=None, workspace=None,
                       union_masks=None, expert_lists=None, union_counts=None,
                       stream=None):
    """y [T, d_h] = chunk-union expert FFN of x masked by scores (see blockffn.h).
    x [T, d_h], w1 [E, d_e, d_h], w2 [E, d_h, d_e] share one dtype; scores [T, E] fp32.
    Optional outputs: union_masks [C, ceil(E/64)] int64 (uint64 bits), expert_lists
    [C, E] int32, union_counts [C] int32, C = ceil(T/n)."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    E, d_e, _ = w1.shape
    if tuple(w1.shape) != (E, d_e, d_h) or tuple(w2.shape) != (E, d_h, d_e):
        raise ValueError("w1 must be [E, d_e, d_h] and w2 [E, d_h, d_e]")
    if tuple(scores.shape) != (T, E):
        raise ValueError("scores must be [T, E]")
    if w1.dtype != x.dtype or w2.dtype != x.dtype:
        raise TypeError("x, w1 and w2 must share a dtype")
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    nbytes = blockffn_chunk_ffn_workspace_bytes(T, d_h, E, d_e, n, code)
    if workspace is None:
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=x.device)
    args = [_dev(x, "x"), _dev(scores, "scores", torch.float32), _dev(w1, "w1"),
            _dev(w2, "w2"), T, d_h, E, d_e, n, code, _dev(y, "y", x.dtype),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _dev(union_masks, "union_masks", torch.int64),
            _dev(expert_lists, "expert_lists", torch.int32),
            _dev(union_counts, "union_counts", torch.int32), _stream(stream)]
    _check(lib.blockffn_chunk_ffn(*args))
    return y


def blockffn_add_layernorm(y, x, gamma=None, beta=None, eps: float = 1e-5, *, out=None,
                           stream=None):
    """out [T, d_h] = LayerNorm(y + x) * gamma + beta over d_h (see blockffn.h). y and x
    share a dtype (float32 or bfloat16); gamma/beta are [d_h] float32. `out` may be y
    or x (in place)."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    if tuple(y.shape) != (T, d_h) or y.dtype != x.dtype:
        raise ValueError("y must be [T, d_h] with the dtype of x")
    if out is None:
        out = torch.empty_like(x)
    args = [_dev(y, "y"), _dev(x, "x"), _dev(gamma, "gamma", torch.float32),
            _dev(beta, "beta", torch.float32), float(eps), T, d_h, _dtype_code(x),
            _dev(out, "out", x.dtype), _stream(stream)]
    _check(lib.blockffn_add_layernorm(*args))
    return out


def blockffn_sparsity_losses_workspace_bytes(B: int, S: int, E: int, L: int) -> int:
    nbytes = load_library().blockffn_sparsity_losses_workspace_bytes(B, S, E, L)
    if nbytes == 0:
        raise BlockFFNError(1, blockffn_last_error())
    return int(nbytes)


def blockffn_sparsity_losses_workspace(B: int, S: int, E: int, L: int, device="cuda"):
    """A zero-filled loss workspace: it must start zeroed and every call returns it to
    that state."""
    import torch
    return torch.zeros(blockffn_sparsity_losses_workspace_bytes(B, S, E, L),
                       dtype=torch.uint8, device=device)


def blockffn_sparsity_losses(probs, alpha: float = 2.0, L: int = 8, lambda_al: float = 1.0,
                             lambda_cs: float = 1.0, *, losses=None, grad=None,
                             want_grad: bool = True, workspace=None, stream=None):
    """(losses [2] fp32 = (activation locality, chunk sparsification), grad) over
    probabilities [B, S, E] (or [S, E]) float32; grad = lambda_al dAL/dp +
    lambda_cs dCS/dp, same shape as probs, or None when want_grad is False and no
    grad tensor is given."""
    import torch
    lib = load_library()
    if probs.dim() == 2:
        B, (S, E) = 1, probs.shape
    elif probs.dim() == 3:
        B, S, E = probs.shape
    else:
        raise ValueError("probs must be [B, S, E] or [S, E]")
    if losses is None:
        losses = torch.empty(2, dtype=torch.float32, device=probs.device)
    if grad is None and want_grad:
        grad = torch.empty_like(probs)
    if grad is not None and tuple(grad.shape) != tuple(probs.shape):
        raise ValueError("grad must have the shape of probs")
    if workspace is None:
        workspace = blockffn_sparsity_losses_workspace(B, S, E, L, probs.device)
    args = [_dev(probs, "probs", torch.float32), B, S, E, float(alpha), int(L),
            float(lambda_al), float(lambda_cs), _dev(losses, "losses", torch.float32),
            _dev(grad, "grad", torch.float32), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    _check(lib.blockffn_sparsity_losses(*args))
    return losses, grad


def blockffn_layer_backward_workspace_bytes(T: int, d_h: int, E: int, d_e: int, n: int,
                                            dtype: int = BLOCKFFN_BF16) -> int:
    nbytes = load_library().blockffn_layer_backward_workspace_bytes(T, d_h, E, d_e, n, dtype)
    if nbytes == 0:
        raise BlockFFNError(2, blockffn_last_error())
    return int(nbytes)


def blockffn_layer_backward(x, w_r, w1, w2, dy, n: int, gain=None, bias=None,
                            eps: float = FP32_EPS, *, dprobs=None, sharpness: float = 1.0,
                            want_gain=True, want_bias=True, out=None, workspace=None,
                            stream=None):
    """Gradients of sum(dy * y) + sum(dprobs * probs) for the layer (see blockffn.h):
    a dict of float32 tensors dx [T, d_h], dw_r [E, d_h], dw1 [E, d_e, d_h],
    dw2 [E, d_h, d_e], dgain [E] and dbias [E] (the last two when asked for). x, w_r,
    w1, w2 and dy are bfloat16. `out` may hold preallocated output tensors under
    those names."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    E, d_e, _ = w1.shape
    if tuple(w_r.shape) != (E, d_h) or tuple(w2.shape) != (E, d_h, d_e) or \
            tuple(dy.shape) != (T, d_h):
        raise ValueError("w_r [E, d_h], w2 [E, d_h, d_e] and dy [T, d_h] expected")
    code = _dtype_code(x)
    dev = x.device
    f32 = torch.float32
    shapes = dict(dx=(T, d_h), dw_r=(E, d_h), dw1=(E, d_e, d_h), dw2=(E, d_h, d_e))
    if want_gain:
        shapes["dgain"] = (E,)
    if want_bias:
        shapes["dbias"] = (E,)
    out = dict(out or {})
    for k, shp in shapes.items():
        if k not in out:
            out[k] = torch.empty(shp, dtype=f32, device=dev)
        elif tuple(out[k].shape) != shp or out[k].dtype != f32:
            raise ValueError(f"out[{k!r}] must be float32 {shp}")
    nbytes = blockffn_layer_backward_workspace_bytes(T, d_h, E, d_e, n, code)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = [_dev(x, "x"), _dev(w_r, "w_r"), _dev(gain, "gain", f32), _dev(bias, "bias", f32),
            float(eps), _dev(w1, "w1"), _dev(w2, "w2"), T, d_h, E, d_e, int(n), code,
            _dev(dy, "dy", x.dtype), _dev(dprobs, "dprobs", f32), float(sharpness),
            _dev(out["dx"], "dx"), _dev(out["dw_r"], "dw_r"), _dev(out.get("dgain"), "dgain"),
            _dev(out.get("dbias"), "dbias"), _dev(out["dw1"], "dw1"), _dev(out["dw2"], "dw2"),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream)]
    _check(lib.blockffn_layer_backward(*args))
    return out


def blockffn_layer_forward_workspace_bytes(T: int, d_h: int, E: int, d_e: int, n: int,
                                           dtype: int) -> int:
    nbytes = load_library().blockffn_layer_forward_workspace_bytes(T, d_h, E, d_e, n, dtype)
    if nbytes == 0:
        raise BlockFFNError(1, blockffn_last_error())
    return int(nbytes)


def blockffn_layer_forward_workspace(T: int, d_h: int, E: int, d_e: int, n: int, dtype: int,
                                     device="cuda"):
    """A zero-filled layer workspace: it must start zeroed and every call returns it to
    that state."""
    import torch
    return torch.zeros(blockffn_layer_forward_workspace_bytes(T, d_h, E, d_e, n, dtype),
                       dtype=torch.uint8, device=device)


def blockffn_layer_forward(x, w_r, w1, w2, n: int, gain=None, bias=None, eps: float = FP32_EPS,
                           *, y=None, scores=None, workspace=None, stream=None):
    """y [T, d_h] = chunk FFN of x under the router's scores (see blockffn.h); `scores`
    ([T, E] float32), when given, receives the scores."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    E, d_e, _ = w1.shape
    if tuple(w_r.shape) != (E, d_h) or tuple(w2.shape) != (E, d_h, d_e):
        raise ValueError("w_r must be [E, d_h], w2 [E, d_h, d_e]")
    if w_r.dtype != x.dtype or w1.dtype != x.dtype or w2.dtype != x.dtype:
        raise TypeError("x, w_r, w1 and w2 must share a dtype")
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = blockffn_layer_forward_workspace(T, d_h, E, d_e, n, code, x.device)
    args = [_dev(x, "x"), _dev(w_r, "w_r"), _dev(gain, "gain", torch.float32),
            _dev(bias, "bias", torch.float32), float(eps), _dev(w1, "w1"), _dev(w2, "w2"),
            T, d_h, E, d_e, int(n), code, _dev(y, "y", x.dtype),
            _dev(scores, "scores", torch.float32), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    _check(lib.blockffn_layer_forward(*args))
    return y


def blockffn_layer_forward_full_workspace_bytes(T: int, d_h: int, E: int, d_e: int, n: int,
                                                dtype: int) -> int:
    nbytes = load_library().blockffn_layer_forward_full_workspace_bytes(T, d_h, E, d_e, n, dtype)
    if nbytes == 0:
        raise BlockFFNError(1, blockffn_last_error())
    return int(nbytes)


def blockffn_layer_forward_full_workspace(T: int, d_h: int, E: int, d_e: int, n: int,
                                          dtype: int, device="cuda"):
    """A zero-filled workspace for blockffn_layer_forward_full."""
    import torch
    return torch.zeros(blockffn_layer_forward_full_workspace_bytes(T, d_h, E, d_e, n, dtype),
                       dtype=torch.uint8, device=device)


def blockffn_layer_forward_full(x, w_r, n: int, *, w1=None, w2=None, packed=None, E=None,
                                d_e=None, gain=None, bias=None, eps: float = FP32_EPS,
                                ln_gamma=None, ln_beta=None, ln_eps: float = 1e-5, out=None,
                                sharpness: float = 1.0, probs=None, y=None, scores=None,
                                workspace=None, stream=None):
    """out [T, d_h] = LayerNorm(layer FFN output + x), and probs = sigmoid(sharpness *
    scores) when `probs` is given (see blockffn.h). Weights: w1/w2 row-major, or packed
    (from blockffn_pack_weights) with E and d_e given."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    if packed is None:
        E, d_e, _ = w1.shape
        if tuple(w2.shape) != (E, d_h, d_e):
            raise ValueError("w2 must be [E, d_h, d_e]")
    elif E is None or d_e is None:
        raise ValueError("packed weights need E and d_e")
    if tuple(w_r.shape) != (E, d_h):
        raise ValueError("w_r must be [E, d_h]")
    code = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = blockffn_layer_forward_full_workspace(T, d_h, E, d_e, n, code, x.device)
    args = [_dev(x, "x"), _dev(w_r, "w_r"), _dev(gain, "gain", torch.float32),
            _dev(bias, "bias", torch.float32), float(eps), _dev(w1, "w1"), _dev(w2, "w2"),
            _dev(packed, "packed"), T, d_h, E, d_e, int(n), code,
            _dev(ln_gamma, "ln_gamma", torch.float32), _dev(ln_beta, "ln_beta", torch.float32),
            float(ln_eps), _dev(out, "out", x.dtype), float(sharpness),
            _dev(probs, "probs", torch.float32), _dev(y, "y", x.dtype),
            _dev(scores, "scores", torch.float32), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    _check(lib.blockffn_layer_forward_full(*args))
    return out


def blockffn_layer_forward_noalloc(x, w_r, w1, w2, n: int, gain=None, bias=None,
                                   eps: float = FP32_EPS, *, y=None, scores=None, stream=None):
    """blockffn_layer_forward with the library's own scratch array instead of a workspace,
    for callers that cannot allocate (see blockffn.h); y must then be given by such
    callers (it is allocated here only when omitted)."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    E, d_e, _ = w1.shape
    if tuple(w_r.shape) != (E, d_h) or tuple(w2.shape) != (E, d_h, d_e):
        raise ValueError("w_r must be [E, d_h], w2 [E, d_h, d_e]")
    if w_r.dtype != x.dtype or w1.dtype != x.dtype or w2.dtype != x.dtype:
        raise TypeError("x, w_r, w1 and w2 must share a dtype")
    if y is None:
        y = torch.empty_like(x)
    args = [_dev(x, "x"), _dev(w_r, "w_r"), _dev(gain, "gain", torch.float32),
            _dev(bias, "bias", torch.float32), float(eps), _dev(w1, "w1"), _dev(w2, "w2"),
            T, d_h, E, d_e, int(n), _dtype_code(x), _dev(y, "y", x.dtype),
            _dev(scores, "scores", torch.float32), _stream(stream)]
    _check(lib.blockffn_layer_forward_noalloc(*args))
    return y


def blockffn_pack_weights_bytes(E: int, d_h: int, d_e: int, dtype: int) -> int:
    return int(load_library().blockffn_pack_weights_bytes(E, d_h, d_e, dtype))


def blockffn_pack_weights(w1, w2, *, packed=None, stream=None):
    """The expert weights W1 [E, d_e, d_h] and W2 [E, d_h, d_e] (bf16) in the tiled
    layout of blockffn_pack_weights (see blockffn.h): a flat bf16 tensor of
    2*E*d_h*d_e elements."""
    import torch
    lib = load_library()
    E, d_e, d_h = w1.shape
    if tuple(w2.shape) != (E, d_h, d_e) or w2.dtype != w1.dtype:
        raise ValueError("w2 must be [E, d_h, d_e] of w1's dtype")
    code = _dtype_code(w1)
    nbytes = blockffn_pack_weights_bytes(E, d_h, d_e, code)
    if nbytes == 0:
        raise BlockFFNError(1, "pack_weights: unsupported sizes or dtype")
    if packed is None:
        packed = torch.empty(nbytes // 2, dtype=w1.dtype, device=w1.device)
    elif packed.numel() * packed.element_size() < nbytes:
        raise ValueError("packed is too small")
    _check(lib.blockffn_pack_weights(_dev(w1, "w1"), _dev(w2, "w2"), E, d_h, d_e, code,
                                     _dev(packed, "packed"), _stream(stream)))
    return packed


def blockffn_layer_forward_packed(x, w_r, packed, E: int, d_e: int, n: int, gain=None,
                                  bias=None, eps: float = FP32_EPS, *, y=None, scores=None,
                                  workspace=None, stream=None):
    """blockffn_layer_forward with W1 and W2 from blockffn_pack_weights (see blockffn.h)."""
    import torch
    lib = load_library()
    T, d_h = x.shape
    if tuple(w_r.shape) != (E, d_h):
        raise ValueError("w_r must be [E, d_h]")
    if w_r.dtype != x.dtype or packed.dtype != x.dtype:
        raise TypeError("x, w_r and packed must share a dtype")
    code = _dtype_code(x)
    if packed.numel() * packed.element_size() < blockffn_pack_weights_bytes(E, d_h, d_e, code):
        raise ValueError("packed is too small for these sizes")
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = blockffn_layer_forward_workspace(T, d_h, E, d_e, n, code, x.device)
    args = [_dev(x, "x"), _dev(w_r, "w_r"), _dev(gain, "gain", torch.float32),
            _dev(bias, "bias", torch.float32), float(eps), _dev(packed, "packed"),
            T, d_h, E, d_e, int(n), code, _dev(y, "y", x.dtype),
            _dev(scores, "scores", torch.float32), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    _check(lib.blockffn_layer_forward_packed(*args))
    return y


def blockffn_layer_forward_fused(T: int, d_h: int, E: int, d_e: int, n: int, dtype: int,
                                 stream=None) -> bool:
    """True when blockffn_layer_forward runs router and FFN in one launch for these
    sizes on the current device."""
    return bool(load_library().blockffn_layer_forward_fused(T, d_h, E, d_e, n, dtype,
                                                            _stream(stream)))
