"""The C ABI library loads, exports every declared symbol, and rejects invalid calls
on the host before touching the device (these run without a GPU).

Invalid calls are given fake non-NULL addresses: validation must return before any
of them is dereferenced or any kernel is launched.
"""
import ctypes
import os
import re

import pytest

import chunk_level_activation_amd as bf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockffn.h")

FAKE = 0x10000          # 256-byte aligned, never dereferenced
FAKE_ODD = 0x10002      # 2-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(blockffn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bf.load_library()


def test_header_declares_every_call():
    names = declared_functions()
    for n in ("blockffn_router", "blockffn_router_workspace_bytes", "blockffn_chunk_ffn",
              "blockffn_chunk_ffn_workspace_bytes", "blockffn_add_layernorm",
              "blockffn_sparsity_losses", "blockffn_sparsity_losses_workspace_bytes",
              "blockffn_last_error", "blockffn_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {bf.library_path}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", nm), name


def test_version(lib):
    assert bf.blockffn_version().startswith("blockffn-gfx950")


def ffn(lib, x=FAKE, scores=FAKE, w1=FAKE, w2=FAKE, T=32, d_h=2048, E=64, d_e=128, n=32,
        dtype=1, y=FAKE, ws=FAKE, ws_bytes=1 << 40, masks=None, lists=None, counts=None):
    return lib.blockffn_chunk_ffn(x, scores, w1, w2, T, d_h, E, d_e, n, dtype, y, ws,
                                  ws_bytes, masks, lists, counts, None)


def router(lib, x=FAKE, w_r=FAKE, gain=None, bias=None, eps=1e-6, T=32, d_h=2048, E=64,
           dtype=1, scores=FAKE, logits=None, sharpness=1.0, probs=None, ws=None,
           ws_bytes=0):
    return lib.blockffn_router(x, w_r, gain, bias, eps, T, d_h, E, dtype, scores, logits,
                               sharpness, probs, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(scores=None), 1), (dict(w1=None), 1), (dict(w2=None), 1),
    (dict(y=None), 1), (dict(ws=None), 1),
    (dict(T=0), 1), (dict(d_h=-1), 1), (dict(E=0), 1), (dict(d_e=0), 1), (dict(n=0), 1),
    (dict(dtype=7), 1),
    (dict(E=257), 2), (dict(d_h=2047), 2), (dict(d_e=100), 2),
    (dict(x=FAKE_ODD), 2), (dict(w1=FAKE_ODD), 2), (dict(y=FAKE_ODD), 2),
    (dict(ws=FAKE + 4), 2), (dict(scores=FAKE_ODD), 2),
    (dict(ws_bytes=0), 3), (dict(ws_bytes=1000), 3),
])
def test_chunk_ffn_rejects(lib, kw, status):
    assert ffn(lib, **kw) == status
    assert bf.blockffn_last_error() != ""


def test_fp32_accepts_unaligned_sizes_but_checks_workspace(lib):
    # fp32 has no d_h / d_e divisibility needs; the tiny workspace still fails
    assert ffn(lib, dtype=0, d_h=250, d_e=60, ws_bytes=16) == 3


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(w_r=None), 1), (dict(scores=None), 1), (dict(T=0), 1),
    (dict(dtype=-1), 1), (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1),
    (dict(E=300), 2), (dict(d_h=100), 2), (dict(x=FAKE_ODD), 2),
    (dict(scores=FAKE_ODD), 2), (dict(ws=FAKE + 4, ws_bytes=1 << 30), 2),
    (dict(ws=FAKE, ws_bytes=0), 3), (dict(ws=FAKE, ws_bytes=255), 3),
    (dict(probs=FAKE + 0x100000, sharpness=float("inf")), 1),
    (dict(probs=FAKE + 0x100000, sharpness=float("nan")), 1),
    (dict(probs=FAKE_ODD), 2),
])
def test_router_rejects(lib, kw, status):
    assert router(lib, **kw) == status


def layernorm(lib, y=FAKE, x=FAKE + (1 << 24), gamma=None, beta=None, eps=1e-5, T=32,
              d_h=2048, dtype=1, out=FAKE + (2 << 24)):
    return lib.blockffn_add_layernorm(y, x, gamma, beta, eps, T, d_h, dtype, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(y=None), 1), (dict(x=None), 1), (dict(out=None), 1), (dict(T=0), 1),
    (dict(d_h=0), 1), (dict(dtype=3), 1), (dict(eps=-1.0), 1), (dict(eps=float("inf")), 1),
    (dict(d_h=2044), 2), (dict(dtype=0, d_h=2046), 2), (dict(y=FAKE + 8), 2),
    (dict(gamma=FAKE + 4), 2), (dict(beta=FAKE + 8), 2),
    # out may be y or x, but not overlap them partially
    (dict(out=FAKE + 4096), 1), (dict(out=FAKE + (1 << 24) - 4096), 1),
])
def test_layernorm_rejects(lib, kw, status):
    assert layernorm(lib, **kw) == status
    assert bf.blockffn_last_error() != ""


def losses(lib, probs=FAKE, B=2, S=4096, E=64, alpha=2.0, L=8, lal=1.0, lcs=1.0,
           out=FAKE + (4 << 24), grad=FAKE + (8 << 24), ws=FAKE + (16 << 24),
           ws_bytes=1 << 20):
    return lib.blockffn_sparsity_losses(probs, B, S, E, alpha, L, lal, lcs, out, grad, ws,
                                        ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(probs=None), 1), (dict(out=None), 1), (dict(ws=None), 1), (dict(B=0), 1),
    (dict(S=0), 1), (dict(E=0), 1), (dict(L=0), 1), (dict(alpha=float("nan")), 1),
    (dict(lal=float("inf")), 1),
    (dict(B=1 << 16, S=1 << 16), 2), (dict(probs=FAKE + 2), 2), (dict(ws=FAKE + (16 << 24) + 4), 2),
    (dict(ws_bytes=100), 3),
    (dict(grad=FAKE + 4096), 1), (dict(out=FAKE + 8), 1),
])
def test_sparsity_losses_rejects(lib, kw, status):
    assert losses(lib, **kw) == status
    assert bf.blockffn_last_error() != ""


def test_sparsity_losses_workspace_query(lib):
    f = lib.blockffn_sparsity_losses_workspace_bytes
    # counter lines (top + 64 groups) + one fp64 pair per workgroup, for the most
    # workgroups a launch
    # may use (4096 tokens, 8-token chunks, 64 experts: 32768 columns -> 512 one-wave
    # workgroups)
    assert f(1, 4096, 64, 8) == 65 * 128 + 512 * 16
    assert f(64, 4096, 64, 8) == 65 * 128 + 2048 * 16
    assert f(1, 4096, 64, 0) == 0
    assert f(1, 0, 64, 8) == 0


def test_router_workspace_query(lib):
    f = lib.blockffn_router_workspace_bytes
    # decode: the d_h sum is split, partial logits of every split need room
    assert f(32, 2048, 64, 1) >= 8 * 32 * 64 * 4
    # many tokens or fp32: no split, the minimum size
    assert f(1 << 16, 2048, 64, 1) == 256
    assert f(32, 2048, 64, 0) == 256
    assert f(0, 2048, 64, 1) == 0
    assert f(32, 2048, 999, 1) == 0


def test_workspace_query(lib):
    f = lib.blockffn_chunk_ffn_workspace_bytes
    decode = f(32, 2048, 64, 128, 32, 1)
    assert decode > 0
    # holds at least one bf16 hidden tile per expert slot
    assert decode >= 64 * 32 * 128 * 2
    assert f(2048, 2048, 64, 128, 32, 1) > decode
    assert f(0, 2048, 64, 128, 32, 1) == 0
    assert f(32, 2048, 999, 128, 32, 1) == 0
    assert "experts" in bf.blockffn_last_error()
    with pytest.raises(bf.BlockFFNError):
        bf.blockffn_chunk_ffn_workspace_bytes(32, 2048, 64, 100, 32, 1)


def test_error_message_is_per_thread(lib):
    import threading
    ffn(lib, T=0)
    seen = {}

    def other():
        seen["msg"] = bf.blockffn_last_error()
    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert bf.blockffn_last_error() != ""


def test_product_path_has_no_oracle_dependency():
    """The package and the library never refer to the oracle."""
    pkg = os.path.join(ROOT, "chunk_level_activation_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn
    deps = os.popen(f"ldd {bf.library_path}").read()
    assert "liboracle" not in deps


def backward(lib, x=FAKE, w_r=FAKE, gain=None, bias=None, eps=1e-6, w1=FAKE, w2=FAKE, T=64,
             d_h=2048, E=64, d_e=128, n=32, dtype=1, dy=FAKE, dprobs=None, sharpness=1.0,
             dx=FAKE, dw_r=FAKE, dgain=None, dbias=None, dw1=FAKE, dw2=FAKE, ws=FAKE,
             ws_bytes=1 << 40):
    return lib.blockffn_layer_backward(x, w_r, gain, bias, eps, w1, w2, T, d_h, E, d_e, n, dtype,
                                       dy, dprobs, sharpness, dx, dw_r, dgain, dbias, dw1, dw2,
                                       ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(dy=None), 1), (dict(dx=None), 1), (dict(dw1=None), 1),
    (dict(ws=None), 1), (dict(T=0), 1), (dict(n=0), 1), (dict(dtype=5), 1),
    (dict(eps=-1.0), 1), (dict(sharpness=float("nan")), 1),
    (dict(dtype=0), 2), (dict(d_h=2080), 2), (dict(d_e=64), 2), (dict(E=300), 2),
    (dict(x=FAKE + 8), 2), (dict(dx=FAKE + 4), 2), (dict(ws=FAKE + 16), 2),
    (dict(ws_bytes=4096), 3),
])
def test_layer_backward_rejects(lib, kw, status):
    assert backward(lib, **kw) == status
    assert bf.blockffn_last_error() != ""


def test_layer_backward_workspace_query(lib):
    f = lib.blockffn_layer_backward_workspace_bytes
    # hidden-activation gradients in three layouts dominate: 3 x CT x E x 32 x d_e bf16
    assert f(2048, 2048, 64, 128, 32, 1) >= 3 * 64 * 64 * 32 * 128 * 2
    assert f(2048, 2048, 64, 128, 32, 0) == 0      # bf16 only
    assert f(2048, 2048, 64, 64, 32, 1) == 0       # d_e % 128
    assert f(0, 2048, 64, 128, 32, 1) == 0


def layer(lib, x=FAKE, w_r=FAKE, gain=None, bias=None, eps=1e-6, w1=FAKE, w2=FAKE, T=32,
          d_h=2048, E=64, d_e=128, n=32, dtype=1, y=FAKE, scores=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.blockffn_layer_forward(x, w_r, gain, bias, eps, w1, w2, T, d_h, E, d_e, n, dtype,
                                      y, scores, ws, ws_bytes, None)


def layer_packed(lib, x=FAKE, w_r=FAKE, gain=None, bias=None, eps=1e-6, packed=FAKE, T=32,
                 d_h=2048, E=64, d_e=128, n=32, dtype=1, y=FAKE, scores=None, ws=FAKE,
                 ws_bytes=1 << 40):
    return lib.blockffn_layer_forward_packed(x, w_r, gain, bias, eps, packed, T, d_h, E, d_e, n,
                                             dtype, y, scores, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(w_r=None), 1), (dict(w1=None), 1), (dict(w2=None), 1),
    (dict(y=None), 1), (dict(ws=None), 1), (dict(T=0), 1), (dict(n=0), 1), (dict(dtype=9), 1),
    (dict(eps=-1.0), 1), (dict(E=257), 2), (dict(x=FAKE_ODD), 2), (dict(w_r=FAKE + 8), 2),
    (dict(ws=FAKE + 16), 2), (dict(ws_bytes=1000), 3),
])
def test_layer_forward_rejects(lib, kw, status):
    assert layer(lib, **kw) == status
    assert bf.blockffn_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(packed=None), 1), (dict(x=None), 1), (dict(y=None), 1), (dict(T=0), 1),
    (dict(packed=FAKE_ODD), 2), (dict(ws_bytes=1000), 3),
    # sizes the one-launch layer never takes (E > 64, several chunks): nothing runs
    (dict(E=128), 2), (dict(T=256), 2),
])
def test_layer_forward_packed_rejects(lib, kw, status):
    assert layer_packed(lib, **kw) == status
    assert bf.blockffn_last_error() != ""


def test_pack_weights_query_and_rejects(lib):
    f = lib.blockffn_pack_weights_bytes
    assert f(64, 2048, 128, 1) == 2 * 64 * 2048 * 128 * 2
    assert f(64, 2048, 128, 0) == 0            # bf16 only
    assert f(64, 2048, 100, 1) == 0            # d_e % 32
    assert f(64, 2050, 128, 1) == 0            # d_h % 32
    assert f(0, 2048, 128, 1) == 0
    assert f(300, 2048, 128, 1) == 0
    p = lib.blockffn_pack_weights
    assert p(FAKE, FAKE, 64, 2048, 128, 0, FAKE, None) == 1
    assert p(None, FAKE, 64, 2048, 128, 1, FAKE, None) == 1
    assert p(FAKE, FAKE, 64, 2048, 128, 1, None, None) == 1
    assert p(FAKE, FAKE_ODD, 64, 2048, 128, 1, FAKE, None) == 2
    assert bf.blockffn_last_error() != ""


def test_workspace_check_rejects_before_touching_the_device(lib):
    assert lib.blockffn_workspace_check(None, 1 << 20, None) == 1          # EINVAL
    assert lib.blockffn_workspace_check(FAKE_ODD, 1 << 20, None) == 2      # EUNSUPPORTED
    assert lib.blockffn_workspace_check(FAKE, 4096, None) == 3             # EWORKSPACE
    assert "control block" in bf.blockffn_last_error()
    assert bf.STATUS_NAMES[5] == "ETIMEOUT"


CONTROL_PROBE = r"""
#include <cstdio>
#include "plan.h"
using namespace blockffn;
int main()
{
    static_assert(kDecodeControlWord < kDecodeControlEnd && kDecodeControlEnd <= kStatusWord &&
                  kStatusWord < kControlWords, "control regions in order");
    const long Es[] = {1, 2, 16, 40, 64, 100, 128, 200, 250, 256};
    const long des[] = {16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 65536};
    const long dhs[] = {32, 128, 512, 1024, 2048, 4096, 8192, 16384};
    const long Ts[] = {1, 32};
    long checked = 0, chunk1 = 0;
    for (long E : Es) for (long de : des) for (long dh : dhs) for (long T : Ts) {
        const FfnPlan p = make_plan(T, dh, E, de, 32, 1);
        ++checked;
        if (p.chunk1) {
            ++chunk1;
            // the single-chunk schedule's counters stay below the decode region
            if (chunk1_control_words(E, dh, de) > kDecodeControlWord) {
                std::printf("overlap E=%ld d_e=%ld d_h=%ld\n", E, de, dh);
                return 1;
            }
        }
    }
    std::printf("ok %ld %ld\n", checked, chunk1);
    return 0;
}
"""


def test_control_block_regions_are_disjoint(tmp_path):
    """Every size the single-chunk schedule takes keeps its counters below the decode
    schedule's flags, whose region ends below the status word (plan.h)."""
    import subprocess
    src = tmp_path / "control_probe.hip"
    src.write_text(CONTROL_PROBE)
    exe = tmp_path / "control_probe"
    csrc = os.path.join(ROOT, "chunk_level_activation_amd", "csrc")
    libdir = os.path.dirname(bf.library_path)
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{csrc}",
           str(src), "-o", str(exe), f"-L{libdir}", "-lblockffn", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    checked, chunk1 = map(int, out.stdout.split()[1:3])
    assert checked > 1000 and chunk1 > 0


def full(lib, x=FAKE, w_r=FAKE, w1=FAKE, w2=FAKE, packed=None, T=32, d_h=2048, E=64, d_e=128,
         n=32, dtype=1, ln_eps=1e-5, out=FAKE + 0x100000, sharpness=1.0, probs=None, y=None,
         scores=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.blockffn_layer_forward_full(x, w_r, None, None, 1e-6, w1, w2, packed, T, d_h, E,
                                           d_e, n, dtype, None, None, ln_eps, out, sharpness,
                                           probs, y, scores, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), 1),
    (dict(packed=FAKE), 1),                       # both row-major and packed weights
    (dict(w1=None, w2=None), 1),                  # neither
    (dict(ln_eps=-1.0), 1),
    (dict(ln_eps=float("inf")), 1),
    (dict(probs=FAKE + 0x200000, sharpness=float("nan")), 1),
    (dict(out=FAKE + 8), 2),                      # misaligned out
    (dict(out=FAKE), 1),                          # out is x
    (dict(ws_bytes=1024), 3),
    (dict(T=0), 1),
])
def test_layer_forward_full_rejects(lib, kw, status):
    assert full(lib, **kw) == status


def test_layer_forward_full_workspace_query(lib):
    a = lib.blockffn_layer_forward_full_workspace_bytes(32, 2048, 64, 128, 32, 1)
    b = lib.blockffn_layer_forward_workspace_bytes(32, 2048, 64, 128, 32, 1)
    assert a >= b + 32 * 2048 * 2
    assert lib.blockffn_layer_forward_full_workspace_bytes(0, 2048, 64, 128, 32, 1) == 0
