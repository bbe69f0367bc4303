#!/usr/bin/env python3
"""Benchmark of the BlockFFN layer forward on one MI355X.

One step = the whole layer over one batch: blockffn_layer_forward (the router, then
the chunked expert FFN on the router's scores). Default workload (the decode /
speculative-verification chunk): d_h=2048, E=64 experts, d_e=128, T = n = 32 tokens,
bf16 weights and activations, fp32 accumulation; at this size router and FFN run in
one launch. No trained router is available, so the inputs are drawn to make the
router's activity follow per-expert two-state Markov masks at 80% token-level and 70%
8-token chunk-level sparsity (the sparsity the pages report for trained BlockFFN
models): W_r has orthonormal rows and every token x_t is built so that W_r x_t has the
mask's signs (positive |N(0,1)| + 0.1 where active), plus Gaussian noise orthogonal
to W_r. The router still computes every logit from x each step.

Inputs are resident in HBM before timing starts. Each step uses the next of several
distinct weight copies (>= 512 MiB in all) and the next of 16 mask draws, so the
256 MB Infinity Cache cannot serve a weight set twice in a row.

Prints ONE JSON line (see the keys below). Timing: W eager warm-up steps, then one
replay of a graph of exactly K captured steps between HIP events on the stream the
kernels run on (--steps K, --warmup W). `roofline` is for the dominant kernel: the
one-launch layer kernel at the decode chunk (its duration is the step's), else the
chunk-FFN launches. For one chunk the bound is HBM: algorithmic bytes per call (the
union experts' W1 and W2 slices, W_r when the router is inside, x and y) over its
average duration. For several chunks the weights are shared by the chunks and stay in
the caches, so the bound is the bf16 MFMA rate: the two expert products' flops
(4 d_h d_e per token and union expert of its chunk) over the average duration.

The union sizes behind the byte counts are read from the timed launch's own scores.
`extras` carries the other configurations (prefill, the larger layer's sparsity sweep
and all-active mode, end-to-end, the recommended shapes), the epilogue, loss and
backward kernels, and the rates of plain streaming kernels measured in the same run.
`cpu_baseline` times the CPU oracle on the host's cores and on one thread, in union
and dense mode, and checks the first timed GPU step's output against it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000,
                    help="steps timed: one replay of a graph of exactly this many steps")
    ap.add_argument("--warmup", type=int, default=200, help="eager steps before timing")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "large", "e2e", "rec256", "rec512",
                             "rec256_prefill"])
    ap.add_argument("--rotate-mib", type=int, default=768,
                    help="total size of the distinct weight copies cycled through")
    ap.add_argument("--draws", type=int, default=16)
    ap.add_argument("--rotation-steps", type=int, default=48,
                    help="steps timed (at least) for each of the other configurations")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--cpu-one-thread-seconds", type=float, default=6.0,
                    help="budget of the one-thread oracle run (0 disables it)")
    ap.add_argument("--cpu-oracle-only", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the all-experts-active comparison run")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configurations, epilogue, loss and backward")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a plain "
                         "kernel of known traffic, for scaling hardware byte counters)")
    return ap.parse_args(argv)


def make_inputs(args, torch, np, inputs, workload=None, tls=0.8, cls=0.7, all_active=False,
                rotate_mib=None, ndraws=None):
    """Weight copies, mask draws, and the x of each of the S steps of one captured
    graph (x depends on the copy's W_r and the draw's mask). Markov workloads draw the
    masks at (tls, cls) with 8-token chunks; all_active makes every expert active for
    every token (the dense FFN of equal parameters)."""
    workload = workload or args.workload
    rotate_mib = args.rotate_mib if rotate_mib is None else rotate_mib
    ndraws = args.draws if ndraws is None else ndraws
    cfg = dict(inputs.WORKLOADS[workload])
    T, d_h, E, d_e = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"]
    dev = torch.device("cuda:0")
    bf16 = torch.bfloat16
    markov = workload != "e2e"

    def to_dev(a, dtype=bf16):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev, dtype)

    copy_bytes = 2 * (2 * E * d_e * d_h + E * d_h)
    ncopies = max(2, math.ceil(rotate_mib * 2 ** 20 / copy_bytes))
    copies, w_r_host = [], []
    for i in range(ncopies):
        rng = np.random.default_rng(args.seed * 1000 + 100 + i)
        w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, True)
        if markov:
            w_r = inputs.router_weight_orthonormal(rng, E, d_h, True)
            bias = None
        else:
            w_r = inputs.gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), True)
            bias = to_dev(inputs.router_shift(w_r, 0.8), torch.float32)
        w_r_host.append(w_r)
        copies.append(dict(w1=to_dev(w1), w2=to_dev(w2), w_r=to_dev(w_r), bias=bias))
        del w1, w2
    draws = []
    for i in range(ndraws):
        rng = np.random.default_rng(args.seed * 1000 + 500 + i)
        if markov:
            act = (np.ones((T, E), bool) if all_active
                   else inputs.markov_active(rng, T, E, tls, cls, 8))
        else:
            act = None
        x = None if markov else to_dev(inputs.gaussian(rng, (T, d_h), 1.0, True))
        dense = to_dev((np.abs(rng.standard_normal((T, E))) + 0.1).astype(np.float32),
                       torch.float32)
        draws.append(dict(act=act, x=x, dense=dense))
    nc, nd = len(copies), len(draws)
    S = nc * nd // math.gcd(nc, nd)
    xs = []
    for i in range(S):
        if markov:
            rng = np.random.default_rng(args.seed * 1000 + 900 + i)
            xs.append(to_dev(inputs.tokens_for_mask(rng, w_r_host[i % nc], draws[i % nd]["act"], True)))
        else:
            xs.append(draws[i % nd]["x"])
    return cfg, copies, draws, xs, S


class Timer:
    """HIP-event timing of work enqueued on torch's current stream (the stream every
    library call here launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, enqueue):
        torch = self.torch
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # a short spin first, so the start event is stamped after the host has queued
        # the timed work, not while the host is still submitting it
        torch.cuda._sleep(200000)
        t0.record()
        enqueue()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)


def upload_graph(torch, g):
    """Moves an instantiated graph's launch resources to the device before its first
    replay (hipGraphUpload), so the one timed replay does not pay for that first-use set-up;
    no step runs. Skipped if the runtime call is not reachable."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
    except (OSError, AttributeError, RuntimeError):
        pass


def measure(args, torch, np, bf, inputs, workload, *, steps, warmup, exact=False, tls=0.8,
            cls=0.7, all_active=False, rotate_mib=None, ndraws=None, want_dense=True):
    """Times the layer step of one workload. exact=True: W eager warm-up steps, then
    one replay of a graph of exactly `steps` captured steps between HIP events.
    exact=False: replays of the S-step rotation graph (at least `steps` steps).
    Returns the figures and the state the other measurements reuse."""
    cfg, copies, draws, xs, S = make_inputs(args, torch, np, inputs, workload, tls, cls,
                                            all_active, rotate_mib, ndraws)
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    C = -(-T // n)
    dev = torch.device("cuda:0")
    gain = torch.ones(E, dtype=torch.float32, device=dev)
    y = torch.empty((T, d_h), dtype=torch.bfloat16, device=dev)
    lws = bf.blockffn_layer_forward_workspace(T, d_h, E, d_e, n, bf.BLOCKFFN_BF16, dev)
    ws = bf.blockffn_chunk_ffn_workspace(T, d_h, E, d_e, n, bf.BLOCKFFN_BF16, dev)
    router_ws = bf.blockffn_router_workspace(T, d_h, E, bf.BLOCKFFN_BF16, dev)
    fused = bf.blockffn_layer_forward_fused(T, d_h, E, d_e, n, bf.BLOCKFFN_BF16)
    if fused:
        # the one-launch layer reads the expert weights in the tiled layout; each copy is
        # packed once here, outside every timed region (as when weights are loaded)
        for w in copies:
            w["packed"] = bf.blockffn_pack_weights(w["w1"], w["w2"])
        torch.cuda.synchronize()
    counts = [torch.zeros(C, dtype=torch.int32, device=dev) for _ in range(S)]
    scores = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in range(S)]
    nc, nd = len(copies), len(draws)
    timer = Timer(torch)

    # step i uses weight copy i % nc and the x drawn for step i % S (S = lcm of the two
    # rotation lengths, so every replay of an S-step graph walks the same sequence)
    def step(i, sc=None):
        w, k = copies[i % nc], i % S
        if fused:
            bf.blockffn_layer_forward_packed(xs[k], w["w_r"], w["packed"], E, d_e, n, gain=gain,
                                             bias=w["bias"], y=y, scores=sc, workspace=lws)
        else:
            bf.blockffn_layer_forward(xs[k], w["w_r"], w["w1"], w["w2"], n, gain=gain,
                                      bias=w["bias"], y=y, scores=sc, workspace=lws)

    def step_rowmajor(i):
        w, k = copies[i % nc], i % S
        bf.blockffn_layer_forward(xs[k], w["w_r"], w["w1"], w["w2"], n, gain=gain, bias=w["bias"],
                                  y=y, workspace=lws)

    def router(i):
        w, k = copies[i % nc], i % S
        bf.blockffn_router(xs[k], w["w_r"], gain, w["bias"], scores=scores[k], workspace=router_ws)

    def ffn(i, dense=False):
        w, k = copies[i % nc], i % S
        s = draws[i % nd]["dense"] if dense else scores[k]
        bf.blockffn_chunk_ffn(xs[k], s, w["w1"], w["w2"], n, y=y, workspace=ws,
                              union_counts=counts[k])

    def capture(body, count=S):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                body(i)
        return g

    replays = max(1, math.ceil(steps / S))

    def rotation_ms(g):
        """Average step time over replays of an S-step graph (one warm replay first): the
        median of three timed samples, so that one stall of the box does not become the
        line."""
        timer(g.replay)
        samples = [timer(lambda: [g.replay() for _ in range(replays)]) / (replays * S)
                   for _ in range(3)]
        return float(np.median(samples))

    # eager warm-up (loads the code objects); the router's scores of every step, for
    # the FFN-alone timing and the realised unions
    for i in range(max(1, warmup)):
        step(i)
    for i in range(S):
        router(i)
    torch.cuda.synchronize()
    res = {"cfg": cfg, "fused": bool(fused), "S": S, "copies": nc,
           "rotation_mib": round(nc * 2 * (2 * E * d_e * d_h + E * d_h) / 2 ** 20)}
    if exact:
        g_k = capture(step, steps)
        upload_graph(torch, g_k)
        res["ms_per_step"] = timer(g_k.replay) / steps
        res["steps"] = steps
        del g_k
        g_step = capture(step)
        res["ms_per_step_rotation"] = rotation_ms(g_step)
        res["rotation_steps_timed"] = replays * S
    else:
        g_step = capture(step)
        res["ms_per_step"] = rotation_ms(g_step)
        res["steps"] = replays * S
    del g_step
    # the chunk-FFN calls alone on the router's scores, same rotation
    g_ffn = capture(ffn)
    res["ffn_ms"] = rotation_ms(g_ffn)
    del g_ffn

    # Realised unions of the timed kernel: from the one-launch layer's own scores when
    # fused, else from the chunk FFN's union counts (the FFN-alone graph wrote them).
    if fused:
        unions = []
        for i in range(S):
            sc = torch.empty((T, E), dtype=torch.float32, device=dev)
            step(i, sc)
            s = sc.cpu().numpy()
            unions.append(float(sum(int((s[c * n:(c + 1) * n] != 0).any(axis=0).sum())
                                    for c in range(C))))
        union_experts = float(np.mean(unions))
    else:
        cnt = np.stack([c.cpu().numpy() for c in counts])            # [S, C]
        union_experts = float(cnt.sum(axis=1).mean())
    res["union_experts_per_step"] = union_experts
    weight_bytes = union_experts * 2 * d_h * d_e * 2                   # W1 + W2, bf16
    act_bytes = T * d_h * 2 + T * d_h * 2                              # x, y
    res["kernel_bytes"] = weight_bytes + act_bytes + (E * d_h * 2 if fused else T * E * 4)
    res["kernel_ms"] = res["ms_per_step"] if fused else res["ffn_ms"]
    res["flops"] = union_experts * min(n, T) * 4 * d_h * d_e + (2 * T * E * d_h if fused else 0)
    res["ffn_flops"] = union_experts * min(n, T) * 4 * d_h * d_e
    if want_dense and workload != "e2e":
        g_dense = capture(lambda i: ffn(i, dense=True))
        res["dense_ffn_ms"] = rotation_ms(g_dense)
        del g_dense
    res["state"] = dict(copies=copies, xs=xs, S=S, gain=gain, y=y, lws=lws, step=step,
                        step_rowmajor=step_rowmajor, router=router, ffn=ffn, capture=capture,
                        rotation_ms=rotation_ms, replays=replays, timer=timer)
    return res


def roofline_of(res, traffic):
    """The roofline object of the dominant kernel (see the module docstring)."""
    cfg = res["cfg"]
    C = -(-cfg["T"] // cfg["n"])
    ms = res["kernel_ms"]
    if res["fused"]:
        name = ("layer forward, router and chunk FFN in one launch, tiled weights "
                "(blockffn_layer_forward_packed)")
        timing = "HIP events around graph replays of the steps (one launch each)"
    else:
        name = "chunk FFN (blockffn_chunk_ffn)"
        timing = ("HIP events around graph replays of the chunk-FFN calls alone (same "
                  "rotation), divided by the number of calls")
    gbs = res["kernel_bytes"] / (ms * 1e-3) / 1e9
    if C == 1:
        # one chunk: the weight stream (each union expert's W1 and W2 read once) bounds it
        return {"kernel": name, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": res["kernel_bytes"], "avg_launch_ms": ms,
                "launch_timing": timing,
                "mfma_frac": res["flops"] / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)}
    # many chunks: every chunk's union experts are multiplied with its 32 tokens while the
    # weights, shared by the chunks, stay in the caches; the products bound it
    tflops = res["ffn_flops"] / (ms * 1e-3) / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS, "traffic": traffic,
            "algorithmic_flops_per_launch": res["ffn_flops"], "avg_launch_ms": ms,
            "launch_timing": timing, "effective_gbs_of_chunk_unions": gbs}


def summary_of(res, label):
    """A compact record of one workload measurement, for the extras."""
    cfg = res["cfg"]
    T = cfg["T"]
    rf = roofline_of(res, None)
    out = {"workload": label, "ms_per_step": res["ms_per_step"],
           "tokens_per_s": T / (res["ms_per_step"] * 1e-3), "fused": res["fused"],
           "chunk_ffn_ms": res["ffn_ms"], "union_experts_per_step": res["union_experts_per_step"],
           "roofline": {k: rf[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac")},
           "steps_timed": res["steps"], "rotation_mib": res["rotation_mib"]}
    if rf["bound"] == "hbm":
        out["roofline"]["mfma_frac"] = rf["mfma_frac"]
    else:
        out["roofline"]["effective_gbs_of_chunk_unions"] = rf["effective_gbs_of_chunk_unions"]
    if "dense_ffn_ms" in res:
        out["dense_ffn_ms"] = res["dense_ffn_ms"]
        out["dense_over_sparse_ffn"] = res["dense_ffn_ms"] / res["ffn_ms"]
    return out


def stream_reference(torch):
    """Measured HBM rates of plain streaming kernels in the same run, as a practical
    ceiling beside the published peak: torch's sum over 1 GiB of fp32 (reads only) and
    torch's copy of 1 GiB (read + write), each alternating two buffers (2 GiB in all,
    beyond the 256 MB Infinity Cache), eager launches between HIP events."""
    n = 2 ** 28
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(2)]
    dst = torch.empty_like(bufs[0])
    timer = Timer(torch)
    reps = 8
    for b in bufs:
        b.sum()
        dst.copy_(b)
    read_ms = timer(lambda: [bufs[i % 2].sum() for i in range(reps)]) / reps
    copy_ms = timer(lambda: [dst.copy_(bufs[i % 2]) for i in range(reps)]) / reps
    del bufs, dst
    torch.cuda.empty_cache()
    nb = 4 * n
    return {"read_gbs": nb / (read_ms * 1e-3) / 1e9, "read_kernel": "torch.sum, 1 GiB fp32",
            "copy_gbs": 2 * nb / (copy_ms * 1e-3) / 1e9,
            "copy_kernel": "torch copy_, 1 GiB fp32 (bytes read + written)"}


def main(argv=None):
    args = parse_args(argv)
    if args.cpu_oracle_only:
        # child process of the CPU baseline (its thread count set in its environment)
        import numpy as np
        from chunk_level_activation_amd import inputs
        cfg = dict(inputs.WORKLOADS[args.workload])
        print(json.dumps(cpu_oracle_rate(args, cfg, np, inputs)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the layer is measured on one MI355X; see DESIGN.md for how it would "
              "shard).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import chunk_level_activation_amd as bf
    from chunk_level_activation_amd import inputs

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        src = torch.ones(args.calibrate_copy_mib * 2 ** 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = measure(args, torch, np, bf, inputs, args.workload, steps=args.steps,
                  warmup=args.warmup, exact=True, want_dense=not args.no_dense)
    cfg, st = res["cfg"], res["state"]
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    fused = res["fused"]
    ms_per_step = res["ms_per_step"]
    tokens_per_s = T / (ms_per_step * 1e-3)

    # the row-major one-launch layer, the unfused pair, the all-active layer step
    extras = {}
    capture, rotation_ms = st["capture"], st["rotation_ms"]
    g_sep = capture(lambda i: (st["router"](i), st["ffn"](i)))
    sep_ms = rotation_ms(g_sep)
    del g_sep
    extras["unfused_layer"] = {
        "what": "blockffn_router + blockffn_chunk_ffn as two launches, same inputs",
        "ms_per_step": sep_ms, "tokens_per_s": T / (sep_ms * 1e-3), "chunk_ffn_ms": res["ffn_ms"]}
    if fused:
        g_rm = capture(st["step_rowmajor"])
        rm_ms = rotation_ms(g_rm)
        del g_rm
        extras["layer_rowmajor_weights"] = {
            "what": "blockffn_layer_forward (one launch) on the row-major W1 and W2",
            "ms_per_step": rm_ms, "tokens_per_s": T / (rm_ms * 1e-3)}

    # Python-launched steps, for comparison (host-bound at these sizes)
    eager_n = min(200, max(1, args.steps))
    torch.cuda.synchronize()
    te = time.perf_counter()
    for i in range(eager_n):
        st["step"](i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te) * 1e3 / eager_n

    # one timed step's output, kept for the CPU baseline leg's check against the oracle
    w0 = st["copies"][0]
    sc0 = torch.empty((T, E), dtype=torch.float32, device="cuda:0")
    st["step"](0, sc0)
    torch.cuda.synchronize()
    gpu_step0 = {"x": st["xs"][0].float().cpu().numpy(), "w_r": w0["w_r"].float().cpu().numpy(),
                 "w1": w0["w1"].float().cpu().numpy(), "w2": w0["w2"].float().cpu().numpy(),
                 "bias": None if w0["bias"] is None else w0["bias"].cpu().numpy(),
                 "y": st["y"].float().cpu().numpy(), "scores": sc0.cpu().numpy()}

    dense = None
    if "dense_ffn_ms" in res:
        dense = {"ffn_ms": res["dense_ffn_ms"],
                 "ratio_dense_over_sparse": res["dense_ffn_ms"] / res["ffn_ms"],
                 "what": "all-active scores through the same chunk-FFN kernels, same rotation"}

    if not args.no_extras:
        timer = st["timer"]

        def time_replays(g, r):
            return timer(lambda: [g.replay() for _ in range(r)])

        extras.update(bench_extras(args, torch, np, bf, inputs, cfg, st["copies"], st["xs"],
                                   st["S"], st["gain"], st["y"], st["lws"], st["replays"],
                                   1, time_replays, capture))
    del st, res["state"]
    torch.cuda.empty_cache()
    if not args.no_extras and args.workload == "decode":
        if fused and dense is not None:
            # the headline launch itself with every expert active (union = E)
            r = measure(args, torch, np, bf, inputs, "decode", steps=args.rotation_steps,
                        warmup=2, all_active=True, want_dense=False)
            dense["layer_all_active_ms"] = r["ms_per_step"]
            dense["layer_ratio_dense_over_sparse"] = r["ms_per_step"] / ms_per_step
            del r
        extras["workloads"] = bench_workloads(args, torch, np, bf, inputs)
        extras["stream_reference"] = stream_reference(torch)
        rf_gbs = res["kernel_bytes"] / (res["kernel_ms"] * 1e-3) / 1e9
        extras["stream_reference"]["headline_frac_of_read"] = (
            rf_gbs / extras["stream_reference"]["read_gbs"])

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args, cfg, np, inputs, gpu_step0)

    roofline = roofline_of(res, read_traffic(args.workload, fused))
    activity = ("router activity following Markov masks at 80% TLS / 70% 8-token CLS "
                "(orthonormal W_r, x drawn for the masks)" if args.workload != "e2e" else
                "router with a logit shift for ~80% zeros, i.i.d. x")
    out = {
        "metric": "tokens/s + effective HBM GB/s (% of peak) of BlockFFN layer, n=32 chunks",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: d_h={d_h} E={E} d_e={d_e} T={T} n={n} bf16, "
                        f"{activity}; router + chunk FFN per step"
                        + (" in one launch" if fused else ""),
            "global_batch": T, "seq_len": n, "parallelism": "none (1 GPU)",
            "weight_copies": res["copies"], "rotation_mib": res["rotation_mib"],
            "union_experts_per_step": res["union_experts_per_step"],
            "timing": (f"{args.warmup} eager warm-up steps, then one replay of a graph of "
                       f"exactly {res['steps']} captured steps (uploaded to the device "
                       f"first, not run) between HIP events (the gap of a few us between the "
                       f"start event and the first step is inside the timed region); replays "
                       f"of the {res['S']}-step rotation graph ({res['rotation_steps_timed']} "
                       f"steps): {res['ms_per_step_rotation']:.5f} ms/step; eager "
                       f"Python-launched step {eager_ms:.4f} ms"),
        },
        "roofline": roofline,
        "dense_ffn": dense,
        "extras": extras or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if cpu is not None and not cpu["parity_vs_gpu"]["ok"]:
        print("bench.py: the GPU step checked against the oracle is outside the tolerance",
              file=sys.stderr)
        return 3
    return 0


def bench_workloads(args, torch, np, bf, inputs):
    """The other configurations, each timed over graph replays of its weight and draw
    rotation (>= 512 MiB of distinct weights): prefill (T=2048), the larger layer
    (d_h=4096, E=128, T=512) at TLS/CLS_8 50/30, 80/70, 90/85 and all-active, the
    end-to-end router + FFN (T=4096, i.i.d. tokens), and the recommended shapes."""
    out = {}
    plan = [("prefill", "prefill", {}),
            ("large_50_30", "large", dict(tls=0.5, cls=0.3)),
            ("large_80_70", "large", dict(tls=0.8, cls=0.7)),
            ("large_90_85", "large", dict(tls=0.9, cls=0.85)),
            ("large_all_active", "large", dict(all_active=True, want_dense=False)),
            ("e2e", "e2e", {}),
            ("rec256", "rec256", {}), ("rec512", "rec512", {}),
            ("rec256_prefill", "rec256_prefill", {})]
    for label, wl, kw in plan:
        kw = dict(kw)
        r = measure(args, torch, np, bf, inputs, wl, steps=args.rotation_steps, warmup=2,
                    rotate_mib=512, ndraws=4, **kw)
        out[label] = summary_of(r, label)
        del r
        torch.cuda.empty_cache()
    return out


def bench_extras(args, torch, np, bf, inputs, cfg, copies, xs, S, gain, y, lws, replays,
                 wreplays, time_replays, capture):
    """The rest of the pages' layer around the hot path, measured the same way:
    (1) the layer step with its residual + LayerNorm epilogue over the same rotation;
    (2) the LayerNorm alone and (3) the sparsity losses with their gradient alone, each
    over rotating input copies of at least 512 MiB; (4) the layer backward; all timed
    with HIP events around graph replays."""
    T, d_h, E, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["n"]
    dev = torch.device("cuda:0")
    nc = len(copies)
    ln_g = torch.ones(d_h, dtype=torch.float32, device=dev)
    ln_b = torch.zeros(d_h, dtype=torch.float32, device=dev)
    out = torch.empty((T, d_h), dtype=torch.bfloat16, device=dev)

    probs = torch.empty((T, E), dtype=torch.float32, device=dev)
    fws = bf.blockffn_layer_forward_full_workspace(T, d_h, E, cfg["d_e"], n, bf.BLOCKFFN_BF16, dev)

    def layer_full(i):
        w, k = copies[i % nc], i % S
        wk = (dict(packed=w["packed"], E=E, d_e=cfg["d_e"]) if "packed" in w else
              dict(w1=w["w1"], w2=w["w2"]))
        bf.blockffn_layer_forward_full(xs[k], w["w_r"], n, gain=gain, bias=w["bias"],
                                       ln_gamma=ln_g, ln_beta=ln_b, out=out, probs=probs,
                                       sharpness=2.0, workspace=fws, **wk)

    def layer_then_ln(i):
        w, k = copies[i % nc], i % S
        if "packed" in w:
            bf.blockffn_layer_forward_packed(xs[k], w["w_r"], w["packed"], E, cfg["d_e"], n,
                                             gain=gain, bias=w["bias"], y=y, workspace=lws)
        else:
            bf.blockffn_layer_forward(xs[k], w["w_r"], w["w1"], w["w2"], n, gain=gain,
                                      bias=w["bias"], y=y, workspace=lws)
        bf.blockffn_add_layernorm(y, xs[k], ln_g, ln_b, out=out)

    res = {}
    for name, body, what in (
            ("layer_with_epilogue", layer_full,
             "blockffn_layer_forward_full: the layer step (as the headline) with the residual "
             "LayerNorm and the router probabilities, fused into the one launch at the decode "
             "chunk; same rotation as the headline step"),
            ("layer_then_add_layernorm", layer_then_ln,
             "the headline layer step followed by blockffn_add_layernorm (two launches)")):
        g = capture(body)
        time_replays(g, wreplays)
        ms = time_replays(g, replays) / (replays * S)
        del g
        res[name] = {"what": what, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3)}

    def rotating_ms(make, launch, bytes_per_set, launches=256):
        """Average duration of one launch over rotating input sets (>= 512 MiB)."""
        sets = max(2, math.ceil(512 * 2 ** 20 / bytes_per_set))
        data = [make(k) for k in range(sets)]
        launch(data[0])
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for k in range(launches):
                launch(data[k % sets])
        time_replays(gr, 2)
        ms = time_replays(gr, 10) / (10 * launches)
        del gr, data
        torch.cuda.empty_cache()
        return ms, sets

    # residual + LayerNorm at the end-to-end token count
    T_ln = 4096
    ln_bytes = 3 * T_ln * d_h * 2 + 2 * d_h * 4

    def make_ln(k):
        r = np.random.default_rng(1000 + k)
        yk = torch.from_numpy(inputs.gaussian(r, (T_ln, d_h), 1.0, True)).to(dev, torch.bfloat16)
        xk = torch.from_numpy(inputs.gaussian(r, (T_ln, d_h), 1.0, True)).to(dev, torch.bfloat16)
        return yk, xk, torch.empty_like(xk)

    ln_ms, ln_sets = rotating_ms(make_ln, lambda a: bf.blockffn_add_layernorm(
        a[0], a[1], ln_g, ln_b, out=a[2]), ln_bytes)
    res["add_layernorm"] = {
        "shape": f"T={T_ln} d_h={d_h} bf16", "avg_launch_us": ln_ms * 1e3,
        "algorithmic_bytes": ln_bytes, "achieved_gbs": ln_bytes / (ln_ms * 1e-3) / 1e9,
        "frac_of_hbm_peak": ln_bytes / (ln_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "rotation_sets": ln_sets}

    # sparsity losses + gradient: one 4096-token sequence and a 16 x 4096 batch
    for B in (1, 16):
        S_l, L = 4096, 8
        l_bytes = 2 * B * S_l * E * 4
        lws = bf.blockffn_sparsity_losses_workspace(B, S_l, E, L, dev)
        lout = torch.empty(2, dtype=torch.float32, device=dev)

        def make_l(k, B=B, S_l=S_l):
            p = torch.from_numpy(inputs.activation_probs(2000 + k, B, S_l, E)).to(dev)
            return p, torch.empty_like(p)

        l_ms, l_sets = rotating_ms(make_l, lambda a, lws=lws, lout=lout:
                                   bf.blockffn_sparsity_losses(a[0], 2.0, L, 0.1, 0.1,
                                                               losses=lout, grad=a[1],
                                                               workspace=lws), l_bytes)
        res[f"sparsity_losses_B{B}"] = {
            "shape": f"probs [{B}, {S_l}, {E}] fp32, L={L}, alpha=2, forward + gradient",
            "avg_launch_us": l_ms * 1e3, "algorithmic_bytes": l_bytes,
            "achieved_gbs": l_bytes / (l_ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": l_bytes / (l_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "rotation_sets": l_sets}
    res.update(bench_backward(args, torch, np, bf, inputs, cfg, copies, xs, S, gain,
                              time_replays))
    return res


def bench_backward(args, torch, np, bf, inputs, cfg, copies, xs, S_all, gain, time_replays):
    """The layer backward (router recomputed, expert pass, weight gradients, dx, router
    backward) at the workload's size over the same rotation, and at 2048 tokens. The
    roofline figures: flops of the five expert products per (chunk, union expert)
    plus the router's two, and the bytes of the unique weights read, x and dy read,
    and dx, dW_r, dW1, dW2 written (fp32)."""
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    dev = torch.device("cuda:0")
    nc = len(copies)
    f32 = torch.float32
    res = {}

    def outputs(Tb):
        return dict(dx=torch.empty((Tb, d_h), dtype=f32, device=dev),
                    dw_r=torch.empty((E, d_h), dtype=f32, device=dev),
                    dw1=torch.empty((E, d_e, d_h), dtype=f32, device=dev),
                    dw2=torch.empty((E, d_h, d_e), dtype=f32, device=dev),
                    dgain=torch.empty(E, dtype=f32, device=dev),
                    dbias=torch.empty(E, dtype=f32, device=dev))

    def figures(Tb, union_sum, used_experts, ms):
        flops = union_sum * 10.0 * d_h * d_e * min(n, Tb) + 4.0 * Tb * E * d_h
        nbytes = (used_experts * 2 * d_h * d_e * 2 + 2 * Tb * d_h * 2 + Tb * d_h * 4 +
                  E * d_h * 4 + 2 * E * d_e * d_h * 4)
        return {"avg_launch_us": ms * 1e3, "algorithmic_flops": flops,
                "algorithmic_bytes": nbytes,
                "achieved_tflops": flops / (ms * 1e-3) / 1e12,
                "mfma_frac": flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                "achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
                "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    # (1) the workload's own size, rotating weight copies and draws (dy = another draw)
    bws = torch.empty(bf.blockffn_layer_backward_workspace_bytes(T, d_h, E, d_e, n),
                      dtype=torch.uint8, device=dev)
    out = outputs(T)

    def bwd(i):
        w = copies[i % nc]
        bf.blockffn_layer_backward(xs[i % S_all], w["w_r"], w["w1"], w["w2"], xs[(i + 1) % S_all],
                                   n, gain=gain, bias=w["bias"], out=out, workspace=bws)

    S = 16
    for i in range(2):
        bwd(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            bwd(i)
    time_replays(g, 2)
    ms = time_replays(g, 10) / (10 * S)
    del g
    # unions of the router's scores: the backward recomputes them; count from a forward
    sc = torch.empty((T, E), dtype=f32, device=dev)
    cnt = torch.zeros(-(-T // n), dtype=torch.int32, device=dev)
    lists = torch.empty((-(-T // n), E), dtype=torch.int32, device=dev)
    union_sum, used = 0.0, 0.0
    y = torch.empty((T, d_h), dtype=torch.bfloat16, device=dev)
    for i in range(S):
        w = copies[i % nc]
        bf.blockffn_router(xs[i % S_all], w["w_r"], gain, w["bias"], scores=sc)
        bf.blockffn_chunk_ffn(xs[i % S_all], sc, w["w1"], w["w2"], n, y=y, union_counts=cnt,
                              expert_lists=lists)
        c = cnt.cpu().numpy()
        union_sum += float(c.sum())
        used += float(len(set(lists.cpu().numpy()[lists.cpu().numpy() >= 0].tolist())))
    res["layer_backward"] = dict(
        shape=f"T={T} d_h={d_h} E={E} d_e={d_e} n={n} bf16, the workload's router inputs, "
              f"fp32 gradients", **figures(T, union_sum / S, used / S, ms))

    # (2) 2048 tokens on two weight copies
    Tp = 2048
    rng = np.random.default_rng(77)

    def tokens(ci):
        w = copies[ci]
        if w["bias"] is not None:          # the logit-shift router: i.i.d. tokens
            return inputs.gaussian(rng, (Tp, d_h), 1.0, True)
        act = inputs.markov_active(rng, Tp, E, 0.8, 0.7, 8)
        return inputs.tokens_for_mask(rng, w["w_r"].float().cpu().numpy(), act, True)

    xs = [torch.from_numpy(tokens(ci)).to(dev, torch.bfloat16) for ci in range(2)]
    dys = [torch.from_numpy(inputs.gaussian(rng, (Tp, d_h), 1.0, True)).to(dev, torch.bfloat16)
           for _ in range(2)]
    bws = torch.empty(bf.blockffn_layer_backward_workspace_bytes(Tp, d_h, E, d_e, n),
                      dtype=torch.uint8, device=dev)
    outp = outputs(Tp)

    def bwdp(i):
        w = copies[i % 2]
        bf.blockffn_layer_backward(xs[i % 2], w["w_r"], w["w1"], w["w2"], dys[i % 2], n,
                                   gain=gain, bias=w["bias"], out=outp, workspace=bws)

    for i in range(2):
        bwdp(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(4):
            bwdp(i)
    time_replays(g, 2)
    ms = time_replays(g, 5) / (5 * 4)
    del g
    scp = torch.empty((Tp, E), dtype=f32, device=dev)
    Cp = -(-Tp // n)
    cntp = torch.zeros(Cp, dtype=torch.int32, device=dev)
    listp = torch.empty((Cp, E), dtype=torch.int32, device=dev)
    yp = torch.empty((Tp, d_h), dtype=torch.bfloat16, device=dev)
    usum, used = 0.0, 0.0
    for i in range(2):
        w = copies[i]
        bf.blockffn_router(xs[i], w["w_r"], gain, w["bias"], scores=scp)
        bf.blockffn_chunk_ffn(xs[i], scp, w["w1"], w["w2"], n, y=yp, union_counts=cntp,
                              expert_lists=listp)
        usum += float(cntp.cpu().numpy().sum())
        lp = listp.cpu().numpy()
        used += float(len(set(lp[lp >= 0].tolist())))
    res["layer_backward_T2048"] = dict(
        shape=f"T={Tp} d_h={d_h} E={E} d_e={d_e} n={n} bf16, router inputs as the "
              f"workload's, fp32 gradients",
        **figures(Tp, usum / 2, used / 2, ms))
    return res


def read_traffic(workload, fused):
    """HBM bytes per launch of the roofline kernel (the one-launch layer when fused,
    else the chunk FFN) from the committed rocprofv3 counter summary, if it was taken
    on the current source of that kernel (the files its `kernel_sources` line names);
    else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{'layer' if fused else 'ffn'}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = os.path.join(ROOT, "chunk_level_activation_amd", "csrc")
    names = kv.get("kernel_sources", "").split()
    if not names or not all(os.path.exists(os.path.join(src, fn)) for fn in names):
        return None
    h = hashlib.sha256()
    for fn in names:
        h.update(open(os.path.join(src, fn), "rb").read())
    if kv.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_oracle_rate(args, cfg, np, inputs, seconds=None):
    """The CPU oracle, as it stands, on a bounded sample of the workload: whole steps
    (router + chunk FFN) on inputs drawn before the clock starts, until the time budget
    is spent; then the chunk FFN alone in dense mode (every expert active, the dense FFN
    of equal parameters) for the CPU's dense/sparse ratio."""
    import oracle
    seconds = args.cpu_seconds if seconds is None else seconds
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    markov = args.workload != "e2e"
    rng = np.random.default_rng(args.seed * 1000 + 100)
    w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, True)
    if markov:
        w_r = inputs.router_weight_orthonormal(rng, E, d_h, True)
        bias = None
    else:
        w_r = inputs.gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), True)
        bias = inputs.router_shift(w_r, 0.8)
    # bounded token sample: at most 4 chunks per oracle step for the large workloads
    Ts = min(T, 4 * n)
    xs = []
    for k in range(8):
        r = np.random.default_rng(args.seed * 1000 + 500 + k)
        if markov:
            xs.append(inputs.tokens_for_mask(r, w_r, inputs.markov_active(r, Ts, E, 0.8, 0.7, 8),
                                             True))
        else:
            xs.append(inputs.gaussian(r, (Ts, d_h), 1.0, True))
    dense = (np.abs(np.random.default_rng(args.seed + 11).standard_normal((Ts, E))) + 0.1
             ).astype(np.float32)
    steps, ffn_s = 0, 0.0
    t0 = time.perf_counter()
    while True:
        x = xs[steps % len(xs)]
        _, s = oracle.router(x, w_r, bias=bias)
        t1 = time.perf_counter()
        oracle.chunk_ffn(x, s.astype(np.float32), w1, w2, n)
        ffn_s += time.perf_counter() - t1
        steps += 1
        el = time.perf_counter() - t0
        if el >= 0.7 * seconds or steps >= 10000:
            break
    dsteps, td = 0, time.perf_counter()
    while True:
        oracle.chunk_ffn(xs[dsteps % len(xs)], dense, w1, w2, n)
        dsteps += 1
        dl = time.perf_counter() - td
        if dl >= 0.3 * seconds or dsteps >= 10000:
            break
    return {"tokens_per_s": steps * Ts / el, "cores": oracle.num_threads(), "steps": steps,
            "tokens_per_step": Ts, "seconds": el,
            "ffn_ms_per_step": 1e3 * ffn_s / steps, "dense_ffn_ms_per_step": 1e3 * dl / dsteps,
            "dense_over_sparse_ffn": (dl / dsteps) / (ffn_s / steps)}


def cpu_baseline(args, cfg, np, inputs, gpu_step):
    """The oracle timed on the host's cores (and on one thread, in a child process,
    since OpenMP fixes its thread count when the library loads), plus the check of
    one timed GPU step's output against the oracle on the same inputs (not timed)."""
    import subprocess

    import oracle
    T, n = cfg["T"], cfg["n"]
    main_rate = cpu_oracle_rate(args, cfg, np, inputs)
    one = None
    if args.cpu_one_thread_seconds > 0:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        cmd = [sys.executable, os.path.abspath(__file__), "--cpu-oracle-only", "--workload",
               args.workload, "--seed", str(args.seed), "--cpu-seconds",
               str(args.cpu_one_thread_seconds)]
        try:
            p = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600)
            one = json.loads(p.stdout.strip().splitlines()[-1])
        except (subprocess.SubprocessError, ValueError, IndexError) as e:
            one = {"error": repr(e)}
    # the GPU's step 0 (same inputs the timed graph's first step used) against the oracle
    g = gpu_step
    logits, s_ref = oracle.router(g["x"], g["w_r"], bias=g["bias"])
    if T <= 256:
        rows = np.arange(T)
        y_ref = oracle.chunk_ffn(g["x"], s_ref.astype(np.float32), g["w1"], g["w2"], n)
    else:
        r = np.random.default_rng(5)
        rows = np.unique(np.concatenate([np.arange(n), np.arange(T - n, T),
                                         r.choice(T, 64, replace=False)]))
        y_ref = oracle.token_ffn(g["x"][rows], s_ref[rows].astype(np.float32), g["w1"], g["w2"])
    err = float(np.abs(g["y"][rows] - y_ref).max() / np.abs(y_ref).max())
    decided = bool(np.abs(logits).min() >= 1e-3)
    union_equal = None
    if decided:
        u_gpu = oracle.chunk_union(g["scores"], n)
        u_ref = oracle.chunk_union(s_ref.astype(np.float32), n)
        union_equal = all(np.array_equal(a, b) for a, b in zip(u_gpu, u_ref))
    ok = err <= 1e-2 and union_equal is not False
    return {"value": main_rate["tokens_per_s"], "unit": "tokens/s", "cores": main_rate["cores"],
            "kind": "oracle",
            "sample": f"{main_rate['steps']} oracle steps (router + chunk FFN, fp64 loops) of "
                      f"{main_rate['tokens_per_step']} tokens each on pre-drawn inputs, "
                      f"{main_rate['seconds']:.1f} s; inputs drawn outside the clock",
            "ffn_ms_per_step": main_rate["ffn_ms_per_step"],
            "dense_ffn_ms_per_step": main_rate["dense_ffn_ms_per_step"],
            "dense_over_sparse_ffn": main_rate["dense_over_sparse_ffn"],
            "one_thread": one,
            "parity_vs_gpu": {"what": "the timed graph's first step (same inputs) against "
                                      "the oracle's router + chunk FFN",
                              "rows_checked": int(len(rows)), "y_max_rel_err": err,
                              "tol": 1e-2, "union_equal": union_equal, "ok": bool(ok)}}


if __name__ == "__main__":
    sys.exit(main())
