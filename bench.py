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

Prints ONE JSON line (see the keys below). `roofline` is for the dominant kernel: the
one-launch layer kernel at the decode chunk (its duration is the step's), else the
chunk-FFN launches. For one chunk the bound is HBM: algorithmic bytes per call (the
union experts' W1 and W2 slices, W_r when the router is inside, x and y) over its
average duration. For several chunks the weights are shared by the chunks and stay in
the caches, so the bound is the bf16 MFMA rate: the five expert products' flops of
every (chunk, union expert) pair over the average duration. Durations are measured
with HIP events around graph replays on the stream the kernels run on.
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
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "large", "e2e", "rec256", "rec512",
                             "rec256_prefill"])
    ap.add_argument("--rotate-mib", type=int, default=768,
                    help="total size of the distinct weight copies cycled through")
    ap.add_argument("--draws", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the all-experts-active comparison run")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the epilogue / loss kernel measurements")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a plain "
                         "kernel of known traffic, for scaling hardware byte counters)")
    return ap.parse_args(argv)


def make_inputs(args, torch, np, inputs):
    """Weight copies, mask draws, and the x of each of the S steps of one captured
    graph (x depends on the copy's W_r and the draw's mask)."""
    cfg = dict(inputs.WORKLOADS[args.workload])
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    dev = torch.device("cuda:0")
    bf16 = torch.bfloat16
    markov = args.workload != "e2e"

    def to_dev(a, dtype=bf16):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev, dtype)

    copy_bytes = 2 * (2 * E * d_e * d_h + E * d_h)
    ncopies = max(2, math.ceil(args.rotate_mib * 2 ** 20 / copy_bytes))
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
    for i in range(args.draws):
        rng = np.random.default_rng(args.seed * 1000 + 500 + i)
        act = inputs.markov_active(rng, T, E, 0.8, 0.7, 8) if markov else None
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


def main(argv=None):
    args = parse_args(argv)
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
    cfg, copies, draws, xs, S = make_inputs(args, torch, np, inputs)
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

    # step i uses weight copy i % nc and the x drawn for step i % S (S = lcm of the two
    # rotation lengths, so every replay of an S-step graph walks the same sequence)
    def step(i):
        w, k = copies[i % nc], i % S
        if fused:
            bf.blockffn_layer_forward_packed(xs[k], w["w_r"], w["packed"], E, d_e, n, gain=gain,
                                             bias=w["bias"], y=y, workspace=lws)
        else:
            bf.blockffn_layer_forward(xs[k], w["w_r"], w["w1"], w["w2"], n, gain=gain,
                                      bias=w["bias"], y=y, workspace=lws)

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

    def capture(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(S):
                body(i)
        return g

    def time_replays(g, replays):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(replays):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    # eager warm-up (loads the code objects); the router's scores of every step, for
    # the FFN-alone timing and the realised unions
    for i in range(min(args.warmup, 2 * S)):
        step(i)
    for i in range(S):
        router(i)
    torch.cuda.synchronize()
    g_step = capture(step)
    g_ffn = capture(ffn)
    replays = max(1, math.ceil(args.steps / S))
    wreplays = max(1, math.ceil(args.warmup / S))
    for _ in range(wreplays):
        g_step.replay()
    total_ms = time_replays(g_step, replays)
    nsteps = replays * S
    ms_per_step = total_ms / nsteps
    # the chunk-FFN calls alone on the router's scores, same rotation
    time_replays(g_ffn, wreplays)
    ffn_avg_ms = time_replays(g_ffn, replays) / nsteps
    # the router and the chunk FFN as separate launches (the unfused layer)
    g_sep = capture(lambda i: (router(i), ffn(i)))
    time_replays(g_sep, wreplays)
    sep_ms = time_replays(g_sep, replays) / nsteps
    del g_sep
    # the one-launch layer on the row-major weights
    rowmajor_ms = None
    if fused:
        g_rm = capture(step_rowmajor)
        time_replays(g_rm, wreplays)
        rowmajor_ms = time_replays(g_rm, replays) / nsteps
        del g_rm

    # Python-launched steps, for comparison (host-bound at these sizes)
    eager_n = min(200, nsteps)
    torch.cuda.synchronize()
    te = time.perf_counter()
    for i in range(eager_n):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te) * 1e3 / eager_n

    # Realised unions (the FFN-alone graph wrote them).
    cnt = np.stack([c.cpu().numpy() for c in counts])            # [S, C]
    union_experts = float(cnt.sum(axis=1).mean())                 # per step
    weight_bytes = union_experts * 2 * d_h * d_e * 2               # W1 + W2, bf16
    act_bytes = T * d_h * 2 + T * d_h * 2                          # x, y
    if fused:
        kernel_bytes = weight_bytes + act_bytes + E * d_h * 2       # + W_r
        kernel_ms = ms_per_step
        kernel_name = ("layer forward, router and chunk FFN in one launch, tiled weights "
                       "(blockffn_layer_forward_packed)")
        timing = "HIP events around graph replays of the steps (one launch each)"
    else:
        kernel_bytes = weight_bytes + act_bytes + T * E * 4         # + scores
        kernel_ms = ffn_avg_ms
        kernel_name = "chunk FFN (blockffn_chunk_ffn)"
        timing = ("HIP events around graph replays of the chunk-FFN calls alone (same "
                  "rotation), divided by the number of calls")
    achieved_gbs = kernel_bytes / (kernel_ms * 1e-3) / 1e9
    flops = union_experts * n * 4 * d_h * d_e + (2 * T * E * d_h if fused else 0)
    tokens_per_s = T / (ms_per_step * 1e-3)

    dense = None
    if not args.no_dense and args.workload != "e2e":
        g_dense = capture(lambda i: ffn(i, dense=True))
        time_replays(g_dense, wreplays)
        dense_ms = time_replays(g_dense, replays) / nsteps
        dense = {"ffn_ms": dense_ms, "ratio_dense_over_sparse": dense_ms / ffn_avg_ms}

    extras = None
    if not args.no_extras:
        extras = bench_extras(args, torch, np, bf, inputs, cfg, copies, xs, S, gain, y, lws,
                              replays, wreplays, time_replays, capture)
        extras["unfused_layer"] = {
            "what": "blockffn_router + blockffn_chunk_ffn as two launches, same inputs",
            "ms_per_step": sep_ms, "tokens_per_s": T / (sep_ms * 1e-3),
            "chunk_ffn_ms": ffn_avg_ms}
        if rowmajor_ms is not None:
            extras["layer_rowmajor_weights"] = {
                "what": "blockffn_layer_forward (one launch) on the row-major W1 and W2",
                "ms_per_step": rowmajor_ms, "tokens_per_s": T / (rowmajor_ms * 1e-3)}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args, cfg, np, inputs)

    traffic = read_traffic(args.workload, fused)
    if C == 1:
        # one chunk: the weight stream (each union expert's W1 and W2 read once) bounds it
        roofline = {
            "kernel": kernel_name, "bound": "hbm", "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic, "algorithmic_bytes_per_launch": kernel_bytes,
            "avg_launch_ms": kernel_ms, "launch_timing": timing,
            "mfma_frac": flops / (kernel_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        }
    else:
        # many chunks: every chunk's union experts are multiplied with its 32 tokens while
        # the weights, shared by the chunks, stay in the caches; the products bound it
        tflops = flops / (kernel_ms * 1e-3) / 1e12
        roofline = {
            "kernel": kernel_name, "bound": "mfma", "achieved": tflops,
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
            "traffic": traffic, "algorithmic_flops_per_launch": flops,
            "avg_launch_ms": kernel_ms, "launch_timing": timing,
            "effective_gbs_of_chunk_unions": achieved_gbs,
        }
    activity = ("router activity following Markov masks at 80% TLS / 70% 8-token CLS "
                "(orthonormal W_r, x drawn for the masks)" if args.workload != "e2e" else
                "router with a logit shift for ~80% zeros, i.i.d. x")
    out = {
        "metric": "tokens/s + effective HBM GB/s (% of peak) of BlockFFN layer, n=32 chunks",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": nsteps,
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
            "weight_copies": nc, "rotation_mib": round(nc * 2 * (2 * E * d_e * d_h + E * d_h) / 2 ** 20),
            "union_experts_per_step": union_experts,
            "timing": f"hipGraph replays of {S} captured steps; eager Python-launched "
                      f"step {eager_ms:.4f} ms",
        },
        "roofline": roofline,
        "dense_ffn": dense,
        "extras": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


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

    def layer_step(i):
        w, k = copies[i % nc], i % S
        if "packed" in w:
            bf.blockffn_layer_forward_packed(xs[k], w["w_r"], w["packed"], E, cfg["d_e"], n,
                                             gain=gain, bias=w["bias"], y=y, workspace=lws)
        else:
            bf.blockffn_layer_forward(xs[k], w["w_r"], w["w1"], w["w2"], n, gain=gain,
                                      bias=w["bias"], y=y, workspace=lws)
        bf.blockffn_add_layernorm(y, xs[k], ln_g, ln_b, out=out)

    g = capture(layer_step)
    time_replays(g, wreplays)
    layer_ms = time_replays(g, replays) / (replays * S)
    del g

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

    res = {"layer_with_epilogue": {
        "what": "the layer step (as the headline) + residual LayerNorm, same rotation as "
                "the headline step",
        "ms_per_step": layer_ms, "tokens_per_s": T / (layer_ms * 1e-3)}}

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


def cpu_baseline(args, cfg, np, inputs):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: whole
    steps (router + chunk FFN) on fresh draws until the time budget is spent."""
    import oracle
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
    tokens = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        rng = np.random.default_rng(args.seed * 1000 + 500 + steps)
        if markov:
            x = inputs.tokens_for_mask(rng, w_r, inputs.markov_active(rng, Ts, E, 0.8, 0.7, 8), True)
        else:
            x = inputs.gaussian(rng, (Ts, d_h), 1.0, True)
        _, s_router = oracle.router(x, w_r, bias=bias)
        oracle.chunk_ffn(x, s_router.astype(np.float32), w1, w2, n)
        tokens += Ts
        steps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or steps >= 10000:
            break
    return {"value": tokens / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{steps} oracle steps (router + chunk FFN, fp64 loops) of "
                      f"{Ts} tokens each on fresh draws, {el:.1f} s"}


if __name__ == "__main__":
    sys.exit(main())
