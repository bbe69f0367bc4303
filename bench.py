#!/usr/bin/env python3
"""Benchmark of the BlockFFN layer forward on one MI355X.

One step = the whole layer over one batch: blockffn_router on the batch's tokens,
then blockffn_chunk_ffn on the same tokens. Default workload (the decode /
speculative-verification chunk): d_h=2048, E=64 experts, d_e=128, T = n = 32
tokens, bf16 weights and activations, fp32 accumulation. The FFN's scores come from
per-expert two-state Markov masks at 80% token-level and 70% 8-token chunk-level
sparsity (the sparsity the pages report for trained BlockFFN models), with active
scores |N(0,1)| + 0.1; they stand in for a trained router, whose weights are not
available. The router still runs every step on the step's tokens (its output goes
to its own buffer), so the step time contains every kernel of the layer.

Inputs are resident in HBM before timing starts. Each step uses the next of several
distinct weight copies (>= 512 MiB in all) and the next of 16 mask/token draws, so
the 256 MB Infinity Cache cannot serve a weight set twice in a row.

Prints ONE JSON line (see the keys below). `roofline` is for the chunk-FFN kernel:
algorithmic bytes per call (the union experts' W1 and W2 slices, plus x, scores and
y) over its average duration, measured with HIP events around each call in the timed
region on the stream it runs on.
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
    cfg = dict(inputs.WORKLOADS[args.workload])
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    dev = torch.device("cuda:0")
    bf16 = torch.bfloat16

    def to_dev(a, dtype=bf16):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev, dtype)

    copy_bytes = 2 * (2 * E * d_e * d_h + E * d_h)
    ncopies = max(2, math.ceil(args.rotate_mib * 2 ** 20 / copy_bytes))
    copies = []
    for i in range(ncopies):
        rng = np.random.default_rng(args.seed * 1000 + 100 + i)
        w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, True)
        w_r = inputs.gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), True)
        bias = inputs.router_shift(w_r, 0.8)
        copies.append(dict(w1=to_dev(w1), w2=to_dev(w2), w_r=to_dev(w_r),
                           bias=to_dev(bias, torch.float32)))
        del w1, w2
    draws = []
    for i in range(args.draws):
        rng = np.random.default_rng(args.seed * 1000 + 500 + i)
        x = inputs.gaussian(rng, (T, d_h), 1.0, True)
        if args.workload == "e2e":
            scores = None
        else:
            act = inputs.markov_active(rng, T, E, 0.8, 0.7, 8)
            scores = to_dev(inputs.scores_for_mask(rng, act), torch.float32)
        dense = to_dev((np.abs(rng.standard_normal((T, E))) + 0.1).astype(np.float32),
                       torch.float32)
        draws.append(dict(x=to_dev(x), scores=scores, dense=dense))
    return cfg, copies, draws


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
    cfg, copies, draws = make_inputs(args, torch, np, inputs)
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    C = -(-T // n)
    dev = torch.device("cuda:0")
    gain = torch.ones(E, dtype=torch.float32, device=dev)
    router_out = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in draws]
    y = torch.empty((T, d_h), dtype=torch.bfloat16, device=dev)
    ws = bf.blockffn_chunk_ffn_workspace(T, d_h, E, d_e, n, bf.BLOCKFFN_BF16, dev)
    router_ws = bf.blockffn_router_workspace(T, d_h, E, bf.BLOCKFFN_BF16, dev)
    counts = [torch.zeros(C, dtype=torch.int32, device=dev) for _ in draws]
    nc, nd = len(copies), len(draws)
    # One captured graph holds S consecutive steps, S a multiple of both rotation
    # lengths, so every replay walks the same sequence of weight copies and draws.
    S = nc * nd // math.gcd(nc, nd)

    def ffn(i, dense=False):
        w = copies[i % nc]
        d = draws[i % nd]
        if args.workload == "e2e":
            s = router_out[i % nd]
        else:
            s = d["dense"] if dense else d["scores"]
        bf.blockffn_chunk_ffn(d["x"], s, w["w1"], w["w2"], n, y=y, workspace=ws,
                              union_counts=counts[i % nd])

    def step(i):
        w = copies[i % nc]
        d = draws[i % nd]
        bf.blockffn_router(d["x"], w["w_r"], gain, w["bias"], scores=router_out[i % nd],
                           workspace=router_ws)
        ffn(i)

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

    # eager warm-up (loads the code objects), then the captured loops
    for i in range(min(args.warmup, 2 * S)):
        step(i)
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
    # the chunk-FFN calls alone, same rotation: average duration of one launch
    time_replays(g_ffn, wreplays)
    ffn_avg_ms = time_replays(g_ffn, replays) / nsteps

    # Python-launched steps, for comparison (host-bound at these sizes)
    eager_n = min(200, nsteps)
    torch.cuda.synchronize()
    te = time.perf_counter()
    for i in range(eager_n):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te) * 1e3 / eager_n

    # Realised unions of the draws (the FFN wrote them during the run).
    cnt = np.stack([c.cpu().numpy() for c in counts])            # [draws, C]
    union_experts = float(np.mean([cnt[i % nd].sum() for i in range(S)]))  # per step
    weight_bytes = union_experts * 2 * d_h * d_e * 2                    # W1 + W2, bf16
    act_bytes = T * d_h * 2 + T * E * 4 + T * d_h * 2                  # x, scores, y
    ffn_bytes = weight_bytes + act_bytes
    achieved_gbs = ffn_bytes / (ffn_avg_ms * 1e-3) / 1e9
    ffn_flops = union_experts * n * 4 * d_h * d_e
    tokens_per_s = T / (ms_per_step * 1e-3)

    dense = None
    if not args.no_dense and args.workload != "e2e":
        g_dense = capture(lambda i: ffn(i, dense=True))
        time_replays(g_dense, wreplays)
        dense_ms = time_replays(g_dense, replays) / nsteps
        dense = {"ffn_ms": dense_ms, "ratio_dense_over_sparse": dense_ms / ffn_avg_ms}

    extras = None
    if not args.no_extras:
        extras = bench_extras(args, torch, np, bf, inputs, cfg, copies, draws, gain,
                              router_out, y, ws, router_ws, counts, S, replays, wreplays,
                              time_replays, capture)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args, cfg, np, inputs)

    traffic = read_traffic(args.workload)
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
            "workload": f"{args.workload}: d_h={d_h} E={E} d_e={d_e} T={T} n={n} bf16"
                        + ("" if args.workload == "e2e" else
                           ", Markov scores 80% TLS / 70% 8-token CLS")
                        + "; router + chunk FFN per step",
            "global_batch": T, "seq_len": n, "parallelism": "none (1 GPU)",
            "weight_copies": nc, "rotation_mib": round(nc * 2 * (2 * E * d_e * d_h + E * d_h) / 2 ** 20),
            "union_experts_per_step": union_experts,
            "timing": f"hipGraph replays of {S} captured steps; eager Python-launched "
                      f"step {eager_ms:.4f} ms",
        },
        "roofline": {
            "kernel": "chunk FFN (blockffn_chunk_ffn)",
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ffn_bytes,
            "avg_launch_ms": ffn_avg_ms,
            "launch_timing": "HIP events around graph replays of the chunk-FFN calls "
                             "alone (same rotation), divided by the number of calls",
            "mfma_frac": ffn_flops / (ffn_avg_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        },
        "dense_ffn": dense,
        "extras": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_extras(args, torch, np, bf, inputs, cfg, copies, draws, gain, router_out, y, ws,
                 router_ws, counts, S, replays, wreplays, time_replays, capture):
    """The rest of the pages' layer around the hot path, measured the same way:
    (1) the whole layer step with its epilogue (router with probabilities, chunk FFN,
    residual + LayerNorm) over the same rotation; (2) the LayerNorm alone and (3) the
    sparsity losses with their gradient alone, each over rotating input copies of at
    least 512 MiB, timed with HIP events around graph replays."""
    T, d_h, E, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["n"]
    dev = torch.device("cuda:0")
    nc, nd = len(copies), len(draws)
    ln_g = torch.ones(d_h, dtype=torch.float32, device=dev)
    ln_b = torch.zeros(d_h, dtype=torch.float32, device=dev)
    probs = torch.empty((T, E), dtype=torch.float32, device=dev)
    out = torch.empty((T, d_h), dtype=torch.bfloat16, device=dev)

    def layer_step(i):
        w = copies[i % nc]
        d = draws[i % nd]
        bf.blockffn_router(d["x"], w["w_r"], gain, w["bias"], scores=router_out[i % nd],
                           probs=probs, workspace=router_ws)
        s = router_out[i % nd] if args.workload == "e2e" else d["scores"]
        bf.blockffn_chunk_ffn(d["x"], s, w["w1"], w["w2"], n, y=y, workspace=ws,
                              union_counts=counts[i % nd])
        bf.blockffn_add_layernorm(y, d["x"], ln_g, ln_b, out=out)

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
        "what": "router (scores + probabilities) + chunk FFN + residual LayerNorm per "
                "step, same rotation as the headline step",
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
    res.update(bench_backward(args, torch, np, bf, inputs, cfg, copies, draws, gain, counts,
                              time_replays))
    return res


def bench_backward(args, torch, np, bf, inputs, cfg, copies, draws, gain, counts, time_replays):
    """The layer backward (router recomputed, expert pass, weight gradients, dx, router
    backward) at the workload's size over the same rotation, and at 2048 tokens. The
    roofline figures: flops of the five expert products per (chunk, union expert)
    plus the router's two, and the bytes of the unique weights read, x and dy read,
    and dx, dW_r, dW1, dW2 written (fp32)."""
    T, d_h, E, d_e, n = cfg["T"], cfg["d_h"], cfg["E"], cfg["d_e"], cfg["n"]
    dev = torch.device("cuda:0")
    nc, nd = len(copies), len(draws)
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
        d = draws[i % nd]
        bf.blockffn_layer_backward(d["x"], w["w_r"], w["w1"], w["w2"], draws[(i + 1) % nd]["x"],
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
        d = draws[i % nd]
        bf.blockffn_router(d["x"], w["w_r"], gain, w["bias"], scores=sc)
        bf.blockffn_chunk_ffn(d["x"], sc, w["w1"], w["w2"], n, y=y, union_counts=cnt,
                              expert_lists=lists)
        c = cnt.cpu().numpy()
        union_sum += float(c.sum())
        used += float(len(set(lists.cpu().numpy()[lists.cpu().numpy() >= 0].tolist())))
    res["layer_backward"] = dict(
        shape=f"T={T} d_h={d_h} E={E} d_e={d_e} n={n} bf16, router scores (logit shift "
              f"for ~80% zeros), fp32 gradients", **figures(T, union_sum / S, used / S, ms))

    # (2) 2048 tokens on two weight copies
    Tp = 2048
    rng = np.random.default_rng(77)
    xs = [torch.from_numpy(inputs.gaussian(rng, (Tp, d_h), 1.0, True)).to(dev, torch.bfloat16)
          for _ in range(2)]
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
        shape=f"T={Tp} d_h={d_h} E={E} d_e={d_e} n={n} bf16, router scores, fp32 gradients",
        **figures(Tp, usum / 2, used / 2, ms))
    return res


def read_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current source of the measured kernel (the files its
    `kernel_sources` line names); else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"ffn_{workload}_traffic.txt")
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
    rng = np.random.default_rng(args.seed * 1000 + 100)
    w1, w2 = inputs.expert_weights(rng, E, d_e, d_h, True)
    w_r = inputs.gaussian(rng, (E, d_h), 1.0 / np.sqrt(d_h), True)
    bias = inputs.router_shift(w_r, 0.8)
    # bounded token sample: at most 4 chunks per oracle step for the large workloads
    Ts = min(T, 4 * n)
    tokens = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        rng = np.random.default_rng(args.seed * 1000 + 500 + steps)
        x = inputs.gaussian(rng, (Ts, d_h), 1.0, True)
        _, s_router = oracle.router(x, w_r, bias=bias)
        if args.workload == "e2e":
            s = s_router.astype(np.float32)
        else:
            s = inputs.scores_for_mask(rng, inputs.markov_active(rng, Ts, E, 0.8, 0.7, 8))
        oracle.chunk_ffn(x, s, w1, w2, n)
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
