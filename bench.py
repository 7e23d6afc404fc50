#!/usr/bin/env python3
"""Throughput of the block-canvas denoising step on one MI355X.

A step is one dg_denoise_step call: schedule constants, embedding +
self-conditioning, q/k/v projection, prefix + canvas attention, output
projection, fused LM head with online softmax, z and Gumbel draw, split merge
and Step select, for every canvas of the batch. Inputs are seeded synthetic
tensors already resident in HBM; t cycles through the 12-step cosine grid,
one Philox seed per step.

Prints one JSON line. `value` is the standard canvas (or --workload).
`roofline` reports the dominant kernel (the fused LM head) from HIP events
recorded around its launches in the timed region; `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload. `workloads` repeats the
throughput measurement for the other workloads (tiny fp32, long prefix,
large vocabulary, batched) on seeded inputs drawn on the GPU, each with its
per-stage algorithmic rates, its LM head's fraction of the MFMA peak and its
own CPU-oracle sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "canvas denoise steps/s & canvas tokens/s (C=256, 1 GPU); % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 vector
WORKLOADS = {
    "c1": "tiny fp32: B=1 C=16 P=8 d=32 2 heads x 16 (MHA) V=64 fp32, linear 8 steps",
    "c2": "standard canvas: B=1 C=256 P=512 d=2048 16q/8kv heads x 128 V=32768 bf16, cosine 12 steps",
    "c3": "long prefix: B=1 C=256 P=32768 d=2048 16q/8kv heads x 128 V=32768 bf16, cosine 12 steps",
    "c4": "large vocabulary: B=1 C=256 P=2048 d=2816 16q/8kv heads x 176 V=262144 bf16, cosine 12 steps",
    "c5": "batched: B=32 C=256 P=4096 d=2048 16q/8kv heads x 128 V=131072 bf16, linear, per-canvas t",
}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "lmhead_counters.txt")
# the LM-head kernel's source: its file and the device helpers it inlines
LMHEAD_SRCS = [os.path.join(ROOT, "discrete_diffusion_decoding_dg_amd", "csrc", n)
               for n in ("k_lmhead.hip", "dg_device.hpp")]


def _sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload):
    """HBM bytes per LM-head launch from committed rocprofv3 counters, if they
    were taken on the current kernel source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            lines = [l for l in f if l.strip() and not l.startswith("#")]
        rec = json.loads(lines[-1]) if lines else {}
        rec = rec.get(workload, rec if rec.get("workload") == workload else {})
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha") != _sha(LMHEAD_SRCS):
        return None
    return (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]) * 1024.0


def cpu_threads():
    """Threads the oracle's BLAS may use: the process's CPU affinity, capped by
    OMP_NUM_THREADS when set (the share of the host this job is given)."""
    aff = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(omp)) if omp.isdigit() and int(omp) > 0 else aff
    return n, aff, os.cpu_count()


def cpu_baseline(cfg, inp, budget_s, canvases=None):
    """The CPU oracle timed on the host cores over a bounded sample of the
    workload: whole denoising steps, or with `canvases` = k one canvas at a
    time, cycling over canvases 0..k-1 of the batch (each with its own Philox
    counters; the K_pre/V_pre arrays may then hold just those k canvases), the
    rate then scaled to the whole batch of cfg.B canvases."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import denoise_step
    n_threads, aff, ncpu = cpu_threads()
    w = {k: inp[k] for k in ["E", "Wq", "Wk", "Wv", "Wo"]}
    t = np.full(cfg.B, 0.5, np.float32) if not cfg.per_canvas_t else inp["t"]
    dt = float(np.float32(1.0 / cfg.steps))
    runs, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=n_threads, user_api="blas"):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
        while True:
            if canvases:
                b = runs % canvases
                sl = slice(b, b + 1)
                denoise_step(cfg, w, inp["x"][sl], inp["z"][sl], inp["K_pre"][sl], inp["V_pre"][sl],
                             t[sl], dt, seed=runs, canvas_ids=[b])
            else:
                denoise_step(cfg, w, inp["x"], inp["z"], inp["K_pre"], inp["V_pre"], t, dt, seed=runs)
            runs += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    if canvases:
        sps = runs / el / cfg.B
        what = (f"{runs} single-canvas oracle steps (cycling over canvases 0..{canvases - 1} of {cfg.B}, "
                f"each with its own prefix cache, z and t) in {el:.1f} s, scaled to the "
                f"{cfg.B}-canvas batch")
    else:
        sps = runs / el
        what = f"{runs} full oracle denoise step(s) of the same workload in {el:.1f} s"
    return {"value": sps, "unit": "denoise steps/s", "cores": int(threads), "kind": "oracle",
            "sample": what + f" (float64 BLAS on {threads} threads)",
            "canvas_tokens_per_s": sps * cfg.B * cfg.C,
            "host_cpu_count": ncpu, "affinity_cpus": aff}


def corrupt_bandwidth(reps=20):
    """dg_corrupt_batch over 2^28 tokens (1 GiB in, 1 GiB out), kappa = 0.5, V = 262144."""
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    B, C, V = 1 << 20, 256, 262144
    x0 = torch.randint(0, V, (B, C), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x0)
    kap = torch.full((B,), 0.5, dtype=torch.float32, device="cuda")
    for _ in range(3):
        dg.dg_corrupt_batch(x0, kap, B, C, V, 1, out)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for r in range(reps):
        dg.dg_corrupt_batch(x0, kap, B, C, V, r, out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    gbs = (8.0 * B * C) / (ms * 1e-3) / 1e9
    del x0, out, kap
    return {"tokens": B * C, "ms": ms, "GB_s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
            "bytes_per_token": 8}


def stage_rates(cfg, stages):
    """Average time per launch of each profiled stage, and for the contraction
    stages their algorithmic TFLOP/s and fraction of the bf16 MFMA peak (a
    stage's time includes its own merge kernel; event pairs add queue time)."""
    fl = cfg.flops_per_step()
    kernels = {k: {"avg_ms": (v[0] / v[1]) if v[1] else None, "launches": v[1]}
               for k, v in stages.items() if v[1]}
    # bf16 stages run on MFMA; the fp32 path is plain VALU (fp32 vector peak)
    peak, key = ((PEAK_BF16_TFLOPS, "frac_mfma_bf16") if cfg.dtype == "bf16"
                 else (PEAK_FP32_TFLOPS, "frac_fp32_vector"))
    for k, f in (("qkv", fl["qkv"]), ("attention", fl["attn"]), ("oproj", fl["oproj"]), ("lmhead", fl["lm"])):
        if k in kernels and kernels[k]["avg_ms"]:
            tf = f / (kernels[k]["avg_ms"] * 1e-3) / 1e12
            kernels[k].update({"algorithmic_flop": f, "tflops": tf, key: tf / peak})
    # the attention's K/V stream (prefix cache plus canvas keys, K and V)
    # against the HBM peak; the stage is MFMA-bound, so this is context
    if "attention" in kernels and kernels["attention"]["avg_ms"]:
        es = 2 if cfg.dtype == "bf16" else 4
        kv = 2.0 * es * cfg.B * cfg.n_kv_heads * (cfg.P + cfg.C) * cfg.head_dim
        gbs = kv / (kernels["attention"]["avg_ms"] * 1e-3) / 1e9
        kernels["attention"].update({"kv_bytes": kv, "kv_GB_s": gbs, "kv_frac_hbm": gbs / PEAK_HBM_GBS})
    return kernels


def time_steps(dg, torch, model, cfg, x, z, Kp, Vp, tvec, steps, warmup, seed0=1000):
    """K timed steps (nothing else on the stream), then the same K steps with
    HIP events around every LM-head launch, then a short pass with every stage
    bracketed. Returns (ms_per_step, LM-head ms per launch, stage profile)."""
    import numpy as np
    xs = [x, torch.empty_like(x)]
    zs = [z, torch.empty_like(z)]
    dt = float(np.float32(1.0 / cfg.steps))

    def step(k):
        a, b = k & 1, (k & 1) ^ 1
        dg.dg_denoise_step(model, xs[a], zs[a], Kp, Vp, tvec(k), dt, seed0 + k, xs[b], zs[b])

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    dg.dg_profile_read(model)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(steps):
        step(warmup + k)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    dg.dg_profile_enable(model, ["lmhead"])
    for k in range(steps):
        step(warmup + steps + k)
    torch.cuda.synchronize()
    dg.dg_profile_enable(model, [])
    lm_ms, lm_n = dg.dg_profile_read(model)["lmhead"]
    dg.dg_profile_enable(model, None)
    for k in range(min(steps, 10)):
        step(k)
    torch.cuda.synchronize()
    dg.dg_profile_enable(model, [])
    stages = dg.dg_profile_read(model)
    return ms, lm_ms / max(1, lm_n), stages


def workload_leg(name, steps, warmup, cpu_budget, with_cpu):
    """Throughput of one more workload on device-drawn inputs of its shape:
    ms per step, steps/s, canvas tokens/s, per-stage algorithmic rates, the LM
    head's fraction of the MFMA peak, and the CPU oracle on a bounded sample."""
    import numpy as np
    import torch

    import discrete_diffusion_decoding_dg_amd as dg
    from tests.dg_harness import config_args
    from workloads import get_config
    from workloads.device_inputs import make_device_inputs, to_host_f32

    cfg = get_config(name)
    t_setup = time.perf_counter()
    d = make_device_inputs(cfg, seed=7)
    model = dg.dg_create(config_args(cfg), d["E"], d["Wq"], d["Wk"], d["Wv"], d["Wo"])
    grid = [np.float32(1.0 - k / cfg.steps) for k in range(cfg.steps)]

    def tvec(k):
        return d["t"] if cfg.per_canvas_t else np.full(cfg.B, grid[k % cfg.steps], np.float32)

    ms, lm_ms, stages = time_steps(dg, torch, model, cfg, d["x"].clone(), d["z"].clone(), d["K_pre"],
                                   d["V_pre"], tvec, steps, warmup)
    model.close()
    fl = cfg.flops_per_step()
    sps = 1000.0 / ms
    lm_tf = fl["lm"] / (lm_ms * 1e-3) / 1e12
    peak, key = ((PEAK_BF16_TFLOPS, "frac_mfma_bf16") if cfg.dtype == "bf16"
                 else (PEAK_FP32_TFLOPS, "frac_fp32_vector"))
    res = {"workload": WORKLOADS[name], "steps": steps, "warmup": warmup, "dtype": cfg.dtype,
           "ms_per_step": ms, "steps_per_s": sps, "canvas_tokens_per_s": sps * cfg.B * cfg.C,
           "step_tflops": fl["total"] / (ms * 1e-3) / 1e12,
           "step_" + key: fl["total"] / (ms * 1e-3) / 1e12 / peak,
           "lmhead": {"avg_ms": lm_ms, "algorithmic_flop_per_launch": fl["lm"], "tflops": lm_tf,
                      key: lm_tf / peak},
           "roofline": {"bound": "mfma" if cfg.dtype == "bf16" else "alu", "kernel": "lmhead_kernel",
                        "achieved": lm_tf, "peak": peak, "unit": "TFLOP/s", "frac": lm_tf / peak,
                        "traffic": _traffic(name) if cfg.dtype == "bf16" else None},
           "kernels": stage_rates(cfg, stages),
           "inputs": "seeded synthetic tensors of the workload's shapes and distributions, drawn on the GPU"}
    if with_cpu:
        # the oracle reads the same tensors, copied to the host
        host = {k: to_host_f32(d[k]) for k in ["E", "Wq", "Wk", "Wv", "Wo", "x", "z"]}
        host["t"] = d["t"]
        # a batch is sampled one canvas at a time: only the first nb canvases'
        # caches travel
        nb = min(cfg.B, 4) if cfg.B > 1 else None
        host["K_pre"] = to_host_f32(d["K_pre"][:nb] if nb else d["K_pre"])
        host["V_pre"] = to_host_f32(d["V_pre"][:nb] if nb else d["V_pre"])
        del d
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(cfg, host, cpu_budget, canvases=nb)
        del host
    else:
        del d
        torch.cuda.empty_cache()
    res["leg_wall_s"] = time.perf_counter() - t_setup
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time per workload")
    ap.add_argument("--workloads", default="c1,c3,c4,c5",
                    help="comma-separated workloads timed after the main one (device-drawn inputs), "
                         "each with its own CPU-oracle sample; empty for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw the main workload's inputs on the GPU (seeded, same shapes and "
                         "distributions; for profiling runs: no CPU baseline)")
    ap.add_argument("--no-corrupt", action="store_true")
    ap.add_argument("--no-ffw", action="store_true", help="skip the feed-forward block timings")
    ap.add_argument("--no-blocks", action="store_true", help="skip the block-autoregressive timings")
    ap.add_argument("--no-stack", action="store_true", help="skip the decoder-stack timings")
    ap.add_argument("--copy-mib", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device to device three times (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the denoising step on exactly one GPU; the library has no "
              "multi-GPU path (no sharding, no collectives). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import discrete_diffusion_decoding_dg_amd as dg
    from workloads import get_config, make_inputs
    from tests.dg_harness import config_args, to_dev

    cfg = get_config(args.workload)
    torch.cuda.set_device(0)
    if args.device_inputs:
        from workloads.device_inputs import make_device_inputs
        inp = make_device_inputs(cfg, seed=7)
    else:
        inp = make_inputs(cfg)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.device_inputs:
        wdev = {n: inp[n] for n in ["E", "Wq", "Wk", "Wv", "Wo"]}
        Kp, Vp, z, x = inp["K_pre"], inp["V_pre"], inp["z"], inp["x"]
    else:
        wdev = {n: to_dev(inp, n, cfg) for n in ["E", "Wq", "Wk", "Wv", "Wo"]}
        Kp, Vp, z = (to_dev(inp, n, cfg) for n in ["K_pre", "V_pre", "z"])
        x = torch.from_numpy(inp["x"]).cuda()
    model = dg.dg_create(config_args(cfg), wdev["E"], wdev["Wq"], wdev["Wk"], wdev["Wv"], wdev["Wo"])
    xs = [x, torch.empty_like(x)]
    zs = [z, torch.empty_like(z)]
    dt = float(np.float32(1.0 / cfg.steps))
    grid = [np.float32(1.0 - k / cfg.steps) for k in range(cfg.steps)]

    def tvec(k):
        if cfg.per_canvas_t:
            return inp["t"]
        return np.full(cfg.B, grid[k % cfg.steps], np.float32)

    def step(k):
        a, b = k & 1, (k & 1) ^ 1
        dg.dg_denoise_step(model, xs[a], zs[a], Kp, Vp, tvec(k), dt, 1000 + k, xs[b], zs[b])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    dg.dg_profile_read(model)          # drop anything recorded so far
    # timed region: K steps with nothing else on the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(args.warmup + k)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    # same K steps again with HIP events around every LM-head launch (on the
    # stream the library launches on): the dominant kernel's duration. The
    # event pairs add queue time between kernels, so this pass is not `value`.
    dg.dg_profile_enable(model, ["lmhead"])
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    for k in range(args.steps):
        step(args.warmup + args.steps + k)
    p1.record()
    torch.cuda.synchronize()
    dg.dg_profile_enable(model, [])
    prof = dg.dg_profile_read(model)
    ms_per_step_profiled = p0.elapsed_time(p1) / args.steps
    # distribution of single-step times: an event pair around each step, in a
    # pass of its own (the pairs add queue time, so it does not touch `value`)
    nd = min(args.steps, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nd)]
    for k in range(nd):
        evs[k][0].record()
        step(args.warmup + 2 * args.steps + k)
        evs[k][1].record()
    torch.cuda.synchronize()
    one = np.sort(np.array([a.elapsed_time(b) for a, b in evs]))
    step_dist = {"steps": nd, "p10_ms": float(np.percentile(one, 10)),
                 "p50_ms": float(np.percentile(one, 50)), "p90_ms": float(np.percentile(one, 90))}
    # per-stage durations from one short pass with every stage bracketed
    dg.dg_profile_enable(model, None)
    for k in range(20):
        step(k)
    torch.cuda.synchronize()
    dg.dg_profile_enable(model, [])
    stages = dg.dg_profile_read(model)

    # generation of one canvas batch end to end (not part of the timed steps)
    xo = torch.empty_like(x)
    dg.dg_generate_canvas(model, Kp, Vp, cfg.steps, 7, xo, None)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    dg.dg_generate_canvas(model, Kp, Vp, cfg.steps, 7, xo, None)
    g1.record()
    torch.cuda.synchronize()
    gen_ms = g0.elapsed_time(g1)

    # one step captured into a HIP graph and replayed K times (the replays
    # repeat the captured arguments: the same t and seed every time), for
    # comparison with the launched steps; not part of `value`
    gxo, gzo = torch.empty_like(x), torch.empty_like(z)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg.dg_denoise_step(model, xs[0], zs[0], Kp, Vp, tvec(0), dt, 1000, gxo, gzo)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.dg_denoise_step(model, xs[0], zs[0], Kp, Vp, tvec(0), dt, 1000, gxo, gzo)
    graph.replay()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(args.steps):
        graph.replay()
    r1.record()
    torch.cuda.synchronize()
    graph_ms = r0.elapsed_time(r1) / args.steps
    del graph, gxo, gzo

    # the entropy-bounded step (the pages' recommended sampler) on the same
    # workload: per-step time, and adaptive generation with at most 48 steps
    # (thresholds in nats; with random weights the entropies sit near ln V, so
    # the canvas accepts a couple of tokens per step and does not stop early)
    import math
    eps_a, eps_s = 2.0 * math.log(cfg.V), 1.0
    det = [torch.empty_like(x), torch.empty_like(x)]
    stop = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")

    def ent_step(k):
        a, b = k & 1, (k & 1) ^ 1
        dg.dg_denoise_step_entropy(model, xs[a], zs[a], Kp, Vp, tvec(k), 2000 + k, eps_a, eps_s,
                                   det[a] if k else None, xs[b], zs[b], det[b], stop)

    for k in range(args.warmup):
        ent_step(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(args.steps):
        ent_step(args.warmup + k)
    e1.record()
    torch.cuda.synchronize()
    ent_ms = e0.elapsed_time(e1) / args.steps
    steps_out = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    dg.dg_generate_canvas_entropy(model, Kp, Vp, 48, 11, eps_a, eps_s, xo, steps_out)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    dg.dg_generate_canvas_entropy(model, Kp, Vp, 48, 11, eps_a, eps_s, xo, steps_out)
    a1.record()
    torch.cuda.synchronize()
    entropy = {"ms_per_step": ent_ms, "steps_per_s": 1000.0 / ent_ms,
               "eps_accept_nats": eps_a, "eps_stop_nats": eps_s,
               "generate_max48_ms": a0.elapsed_time(a1),
               "generate_steps_taken": steps_out.cpu().tolist()[:8]}

    # the step with the gated self-conditioning block z = FFW(p0 E) attached,
    # at hidden widths d and 4 d (not part of `value`, whose workload keeps
    # the identity block)
    ffw_res = None
    if not args.no_ffw:
        ffw_res = {}
        nsteps = min(args.steps, 100)
        for F in (cfg.d, 4 * cfg.d):
            cf = cfg.with_(ffw_hidden=F)
            fw = {n: to_dev(make_inputs(cf, [n]), n, cf) for n in ["W_gate", "W_up", "W_down"]}
            dg.dg_set_ffw(model, fw["W_gate"], fw["W_up"], fw["W_down"])
            for k in range(args.warmup):
                step(k)
            torch.cuda.synchronize()
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record()
            for k in range(nsteps):
                step(args.warmup + k)
            f1.record()
            torch.cuda.synchronize()
            dg.dg_profile_read(model)
            dg.dg_profile_enable(model, ["ffw"])
            for k in range(nsteps):
                step(k)
            torch.cuda.synchronize()
            dg.dg_profile_enable(model, [])
            b_ms, b_n = dg.dg_profile_read(model)["ffw"]
            blk_ms = b_ms / max(1, b_n)
            flop = 6.0 * cfg.R * cfg.d * F
            wbytes = 3.0 * F * cfg.d * 2
            ffw_res[f"hidden_{F}"] = {
                "ms_per_step": f0.elapsed_time(f1) / nsteps,
                "block_ms": blk_ms,
                "block_tflops": flop / (blk_ms * 1e-3) / 1e12,
                "block_weight_gbs": wbytes / (blk_ms * 1e-3) / 1e9,
                "block_gflop": flop / 1e9, "block_weight_mb": wbytes / 1e6}
            dg.dg_set_ffw(model)
            del fw

    # block-autoregressive pipeline on the same shapes: prefill of the P-token
    # prompt into a cache with room for 4 more canvases, then 4 canvases of
    # cfg.steps steps, each committed to the cache before the next starts
    blocks_res = None
    if not args.no_blocks and cfg.B * (cfg.P + 4 * cfg.C) * cfg.n_kv_heads * cfg.head_dim * 2 < (8 << 30):
        nb = 4
        cb = cfg.with_(P=cfg.P + nb * cfg.C)
        mb = dg.dg_create(config_args(cb), wdev["E"], wdev["Wq"], wdev["Wk"], wdev["Wv"], wdev["Wo"])
        shape = (cfg.B, cfg.n_kv_heads, cb.P, cfg.head_dim)
        Kc = torch.zeros(shape, dtype=Kp.dtype, device="cuda")
        Vc = torch.zeros(shape, dtype=Kp.dtype, device="cuda")
        prompt = torch.from_numpy(
            np.random.default_rng(1).integers(0, cfg.V, size=(cfg.B, cfg.P)).astype(np.int32)).cuda()
        xb = torch.empty((cfg.B, nb, cfg.C), dtype=torch.int32, device="cuda")
        dg.dg_encode_kv(mb, prompt, 0, Kc, Vc)
        dg.dg_generate_blocks(mb, Kc, Vc, cfg.P, nb, cfg.steps, 5, xb)
        torch.cuda.synchronize()
        b0, b1, b2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        b0.record()
        dg.dg_encode_kv(mb, prompt, 0, Kc, Vc)
        b1.record()
        dg.dg_generate_blocks(mb, Kc, Vc, cfg.P, nb, cfg.steps, 5, xb)
        b2.record()
        torch.cuda.synchronize()
        dg.dg_profile_enable(mb, ["encode"])
        dg.dg_generate_blocks(mb, Kc, Vc, cfg.P, nb, cfg.steps, 5, xb)
        torch.cuda.synchronize()
        dg.dg_profile_enable(mb, [])
        enc_ms, enc_n = dg.dg_profile_read(mb)["encode"]
        gen_blocks_ms = b1.elapsed_time(b2)
        blocks_res = {"prompt_tokens": cfg.P, "canvases": nb, "steps_per_canvas": cfg.steps,
                      "prefill_ms": b0.elapsed_time(b1), "generate_ms": gen_blocks_ms,
                      "commit_ms": enc_ms / max(1, enc_n),
                      "canvas_tokens_per_s": cfg.B * nb * cfg.C / (gen_blocks_ms * 1e-3)}
        mb.close()
        del Kc, Vc

    # the step through a 4-layer pre-norm stack with gated MLPs of width 4 d
    # (per-layer caches of the workload's prefix length); not part of `value`
    stack_res = None
    if not args.no_stack and 4 * cfg.B * cfg.n_kv_heads * cfg.P * cfg.head_dim <= (64 << 20):
        L = 4
        cs = cfg.with_(n_layers=L, mlp_hidden=4 * cfg.d)
        names = ["S_Wq", "S_Wk", "S_Wv", "S_Wo", "S_g_attn", "S_g_mlp", "S_g_final", "S_W_gate",
                 "S_W_up", "S_W_down", "S_K_pre", "S_V_pre"]
        sin = make_inputs(cs, names)
        sdev = {n: to_dev(sin, n, cs) for n in names}
        layers = [{n: sdev["S_" + n][l].contiguous() for n in
                   ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down"]} for l in range(L)]
        dg.dg_set_stack(model, layers, sdev["S_g_final"])
        Ks, Vs = sdev["S_K_pre"], sdev["S_V_pre"]

        def sstep(k):
            a, b = k & 1, (k & 1) ^ 1
            dg.dg_denoise_step(model, xs[a], zs[a], Ks, Vs, tvec(k), dt, 3000 + k, xs[b], zs[b])

        nsteps = min(args.steps, 50)
        for k in range(args.warmup):
            sstep(k)
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for k in range(nsteps):
            sstep(k)
        s1.record()
        torch.cuda.synchronize()
        dg.dg_profile_read(model)
        dg.dg_profile_enable(model, None)
        for k in range(10):
            sstep(k)
        torch.cuda.synchronize()
        dg.dg_profile_enable(model, [])
        sp = dg.dg_profile_read(model)
        dg.dg_set_stack(model)
        sfl = cs.flops_per_step()
        sms = s0.elapsed_time(s1) / nsteps
        stack_res = {"layers": L, "mlp_hidden": 4 * cfg.d, "ms_per_step": sms,
                     "step_tflops": sfl["total"] / (sms * 1e-3) / 1e12,
                     "stage_ms_per_step": {k: v[0] / 10 for k, v in sp.items() if v[1]}}
        del layers, sdev
        # the same stack with a mixture of 8 experts of width d per layer, top 2
        X, TK = 8, 2
        cm = cfg.with_(n_layers=L, mlp_hidden=cfg.d, n_experts=X, top_k=TK)
        mnames = ["S_Wq", "S_Wk", "S_Wv", "S_Wo", "S_g_attn", "S_g_mlp", "S_g_final", "S_W_gate",
                  "S_W_up", "S_W_down", "S_W_router"]
        min_ = make_inputs(cm, mnames)
        mdev = {n: to_dev(min_, n, cm) for n in mnames}
        mlayers = [{n: mdev["S_" + n][l].contiguous() for n in
                    ["Wq", "Wk", "Wv", "Wo", "g_attn", "g_mlp", "W_gate", "W_up", "W_down", "W_router"]}
                   for l in range(L)]
        dg.dg_set_stack(model, mlayers, mdev["S_g_final"], top_k=TK)
        for k in range(args.warmup):
            sstep(k)
        torch.cuda.synchronize()
        s0.record()
        for k in range(nsteps):
            sstep(k)
        s1.record()
        torch.cuda.synchronize()
        dg.dg_set_stack(model)
        mms = s0.elapsed_time(s1) / nsteps
        mfl = cm.flops_per_step()
        stack_res["moe"] = {"experts": X, "top_k": TK, "expert_hidden": cfg.d, "ms_per_step": mms,
                            "step_tflops_activated": mfl["total"] / (mms * 1e-3) / 1e12}
        del mlayers, mdev, Ks, Vs

    fl = cfg.flops_per_step()
    lm_ms, lm_n = prof["lmhead"]
    lm_avg_ms = lm_ms / max(1, lm_n)
    achieved = fl["lm"] / (lm_avg_ms * 1e-3) / 1e12
    traffic = _traffic(args.workload)
    kernels = stage_rates(cfg, stages)
    steps_per_s = 1000.0 / ms_per_step
    result = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "B": cfg.B, "C": cfg.C, "P": cfg.P,
                   "d": cfg.d, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "V": cfg.V, "schedule": cfg.schedule,
                   "parallelism": "single GPU"},
        "canvas_tokens_per_s": steps_per_s * cfg.B * cfg.C,
        "step_tflops": fl["total"] / (ms_per_step * 1e-3) / 1e12,
        "step_frac_mfma": fl["total"] / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "generate_canvas_ms": gen_ms,
        "graph_replay_ms_per_step": graph_ms,
        "ms_per_step_with_lmhead_events": ms_per_step_profiled,
        "step_ms_distribution": step_dist,
        "roofline": {"bound": "mfma", "kernel": "lmhead_kernel", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "avg_ms": lm_avg_ms,
                     "algorithmic_flop_per_launch": fl["lm"]},
        "kernels": kernels,
        "entropy_step": entropy,
    }
    if ffw_res is not None:
        result["ffw_block"] = ffw_res
    if blocks_res is not None:
        result["blocks"] = blocks_res
    if stack_res is not None:
        result["stack"] = stack_res
    if not args.no_corrupt:
        result["corrupt"] = corrupt_bandwidth()
    model.close()
    del wdev, Kp, Vp, z, x, xs, zs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not args.device_inputs:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    del inp
    # the other workloads, one after another (each frees its tensors)
    legs = [w for w in args.workloads.split(",") if w and w != args.workload]
    if legs:
        wl = {args.workload: {
            "workload": WORKLOADS[args.workload], "ms_per_step": ms_per_step,
            "steps_per_s": steps_per_s, "canvas_tokens_per_s": steps_per_s * cfg.B * cfg.C,
            "lmhead": {"avg_ms": lm_avg_ms, "frac_mfma_bf16": achieved / PEAK_BF16_TFLOPS},
            "note": "the main measurement (value, roofline, cpu_baseline above)"}}
        for w in legs:
            print(f"[bench] workload {w}", file=sys.stderr, flush=True)
            wl[w] = workload_leg(w, args.steps, args.warmup, args.cpu_budget,
                                 not args.no_cpu_baseline)
        result["workloads"] = wl
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
