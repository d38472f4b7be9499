#!/usr/bin/env python3
"""Throughput of the fused MXFP4 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode] [--no-sweep]

A step is one whole layer call (routing, shared append, sort, gate, GEMM1 +
SwiGLU, GEMM2, finalize) on one batch of seeded synthetic inputs that are
resident in HBM before timing starts. Steps are replayed from captured
graphs that cycle through enough copies of the weights that no step finds
the weights it reads in L2 or the 256 MB Infinity Cache (cold weights, as
the decode page measures). One graph holds CHAIN_STEPS or more steps in
turn, cycling the copies, as a model's decode graph holds all of its MoE
layers: a graph launch is paid once per replay, not once per layer. The K
timed steps (whole replays of that graph, then single-step graphs for the
remainder) follow SETTLE_S seconds of replays (clocks settle after idle)
and the W warmup steps, and are bracketed by one pair of HIP events and a
synchronisation on both sides; more replays, each between its own pair of
events, give the distribution of the per-step time. The mean of K
single-step graph replays is reported beside it (`single_step_graph_us`).
Prints one JSON line.

The headline is the 64-token decode layer (T=64, E=896, top-16, H=3584,
I=384, BlockN=32): `value` is its tokens/s over the K timed steps. The line
also carries, under "configs", the same measurement for the EP decode, the
64-token decode in W4A8, the shared-expert + clamp layer and the 32k-token
prefill in bf16, W4A8 and W4A4 (skip with --no-sweep). For every workload:
  * layer time: the mean over the K timed steps, and the median, p10 and
    p90 over replays of the per-step time;
  * layer_roofline: the whole layer's algorithmic HBM bytes (decode shapes:
    touched experts' weights and scales, x, out, router logits) or FLOPs
    (prefill: 6 R H I) over the median replay time, against 8 TB/s HBM or
    the dense MFMA peak of the compute type;
  * kernels: GEMM1 and GEMM2 timed with HIP events recorded by the library
    between the stages of the same chain on the stream the kernels run on,
    their algorithmic bytes or FLOPs per launch over that time;
  * roofline (headline) is the dominant kernel's (GEMM1), with its HBM
    traffic from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary when
    the kernel sources still hash to the profiled version;
  * cpu_baseline: the fp64 oracle timed on a bounded token sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
METRIC = "MoE layer tokens/s and µs/layer; achieved HBM GB/s (decode), MFMA % (prefill)"
# The Infinity Cache holds 256 MB: cycle through enough weight copies that
# the other copies' touched weights between two uses of one copy exceed
# twice that.
MALL_FLUSH_BYTES = 512 << 20
# Steps per replayed graph (at least; a whole number of weight-copy cycles).
CHAIN_STEPS = 10
# After idle time (input generation, the CPU baseline) the GPU's clocks and
# power state take tens of milliseconds of work to settle: every workload
# replays its graph this long before its warmup steps.
SETTLE_S = 1.0
SWEEP = [("decode_ep", "bf16"), ("decode", "mxfp8"), ("shared_clamp", "bf16"), ("prefill", "bf16"),
         ("prefill", "mxfp8"), ("prefill", "mxfp4")]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--a-dtype", default="bf16", choices=["bf16", "mxfp8", "mxfp4"],
                   help="activation format of the headline workload: bf16 (W4A16), mxfp8 (W4A8) "
                        "or mxfp4 (W4A4)")
    p.add_argument("--activation", default=None, choices=["swiglu", "situ"],
                   help="GEMM1 epilogue (default: the workload's; situ uses beta 4, linear beta 25)")
    p.add_argument("--config", default="decode",
                   help="headline workload: tiny | decode | decode_ep | shared_clamp | prefill")
    p.add_argument("--no-sweep", action="store_true",
                   help="measure only the headline workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the headline's oracle sample run")
    p.add_argument("--sweep-cpu-seconds", type=float, default=6.0,
                   help="target CPU time of each sweep workload's oracle sample run")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="first run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(config: str, kernel: str):
    """HBM bytes per launch of `kernel` on this workload, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/, scaled by the
    counters' reading for a 1 GiB copy; None when no summary matches or the
    kernel's sources changed since the counters were taken."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "mxfp4_weight_expert_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-json: "):
                    continue
                rec = json.loads(line[len("traffic-json: "):])
                rk = rec.get("kernel", "")
                rk = rk[len("moe::"):] if rk.startswith("moe::") else rk
                if rec.get("workload") != config or rk.split("<")[0] != kernel.split("<")[0]:
                    continue
                if ("<true" in kernel) != ("<true" in rk):  # tiled GEMM1 vs tiled dense GEMM2
                    continue
                h = hashlib.sha256()
                for src in rec["src"]:
                    with open(os.path.join(csrc, src), "rb") as g:
                        h.update(g.read())
                if h.hexdigest()[:16] == rec["src_sha256_16"]:
                    return rec.get("traffic_bytes")
    return None


def workload_name(s) -> str:
    parts = [f"T={s.T}", f"E={s.E}" + (f"/{s.E_g}@{s.expert_offset}" if s.E != s.E_g else ""),
             f"topk={s.topk}"]
    if s.S:
        parts.append(f"shared={s.S}")
    parts += [f"H={s.H}", f"I={s.I}", f"BlockN={s.B}"]
    if s.swiglu_limit > 0:
        parts.append(f"clamp={s.swiglu_limit:g}")
    if s.activation == "situ":
        parts.append(f"SiTU(beta={s.act_beta:g}, linear_beta={s.act_linear_beta:g})")
    if s.routing == "zipf":
        parts.append(f"zipf={s.zipf_s:g}")
    act = {"mxfp8": "W4A8 MXFP8 (E4M3) activations", "mxfp4": "W4A4 MXFP4 (E2M1) activations"}.get(
        s.a_dtype, "W4A16 bf16 activations")
    return f"MXFP4 MoE layer ({s.name}): " + " ".join(parts) + f", {act}"


def cpu_baseline(s, inp, target_s: float) -> dict:
    """The oracle (as it stands) on a prefix of the tokens, doubling the prefix
    until one run takes at least half the target time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report what numpy could use
        cores = os.cpu_count() or 1
    n, best = 1, None
    while True:
        n = min(n, s.T)
        sub = s.replace(T=n)
        sl = {k: (v[:n] if k in ("x", "logits", "shared", "topk_ids", "topk_w") else v)
              for k, v in inp.items()}
        t0 = time.perf_counter()
        oracle.reference_forward(sub, sl)
        dt = time.perf_counter() - t0
        best = (n, dt)
        if dt >= target_s / 2 or n >= s.T:
            break
        n *= 2
    n, dt = best
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} of {s.T} tokens of the {s.name} workload, whole layer in fp64 "
                      f"NumPy, one run of {dt:.1f} s"}


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def measure(name: str, a_dtype: str, args, activation=None, cpu_seconds=None) -> dict:
    """One workload: graph-replayed layer steps, stage kernels, roofline."""
    import numpy as np
    import torch

    import mxfp4_weight_expert_amd as moe
    from workloads import CONFIGS, config_seed, make_inputs

    s = CONFIGS[name].replace(a_dtype=a_dtype)
    if activation:
        s = s.replace(activation=activation)
    a8 = s.a_dtype in ("mxfp8", "mxfp4")  # MX activations (W4A8 or W4A4)
    a4 = s.a_dtype == "mxfp4"
    log(f"[bench] {name}/{a_dtype}: generating inputs")
    inp = make_inputs(s, config_seed(name))
    shp = moe.Shape(T=s.T, E=s.E, E_global=s.E_g, topk=s.topk, H=s.H, I=s.I, block_n=s.B, S=s.S,
                    expert_offset=s.expert_offset, swiglu_limit=s.swiglu_limit,
                    shared_scale=s.shared_scale, a_dtype=s.a_dtype, activation=s.activation,
                    act_beta=s.act_beta, act_linear_beta=s.act_linear_beta)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    x = bf16(inp["x"])
    logits = torch.from_numpy(inp["logits"]).cuda()
    shared = bf16(inp["shared"]) if s.S else None

    def upload():  # prepacked once, outside the timed region (a load-time step)
        return {k: (moe.prepack(torch.from_numpy(inp[k]).cuda()) if k in ("w13", "w2")
                    else torch.from_numpy(inp[k]).cuda()) for k in ("w13", "s13", "w2", "s2")}

    sets = [upload()]
    ws = torch.empty(moe.query(shp), dtype=torch.uint8, device="cuda")
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")

    def step(i, stream=None):
        w = sets[i % len(sets)]
        moe.forward(x, w["w13"], w["s13"], w["w2"], w["s2"], shp, router_logits=logits,
                    shared_logits=shared, out=out, workspace=ws, stream=stream)

    # one eager call gives the routing: touched experts decide how many
    # weight copies keep every replay's weights cold
    step(0)
    torch.cuda.synchronize()
    maps = moe.read_maps(ws, shp)
    gate = [int(v) for v in maps["counters"][4:8].cpu().tolist()]
    U, R = gate[1], gate[2]
    w13_e = 2 * s.I * (s.H // 2 + s.H // 32)  # W13 codes + scales of one expert
    w2_e = s.H * (s.I // 2 + s.I // 32)
    touched = max(U * (w13_e + w2_e), 1)
    nsets = min(64, max(2, -(-MALL_FLUSH_BYTES // touched) + 1))
    while len(sets) < nsets:
        sets.append(upload())
    for i in range(1, nsets):
        step(i)
    torch.cuda.synchronize()
    # one single-step graph per weight copy, and one graph of `chain` steps
    # that cycles through the copies (whole cycles, so that two uses of a
    # copy stay nsets - 1 steps apart across replays too)
    graphs = []
    cap = torch.cuda.Stream()
    for i in range(nsets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(i)
        graphs.append(g)
    chain = nsets * -(-CHAIN_STEPS // nsets)
    chain_g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chain_g, stream=cap):
        for i in range(chain):
            step(i)
    torch.cuda.synchronize()

    def run_steps(n):  # n layer steps: whole chain replays, then single-step graphs
        for _ in range(n // chain):
            chain_g.replay()
        for i in range(n % chain):
            graphs[i % nsets].replay()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        chain_g.replay()
        torch.cuda.synchronize()
    run_steps(max(args.warmup, 1))
    torch.cuda.synchronize()

    # The K timed steps, bracketed by one event pair and a synchronisation on
    # both sides.
    log(f"[bench] {name}/{a_dtype}: timing {args.steps} steps ({nsets} weight sets, "
        f"{chain} steps per graph)")
    t0 = time.perf_counter()
    ms_per_step = timed(lambda: run_steps(args.steps)) / args.steps
    wall = time.perf_counter() - t0
    # the same K steps as single-step graph replays (a graph launch per step)
    single_ms = timed(lambda: [graphs[i % nsets].replay() for i in range(args.steps)]) / args.steps
    # The distribution of the per-step time: chain replays, each between its
    # own pair of events.
    nrep = max(10, args.steps // chain)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nrep)]
    for i in range(nrep):
        ev[i][0].record()
        chain_g.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    rep_us = [a.elapsed_time(b) * 1e3 / chain for a, b in ev]
    med = pct(rep_us, 50)
    log(f"[bench] {name}/{a_dtype}: {ms_per_step * 1e3:.1f} us/step mean, median {med:.1f} us "
        f"(wall {wall / args.steps * 1e6:.1f} us/step; single-step graphs {single_ms * 1e3:.1f} us/step)")

    # Stage kernels: the same chain with the library's per-stage HIP events
    # on its stream (eager calls, same weight rotation).
    nst = moe.NUM_STAGES
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    for i in range(min(args.warmup, 3)):
        step(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        w = sets[i % nsets]
        moe.forward_timed(sev[i], x, w["w13"], w["s13"], w["w2"], w["s2"], shp,
                          router_logits=logits, shared_logits=shared, out=out, workspace=ws)
    torch.cuda.synchronize()
    stage_ms = [sum(sev[i][k].elapsed_time(sev[i][k + 1]) for i in range(args.steps)) / args.steps
                for k in range(nst)]
    stages = {n: round(v * 1e3, 2) for n, v in zip(moe.STAGE_NAMES, stage_ms)}
    log(f"[bench] {name}/{a_dtype}: stage us {stages}")
    counts = maps["counts"].cpu().numpy()
    U_routed = int(np.count_nonzero(counts[: s.E]))
    dense = gate[0] == 1

    # algorithmic work (bytes: read once or written once; FLOPs: 2 per MAC)
    # activations: bf16, or MX codes (1 byte E4M3, half a byte E2M1) plus one
    # scale byte per 32
    x_bytes = s.T * ((s.H // 2 if a4 else s.H) + s.H // 32) if a8 else s.T * s.H * 2
    act_bytes = R * ((s.I // 2 if a4 else s.I) + s.I // 32) if a8 else R * s.I * 2
    gemm1_bytes = U * w13_e + x_bytes + act_bytes + R * 4
    gemm2_bytes = U * w2_e + act_bytes + R * s.H * 2
    gemm1_flops = 2.0 * R * s.H * 2 * s.I
    gemm2_flops = 2.0 * R * s.I * s.H
    layer_bytes = U * (w13_e + w2_e) + s.T * s.H * 4 + s.T * s.E_g * 4
    layer_flops = gemm1_flops + gemm2_flops
    mfma_peak = MFMA_PEAK_TFLOPS["fp4" if a4 else ("fp8" if a8 else "bf16")]
    compute_bound = R >= 64 * max(U, 1)  # prefill-like: the contraction dominates

    def roof(bytes_, flops, us, bound_mfma):
        if bound_mfma:
            a = flops / (us * 1e-6) / 1e12
            return {"bound": "mfma", "achieved": round(a, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                    "frac": round(a / mfma_peak, 4), "algorithmic_flops": flops}
        a = bytes_ / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(bytes_)}

    if s.B <= 32:
        k1 = "gemm1_decode_a8_kernel" if a8 else "gemm1_decode_kernel"
    else:
        k1 = "gemm_tiled_a8_kernel<true>" if a8 else "gemm_tiled_kernel<true>"
    # GEMM2: one gated launch runs either path (MX act, or bf16 act with
    # I <= 384); beyond that the split kernel and the generic tiled dense one
    if a8:
        k2 = "gemm2_gated_mx_kernel"
    elif s.I <= 384:
        k2 = "gemm2_gated_kernel"
    elif dense:
        k2 = "gemm_tiled_kernel<false>"
    else:
        k2 = "gemm2_stream_kernel" if s.I == 512 else "gemm2_split_kernel"
    kernels = {}
    for label, kname, us, b, f in (("gemm1", k1, stages["gemm1"], gemm1_bytes, gemm1_flops),
                                   ("gemm2", k2, stages["gemm2"], gemm2_bytes, gemm2_flops)):
        r = roof(b, f, us, compute_bound)
        r.update(kernel=kname, kernel_us=us,
                 traffic=measured_traffic(s.name if s.a_dtype == "bf16" else f"{s.name}/{s.a_dtype}",
                                          kname))
        kernels[label] = r
    layer = roof(layer_bytes, layer_flops, med, compute_bound)
    layer["basis"] = "median per-step time of the whole layer"

    res = {
        "workload": workload_name(s),
        "T": s.T, "E": s.E, "E_global": s.E_g, "topk": s.topk, "S": s.S, "H": s.H, "I": s.I,
        "block_n": s.B, "a_dtype": s.a_dtype,
        "touched_experts": U_routed, "rows": R, "gemm2_path": "dense" if dense else "split",
        "tokens_per_s": round(s.T / (ms_per_step * 1e-3), 1),
        "ms_per_step": round(ms_per_step, 4),
        "layer_us": {"median": round(med, 2), "p10": round(pct(rep_us, 10), 2),
                     "p90": round(pct(rep_us, 90), 2), "mean": round(ms_per_step * 1e3, 2),
                     "basis": f"steps run {chain} to a graph"},
        "single_step_graph_us": round(single_ms * 1e3, 2),
        "stage_us": stages,
        "weight_sets": nsets,
        "layer_roofline": layer,
        "kernels": kernels,
    }
    del graphs, chain_g, sets, ws, out, x, logits, shared
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and cpu_seconds:
        log(f"[bench] {name}/{a_dtype}: CPU baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(s, inp, cpu_seconds)
    else:
        res["cpu_baseline"] = None
    del inp
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported: the layer "
              "runs on one GPU, and splitting experts over GPUs (expert_offset) is the "
              "caller's part", file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp4_weight_expert_amd as moe

    moe.load_library()  # fails loudly if the HIP library is not built
    torch.cuda.set_device(0)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # The sweep runs first, then the headline (each workload settles the
    # clocks itself before its warmup steps).
    sweep = {}
    if not args.no_sweep:
        for name, adt in SWEEP:
            if name == args.config and adt == args.a_dtype:
                continue
            key = name if adt == "bf16" else f"{name}_{'w4a8' if adt == 'mxfp8' else 'w4a4'}"
            sweep[key] = measure(name, adt, args, None, args.sweep_cpu_seconds)
    head = measure(args.config, args.a_dtype, args, args.activation, args.cpu_seconds)
    k1 = head["kernels"]["gemm1"]
    roofline = {key: k1[key] for key in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                         "kernel", "kernel_us")}
    roofline["algorithmic_bytes" if k1["bound"] == "hbm" else "algorithmic_flops"] = \
        k1.get("algorithmic_bytes", k1.get("algorithmic_flops"))
    config = {key: v for key, v in head.items() if key not in ("cpu_baseline", "kernels",
                                                               "layer_roofline", "tokens_per_s",
                                                               "ms_per_step")}
    config["gemm2"] = head["kernels"]["gemm2"]
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp8": "e4m3 x e2m1 (fp32 acc)", "mxfp4": "e2m1 x e2m1 (fp32 acc)"}.get(
            args.a_dtype, "bf16"),
        "data": "synthetic (seeded PCG64: N(0,1) bf16 x, N(0,1) router logits (Zipf-skewed for "
                "the EP decode), uniform E2M1 nibbles, E8M0 scales uniform in [118,127])",
        "config": config,
        "roofline": roofline,
        "layer_roofline": head["layer_roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    if not args.no_sweep:
        res["configs"] = sweep
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
