#!/usr/bin/env python3
"""Throughput of the gpt-oss MoE FFN layer (fp32 router, MXFP4 experts) on one MI355X.

A step is one moe_forward call -- router, top-k, permutation, gate/up GEMM +
SwiGLU, down GEMM + weighted combine -- over one batch of seeded synthetic
input already resident in HBM. Prints one JSON line on stdout.

Default workload: the 120b layer on the mixed batch, T=16384 (256 decode + 16128
prefill tokens), E=128, k=4, Zipf(1.3) expert load -- the largest of the five
configurations, bound by the bf16 matrix cores. The same run also measures the
other four configurations (the `per_config` key: tokens/s, dominant-kernel and
whole-layer roofline fractions). For the weight-bound (decode) shapes the step
rotates over enough device copies of the layer's weights (>= 1 GB in total)
that they cannot be served from the 256 MB Infinity Cache.

Roofline: the dominant kernel (the gate/up GEMM) is timed with HIP events on
the stream it runs on, in a second timed region of back-to-back launches of
the same kernel through the layer's moe_gate_up entry point. Its algorithmic
bytes (decode) or FLOPs (prefill) divided by that time give `achieved`.

cpu_baseline: the fp64 oracle on a bounded sample of the same workload, on
the host cores (BLAS threads = the cores this process may run on; not a tuned
CPU implementation).

Also reported: p10/p50/p90 of single steps (a second pass with one event
pair per step) and, for the weight-bound shapes, the step time without
rotating weight copies and the time per layer step when 24 steps (a decode
pass through gpt-oss-20b's 24 MoE layers) are captured as one HIP graph and
replayed (`graph_ms_per_step`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec; % HBM BW (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
FP6_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP6 / FP4 matrix cores
H = I = 2880
W13_EXPERT_BYTES = 2 * I * H // 2 + 2 * I * H // 32 + 2 * I * 2   # codes + scales + bf16 bias
W2_EXPERT_BYTES = H * I // 2 + H * I // 32 + H * 2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["sparse_moe_ffn_fp32_amd/csrc/ffn.hip", "sparse_moe_ffn_fp32_amd/csrc/moe_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    ent = d.get(workload)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("traffic_bytes")


def measured_peaks(dev):
    """Reference rates measured on this device in the same run (not part of
    the layer): a 2 GiB device-to-device copy through torch (bytes read +
    written per second) and a 8192^3 bf16 matrix product through torch
    (hipBLASLt). The roofline fractions are also given against these."""
    import torch
    n = (2 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * 4 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    b = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    return {"hbm_copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tf, 1),
            "how": "torch device copy of 2 GiB (read + write bytes); torch bf16 8192^3 matmul"}


def cpu_baseline(inp, cfg, n_tokens):
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    blas, limits = "unknown", None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
        limits = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        pass
    sample = np.arange(min(n_tokens, cfg.T))
    # repeat a short sample until about 10 s of CPU work (at most 8 passes)
    reps, dt = 0, 0.0
    try:
        while reps < 8 and (reps == 0 or dt < 10.0):
            t0 = time.perf_counter()
            oracle.forward(inp, cfg.k, tokens=sample)
            dt += time.perf_counter() - t0
            reps += 1
    finally:
        if limits is not None:
            limits.restore_original_limits()
    return {"value": round(reps * sample.size / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "blas": blas,
            "sample": (f"first {sample.size} of {cfg.T} tokens, {reps} pass(es): router over all "
                       f"{cfg.T} tokens, experts for the sample, fp64 numpy ({blas}, "
                       f"{cores} threads), {dt:.1f} s wall")}


def measure(idx, args, dev, steps, warmup, want_kernel=True):
    """Time the layer on configuration `idx` (and its dominant kernel); returns
    (result dict, host inputs)."""
    import numpy as np
    import torch

    import sparse_moe_ffn_fp32_amd as moe
    from moe_inputs import LAYER_CONFIGS, make_config_inputs

    cfg = LAYER_CONFIGS[idx]
    T, E, k = cfg.T, cfg.E, cfg.k
    log(f"bench: config {idx} ({cfg.name}) T={T} E={E} k={k}")
    inp = make_config_inputs(idx, seed=args.seed)

    def dev_t(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    layer_bytes = E * (W13_EXPERT_BYTES + W2_EXPERT_BYTES)
    copies = args.copies or (max(1, math.ceil(1.0e9 / layer_bytes)) if cfg.regime == "decode" else 1)
    x = dev_t(inp["x"])
    sets = []
    for _ in range(copies):
        w = {key: dev_t(inp[key]) for key in ("Wr", "br")}
        # one-time layout conversion of the static expert weights (MXFP4 packing)
        w["experts"] = moe.pack_experts(dev_t(inp["w13_codes"]), dev_t(inp["w13_scales"]),
                                        dev_t(inp["b13"]), dev_t(inp["w2_codes"]),
                                        dev_t(inp["w2_scales"]), dev_t(inp["b2"]))
        sets.append(w)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.workspace_size(T, E, k), dtype=torch.uint8, device=dev)
    log(f"bench: {copies} weight copies ({copies * layer_bytes / 1e9:.2f} GB)")

    fwd = moe.forward_mx6 if args.path == "mx6" else moe.forward
    gnorm = torch.ones(H, dtype=torch.float32, device=dev)

    def step(i):
        w = sets[i % copies]
        if args.block:
            moe.forward_block(x, gnorm, w["Wr"], w["br"], w["experts"], k=k, out=out, workspace=ws)
            return
        fwd(x, w["Wr"], w["br"], w["experts"], k=k, out=out, workspace=ws)

    eager_step = step

    def capture_pass(n_layers):
        """One HIP graph of n_layers consecutive layer steps (a decode pass
        through that many MoE layers; the weight copies rotate as the layers'
        weights would)."""
        for i in range(copies):
            eager_step(i)
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for i in range(copies):
                eager_step(i)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for i in range(n_layers):
                eager_step(i)
        return gph

    def graph_ms_per_layer(n_layers, layer_steps):
        gph = capture_pass(n_layers)
        reps = max(2, layer_steps // n_layers)
        for _ in range(2):
            gph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            gph.replay()
        g1.record()
        torch.cuda.synchronize()
        del gph
        return g0.elapsed_time(g1) / (reps * n_layers)

    stream = torch.cuda.current_stream(dev)
    if args.graph:
        # whole captured passes replayed: time per layer step = replay time /
        # layers in the pass (no per-step distribution: a replay is one unit)
        ms_per_step = graph_ms_per_layer(args.graph_layers, steps)
        p10 = p50 = p90 = ms_per_step
        log(f"bench: {ms_per_step * 1e3:.1f} us per layer step ({args.graph_layers}-layer graphs)")
    else:
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t0.elapsed_time(t1) / steps
        log(f"bench: {ms_per_step * 1e3:.1f} us per step")

        # Distribution of single steps (a second pass, one event pair per
        # step), and for the weight-bound shapes the same layer without
        # rotating the weight copies (one copy, partly served from the
        # Infinity Cache).
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            step(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
        p10, p50, p90 = (float(v) for v in np.percentile(per_step, [10, 50, 90]))
    assert torch.isfinite(out).all().item(), "non-finite layer output"
    nonrot_ms = None
    if copies > 1 and not args.graph:
        n0 = torch.cuda.Event(enable_timing=True)
        n1 = torch.cuda.Event(enable_timing=True)
        n0.record(stream)
        for i in range(steps):
            step(0)
        n1.record(stream)
        torch.cuda.synchronize()
        nonrot_ms = n0.elapsed_time(n1) / steps

    # Decode shapes: the same layer steps captured as one HIP graph per decode
    # pass through the model's MoE layers (gpt-oss-20b: 24 layers, its raw
    # config.json), replayed; time per layer step.
    graph_ms = None
    if cfg.regime == "decode" and not args.graph:
        graph_ms = graph_ms_per_layer(24, 24 * 20)
        log(f"bench: {graph_ms * 1e3:.1f} us per layer step replaying 24-layer graphs")

    # Dominant kernel: the gate/up GEMM, timed by HIP events on its stream
    # around back-to-back launches (the routing is computed once; each launch
    # streams the next weight copy).
    w0 = sets[0]
    ids, tw = moe.route(x, w0["Wr"], w0["br"], k=k, workspace=ws)
    counts, offsets, rows = moe.permute(ids, E, workspace=ws)
    touched = int((counts > 0).sum().item())
    mx6 = args.path == "mx6" and cfg.regime != "decode"
    kern_ms = None
    if want_kernel:
        h = torch.empty((T * k, I), dtype=torch.int16, device=dev)
        xrec = moe.encode_mx6(x) if mx6 else None

        def gate_up(i):
            w = sets[i % copies]
            if mx6:
                moe.gate_up_mx6(xrec, offsets, rows, w["experts"], k=k, h=h)
            else:
                moe.gate_up(x, offsets, rows, w["experts"], k=k, h=h)

        for i in range(warmup):
            gate_up(i)
        torch.cuda.synchronize()
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        for i in range(steps):
            gate_up(i)
        k1.record(stream)
        torch.cuda.synchronize()
        kern_ms = k0.elapsed_time(k1) / steps
        log(f"bench: gate/up kernel {kern_ms * 1e3:.1f} us per launch, {touched} experts touched")
        del h, xrec

    workload = f"{cfg.name} (E={E}, k={k})" + (" + RMSNorm + residual" if args.block else "")
    layer_flop = 2.0 * T * k * (H * 2 * I + H * I) + 2.0 * T * H * E
    layer_alg_bytes = touched * (W13_EXPERT_BYTES + W2_EXPERT_BYTES) + E * (H * 4 + 4) \
        + T * H * 2 + T * H * 4 + T * k * 8
    roof = None
    if cfg.regime == "decode":
        if kern_ms is not None:
            alg = touched * W13_EXPERT_BYTES + T * H * 2 + T * k * I * 2
            achieved = alg / (kern_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(workload),
                    "kernel": "ffn_skinny_kernel<EPI_SWIGLU> (gate/up + SwiGLU)",
                    "algorithmic_bytes_per_launch": alg}
        layer_frac = layer_alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
        layer_unit = "of 8 TB/s HBM (algorithmic bytes / step time)"
    else:
        if kern_ms is not None:
            alg = 2.0 * T * k * H * 2 * I
            achieved = alg / (kern_ms * 1e-3) / 1e12
            if mx6:
                # block-scaled FP4 x FP6 matrix cores: two MFMAs per product (one
                # per activation piece), priced against the FP6/FP4 dense peak
                roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP6_FP4_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / FP6_FP4_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic(workload + " mx6"),
                        "kernel": "ffn_wide6_kernel<EPI_SWIGLU> (gate/up + SwiGLU, FP4 x FP6 pieces)",
                        "algorithmic_flop_per_launch": alg,
                        "mfma_flop_issued_per_launch": 2 * alg,
                        "issued_frac": round(2 * achieved / FP6_FP4_PEAK_TFLOPS, 4),
                        "bf16_peak_frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
            else:
                roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic(workload),
                        "kernel": "ffn_tile_kernel<EPI_SWIGLU> (gate/up + SwiGLU)",
                        "algorithmic_flop_per_launch": alg}
        layer_frac = layer_flop / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
        layer_unit = "of 2.5 PFLOP/s dense bf16 (algorithmic FLOP / step time)"

    res = {
        "workload": workload, "T": T, "E": E, "k": k, "copies": copies, "ms_per_step": ms_per_step,
        "value": T / (ms_per_step * 1e-3), "roofline": roof, "layer_roofline_frac": layer_frac,
        "layer_roofline_unit": layer_unit, "experts_touched": touched,
        "p10_p50_p90": [p10, p50, p90], "nonrot_ms": nonrot_ms,
        "kernel_ms": kern_ms, "layer_flop": layer_flop, "layer_alg_bytes": layer_alg_bytes,
        "graph_ms": graph_ms,
    }
    del sets, x, out, ws
    torch.cuda.empty_cache()
    return res, inp


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4, help="layer configuration index (0-4)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0,
                    help="device copies of the weights to rotate over (0: automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip the reference copy / matrix-product rates")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure only --config (not the other configurations)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0: automatic)")
    ap.add_argument("--path", choices=("bf16", "mx6"), default="bf16",
                    help="tiled expert GEMMs on bf16 activations (moe_forward) or on two-piece "
                         "MX FP6 activations with the block-scaled FP4 matrix cores "
                         "(moe_forward_mx6)")
    ap.add_argument("--graph", action="store_true",
                    help="capture --graph-layers consecutive steps (a decode pass through that many "
                         "MoE layers, weight copies rotating) into one HIP graph and time its "
                         "replays per layer step")
    ap.add_argument("--graph-layers", type=int, default=24,
                    help="layer steps per captured graph (gpt-oss-20b has 24 layers)")
    ap.add_argument("--block", action="store_true",
                    help="time the decoder sublayer x + layer(RMSNorm(x)) (moe_forward_block) "
                         "instead of the layer alone")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the bench, run a plain device copy of this size "
                         "(reference kernel for the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs the layer on one GPU only: the library has no multi-GPU path "
              "(expert-parallel sharding is a design note). Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.block and args.path == "mx6":
        print("--block runs the bf16 path (moe_forward_block)", file=sys.stderr)
        return 2

    import torch

    from moe_inputs import LAYER_CONFIGS

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = LAYER_CONFIGS[args.config]
    r, inp = measure(args.config, args, dev, args.steps, args.warmup)
    roof = r["roofline"]
    res = {
        "metric": METRIC,
        "value": round(r["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 x mxfp6 (2 pieces)" if args.path == "mx6" else "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"], "T": cfg.T, "E": cfg.E, "k": cfg.k, "hidden": H,
                   "intermediate": I, "weights": "MXFP4 (E2M1 + E8M0 per 32)",
                   "weight_copies_rotated": r["copies"], "seed": args.seed,
                   "hip_graph": bool(args.graph)},
        "roofline": roof,
        "layer_roofline_frac": round(r["layer_roofline_frac"], 4),
        "layer_roofline_unit": r["layer_roofline_unit"],
        "experts_touched": r["experts_touched"],
        "step_ms_p10_p50_p90": [round(v, 5) for v in r["p10_p50_p90"]],
        "ms_per_step_one_weight_copy": None if r["nonrot_ms"] is None else round(r["nonrot_ms"], 5),
        "graph_ms_per_step": None if r["graph_ms"] is None else round(r["graph_ms"], 5),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_per_config:
        # the other configurations, same path and kernels, fewer steps
        per = {}
        for idx in range(len(LAYER_CONFIGS)):
            if idx == args.config:
                continue
            ri, _ = measure(idx, args, dev, max(5, min(args.steps, 50)), max(2, min(args.warmup, 5)))
            rr = ri["roofline"] or {}
            per[str(idx)] = {
                "workload": ri["workload"], "tokens_per_s": round(ri["value"], 1),
                "ms_per_step": round(ri["ms_per_step"], 5),
                "kernel": rr.get("kernel"), "kernel_us": round(ri["kernel_ms"] * 1e3, 2),
                "kernel_frac": rr.get("frac"), "kernel_bound": rr.get("bound"),
                "layer_roofline_frac": round(ri["layer_roofline_frac"], 4),
                "layer_roofline_unit": ri["layer_roofline_unit"],
                "weight_copies_rotated": ri["copies"],
            }
            if ri["graph_ms"] is not None:
                g = ri["graph_ms"]
                per[str(idx)].update({
                    "graph_ms_per_step": round(g, 5),
                    "graph_tokens_per_s": round(ri["T"] / (g * 1e-3), 1),
                    "graph_layer_roofline_frac": round(ri["layer_alg_bytes"] / (g * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "graph": "24 layer steps per HIP graph (one decode pass), replayed"})
        res["per_config"] = per
    if not args.no_peak_probe:
        peaks = measured_peaks(dev)
        res["measured_peaks"] = peaks
        if roof["unit"] == "GB/s":
            roof["frac_of_measured_copy"] = round(roof["achieved"] / peaks["hbm_copy_GBps"], 4)
        elif args.path != "mx6":
            roof["frac_of_measured_gemm"] = round(roof["achieved"] / peaks["bf16_gemm_TFLOPs"], 4)
        else:
            roof["bf16_equivalent_frac_of_measured_gemm"] = round(roof["achieved"] / peaks["bf16_gemm_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        n = args.cpu_tokens or (cfg.T if cfg.T <= 64 else (32 if cfg.E <= 32 else 16))
        log(f"bench: oracle on {n} tokens")
        res["cpu_baseline"] = cpu_baseline(inp, cfg, n)
    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = nbytes
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
