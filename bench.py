"""Benchmark of one GPU's trainable MoE layer (forward + backward) on MI355X.

    python bench.py [--gpus 1] [--steps 15] [--warmup 5] [--config 30b]

A step is one forward and one backward pass of the whole layer (routing,
dispatch, both expert GEMMs with fused SwiGLU, combine; dy dispatch, the four
backward GEMMs with fused SwiGLU-backward and routing-weight gradient,
un-permute reduction) over one batch of synthetic inputs already resident in
HBM.  The default workload is the Qwen3-30B-A3B-shaped layer (T=16384 tokens,
D=2048, F=768, 128 experts, top-8, uniform random routing, bf16).  Timing
follows the pages' averaging rule (mean over steps after a warm-up: Prime Mega
MoE news item, "How fast is Prime Mega MoE?").

Prints one JSON line.  `value` is achieved TFLOP/s of the algorithmic fwd+bwd
FLOPs (18 * T * K * D * F).  `roofline` covers the kernel with the largest
share of the step, timed with HIP events on the stream it is launched on;
`cpu_baseline` times the CPU oracle's forward and backward on a bounded sample
of the same workload.  With the default 30B main line, the same run also times
the Qwen3-235B-A22B-shaped layer in bf16 and in fp8_bwd, and the 30B shape in
MXFP8 with Zipf routing, each under `configs` with its own step time, fwd/bwd
split, kernel table and roofline entry (`--extra none` skips them).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd ms and TFLOP/s (% MFMA peak), Qwen3-30B/235B shapes"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0


FWD_GEMMS = ("gemm_w1_swiglu", "gemm_w2")


def gemm_peak(cfg, name: str) -> float:
    """Dense MFMA peak (TFLOP/s) of the operand type a GEMM runs in for this mode."""
    fp8 = (cfg.mode in (4, 5)) or (cfg.mode == 3 and name not in FWD_GEMMS)
    return PEAK_TFLOPS["fp8" if fp8 else "bf16"]


def gemm_flops(cfg) -> dict:
    """Algorithmic FLOPs per launch of each GEMM kernel (2 per multiply-add)."""
    ndf = float(cfg.N) * cfg.D * cfg.F
    return {"gemm_w1_swiglu": 4 * ndf, "gemm_w2": 2 * ndf, "gemm_w2_dgrad_dswiglu": 2 * ndf,
            "gemm_w2_wgrad": 2 * ndf, "gemm_w1_dgrad": 4 * ndf, "gemm_w1_wgrad": 4 * ndf,
            # paired backward launches: each dgrad with its weight gradient
            "pair_w2": 4 * ndf, "pair_w1": 8 * ndf}


def weights_in_gemms(cfg) -> bool:
    """bf16 at the shapes whose GEMMs carry the routing weights and the dispatch
    (the library's own condition: 2F % 256 == 0 and D % 64 == 0)."""
    return cfg.mode == 2 and (2 * cfg.F) % 256 == 0 and cfg.D % 64 == 0


def row_bytes(cfg, b=2, recompute=False) -> dict:
    """Algorithmic HBM bytes per launch of the row movers (bf16 rows).  In the FP8
    forward modes (MXFP8, blockwise FP8) the dispatch writes the e4m3 row codes
    of x_perm and one 4-byte scale entry per 128 columns instead of the bf16
    rows (which it writes too under activation recompute; in MXFP8 without
    recompute no dispatch runs).  The combine-backward writes dYw's codes in
    blockwise FP8 and fp8_bwd instead of its bf16 rows, and in MXFP8 neither
    (it computes only dtopk_w).  Where the GEMMs carry the routing weights (bf16
    at the wide shapes) no forward dispatch runs, the combine is an unweighted
    sum, the backward's dispatch copies dy unscaled and dtopk_w is the sum of
    the W2 dgrad's partials (F / 64 per row)."""
    T, N, D = cfg.T, cfg.N, cfg.D
    codes = N * D + N * (D // 128) * 4
    fwd_q = cfg.mode in (4, 5)   # MXFP8, blockwise FP8 in both passes
    dyw_out = {4: 0, 3: codes, 5: codes}.get(cfg.mode, N * D * b)
    xrows = N * D * b if (not fwd_q or recompute) else 0
    if weights_in_gemms(cfg):
        return {"combine": N * D * b + T * D * b + N * 4,
                # dy once, each pair's row written, pos read
                "dispatch_dy": T * D * b + N * D * b + N * 4,
                "dprob_reduce": N * 4 + N * (cfg.F // 64) * 4 + N * 4,
                "unpermute": N * D * b + T * D * b + N * 4}
    return {"dispatch": T * D * b + xrows + 2 * N * 4 + N * 4 + (codes if fwd_q else 0),
            "combine": N * D * b + T * D * b + N * 8,
            # dy once, each pair's expert-output row read and its w*dy row (or its
            # codes) written, pos and topk_w read, dtopk_w written
            "dispatch_dy": T * D * b + N * D * b + dyw_out + 3 * N * 4,
            "unpermute": N * D * b + T * D * b + N * 4}


def measured_traffic(cfg, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (already scaled by the copy-kernel calibration), or None when there is no
    summary for this workload or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}_bf16.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for p in rec["sources"]:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    if h.hexdigest()[:16] != rec["source_sha256_16"] or kernel not in rec["kernels"]:
        return None
    k = rec["kernels"][kernel]
    return k["fetch_bytes"] + k["write_bytes"]


def host_info() -> dict:
    """CPU model, host memory and usable cores of the machine the oracle runs on."""
    model, ram = "unknown", None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    return {"cpu_model": model, "ram_gib": ram, "cores": len(os.sched_getaffinity(0))}


def cpu_baseline(cfg, inp, budget_s: float) -> dict:
    """Times the CPU oracle's forward and backward, separately, on the first S
    tokens of the workload (S sized so both take about budget_s), and scales
    each to the whole layer's T tokens (the oracle's work is linear in T)."""
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as orc

    info = host_info()
    cores = info["cores"]

    def run(S):
        sl = slice(0, S)
        t0 = time.perf_counter()
        f = orc.forward(inp["x"][sl], inp["topk_idx"][sl], inp["topk_w"][sl], inp["w1"], inp["w2"])
        t1 = time.perf_counter()
        orc.backward(inp["dy"][sl], inp["x"][sl], inp["topk_idx"][sl], inp["topk_w"][sl],
                     inp["w1"], inp["w2"], f)
        return t1 - t0, time.perf_counter() - t1

    with threadpool_limits(limits=cores):
        t_small = sum(run(2))
        S = int(max(2, min(cfg.T, 2 * budget_s / max(t_small, 1e-3))))
        S = min(S, 512)
        tf, tb = run(S)
    flops = 18.0 * S * cfg.K * cfg.D * cfg.F
    scale = cfg.T / S
    return {"value": flops / (tf + tb) / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"forward and backward of the first {S} of {cfg.T} tokens (all {cfg.K} routed "
                      f"pairs each), numpy float64, {tf:.1f} s + {tb:.1f} s",
            "dtype": "float64", "tokens": S, "fwd_s": round(tf, 2), "bwd_s": round(tb, 2),
            "fwd_tflops": round(6.0 * S * cfg.K * cfg.D * cfg.F / tf / 1e12, 5),
            "bwd_tflops": round(12.0 * S * cfg.K * cfg.D * cfg.F / tb / 1e12, 5),
            "fwd_ms_whole_layer_est": round(tf * scale * 1e3, 0),
            "bwd_ms_whole_layer_est": round(tb * scale * 1e3, 0),
            "cpu_model": info["cpu_model"], "ram_gib": info["ram_gib"]}


def queue_capable(cfg) -> bool:
    """Whether the forward of this workload runs as the overlapped one-launch kernel."""
    return cfg.mode in (1, 2, 3) and cfg.D % 256 == 0 and (2 * cfg.F) % 256 == 0


def run_config(name: str, args, flags: int, main_line: bool) -> tuple:
    """Times one workload: warm-up, then K steps without per-kernel events (the
    step time), then K steps with them (kernel table and roofline entry).  The
    main line also times the overlapped forward and the router.  Returns the
    result dictionary and the host inputs (for the CPU baseline)."""
    import torch

    import mixture_experts_layer_31_amd as moe
    import moe_inputs as mi
    from tests.layer_harness import Layer, desc_of

    cfg = mi.CONFIGS[name]
    t0 = time.perf_counter()
    inp = mi.make_inputs(cfg, threads=16)
    gen_s = time.perf_counter() - t0
    L = Layer(cfg, inp, flags=flags, device="cuda:0")
    stream = torch.cuda.current_stream()
    # weight preparation (FP8 quantised copies) is timed on its own, outside the step
    prep_ms = None
    if L.wprep is not None:
        L.prepare()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        L.prepare()
        b.record(stream)
        torch.cuda.synchronize()
        prep_ms = round(a.elapsed_time(b), 4)
    if main_line and args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        L.fwd()
        L.bwd()
    torch.cuda.synchronize()
    status = L.check()
    if status != moe.MOE_OK:
        raise RuntimeError(f"{name}: {moe.strerror(status)}")

    def timed_steps(profile: bool):
        """K steps between a start and a stop event (fwd/bwd split by events between
        them); with `profile`, the library also brackets every kernel with events."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        if profile:
            moe.moe_profile_reset()
            moe.moe_profile_enable(True)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for a, b, c in ev:
            a.record(stream)
            L.fwd()
            b.record(stream)
            L.bwd()
            c.record(stream)
        stop.record(stream)
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        kern = moe.moe_profile_collect() if profile else {}
        status = L.check()
        if status != moe.MOE_OK:
            raise RuntimeError(f"{name}: {moe.strerror(status)}")
        return (start.elapsed_time(stop) / args.steps,
                sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps,
                sum(b.elapsed_time(c) for _, b, c in ev) / args.steps, kern)

    # the step time is taken without per-kernel events (they add about 80 us to a
    # 30B step); the same K steps then run again with them for the per-kernel
    # durations behind the roofline entry
    ms_step, fwd_ms, bwd_ms, _ = timed_steps(False)
    kernels, ms_step_profiled = {}, None
    if not args.no_profile:
        ms_step_profiled, _, _, kernels = timed_steps(True)

    f5 = router = None
    if main_line and queue_capable(cfg):
        # the overlapped one-launch forward against the one-kernel-per-step forward
        f5 = {"reps": 10}
        for key, fl in (("fwd_ms_overlapped", moe.MOE_FLAG_OVERLAP), ("fwd_ms_per_step", 0)):
            L.desc = desc_of(cfg, fl | (flags & moe.MOE_FLAG_RECOMPUTE))
            L.fwd()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(f5["reps"]):
                L.fwd()
            b.record(stream)
            torch.cuda.synchronize()
            f5[key] = round(a.elapsed_time(b) / f5["reps"], 4)
        L.desc = desc_of(cfg, flags)
        status = L.check()
        if status != moe.MOE_OK:
            raise RuntimeError(moe.strerror(status))

    if main_line and cfg.E <= 512 and cfg.K <= 64:
        # the router ahead of the layer (softmax -> top-k -> renormalise, and its
        # backward to the logits), timed on its own: not part of the layer step
        r = mi.make_router_inputs(cfg)
        rd = moe.make_desc(cfg.T, 0, 0, cfg.E, cfg.K)
        z = torch.from_numpy(r["logits"]).to("cuda:0")
        rdw = torch.from_numpy(r["dtopk_w"]).to("cuda:0")
        ridx = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda:0")
        rw = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda:0")
        rdz = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda:0")
        router = {"reps": 50,
                  "bytes_fwd": cfg.T * cfg.E * 4 + cfg.T * cfg.K * 8,
                  "bytes_bwd": cfg.T * cfg.K * 12 + cfg.T * cfg.E * 4}
        calls = {"fwd": lambda: moe.moe_router_fwd(rd, z, ridx, rw),
                 "bwd": lambda: moe.moe_router_bwd(rd, ridx, rw, rdw, rdz)}
        for key, call in calls.items():
            if call() != moe.MOE_OK:
                raise RuntimeError(f"router {key} failed")
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(router["reps"]):
                call()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / router["reps"] * 1e3
            router[f"{key}_us"] = round(us, 2)
            router[f"{key}_gbs"] = round(router[f"bytes_{key}"] / (us * 1e-6) / 1e9, 1)

    flops = cfg.fwd_flops() + cfg.bwd_flops()
    tflops = flops / (ms_step * 1e-3) / 1e12
    dtype = {0: "fp32", 1: "fp32", 2: "bf16", 3: "bf16+fp8(bwd)", 4: "mxfp8", 5: "fp8"}[cfg.mode]
    # whole-layer fraction: algorithmic flops over the time the same flops take at each GEMM's peak
    peak = (cfg.fwd_flops() + cfg.bwd_flops()) / (
        cfg.fwd_flops() / gemm_peak(cfg, "gemm_w1_swiglu") + cfg.bwd_flops() / gemm_peak(cfg, "gemm_w1_dgrad"))

    roof = None
    per_kernel = {}
    if kernels:
        gf = gemm_flops(cfg)
        rb = row_bytes(cfg, recompute=bool(flags & moe.MOE_FLAG_RECOMPUTE))
        for kname, (ms, n) in kernels.items():
            avg = ms / n
            entry = {"avg_ms": round(avg, 4), "launches": n}
            if kname in gf:
                entry["tflops"] = round(gf[kname] / (avg * 1e-3) / 1e12, 1)
                entry["frac_peak"] = round(gf[kname] / (avg * 1e-3) / 1e12 / gemm_peak(cfg, kname), 3)
            if kname in rb:
                entry["gbs"] = round(rb[kname] / (avg * 1e-3) / 1e9, 1)
                entry["frac_hbm"] = round(rb[kname] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)
            per_kernel[kname] = entry
        dom = max((k for k in kernels if k in gf), key=lambda k: kernels[k][0])
        avg = kernels[dom][0] / kernels[dom][1]
        ach = gf[dom] / (avg * 1e-3) / 1e12
        dpeak = gemm_peak(cfg, dom)
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": dpeak,
                "unit": "TFLOP/s", "frac": round(ach / dpeak, 4),
                "traffic": measured_traffic(cfg, dom),
                "flops_per_launch": gf[dom], "avg_ms": round(avg, 4)}

    res = {
        "value": round(tflops, 2), "ms_per_step": round(ms_step, 4), "dtype": dtype,
        "config": {"workload": f"{cfg.name}: Qwen3 MoE layer T={cfg.T} D={cfg.D} F={cfg.F} "
                               f"E={cfg.E} top-{cfg.K}, {cfg.routing} routing",
                   "T": cfg.T, "D": cfg.D, "F": cfg.F, "E": cfg.E, "K": cfg.K, "mode": cfg.mode,
                   "recompute": bool(flags & moe.MOE_FLAG_RECOMPUTE)},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(cfg.fwd_flops() / (fwd_ms * 1e-3) / 1e12, 1),
        "bwd_tflops": round(cfg.bwd_flops() / (bwd_ms * 1e-3) / 1e12, 1),
        "peak_tflops": round(peak, 1),
        "frac_mfma_peak": round(tflops / peak, 4),
        "weight_prep_ms": prep_ms,
        "roofline": roof,
        "ms_per_step_profiled": None if ms_step_profiled is None else round(ms_step_profiled, 4),
        "kernels": per_kernel,
        "input_gen_s": round(gen_s, 1),
    }
    if main_line:
        res["f5_overlap"] = f5
        res["router"] = router
    del L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, inp


# the other workloads of the metric, timed in the same run as extra entries
EXTRA_CONFIGS = ("235b", "235b_fp8bwd", "30b_mxfp8")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="30b")
    ap.add_argument("--extra", default=None,
                    help="comma-separated extra workloads timed after the main one (default: "
                         f"{','.join(EXTRA_CONFIGS)} with the 30b main line, none otherwise; 'none')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (reference for HBM counters)")
    ap.add_argument("--no-profile", action="store_true",
                    help="time without per-kernel events (no roofline entry)")
    ap.add_argument("--overlap", action="store_true",
                    help="time the overlapped one-launch forward instead of one kernel per step")
    ap.add_argument("--recompute", action="store_true",
                    help="activation recompute: the forward keeps no H, the backward rebuilds it")
    ap.add_argument("--overlap-bwd", action="store_true",
                    help="backward with each dgrad beside its weight gradient in one launch "
                         "(the default in bf16)")
    ap.add_argument("--serial-bwd", action="store_true",
                    help="backward with one kernel per GEMM")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's layer only: the expert-parallel exchange between "
              "GPUs is outside this library, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import mixture_experts_layer_31_amd as moe
    import moe_inputs as mi

    cfg = mi.CONFIGS[args.config]
    flags = ((moe.MOE_FLAG_OVERLAP if args.overlap else 0) |
             (moe.MOE_FLAG_RECOMPUTE if args.recompute else 0) |
             (moe.MOE_FLAG_OVERLAP_BWD if args.overlap_bwd else 0) |
             (moe.MOE_FLAG_SERIAL_BWD if args.serial_bwd else 0))
    if args.extra is None:
        extra = list(EXTRA_CONFIGS) if args.config == "30b" and not flags else []
    else:
        extra = [] if args.extra == "none" else [e for e in args.extra.split(",") if e]
    main_res, inp = run_config(args.config, args, flags, True)
    print(f"[bench] {args.config}: {main_res['ms_per_step']} ms/step", file=sys.stderr, flush=True)
    others = {}
    for name in extra:
        if name == args.config:
            continue
        others[name], _ = run_config(name, args, flags, False)
        print(f"[bench] {name}: {others[name]['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC, "value": main_res["value"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": main_res["dtype"], "data": "synthetic",
    }
    out.update({k: v for k, v in main_res.items() if k not in ("value", "ms_per_step", "dtype")})
    if others:
        out["configs"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
