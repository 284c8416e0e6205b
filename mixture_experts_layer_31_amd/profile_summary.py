"""Summarises rocprofv3 output of `bench.py` into the committed profile files.

Inputs (CSV output of three rocprofv3 runs of the same bench command, which
must include `--calib-copy-mib M`):
  * `--kernel-trace --stats`  -> <trace>_kernel_trace.csv
  * `--pmc FETCH_SIZE`        -> <fetch>_counter_collection.csv
  * `--pmc WRITE_SIZE`        -> <write>_counter_collection.csv
With --stats-only, only the trace run is read and profiles/kernels_<config>.md
lists every kernel's launches and durations (the FP8 workloads).
Outputs: profiles/layer_<config>_bf16.md (per-kernel durations and calibrated
HBM bytes, with the commands) and profiles/traffic_<config>_bf16.json (the
bytes per launch that bench.py reports as roofline traffic, keyed to a hash of
the GEMM sources so a stale file is ignored).

Kernels are named after the layer step they run: the GEMMs by their template
arguments (operand layout and epilogue), the two weight-gradient GEMMs by grid
size (the W1 one has twice the output tiles of the W2 one).  The calibration
scales each counter so that the device copy of M MiB reads and writes M MiB.

    python -m mixture_experts_layer_31_amd.profile_summary --config 30b \\
        --trace <dir>/trace --fetch <dir>/fetch \\
        --write <dir>/write --calib-mib 512 --commands "..."
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GEMM_SOURCES = [
    "mixture_experts_layer_31_amd/csrc/moe_common.h",
    "mixture_experts_layer_31_amd/csrc/moe_gemm.hip",
    "mixture_experts_layer_31_amd/csrc/moe_gemm_common.h",
    "mixture_experts_layer_31_amd/csrc/moe_fp8_codec.h",
    "mixture_experts_layer_31_amd/csrc/moe_grouped.h",
    "mixture_experts_layer_31_amd/csrc/moe_pair.h",
]
_GROUPED = {("false", "1"): "gemm_w1_swiglu", ("false", "0"): "gemm_w2",
            ("true", "2"): "gemm_w2_dgrad_dswiglu", ("true", "0"): "gemm_w1_dgrad"}
_PLAIN = [("clear_err_kernel", "clear_err"), ("route_count_kernel", "route_count"),
          ("route_scan_kernel", "route_scan"), ("route_scatter_kernel", "route_scatter"),
          ("dispatch_dy_kernel", "dispatch_dy"), ("dispatch_kernel", "dispatch"),
          ("dprob_reduce_kernel", "dprob_reduce"), ("zero16_kernel", "zero"),
          ("fwd_queue_kernel", "fwd_queue"), ("queue_build_kernel", "queue_build"),
          ("convert_bf16_kernel", "convert_bf16"), ("__amd_rocclr_copyBuffer", "copyBuffer")]
# Where the GEMMs carry the routing weights (bf16 at the Qwen3 shapes) the row
# dispatch kernel runs once per step, on dy (the forward's dispatch is inside W1).
DY_DISPATCH = {"flag": False}


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def step_name(kernel: str) -> str | None:
    # paired backward launches: <A tile, B_T or MX, epilogue, B tile...>
    m = re.search(r"pair_kernel<[^,]*Tile<[^>]*>, (true|false), (\d),", kernel)
    if m:
        return {"2": "pair_w2", "0": "pair_w1"}.get(m.group(2))
    m = re.search(r"grouped_gemm_kernel<.*Tile<[^>]*>, (true|false), (\d)>", kernel)
    if m:
        return _GROUPED.get((m.group(1), m.group(2)))
    if "wgrad_gemm_kernel" in kernel:
        return "wgrad"
    m = re.search(r"gather_reduce_kernel<[^>]*\b(true|false), \d+>", kernel)  # weighted, batch
    if m:
        return "combine" if m.group(1) == "true" else "unpermute"
    # wide rows (D = 4096, 8192): <element type, weighted, chunks per thread, batch>
    m = re.search(r"gather_reduce_wide_kernel<[^,>]*, (true|false),", kernel)
    if m:
        return "combine" if m.group(1) == "true" else "unpermute"
    if "dispatch_rows_kernel" in kernel:  # whole rows per wave (D = 2048, 4096; K >= 4)
        return "dispatch_dy" if DY_DISPATCH["flag"] else "dispatch"
    for key, name in _PLAIN:
        if key in kernel:
            return name
    return None


def _grid(row) -> int:
    for k in ("Grid_Size", "Grid_Size_X"):
        if k in row and row[k] != "":
            return int(float(row[k]))
    return 0


def _wgrad_split(rows):
    """Names the two wgrad GEMMs: larger grid -> W1, smaller -> W2."""
    grids = sorted({_grid(r) for r in rows if step_name(r["Kernel_Name"]) == "wgrad"})
    names = {}
    if len(grids) == 2:
        names = {grids[0]: "gemm_w2_wgrad", grids[1]: "gemm_w1_wgrad"}
    return names


def name_rows(rows):
    """(step name, row) for every named launch, in dispatch order.  Where the
    rows carry their routing weights (--dy-dispatch) the combine and the
    un-permute are the same unweighted gather-reduce kernel: a launch after W2
    (or the persistent forward) is the combine, any other the un-permute."""
    split = _wgrad_split(rows)
    out = []
    prev = None
    for r in sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or 0)):
        n = step_name(r["Kernel_Name"])
        if n == "wgrad":
            n = split.get(_grid(r), "gemm_wgrad")
        if n == "unpermute" and DY_DISPATCH["flag"] and prev in ("gemm_w2", "fwd_queue"):
            n = "combine"
        if n:
            out.append((n, r))
            prev = n
    return out


def trace_table(prefix: str):
    rows = list(csv.DictReader(open(prefix + "_kernel_trace.csv")))
    dur = collections.defaultdict(list)
    for n, r in name_rows(rows):
        dur[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return dur


def counter_table(prefix: str, counter: str):
    rows = [r for r in csv.DictReader(open(prefix + "_counter_collection.csv"))
            if r["Counter_Name"] == counter]
    per = collections.defaultdict(list)
    for n, r in name_rows(rows):
        per[n].append(float(r["Counter_Value"]))  # KiB per dispatch
    return per


def stats_summary(args):
    """profiles/kernels_<config>.md from a --kernel-trace --stats run alone: every
    kernel of the run by total time (for workloads without a traffic summary)."""
    rows = list(csv.DictReader(open(args.trace + "_kernel_stats.csv")))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# {args.config} layer: per-kernel time", "",
             f"Workload: {args.workload or args.config}.", "",
             "Commands (run from the repository root on the MI355X):", ""]
    lines += [f"    {c.strip()}" for c in args.commands.split(";") if c.strip()]
    lines += ["", "## Kernel statistics (rocprofv3 --kernel-trace --stats)", "",
              "Every launch of the run, warm-up included (the bench also times the overlapped "
              "forward and the router after its steps).", "",
              "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = re.sub(r"\(anonymous namespace\)::", "", r["Name"]).split("(")[0]
        name = name.replace("void ", "").replace("moe::", "").replace("gemm::", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f} |")
    with open(os.path.join(ROOT, "profiles", f"kernels_{args.config}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def clock_summary(args):
    """profiles/clock_<config>.md from a --kernel-trace --pmc GRBM_GUI_ACTIVE GRBM_COUNT
    SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES run: per kernel, the shader clock over its
    dispatches (GRBM cycles, summed over the 8 XCD instances, divided by 8 and by the
    duration) and the MFMA-busy fraction (busy cycles over active cycles x 1024 SIMDs)."""
    rows = list(csv.DictReader(open(args.trace + "_counter_collection.csv")))
    by, meta = collections.defaultdict(dict), {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        by[d][r["Counter_Name"]] = float(r["Counter_Value"])
        meta[d] = r
    agg = collections.defaultdict(list)
    named = {int(r["Dispatch_Id"]): n for n, r in name_rows(list(meta.values()))}
    for d, r in meta.items():
        # kernels without a layer-step name (the FP8 GEMMs and quantisers) keep
        # their own, without namespace and argument list
        n = named.get(d) or "`" + re.sub(r"^void |moe::|\(anonymous namespace\)::|gemm::|\(.*\)$",
                                         "", r["Kernel_Name"]) + "`"
        if n == "copyBuffer" or "copyBuffer" in n:
            continue
        c = by[int(r["Dispatch_Id"])]
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        agg[n].append((dur, c.get("GRBM_COUNT", 0.0), c.get("GRBM_GUI_ACTIVE", 0.0),
                       c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)))
    lines = [f"# {args.config} layer: shader clock and MFMA busy per kernel", "",
             f"Workload: {args.workload or args.config}.", "",
             "Commands (run from the repository root on the MI355X):", ""]
    lines += [f"    {c.strip()}" for c in args.commands.split(";") if c.strip()]
    lines += ["", "GRBM counters are summed over the 8 XCD instances, so the clock is "
              "GRBM_COUNT / 8 / duration; MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES / "
              "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).  Kernels shorter than 50 us are "
              "dominated by counter set-up and are left out.", "",
              "| kernel | dispatches | avg us | clock GHz | MFMA busy % |", "|---|---|---|---|---|"]
    for n, v in sorted(agg.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        dur = sum(x[0] for x in v) / len(v)
        if dur < 50e3:
            continue
        cnt = sum(x[1] for x in v) / len(v)
        act = sum(x[2] for x in v) / len(v)
        mf = sum(x[3] for x in v) / len(v)
        lines.append(f"| {n} | {len(v)} | {dur / 1e3:.1f} | {cnt / 8 / dur:.2f} | "
                     f"{100 * mf / (act / 8 * 1024) if act else 0:.1f} |")
    with open(os.path.join(ROOT, "profiles", f"clock_{args.config}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-mib", type=int)
    ap.add_argument("--stats-only", action="store_true",
                    help="only the kernel statistics of the trace run (profiles/kernels_<config>.md)")
    ap.add_argument("--clock", action="store_true",
                    help="clock and MFMA-busy table of a GRBM/SQ counter run (profiles/clock_<config>.md)")
    ap.add_argument("--commands", required=True, help="the rocprofv3 commands, ';'-separated")
    ap.add_argument("--workload", default="")
    ap.add_argument("--skip", type=int, default=0,
                    help="warm-up launches per kernel left out of the 'timed avg' column")
    ap.add_argument("--dy-dispatch", action="store_true",
                    help="the row dispatch kernel moves dy (no forward dispatch kernel runs)")
    args = ap.parse_args()
    DY_DISPATCH["flag"] = args.dy_dispatch
    if args.stats_only:
        return stats_summary(args)
    if args.clock:
        return clock_summary(args)
    if not (args.fetch and args.write and args.calib_mib):
        raise SystemExit("--fetch, --write and --calib-mib are required without --stats-only")

    dur = trace_table(args.trace)
    fetch = counter_table(args.fetch, "FETCH_SIZE")
    write = counter_table(args.write, "WRITE_SIZE")
    mib_kib = args.calib_mib * 1024.0
    rf = mib_kib / max(fetch["copyBuffer"]) if fetch.get("copyBuffer") else None
    wf = mib_kib / max(write["copyBuffer"]) if write.get("copyBuffer") else None
    if rf is None or wf is None:
        raise SystemExit("no calibration copy in the counter runs (bench.py --calib-copy-mib)")

    total = sum(sum(v) for k, v in dur.items() if k != "copyBuffer")
    h = sources_hash()
    kernels = {}
    for n in sorted(fetch):
        if n == "copyBuffer" or n not in write:
            continue
        f = sum(fetch[n]) / len(fetch[n]) * 1024 * rf
        w = sum(write[n]) / len(write[n]) * 1024 * wf
        kernels[n] = {"fetch_bytes": int(f), "write_bytes": int(w)}
    rec = {"workload": args.workload or args.config, "source_sha256_16": h,
           "sources": GEMM_SOURCES, "read_factor": round(rf, 4), "write_factor": round(wf, 4),
           "kernels": kernels}
    base = os.path.join(ROOT, "profiles")
    with open(os.path.join(base, f"traffic_{args.config}_bf16.json"), "w") as fh:
        json.dump(rec, fh, indent=1)

    lines = [f"# {args.config} layer, bf16: per-kernel time and HBM traffic", "",
             f"Workload: {args.workload or args.config}.  GEMM source hash (sha256 of "
             f"{', '.join(os.path.basename(p) for p in GEMM_SOURCES)}, first 16 hex digits): "
             f"`{h}`.", "", "Commands (run from the repository root on the MI355X):", ""]
    lines += [f"    {c.strip()}" for c in args.commands.split(";") if c.strip()]
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              f"'timed avg' leaves out the first {args.skip} launches of each kernel (the bench's "
              "warm-up steps), matching the steps bench.py times.", "",
              "| kernel | calls | avg us | timed avg us | min us | max us | % of GPU time |",
              "|---|---|---|---|---|---|---|"]
    for n, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        if n == "copyBuffer":
            continue
        per_step = len(v) // (len(dur["combine"]) if dur.get("combine") else len(v)) or 1
        timed = v[args.skip * per_step:] or v
        lines.append(f"| {n} | {len(v)} | {sum(v) / len(v):.1f} | {sum(timed) / len(timed):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} | {100 * sum(v) / total:.1f} |")
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"Calibration: the runs copy {args.calib_mib} MiB device-to-device first; FETCH_SIZE "
              f"reads {max(fetch['copyBuffer']):.0f} KiB and WRITE_SIZE {max(write['copyBuffer']):.0f} "
              f"KiB for it, so reads are scaled by {rf:.3f} and writes by {wf:.3f}.", "",
              "| kernel | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | scaled read GB | scaled write GB |",
              "|---|---|---|---|---|"]
    for n, k in kernels.items():
        fk = sum(fetch[n]) / len(fetch[n])
        wk = sum(write[n]) / len(write[n])
        lines.append(f"| {n} | {fk:.0f} | {wk:.0f} | {k['fetch_bytes'] / 1e9:.3f} | "
                     f"{k['write_bytes'] / 1e9:.3f} |")
    with open(os.path.join(base, f"layer_{args.config}_bf16.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
