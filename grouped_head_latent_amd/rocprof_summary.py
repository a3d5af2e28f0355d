"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    # per-kernel durations (rocprofv3 --kernel-trace --stats ... --output-format csv);
    # with the traced bench.py run's JSON line, also the workload's rate from the trace
    python -m grouped_head_latent_amd.rocprof_summary trace <out_dir> <summary.md> --command "..." \\
        [--bench-json <bench_stdout>]
    # counters of one --pmc run (FETCH_SIZE, WRITE_SIZE, SQ_* ...)
    python -m grouped_head_latent_amd.rocprof_summary pmc <out_dir> <summary.md> --command "..."
    # a plain copy of known size, profiled to calibrate FETCH_SIZE / WRITE_SIZE
    python -m grouped_head_latent_amd.rocprof_summary copy
    # HBM traffic record for bench.py (fetch run, write run, copy calibration runs)
    python -m grouped_head_latent_amd.rocprof_summary traffic <fetch_dir> <write_dir> \\
        <copy_fetch_dir> <copy_write_dir> <kernel_substring> <source_file> <out.json>

Nothing here runs on import; the module only reads CSV files that rocprofv3
wrote and writes text.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

COPY_BYTES = 2 * 1024 * 1024 * 1024  # bytes read and bytes written by the calibration copy


def _find(out_dir: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(out_dir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {out_dir}")
    return hits[0]


def _short(name: str, width: int = 90) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= width else name[: width - 3] + "..."


def trace_summary(out_dir: str) -> list[dict]:
    """Per-kernel dispatch count and durations from a --kernel-trace CSV."""
    path = _find(out_dir, "kernel_trace.csv")
    per = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = []
    for name, d in per.items():
        rows.append({"kernel": name, "calls": len(d), "total_us": sum(d), "avg_us": statistics.mean(d),
                     "min_us": min(d), "max_us": max(d)})
    rows.sort(key=lambda r: -r["total_us"])
    return rows


def pmc_summary(out_dir: str) -> dict:
    """Counter value per dispatch (mean over dispatches) per kernel."""
    path = _find(out_dir, "counter_collection.csv")
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: statistics.mean(v) for c, v in d.items()} for k, d in per.items()}


PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2516.6


def _md_trace(rows, command, bench=None):
    out = ["# rocprofv3 kernel trace", "", f"Command: `{command}`", "",
           "| kernel | calls | avg us | min us | max us | total us |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['kernel'])}` | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | "
                   f"{r['max_us']:.1f} | {r['total_us']:.1f} |")
    if bench:
        # one workload per traced run: a call of the path is one dispatch of
        # each of the library's kernels, so its time from the trace is the sum
        # of their average durations (torch's input-preparation kernels left out)
        lib = [r for r in rows if r["kernel"].lstrip().split("(")[0].split("<")[0].split()[-1].startswith("gha::")]
        t_us = sum(r["avg_us"] for r in lib)
        out += ["", "Roofline from this trace (algorithmic work of the workload from the same run's bench line; "
                "the path's time per call = the sum of the library kernels' average durations above; the bound "
                "is MFMA when FLOP per byte exceeds the ridge of the two peaks, else HBM):", "",
                "| workload | HIP-event ms per call | trace us per call | algorithmic | bound | rate from trace | of peak |",
                "|---|---|---|---|---|---|---|"]
        ridge = PEAK_BF16_TFLOPS * 1e3 / PEAK_HBM_GBPS  # FLOP per byte
        for name, e in bench.items():
            nbytes, flops = e.get("bytes"), e.get("flops")
            work = " + ".join(x for x in (f"{nbytes:.4g} B" if nbytes else "", f"{flops:.4g} FLOP" if flops else "") if x)
            if nbytes and not (flops and flops / nbytes > ridge):
                rate = nbytes / (t_us * 1e3)
                bound, frac, unit = "HBM", rate / PEAK_HBM_GBPS, "GB/s"
            else:
                rate = (flops or 0.0) / (t_us * 1e6)
                bound, frac, unit = "MFMA", rate / PEAK_BF16_TFLOPS, "TFLOP/s"
            out.append(f"| {name} | {e['ms']:.4f} | {t_us:.1f} | {work} | {bound} | {rate:.1f} {unit} | {frac:.3f} |")
    return "\n".join(out) + "\n"


def _bench_workloads(path):
    """The workloads of one bench.py JSON line: {name: record}."""
    line = [l for l in open(path) if l.startswith("{")][-1]
    d = json.loads(line)
    w = dict(d.get("extras", {}))
    if "ms_per_step" in d:
        w["gqa_prefill"] = {"ms": d["ms_per_step"], "flops": d["roofline"]["achieved"] * d["ms_per_step"] * 1e9}
    return w


def _md_pmc(d, command):
    out = ["# rocprofv3 counters (mean per dispatch)", "", f"Command: `{command}`", ""]
    for k, cs in d.items():
        out.append(f"## `{_short(k)}`")
        out.append("")
        out.append("| counter | value |")
        out.append("|---|---|")
        for c, v in sorted(cs.items()):
            out.append(f"| {c} | {v:.6g} |")
        out.append("")
    return "\n".join(out)


def copy_for_calibration(nbytes: int = COPY_BYTES):
    """One device copy of nbytes (reads nbytes, writes nbytes).  A streaming
    copy much larger than the 256 MB last-level cache, so its reads reach HBM
    with the same request sizes as the kernels' streaming reads."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def _kernel_value(d: dict, substr: str, counter: str) -> float:
    hits = [cs[counter] for k, cs in d.items() if substr in k and counter in cs]
    if not hits:
        raise KeyError(f"{counter} for a kernel matching {substr!r}")
    return hits[0]


def _largest_dispatch(out_dir: str, substr: str, counter: str) -> float:
    """The largest per-dispatch value of a counter for kernels matching substr
    (the calibration copy is the largest copy in its run)."""
    path = _find(out_dir, "counter_collection.csv")
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise KeyError(f"{counter} for a kernel matching {substr!r}")
    return max(vals)


def traffic_record(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernel, source) -> dict:
    fetch = pmc_summary(fetch_dir)
    write = pmc_summary(write_dir)
    cf = _largest_dispatch(copy_fetch_dir, "copyBuffer", "FETCH_SIZE")
    cw = _largest_dispatch(copy_write_dir, "copyBuffer", "WRITE_SIZE")
    f_kib = _kernel_value(fetch, kernel, "FETCH_SIZE")
    w_kib = _kernel_value(write, kernel, "WRITE_SIZE")
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    src = open(source, "rb").read()
    return {"kernel": kernel, "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
            "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "bytes_per_dispatch": f_kib * 1024 * f_scale + w_kib * 1024 * w_scale,
            "source": os.path.relpath(source, os.path.dirname(os.path.dirname(os.path.abspath(__file__)))),
            "source_sha256": hashlib.sha256(src).hexdigest()}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace"); t.add_argument("out_dir"); t.add_argument("md"); t.add_argument("--command", default="")
    t.add_argument("--bench-json", default=None, help="the traced bench.py run's JSON line (one workload)")
    p = sub.add_parser("pmc"); p.add_argument("out_dir"); p.add_argument("md"); p.add_argument("--command", default="")
    sub.add_parser("copy")
    tr = sub.add_parser("traffic")
    for n in ("fetch_dir", "write_dir", "copy_fetch_dir", "copy_write_dir", "kernel", "source", "out"):
        tr.add_argument(n)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        bench = _bench_workloads(a.bench_json) if a.bench_json else None
        open(a.md, "w").write(_md_trace(trace_summary(a.out_dir), a.command, bench))
    elif a.cmd == "pmc":
        open(a.md, "w").write(_md_pmc(pmc_summary(a.out_dir), a.command))
    elif a.cmd == "copy":
        copy_for_calibration()
    elif a.cmd == "traffic":
        rec = traffic_record(a.fetch_dir, a.write_dir, a.copy_fetch_dir, a.copy_write_dir, a.kernel, a.source)
        db = json.load(open(a.out)) if os.path.exists(a.out) else {}
        db[a.kernel] = rec
        json.dump(db, open(a.out, "w"), indent=1, sort_keys=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
