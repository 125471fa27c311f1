"""Summaries of rocprofv3 CSV output (host-side text processing only).

    python -m post_weight_quantization_19_amd.profiling stats DIR --command CMD --out FILE.md
        per-kernel call count / average / total from DIR/*_kernel_stats.csv
    python -m post_weight_quantization_19_amd.profiling traffic --fetch DIR --write DIR \
            --kernel NAME --algorithmic-bytes B --source FILE --command CMD ... --out FILE.json
    python -m post_weight_quantization_19_amd.profiling kernels --trace DIR --sq DIR \
            --fetch DIR --write DIR --kernel NAME[=PEAK] ... --command CMD ... --out FILE.md
        per-kernel MFMA rate, MFMA busy fraction, clock and HBM bytes
        HBM bytes per launch of one kernel from two --pmc runs (FETCH_SIZE,
        WRITE_SIZE in KiB per dispatch), each scaled by what the same counter
        reads for the 1 GiB device copy in the same run.

The scale factors exist because FETCH_SIZE/WRITE_SIZE count cache-line
requests of particular sizes; a plain copy of known size calibrates them.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

COPY_KERNEL = "copyBuffer"
COPY_KIB = 1 << 20          # the calibration copy moves 1 GiB each way


def _one(pattern):
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def short_name(name: str) -> str:
    """Kernel name without namespaces and argument list (template arguments kept)."""
    s = re.sub(r"^void\s+", "", name.replace("(anonymous namespace)::", ""))
    depth = 0
    for i, ch in enumerate(s):
        depth += (ch == "<") - (ch == ">")
        if ch == "(" and depth == 0:
            s = s[:i]
            break
    head = s.split("<", 1)[0]
    return head.split("::")[-1] + s[len(head):]


def kernel_stats(d):
    rows = []
    with open(_one(os.path.join(d, "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3,
                         "total_ms": float(r["TotalDurationNs"]) / 1e6,
                         "pct": float(r["Percentage"]),
                         "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3})
    return rows


def launch_durations_us(d, kernel):
    """Durations of every launch of one kernel, in launch order (kernel trace)."""
    out = []
    with open(_one(os.path.join(d, "*kernel_trace.csv"))) as f:
        for r in csv.DictReader(f):
            if short_name(r["Kernel_Name"]) == kernel:
                out.append((int(r["Start_Timestamp"]),
                            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    return [x for _, x in sorted(out)]


def stats_markdown(d, command, title, launches=None, bench_log=None):
    rows = kernel_stats(d)
    out = [f"# {title}", "", "Command (from the repository root):", "", "```", command, "```",
           "", "| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | % |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {r['name']} | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | "
                   f"{r['max_us']:.1f} | {r['total_ms']:.3f} | {r['pct']:.2f} |")
    if launches:
        d_us = launch_durations_us(d, launches)
        out += ["", f"Every launch of {launches}, in order (us):", "",
                " ".join(f"{x:.1f}" for x in d_us)]
        if bench_log:
            line = None
            with open(bench_log) as f:
                for ln in f:
                    if ln.startswith("{"):
                        line = json.loads(ln)
            if line is not None:
                rf = line["roofline"]
                k, w = line["steps"], line["warmup"]
                # launches before the timed steps: the first call and the warmup steps
                timed = d_us[1 + w:1 + w + k]
                out += ["", f"bench.py's own HIP-event average over its {k} timed launches: "
                        f"{rf['avg_launch_ms'] * 1e3:.1f} us; the same {len(timed)} launches "
                        f"in this trace (launches {2 + w}..{1 + w + k}): "
                        f"{sum(timed) / max(len(timed), 1):.1f} us; "
                        f"achieved {rf['achieved']:.1f} {rf['unit']} = "
                        f"{100 * rf['frac']:.1f}% of {rf['peak']:.0f}."]
    return "\n".join(out) + "\n"


def counter_per_dispatch(d, counter):
    """{short kernel name: [value per dispatch ...]} for one counter."""
    vals = {}
    with open(_one(os.path.join(d, "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_dir, write_dir, kernel, algorithmic_bytes, source, commands, title,
            workload, x_layout=None):
    fv = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    wv = counter_per_dispatch(write_dir, "WRITE_SIZE")

    def pick(vals, key):
        for k, v in vals.items():
            if key in k:
                return v
        raise SystemExit(f"kernel {key} not in the counter run")
    kf, kw = pick(fv, kernel), pick(wv, kernel)
    cf, cw = pick(fv, COPY_KERNEL), pick(wv, COPY_KERNEL)
    f_fac = COPY_KIB / max(cf)
    w_fac = COPY_KIB / max(cw)
    fkib = sum(kf) / len(kf)
    wkib = sum(kw) / len(kw)
    rd = fkib * f_fac * 1024
    wr = wkib * w_fac * 1024
    with open(source, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    return {
        "title": title, "kernel": kernel, "workload": workload, "x_layout": x_layout,
        "commands": commands,
        "fetch_size_kib_per_dispatch": fkib, "fetch_dispatches": len(kf),
        "write_size_kib_per_dispatch": wkib, "write_dispatches": len(kw),
        "calibration": {"kernel": "1 GiB device-to-device copy (bench.py --copy-calibration)",
                        "fetch_size_kib": max(cf), "write_size_kib": max(cw),
                        "known_kib_each_way": COPY_KIB, "fetch_factor": f_fac,
                        "write_factor": w_fac},
        "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": algorithmic_bytes,
        "kernel_source": os.path.relpath(source), "kernel_source_sha256": sha,
    }


def _dispatches(d, counters=None):
    """{short kernel name: {dispatch id: {counter: value, "_ns": duration}}}
    from one counter-collection run."""
    out = {}
    with open(_one(os.path.join(d, "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if counters and r["Counter_Name"] not in counters:
                continue
            k = short_name(r["Kernel_Name"])
            disp = out.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
            disp[r["Counter_Name"]] = disp.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            disp["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def kernels_markdown(trace, sq, fetch, write, kernels, commands, title, peaks):
    """Per kernel: launch statistics from the kernel trace; MFMA work, MFMA
    busy cycles and the shader clock from the SQ run; HBM bytes from the
    FETCH_SIZE / WRITE_SIZE runs, each scaled by what the same counter reads
    for the 1 GiB device copy of that run.  Rates are totals over every
    dispatch of the kernel in the counter run divided by the summed dispatch
    durations of that run."""
    st = {r["name"]: r for r in kernel_stats(trace)}
    sqd = _dispatches(sq)
    fd = _dispatches(fetch, {"FETCH_SIZE"})
    wd = _dispatches(write, {"WRITE_SIZE"})

    def copy_factor(dd, counter):
        for k, v in dd.items():
            if COPY_KERNEL in k:
                return COPY_KIB / max(x[counter] for x in v.values())
        raise SystemExit(f"no {COPY_KERNEL} dispatch in the {counter} run")
    ff, wf = copy_factor(fd, "FETCH_SIZE"), copy_factor(wd, "WRITE_SIZE")

    def pick(dd, key):
        for k, v in dd.items():
            if k == key:
                return list(v.values())
        raise SystemExit(f"kernel {key} not in a counter run")
    out = [f"# {title}", "", "Commands (from the repository root):", "", "```"] + commands + [
        "```", "",
        "Launch statistics come from the kernel trace; every other column is a total over all "
        "dispatches of the kernel in the counter run (MOPS x 512 = flop) divided by their summed "
        "durations in that run.  MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x the "
        "summed duration x 2.4 GHz.  Clock: GRBM_GUI_ACTIVE / (8 XCDs x duration), "
        "the shader clock the kernel ran at, shown for kernels of 1 ms or more (the counters "
        "of shorter dispatches include cycles outside them).  HBM "
        f"bytes: FETCH_SIZE x {ff:.3f} and WRITE_SIZE x {wf:.3f} KiB (factors from the 1 GiB "
        "device copy of each run).", "",
        "| kernel | calls | avg (us) | total (ms) | MFMA TFLOP/s | % of peak | MFMA busy "
        "| clock (GHz) | read GB/dispatch | write GB/dispatch | HBM GB/s |",
        "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k in kernels:
        t = st.get(k)
        sq_v = pick(sqd, k)
        ns = sum(x["_ns"] for x in sq_v)
        flop = 512.0 * sum(x.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) +
                           x.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) +
                           x.get("SQ_INSTS_VALU_MFMA_MOPS_F64", 0.0) for x in sq_v)
        busy = sum(x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in sq_v) / (1024 * ns * 2.4)
        gui = sum(x.get("GRBM_GUI_ACTIVE", 0.0) for x in sq_v)
        clk = f"{gui / (8 * ns):.2f}" if gui > 0 and ns / len(sq_v) >= 1e6 else "—"
        peak = peaks.get(k)
        tf = flop / ns / 1e3
        fv, wv = pick(fd, k), pick(wd, k)
        rd = sum(x["FETCH_SIZE"] for x in fv) * ff * 1024
        wr = sum(x["WRITE_SIZE"] for x in wv) * wf * 1024
        fns = sum(x["_ns"] for x in fv) + sum(x["_ns"] for x in wv)
        out.append(
            f"| {k} | {t['calls'] if t else '-'} | {t['avg_us'] if t else 0:.1f} | "
            f"{t['total_ms'] if t else 0:.3f} | {tf:.1f} | "
            f"{(100 * tf / peak) if peak else float('nan'):.1f} | {busy:.3f} | {clk} | "
            f"{rd / len(fv) / 1e9:.4f} | {wr / len(wv) / 1e9:.4f} | "
            f"{(rd + wr) / (fns / 2) :.1f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--launches", help="list every launch of this kernel")
    s.add_argument("--bench-log", help="bench.py output of the same run (JSON line)")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--algorithmic-bytes", type=float, required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--command", action="append", required=True)
    t.add_argument("--title", default="HBM traffic per launch")
    t.add_argument("--workload", default="")
    t.add_argument("--x-layout", default=None, help="X layout the counters were taken with")
    t.add_argument("--out", required=True)
    kk = sub.add_parser("kernels")
    kk.add_argument("--trace", required=True)
    kk.add_argument("--sq", required=True)
    kk.add_argument("--fetch", required=True)
    kk.add_argument("--write", required=True)
    kk.add_argument("--kernel", action="append", required=True,
                    help="short kernel name, optionally NAME=PEAK_TFLOPS")
    kk.add_argument("--command", action="append", required=True)
    kk.add_argument("--title", default="rocprofv3 counters per kernel")
    kk.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        txt = stats_markdown(a.dir, a.command, a.title, a.launches, a.bench_log)
    elif a.cmd == "kernels":
        names, peaks = [], {}
        for spec in a.kernel:
            nm, _, pk = spec.partition("=")
            names.append(nm)
            if pk:
                peaks[nm] = float(pk)
        txt = kernels_markdown(a.trace, a.sq, a.fetch, a.write, names, a.command, a.title, peaks)
    else:
        txt = json.dumps(traffic(a.fetch, a.write, a.kernel, a.algorithmic_bytes, a.source,
                                 a.command, a.title, a.workload, a.x_layout), indent=1) + "\n"
    with open(a.out, "w") as f:
        f.write(txt)
    sys.stdout.write(txt)


if __name__ == "__main__":
    main()
