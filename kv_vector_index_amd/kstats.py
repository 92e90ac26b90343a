"""Kernel durations and matrix-core use from rocprofv3 runs of bench.py, as markdown summaries.

    python -m kv_vector_index_amd.kstats times --trace DIR --bench FILE [--cmd "..."] --out FILE.md
        reads the kernel trace (`rocprofv3 --kernel-trace --stats --output-format csv -d DIR`) of
        a bench.py run and the JSON line that run printed; for each decode kernel it reports the
        dispatches that ran as single launches inside decode steps (graph replays, warm-up) and
        those the profiling pass launched back to back (each repeat reading another copy of the
        index), their average durations, and the roofline position the bench's algorithmic bytes
        per launch give with each, next to the figure the bench measured live with HIP events.

    python -m kv_vector_index_amd.kstats mfma --pmc DIR --trace DIR --kernel NAME --flops F \\
            --peak-tflops P [--cmd "..."] --out FILE.md
        reads a counter run (`rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
        SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES ...`) and a kernel trace of the same command;
        for the kernels whose name contains NAME it reports the matrix operations the counters
        saw (MOPS x 512 flops) against the algorithmic F flops per launch, the duration, the
        achieved rate against the peak, and the matrix cores' busy share of the busy CU cycles.

    python -m kv_vector_index_amd.kstats build --trace DIR --bench FILE [--cmd "..."] --out FILE.md
        reads the kernel trace of a `bench.py --build-only` run and lists every library kernel
        with its calls, average and total duration.
"""
import argparse
import csv
import glob
import json
import os
import sys

DECODE_KERNELS = {"score": "k_score", "select": "k_select", "attend": "k_attend", "merge": "k_merge"}


def _rows(directory: str, suffix: str):
    files = glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    for fn in sorted(files):
        with open(fn, newline="") as f:
            yield from csv.DictReader(f)


def dispatches(trace_dir: str):
    """[(dispatch id, kernel name, start ns, end ns)] in dispatch order."""
    out = []
    for r in _rows(trace_dir, "kernel_trace.csv"):
        out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out.sort()
    return out


def split_single_and_repeat(ds):
    """Per kernel name: durations (us) of dispatches launched alone between other kernels, and of
    those launched back to back with the same kernel (the profiling pass's repeats)."""
    single, rep = {}, {}
    for i, (_, name, t0, t1) in enumerate(ds):
        same = (i > 0 and ds[i - 1][1] == name) or (i + 1 < len(ds) and ds[i + 1][1] == name)
        (rep if same else single).setdefault(name, []).append((t1 - t0) / 1e3)
    return single, rep


def _find(table: dict, frag: str):
    vals = [v for k, vs in table.items() if frag in k for v in vs]
    names = sorted(k for k in table if frag in k)
    return vals, names


def kernel_stats(trace_dir: str):
    """[(kernel name, calls, average us, min us, max us)] from the --stats summary of a trace."""
    try:
        rows = list(_rows(trace_dir, "kernel_stats.csv"))
    except FileNotFoundError:
        return []
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
             float(r["MaxNs"]) / 1e3) for r in rows]


def cmd_times(args):
    with open(args.bench) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    single, rep = split_single_and_repeat(dispatches(args.trace))
    peak = float(bench["roofline"]["peak"])
    live = bench.get("kernel_avg_us", {})
    nbytes = bench.get("kernel_algorithmic_bytes", {})
    lines = [f"# Decode kernel durations, {bench['config']['workload']} (rocprofv3 kernel trace)", ""]
    if args.cmd:
        lines += ["Command (repo root, one MI355X):", "", "    " + args.cmd, ""]
    lines += [f"Step: {bench['ms_per_step'] * 1e3:.2f} us ({bench['value']:.0f} steps/s, "
              f"{bench['config'].get('timing', '')}, {bench['config'].get('instances')} index copies).", "",
              "| kernel | in steps: dispatches | avg us | back-to-back repeats: dispatches | avg us | "
              "bench live (HIP events) us | algorithmic bytes / launch | GB/s (repeats) | frac of "
              f"{peak:.0f} GB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for key, frag in DECODE_KERNELS.items():
        s, names = _find(single, frag)
        r, _ = _find(rep, frag)
        if not names and not r:
            continue
        avg_s = sum(s) / len(s) if s else float("nan")
        avg_r = sum(r) / len(r) if r else float("nan")
        b = nbytes.get(key)
        gbs = b / (avg_r * 1e-6) / 1e9 if (b and r) else None
        lines.append(f"| {key} | {len(s)} | {avg_s:.2f} | {len(r)} | {avg_r:.2f} | "
                     f"{live.get(key, float('nan')):.2f} | {b if b is not None else '-'} | "
                     f"{'-' if gbs is None else f'{gbs:.0f}'} | {'-' if gbs is None else f'{gbs / peak:.3f}'} |")
    rl = bench["roofline"]
    lines += ["", f"Bench roofline line: kernel {rl['kernel']}, {rl['achieved']:.0f} GB/s, frac {rl['frac']:.3f} "
              f"({rl.get('bytes_per_launch')} bytes / {rl.get('avg_launch_us', float('nan')):.2f} us)."]
    stats = kernel_stats(args.trace)
    if stats:
        lines += ["", "rocprofv3 --stats (every dispatch of the run, decode kernels):", "",
                  "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        for name, calls, avg, mn, mx in stats:
            if any(frag in name for frag in DECODE_KERNELS.values()):
                lines.append(f"| `{name}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_build(args):
    """Every library kernel of an index-build bench run: calls, average and total duration."""
    with open(args.bench) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    cfg = bench["config"]
    lines = [f"# Index build kernels, {cfg['workload']} (rocprofv3 kernel trace)", ""]
    if args.cmd:
        lines += ["Command (repo root, one MI355X):", "", "    " + args.cmd, ""]
    lines += [f"Build: {bench['ms_per_step']:.3f} ms per index ({cfg['batch']} x {cfg['kv_heads']} KV heads, "
              f"{cfg['context']} tokens, segments of {cfg['segment']}, {cfg['clusters_per_segment']} clusters each, "
              f"{cfg['iterations']} iterations); k_assign {bench['roofline']['achieved']:.0f} TFLOP/s on the "
              f"algorithmic flops (frac {bench['roofline']['frac']:.3f} of {bench['roofline']['peak']:.0f}).", "",
              "| kernel | calls | average us | total us | share of the library's kernel time |", "|---|---|---|---|---|"]
    stats = [s for s in kernel_stats(args.trace) if s[0].startswith(("void wi::", "wi::"))]
    total = sum(c * a for _, c, a, _, _ in stats)
    for name, calls, avg, _, _ in stats:
        lines.append(f"| `{name}` | {calls} | {avg:.2f} | {calls * avg:.1f} | {calls * avg / total:.3f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def per_dispatch_counters(pmc_dir: str):
    """{dispatch id: (kernel name, {counter: value summed over the dispatch's rows})}."""
    out = {}
    for r in _rows(pmc_dir, "counter_collection.csv"):
        key = int(r["Dispatch_Id"])
        name, cs = out.setdefault(key, (r["Kernel_Name"], {}))
        c = r["Counter_Name"]
        cs[c] = cs.get(c, 0.0) + float(r["Counter_Value"])
    return out


def cmd_mfma(args):
    pmc = per_dispatch_counters(args.pmc)
    sel = [(n, cs) for n, cs in pmc.values() if args.kernel in n]
    if not sel:
        raise SystemExit(f"no dispatch of a kernel matching {args.kernel!r}")
    counters = sorted({c for _, cs in sel for c in cs})
    avg = {c: sum(cs.get(c, 0.0) for _, cs in sel) / len(sel) for c in counters}
    single, rep = split_single_and_repeat(dispatches(args.trace))
    durs, _ = _find(single, args.kernel)
    r, _ = _find(rep, args.kernel)
    durs = durs + r
    dur = sum(durs) / len(durs)
    lines = [f"# Matrix-core use of {args.kernel} (rocprofv3 counters)", ""]
    if args.cmd:
        lines += ["Commands (repo root, one MI355X):", ""] + ["    " + c for c in args.cmd] + [""]
    lines += [f"Dispatches: {len(sel)} counted, {len(durs)} timed; kernels: {sorted({n for n, _ in sel})}", "",
              "| counter | average per dispatch |", "|---|---|"]
    lines += [f"| {c} | {avg[c]:.6g} |" for c in counters]
    lines += ["", f"Average duration: {dur:.2f} us."]
    mops = [c for c in counters if c.startswith("SQ_INSTS_VALU_MFMA_MOPS")]
    if mops:
        flops_ctr = 512.0 * sum(avg[c] for c in mops)
        lines.append(f"Matrix flops by the counters (MOPS x 512): {flops_ctr:.6g} per dispatch; "
                     f"algorithmic flops per launch: {args.flops:.6g} (ratio {flops_ctr / args.flops:.3f}).")
        lines.append(f"Rate on the counted flops: {flops_ctr / (dur * 1e-6) / 1e12:.1f} TFLOP/s = "
                     f"{flops_ctr / (dur * 1e-6) / 1e12 / args.peak_tflops:.3f} of {args.peak_tflops:.0f}; on the "
                     f"algorithmic flops: {args.flops / (dur * 1e-6) / 1e12:.1f} TFLOP/s = "
                     f"{args.flops / (dur * 1e-6) / 1e12 / args.peak_tflops:.3f}.")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "SQ_BUSY_CU_CYCLES" in avg and avg["SQ_BUSY_CU_CYCLES"] > 0:
        lines.append(f"SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES = "
                     f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_BUSY_CU_CYCLES']:.3f}.")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("times")
    t.add_argument("--trace", required=True)
    t.add_argument("--bench", required=True)
    t.add_argument("--cmd", default="")
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--trace", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--flops", type=float, required=True)
    m.add_argument("--peak-tflops", type=float, required=True)
    m.add_argument("--cmd", action="append", default=[])
    m.add_argument("--out", required=True)
    bl = sub.add_parser("build")
    bl.add_argument("--trace", required=True)
    bl.add_argument("--bench", required=True)
    bl.add_argument("--cmd", default="")
    bl.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    return {"times": cmd_times, "mfma": cmd_mfma, "build": cmd_build}[args.cmd_name](args)


if __name__ == "__main__":
    sys.exit(main())
