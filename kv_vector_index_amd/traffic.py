"""HBM traffic records from rocprofv3 counter runs.

Two sub-commands:

    python -m kv_vector_index_amd.traffic copy --mib 512 --reps 4
        runs a plain device-to-device copy of a known size, the calibration kernel for the
        FETCH_SIZE / WRITE_SIZE counters;

    python -m kv_vector_index_amd.traffic record --fetch DIR --write DIR \\
            --copy-fetch DIR --copy-write DIR --copy-mib 512 --workload W --instances N --out FILE
        reads the counter CSVs that `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` wrote
        for a decode run and for the copy run, scales every kernel's per-dispatch KiB by the
        factor that makes the copy kernel read and write exactly its known size, and writes a
        JSON record of HBM bytes per launch for the decode kernels, tagged with a hash of the
        decode kernels' source so that a record taken from older kernels is not reported.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE_KERNELS = {"score": "k_score", "select": "k_select", "attend": "k_attend", "merge": "k_merge"}


DECODE_SOURCES = ("wi_decode.hip", "wi_device.h", "wi_internal.h", "wi_api.hip")


def decode_source_hash() -> str:
    """sha256 (first 16 hex digits) over every source the decode kernels and their launch
    configuration are compiled from."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "kv_vector_index_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def per_kernel_kib(directory: str, counter: str) -> dict:
    """Average per-dispatch value of `counter` for every kernel name in a rocprofv3 CSV run."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    per_dispatch = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (fn, row["Dispatch_Id"])
                name = row["Kernel_Name"]
                v = float(row["Counter_Value"])
                if key in per_dispatch:
                    per_dispatch[key] = (name, per_dispatch[key][1] + v)
                else:
                    per_dispatch[key] = (name, v)
    sums = {}
    for name, v in per_dispatch.values():
        s, n = sums.get(name, (0.0, 0))
        sums[name] = (s + v, n + 1)
    return {name: {"kib": s / n, "dispatches": n} for name, (s, n) in sums.items()}


def match(table: dict, fragment: str) -> dict:
    hits = {k: v for k, v in table.items() if fragment in k}
    if not hits:
        raise KeyError(f"no kernel matching {fragment!r}")
    kib = sum(v["kib"] * v["dispatches"] for v in hits.values())
    n = sum(v["dispatches"] for v in hits.values())
    return {"kib": kib / n, "dispatches": n, "names": sorted(hits)}


def cmd_copy(args):
    import torch
    n = args.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": args.reps}), flush=True)


def cmd_record(args):
    nbytes = args.copy_mib << 20
    cf = per_kernel_kib(args.copy_fetch, "FETCH_SIZE")
    cw = per_kernel_kib(args.copy_write, "WRITE_SIZE")
    # the calibration kernel: the one that moved the most bytes in the copy run
    copy_name = max(cf, key=lambda k: cf[k]["kib"])
    f_fetch = nbytes / (cf[copy_name]["kib"] * 1024.0)
    f_write = nbytes / (cw[copy_name]["kib"] * 1024.0)
    df = per_kernel_kib(args.fetch, "FETCH_SIZE")
    dw = per_kernel_kib(args.write, "WRITE_SIZE")
    out = {"kernel_source_sha256_16": decode_source_hash(), "kernel_sources": list(DECODE_SOURCES),
           "workload": args.workload, "instances": args.instances,
           "calibration": {"kernel": copy_name, "bytes": nbytes,
                           "fetch_kib": cf[copy_name]["kib"], "write_kib": cw[copy_name]["kib"],
                           "fetch_factor": f_fetch, "write_factor": f_write},
           "hbm_bytes_per_launch": {}, "raw": {}}
    for key, frag in DECODE_KERNELS.items():
        try:
            a, b = match(df, frag), match(dw, frag)
        except KeyError:
            continue
        fetch_b = a["kib"] * 1024.0 * f_fetch
        write_b = b["kib"] * 1024.0 * f_write
        out["hbm_bytes_per_launch"][key] = fetch_b + write_b
        out["raw"][key] = {"fetch_kib": a["kib"], "write_kib": b["kib"], "dispatches": a["dispatches"],
                           "fetch_bytes": fetch_b, "write_bytes": write_b, "kernels": a["names"]}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out["hbm_bytes_per_launch"]))
    if args.md:
        write_md(out, args)


def write_md(rec: dict, args):
    """A markdown summary of a record: measured HBM bytes per launch of each decode kernel beside
    the algorithmic bytes the bench run of the same workload reported."""
    algo = {}
    if args.bench:
        with open(args.bench) as f:
            algo = json.loads(f.read().strip().splitlines()[-1]).get("kernel_algorithmic_bytes", {})
    cal = rec["calibration"]
    lines = [f"# HBM traffic of the decode kernels, {rec['workload']} (rocprofv3 FETCH_SIZE / WRITE_SIZE)", ""]
    if args.cmd:
        lines += ["Commands (repo root, one MI355X):", ""] + ["    " + c for c in args.cmd] + [""]
    lines += [f"Decode kernel sources sha256/16: {rec['kernel_source_sha256_16']}; index copies cycled: "
              f"{rec['instances']}.", "",
              f"Calibration: `{cal['kernel']}` copying {cal['bytes']} bytes reads {cal['fetch_kib']:.0f} KiB "
              f"(FETCH_SIZE) and writes {cal['write_kib']:.0f} KiB (WRITE_SIZE) per dispatch: factors "
              f"{cal['fetch_factor']:.4f} and {cal['write_factor']:.4f} turn the counters into bytes.", "",
              "| kernel | dispatches | FETCH bytes | WRITE bytes | HBM bytes / launch | algorithmic bytes / launch | "
              "HBM / algorithmic |", "|---|---|---|---|---|---|---|"]
    for key, r in rec["raw"].items():
        tot = rec["hbm_bytes_per_launch"][key]
        a = algo.get(key)
        ratio = f"{tot / a:.3f}" if a else "-"
        lines.append(f"| {key} | {r['dispatches']} | {r['fetch_bytes']:.4g} | {r['write_bytes']:.4g} | {tot:.4g} | "
                     f"{a if a is not None else '-'} | {ratio} |")
    with open(args.md, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=512)
    c.add_argument("--reps", type=int, default=4)
    r = sub.add_parser("record")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        r.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    r.add_argument("--copy-mib", type=int, default=512)
    r.add_argument("--workload", required=True, help="the bench workload the decode run measured")
    r.add_argument("--instances", type=int, required=True, help="index copies that bench run cycled through")
    r.add_argument("--out", required=True)
    r.add_argument("--md", default="", help="also write a markdown summary here")
    r.add_argument("--bench", default="", help="a bench.py JSON line of the same workload (algorithmic bytes)")
    r.add_argument("--cmd", action="append", default=[], help="commands to list in the summary")
    args = ap.parse_args(argv)
    return cmd_copy(args) if args.cmd == "copy" else cmd_record(args)


if __name__ == "__main__":
    sys.exit(main())
