"""Summarise rocprofv3 CSV output of bench.py into a short markdown file.

Inputs are three rocprofv3 output folders made from bench.py:
  --trace  a `--kernel-trace --stats --output-format csv` run (kernel durations),
  --fetch  a `--pmc FETCH_SIZE --output-format csv` run with `--copy-mb N`,
  --write  a `--pmc WRITE_SIZE --output-format csv` run with `--copy-mb N`.

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch. They are scaled
by what the same counter reads for the plain device copy of N MiB that
`bench.py --copy-mb N` launches (`__amd_rocclr_copyBuffer`, N MiB read and N
MiB written): factor = N MiB / counter reading. The summary records the
SHA-256 of the decode kernel's source, so a reader (bench.py) can tell when
the kernel has changed since the counters were taken.

usage: python -m mla_decode_fwd_amd.profile_summary --trace D1 --fetch D2 --write D3
           --copy-mb N --command "..." --out profiles/<kernel>_<workload>.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ("csrc/mla_decode_bf16.hip", "csrc/mla_decode_common.h", "csrc/mla_internal.h")
DECODE_KERNEL = "mla_decode_bf16_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def decode_source_sha256() -> str:
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _one(folder: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(folder, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {folder}")
    return hits[0]


def _short(name: str) -> str:
    base = name.replace("(anonymous namespace)", "").split("(")[0]
    return base.split("::")[-1].replace("void ", "")


def kernel_stats(folder: str):
    rows = list(csv.DictReader(open(_one(folder, "*kernel_stats.csv"))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
             float(r["Percentage"])) for r in rows]


def counter_medians(folder: str, counter: str):
    """Median counter value (KiB) per kernel name, and the largest copy kernel's value."""
    rows = [r for r in csv.DictReader(open(_one(folder, "*counter_collection.csv")))
            if r["Counter_Name"] == counter]
    per = {}
    copy = []
    for r in rows:
        v = float(r["Counter_Value"])
        if r["Kernel_Name"].startswith(COPY_KERNEL):
            copy.append((int(r["Grid_Size"]), v))
        else:
            per.setdefault(r["Kernel_Name"], []).append(v)
    big_grid = max(g for g, _ in copy)
    copy_vals = [v for g, v in copy if g == big_grid]
    return {k: statistics.median(v) for k, v in per.items()}, statistics.median(copy_vals)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mb", type=int, required=True)
    ap.add_argument("--command", required=True, help="the bench command line of the kernel-trace run")
    ap.add_argument("--pmc-command", default=None,
                    help="the bench command line of the counter runs, without --copy-mb (default: --command)")
    ap.add_argument("--workload", default="batched decode B=64 x ctx 4096, s_q=1, H=128, bf16")
    ap.add_argument("--algorithmic-bytes", type=float, default=None)
    ap.add_argument("--bench-output", default=None,
                    help="stdout of the kernel-trace run (bench.py's JSON line), for the event-vs-trace check")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()

    stats = kernel_stats(args.trace)
    fetch, copy_fetch = counter_medians(args.fetch, "FETCH_SIZE")
    write, copy_write = counter_medians(args.write, "WRITE_SIZE")
    pmc_cmd = args.pmc_command or args.command
    copy_kib = args.copy_mb * 1024.0
    f_fetch = copy_kib / copy_fetch
    f_write = copy_kib / copy_write

    lines = [f"# rocprofv3 summary: {DECODE_KERNEL}, {args.workload}", ""]
    lines += ["Commands (from the repository root, on one MI355X):", "", "```"]
    lines += [f"rocprofv3 --kernel-trace --stats --output-format csv -d <trace> -o run -- {args.command}",
              f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o run -- {pmc_cmd} --copy-mb {args.copy_mb}",
              f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- {pmc_cmd} --copy-mb {args.copy_mb}",
              "python -m mla_decode_fwd_amd.profile_summary --trace <trace> --fetch <fetch> --write <write> "
              f"--copy-mb {args.copy_mb} --command '{args.command}' --pmc-command '{pmc_cmd}' --out <this file>",
              "```", ""]
    lines += ["## Kernel durations (kernel trace)", "",
              "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in stats:
        lines.append(f"| {_short(name)} | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {pct:.1f} |")
    if args.bench_output:
        import json
        rec = None
        for line in open(args.bench_output, encoding="utf-8", errors="replace"):
            if line.startswith("{") and '"roofline"' in line:
                rec = json.loads(line)
        if rec:
            ev_us = rec["roofline"]["kernel_us"]
            tr_us = next(avg for name, _, avg, _, _, _ in stats if DECODE_KERNEL in name) / 1e3
            lines += ["", f"Cross-check in the same run: bench.py's HIP events give the decode kernel {ev_us:.2f} us "
                          f"per launch, the kernel trace {tr_us:.2f} us ({100 * (ev_us / tr_us - 1):+.1f}%)."]
    lines += ["", "## HBM traffic per dispatch (memory counters)", "",
              f"Copy calibration: a device copy of {args.copy_mb} MiB reads FETCH_SIZE = {copy_fetch:.0f} KiB and "
              f"WRITE_SIZE = {copy_write:.0f} KiB, so the counters are scaled by {f_fetch:.3f} (fetch) and "
              f"{f_write:.3f} (write).", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | total MB |",
              "|---|---|---|---|---|---|"]
    decode_total = None
    for name in sorted(n for n in set(fetch) | set(write) if n.lstrip("void ").startswith("mla::")):
        fk, wk = fetch.get(name, 0.0), write.get(name, 0.0)
        rb, wb = fk * 1024 * f_fetch, wk * 1024 * f_write
        lines.append(f"| {_short(name)} | {fk:.0f} | {wk:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / 1e6:.1f} |")
        if DECODE_KERNEL in name:
            decode_total = rb + wb
    lines += [""]
    if args.algorithmic_bytes:
        lines += [f"Algorithmic bytes per decode launch: {args.algorithmic_bytes / 1e6:.1f} MB.", ""]
    lines += ["Machine-readable (read by bench.py; valid only while the source hash matches):", "",
              f"traffic_bytes_per_launch: {decode_total:.0f}",
              f"kernel_source_sha256: {decode_source_sha256()}", ""]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
