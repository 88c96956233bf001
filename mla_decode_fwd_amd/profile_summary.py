"""Summarise rocprofv3 CSV output of bench.py into a short markdown file.

Inputs are rocprofv3 output folders made from bench.py:
  --trace  a `--kernel-trace --stats --output-format csv` run (kernel durations),
  --fetch  a `--pmc FETCH_SIZE --output-format csv` run with `--copy-mb N`,
  --write  a `--pmc WRITE_SIZE --output-format csv` run with `--copy-mb N`.
The two counter runs are optional (both or neither).

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch. They are scaled
by what the same counter reads for the plain device copy of N MiB that
`bench.py --copy-mb N` launches (`__amd_rocclr_copyBuffer`, N MiB read and N
MiB written): factor = N MiB / counter reading. The summary records the
SHA-256 of the dominant kernel's sources (code only: comments and spacing are
left out), so a reader (bench.py) can tell when the kernel has changed since
the counters were taken.

usage: python -m mla_decode_fwd_amd.profile_summary --trace D1 [--fetch D2 --write D3 --copy-mb N]
           --command "..." [--kernel NAME --sources a.hip,b.h] --out profiles/<kernel>_<workload>.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ("csrc/mla_decode_bf16.hip", "csrc/mla_decode_common.h", "csrc/mla_internal.h")
DECODE_KERNEL = "mla_decode_bf16_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _code_only(text: str) -> str:
    """The source without comments or blank space, so that a change of wording
    does not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def decode_source_sha256(sources=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def _one(folder: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(folder, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {folder}")
    return hits[0]


def _demangle_nested(name: str) -> str:
    """'mla::(anonymous namespace)::f' from an Itanium nested name '_ZN3mla12_GLOBAL__N_11fE...'
    (the trace leaves some kernel names mangled)."""
    if not name.startswith("_ZN"):
        return name
    parts, i = [], 3
    while i < len(name) and name[i].isdigit():
        j = i
        while name[j].isdigit():
            j += 1
        n = int(name[i:j])
        part = name[j:j + n]
        parts.append("(anonymous namespace)" if part.startswith("_GLOBAL__N") else part)
        i = j + n
    return "::".join(parts) + "(...)" if parts else name


def _short(name: str) -> str:
    base = _demangle_nested(name).replace("(anonymous namespace)", "").split("(")[0]
    return base.split("::")[-1].replace("void ", "")


def _ours(name: str) -> bool:
    return _demangle_nested(name).lstrip("void ").startswith("mla::")


def kernel_stats(folder: str):
    rows = list(csv.DictReader(open(_one(folder, "*kernel_stats.csv"))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
             float(r["Percentage"])) for r in rows]


def dispatch_durations(folder: str, kernel: str):
    """Durations (ns) of the dispatches of `kernel`, in dispatch order, from the kernel trace."""
    paths = glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        return []
    rows = [r for r in csv.DictReader(open(paths[0])) if kernel in _demangle_nested(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def counter_medians(folder: str, counter: str, need_copy: bool = True):
    """Median counter value per kernel name, and the largest copy kernel's value."""
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
    meds = {k: statistics.median(v) for k, v in per.items()}
    if not need_copy:
        return meds, None
    big_grid = max(g for g, _ in copy)
    copy_vals = [v for g, v in copy if g == big_grid]
    return meds, statistics.median(copy_vals)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", default=None)
    ap.add_argument("--write", default=None)
    ap.add_argument("--copy-mb", type=int, default=0)
    ap.add_argument("--command", required=True, help="the bench command line of the kernel-trace run")
    ap.add_argument("--pmc-command", default=None,
                    help="the bench command line of the counter runs, without --copy-mb (default: --command)")
    ap.add_argument("--workload", default="batched decode B=64 x ctx 4096, s_q=1, H=128, bf16")
    ap.add_argument("--kernel", default=DECODE_KERNEL, help="the dominant kernel (a substring of its name)")
    ap.add_argument("--sources", default=",".join(DECODE_SOURCES),
                    help="its sources, relative to the package, for the hash")
    ap.add_argument("--mfma", default=None,
                    help="a `--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv` run of --pmc-command")
    ap.add_argument("--algorithmic-bytes", type=float, default=None)
    ap.add_argument("--call-kernels", default=None,
                    help="comma-separated kernel names that make up one library call (default: all of ours)")
    ap.add_argument("--bench-output", default=None,
                    help="stdout of the kernel-trace run (bench.py's JSON line), for the event-vs-trace check")
    ap.add_argument("--skip", type=int, default=0,
                    help="leading dispatches of --kernel (the warm-up) left out of the steady-state average")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    if (args.fetch is None) != (args.write is None) or (args.fetch and args.copy_mb <= 0):
        raise SystemExit("--fetch and --write go together, with --copy-mb")
    sources = tuple(x for x in args.sources.split(",") if x)

    stats = kernel_stats(args.trace)
    pmc_cmd = args.pmc_command or args.command

    lines = [f"# rocprofv3 summary: {args.kernel}, {args.workload}", ""]
    lines += ["Commands (from the repository root, on one MI355X):", "", "```"]
    redirect = " > <stdout>" if args.bench_output else ""
    lines += [f"rocprofv3 --kernel-trace --stats --output-format csv -d <trace> -o run -- {args.command}{redirect}"]
    summary = (f"python -m mla_decode_fwd_amd.profile_summary --trace <trace> --command '{args.command}' "
               f"--kernel {args.kernel} --sources {args.sources} --workload '{args.workload}'")
    if args.bench_output:
        summary += " --bench-output <stdout>"
    if args.skip:
        summary += f" --skip {args.skip}"
    if args.call_kernels:
        summary += f" --call-kernels {args.call_kernels}"
    if args.fetch:
        lines += [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o run -- {pmc_cmd} --copy-mb {args.copy_mb}",
                  f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- {pmc_cmd} --copy-mb {args.copy_mb}"]
        summary += f" --fetch <fetch> --write <write> --copy-mb {args.copy_mb} --pmc-command '{pmc_cmd}'"
    if args.mfma:
        lines += [f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d <mfma> -o run -- {pmc_cmd}"]
        summary += " --mfma <mfma>"
    lines += [summary + " --out <this file>", "```", ""]
    lines += ["## Kernel durations (kernel trace)", "",
              "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in stats:
        lines.append(f"| {_short(name)} | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {pct:.1f} |")
    steady_us = None
    if args.skip:
        durs = dispatch_durations(args.trace, args.kernel)[args.skip:]
        if durs:
            steady_us = statistics.mean(durs) / 1e3
            lines += ["", f"Steady state: the {len(durs)} dispatches of {args.kernel} after the first {args.skip} "
                          f"(the warm-up, which spans the clock transient of a burst of launches) average "
                          f"{steady_us:.2f} us (median {statistics.median(durs) / 1e3:.2f} us)."]
    if args.bench_output:
        import json
        rec = None
        for line in open(args.bench_output, encoding="utf-8", errors="replace"):
            if line.startswith("{") and '"roofline"' in line:
                rec = json.loads(line)
        if rec and "kernel_us" in rec["roofline"]:
            ev_us = rec["roofline"]["kernel_us"]
            tr_us = steady_us if steady_us is not None else \
                next(avg for name, _, avg, _, _, _ in stats if args.kernel in _demangle_nested(name)) / 1e3
            which = "steady-state average" if steady_us is not None else "average"
            lines += ["", f"Cross-check in the same run: bench.py's HIP events give {args.kernel} {ev_us:.2f} us "
                          f"per launch, the kernel trace's {which} {tr_us:.2f} us ({100 * (ev_us / tr_us - 1):+.1f}%)."]
        elif rec and "call_us" in rec["roofline"]:
            # One library call launches several kernels: compare the events'
            # time per call with the traced kernel time per call.
            n_calls = rec["steps"] + rec["warmup"]
            picked = [k for k in args.call_kernels.split(",")] if args.call_kernels else None
            tr_us = sum(avg * calls for name, calls, avg, _, _, _ in stats
                        if _ours(name) and (picked is None or _short(name) in picked)) / n_calls / 1e3
            ev_us = rec["roofline"]["call_us"]
            lines += ["", f"Cross-check in the same run: bench.py's HIP events give {ev_us:.2f} us per library call "
                          f"(back to back), the kernel trace {tr_us:.2f} us of kernel time per call over "
                          f"{n_calls} calls ({100 * (ev_us / tr_us - 1):+.1f}%)."]
    total = None
    if args.fetch:
        fetch, copy_fetch = counter_medians(args.fetch, "FETCH_SIZE")
        write, copy_write = counter_medians(args.write, "WRITE_SIZE")
        copy_kib = args.copy_mb * 1024.0
        f_fetch = copy_kib / copy_fetch
        f_write = copy_kib / copy_write
        lines += ["", "## HBM traffic per dispatch (memory counters)", "",
                  f"Copy calibration: a device copy of {args.copy_mb} MiB reads FETCH_SIZE = {copy_fetch:.0f} KiB and "
                  f"WRITE_SIZE = {copy_write:.0f} KiB, so the counters are scaled by {f_fetch:.3f} (fetch) and "
                  f"{f_write:.3f} (write).", "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | total MB |",
                  "|---|---|---|---|---|---|"]
        for name in sorted(n for n in set(fetch) | set(write) if _ours(n)):
            fk, wk = fetch.get(name, 0.0), write.get(name, 0.0)
            rb, wb = fk * 1024 * f_fetch, wk * 1024 * f_write
            lines.append(f"| {_short(name)} | {fk:.0f} | {wk:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | "
                         f"{(rb + wb) / 1e6:.1f} |")
            if args.kernel in _demangle_nested(name):
                total = rb + wb
    if args.mfma:
        busy, _ = counter_medians(args.mfma, "SQ_VALU_MFMA_BUSY_CYCLES", need_copy=False)
        active, _ = counter_medians(args.mfma, "GRBM_GUI_ACTIVE", need_copy=False)
        lines += ["", "## MFMA busy time (counters)", "",
                  "SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) over 1024 x the kernel's cycles, where "
                  "the kernel's cycles are GRBM_GUI_ACTIVE / 8 (the counter reads summed over the 8 XCDs): the "
                  "share of SIMD-cycles with the matrix unit busy while the kernel ran, prologue and tail included.",
                  "", "| kernel | MFMA busy | MFMA busy cycles per SIMD | kernel cycles |", "|---|---|---|---|"]
        for name in sorted(n for n in busy if _ours(n)):
            if active.get(name):
                cyc = active[name] / 8
                lines.append(f"| {_short(name)} | {100 * busy[name] / (cyc * 1024):.1f}% | {busy[name] / 1024:.0f} | "
                             f"{cyc:.0f} |")
    lines += [""]
    if args.algorithmic_bytes:
        lines += [f"Algorithmic bytes per launch of {args.kernel}: {args.algorithmic_bytes / 1e6:.1f} MB.", ""]
    lines += ["Machine-readable (read by bench.py; valid only while the source hash matches):", ""]
    if total is not None:
        lines += [f"traffic_bytes_per_launch: {total:.0f}"]
    lines += [f"kernel_source_sha256: {decode_source_sha256(sources)}", ""]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
