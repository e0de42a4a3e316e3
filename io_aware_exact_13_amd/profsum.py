"""Summaries of rocprofv3 output (CSV) as the short text kept with the sources.

Usage (repo root):
  python -m io_aware_exact_13_amd.profsum trace DIR --kernel fa_fwd_kernel [--flops F] [--skip-first | --skip N | --last N]
  python -m io_aware_exact_13_amd.profsum counters DIR [DIR ...] --kernel fa_fwd_kernel
  python -m io_aware_exact_13_amd.profsum traffic --fetch DIR --write DIR --fetch-copy DIR --write-copy DIR
        --kernel fa_fwd_kernel --workload NAME --pass fwd --source fa_fwd.hip [--algorithmic BYTES]

DIR is a rocprofv3 output folder (-d); the CSV files in it are found by
their suffix.  `traffic` scales the per-dispatch FETCH_SIZE and WRITE_SIZE of
the kernel by what the same counters read for a plain device-to-device copy
of COPY_BYTES (bench.py --copy-calibration), and prints a `traffic-record:`
line that bench.py reports while the kernel source's sha256 is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 512 << 20          # bench.py --copy-calibration copies 512 MiB


def _csv(folder: str, suffix: str) -> list[str]:
    hits = sorted(glob.glob(os.path.join(folder, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {folder}")
    return hits


def _short(name: str) -> str:
    name = name.replace("void (anonymous namespace)::", "")
    return name.split("(")[0] if "(" in name else name


def kernel_durations(folder: str, kernel: str) -> dict[str, list[float]]:
    """Per kernel instance whose name contains `kernel`: durations in ns, in dispatch order."""
    out: dict[str, list[tuple[int, float]]] = defaultdict(list)
    for path in _csv(folder, "kernel_trace.csv"):
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                out[_short(r["Kernel_Name"])].append(
                    (int(r["Dispatch_Id"]), float(r["End_Timestamp"]) - float(r["Start_Timestamp"])))
    return {k: [d for _, d in sorted(v)] for k, v in out.items()}


def counter_means(folder: str, kernel: str) -> dict[str, dict[str, float]]:
    """Per kernel instance: mean per dispatch of every counter collected."""
    tot: dict[str, dict[str, float]] = defaultdict(lambda: defaultdict(float))
    disp: dict[str, set] = defaultdict(set)
    for path in _csv(folder, "counter_collection.csv"):
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                k = _short(r["Kernel_Name"])
                tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
                disp[k].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k]) for c, v in d.items()} for k, d in tot.items()}


def source_sha256(name: str) -> str:
    with open(os.path.join(PKG, "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def cmd_trace(a) -> None:
    skip = max(a.skip, 1 if a.skip_first else 0)
    for k, durs in kernel_durations(a.dir, a.kernel).items():
        if a.last:
            n = max(0, len(durs) - a.last)
            note = f" (the last {len(durs) - n} in the figures below)"
        else:
            n = skip if len(durs) > skip else 0
            note = {0: "", 1: " (first left out of the figures below)"}.get(
                n, f" (first {n} left out of the figures below)")
        body = durs[n:]
        mean = statistics.fmean(body)
        print(f"{k}: {len(durs)} dispatches{note}")
        print(f"  mean {mean / 1e6:.4f} ms, median {statistics.median(body) / 1e6:.4f} ms, "
              f"min {min(body) / 1e6:.4f} ms, max {max(body) / 1e6:.4f} ms; first dispatch {durs[0] / 1e6:.4f} ms")
        if a.flops:
            print(f"  {a.flops:.4e} FLOP / mean -> {a.flops / (mean * 1e-9) / 1e12:.1f} TFLOP/s")


def cmd_counters(a) -> None:
    for folder in a.dirs:
        for k, d in counter_means(folder, a.kernel).items():
            print(f"{k} ({os.path.basename(os.path.normpath(folder))}), mean per dispatch:")
            for c, v in sorted(d.items()):
                print(f"  {c:28s} {v:.5e}")


def _one(folder: str, kernel: str, counter: str) -> float:
    vals = [d[counter] for d in counter_means(folder, kernel).values() if counter in d]
    if len(vals) != 1:
        raise ValueError(f"expected one kernel matching {kernel!r} with {counter} in {folder}, found {len(vals)}")
    return vals[0]


def cmd_traffic(a) -> None:
    fetch = _one(a.fetch, a.kernel, "FETCH_SIZE")
    write = _one(a.write, a.kernel, "WRITE_SIZE")
    fetch_copy = _one(a.fetch_copy, a.copy_kernel, "FETCH_SIZE")
    write_copy = _one(a.write_copy, a.copy_kernel, "WRITE_SIZE")
    fs = COPY_BYTES / (fetch_copy * 1024)
    ws = COPY_BYTES / (write_copy * 1024)
    rd, wr = fetch * 1024 * fs, write * 1024 * ws
    print(f"copy calibration ({COPY_BYTES} B read and written): FETCH_SIZE {fetch_copy:.5e} KiB -> scale {fs:.3f}; "
          f"WRITE_SIZE {write_copy:.5e} KiB -> scale {ws:.3f}")
    print(f"kernel, per dispatch: FETCH_SIZE {fetch:.5e} KiB -> read {rd:.4e} B; "
          f"WRITE_SIZE {write:.5e} KiB -> written {wr:.4e} B; total {rd + wr:.4e} B")
    if a.algorithmic:
        print(f"algorithmic bytes {a.algorithmic:.4e} B: traffic / algorithmic = {(rd + wr) / a.algorithmic:.3f}")
    print(f"traffic-record: workload={a.workload} pass={a.pass_} source={a.source} "
          f"source_sha256={source_sha256(a.source)} read_bytes={rd:.6e} write_bytes={wr:.6e}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--flops", type=float, default=None)
    t.add_argument("--skip-first", action="store_true", help="leave the first dispatch out")
    t.add_argument("--skip", type=int, default=0, help="leave the first N dispatches out (e.g. the warm-up calls)")
    t.add_argument("--last", type=int, default=0,
                   help="keep only the last N dispatches (e.g. the timed calls after a time-based warm-up)")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    f = sub.add_parser("traffic")
    for opt in ("--fetch", "--write", "--fetch-copy", "--write-copy", "--kernel", "--workload", "--source"):
        f.add_argument(opt, required=True)
    f.add_argument("--pass", dest="pass_", required=True)
    f.add_argument("--copy-kernel", default="copyBuffer")
    f.add_argument("--algorithmic", type=float, default=None)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "counters": cmd_counters, "traffic": cmd_traffic}[a.what](a)


if __name__ == "__main__":
    main(sys.argv[1:])
