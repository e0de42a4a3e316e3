"""Compile the HIP library for gfx950 in-tree (hipcc cross-compiles without a GPU).

Each source is compiled to its own object (with its own embedded gfx950 code
object), in parallel, and the objects are linked into one shared library.
A build variant overrides compile-time constants of one source (the forward
unless VARIANT_SOURCE names another) and reuses the other objects.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_NAME = "libfa_mi355x.so"
OBJ_DIR = os.path.join(PKG, "_build")
FWD_SOURCE = "fa_fwd.hip"
SOURCE_NAMES = (FWD_SOURCE, "fa_bwd.hip", "fa_fa1.hip", "fa_fp8.hip", "fa_quant8.hip")
SOURCES = [os.path.join(PKG, "csrc", name) for name in SOURCE_NAMES]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"),
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Variants of the bf16 forward, each overriding compile-time constants of
# fa_fwd.hip (the default build overrides none).  The tile candidates are for
# measurement only; TEST_VARIANTS are also built by the default build, because
# GPU tests compare them with the default library or the oracle.
TILE_VARIANTS = {
    "w4d128": ["-DFA_WAVES_D128=4"],       # 4 waves (128 query rows) per workgroup at d = 128
    "w8d64": ["-DFA_WAVES_D64=8"],         # 8 waves (256 query rows) per workgroup at d = 64
    "ahead1": ["-DFA_OPERAND_AHEAD=1"],    # MFMA operands requested one step pair ahead
    "ahead3": ["-DFA_OPERAND_AHEAD=3"],    # three step pairs ahead
    "exactmax": ["-DFA_EXACT_MAX=1"],      # reference maximum = running row maximum (no lag)
    "noshare": ["-DFA_LAG_SHARE=0"],       # lag bounded by size only (no share-of-sum rule)
    "share50": ["-DFA_LAG_SHARE=0.5f"],    # share-of-sum rule at 1/2
    "share12": ["-DFA_LAG_SHARE=0.125f"],  # share-of-sum rule at 1/8
    "d64max0": ["-DFA_D64_MAX_TILES=0"],   # d = 64: no row maximum from the first tile on
    "d64max16": ["-DFA_D64_MAX_TILES=16"],  # d = 64: the row maximum on the first 16 tiles
    "d64maxall": ["-DFA_D64_MAX_TILES=1000000"],  # d = 64: the row maximum on every tile
    "valu2": ["-DFA_VALU_PER_MFMA=2"],     # softmax VALU instructions placed after each MFMA: 2
    "valu4": ["-DFA_VALU_PER_MFMA=4"],     # 4
    "valu5": ["-DFA_VALU_PER_MFMA=5"],     # 5 (all of a d = 128 step's softmax between its MFMAs)
    "racecheck": ["-DFA_EXTRA_BARRIER=1"],  # a wait and a workgroup barrier after every step's LDS reads
    "g2": ["-DFA_GROUPS_D128=2"],          # d = 128: 4 waves of 64 rows (two row groups), 32-key tiles
    "g2racecheck": ["-DFA_GROUPS_D128=2", "-DFA_EXTRA_BARRIER=1"],
    "g2v4": ["-DFA_GROUPS_D128=2", "-DFA_VALU_PER_MFMA=4"],
    "g2v5": ["-DFA_GROUPS_D128=2", "-DFA_VALU_PER_MFMA=5"],
    "g2v6": ["-DFA_GROUPS_D128=2", "-DFA_VALU_PER_MFMA=6"],
    "g2v7": ["-DFA_GROUPS_D128=2", "-DFA_VALU_PER_MFMA=7"],
    "g2nomax": ["-DFA_GROUPS_D128=2", "-DFA_NOMAX_D128=1"],
    "nomax128": ["-DFA_NOMAX_D128=1"],
    # the gradient kernels with a wait and a workgroup barrier after every tile's LDS reads
    "bwdracecheck": ["-DFA_BWD_EXTRA_BARRIER=1"],
    # the FP8 forward with a wait and a workgroup barrier after every step's LDS reads
    "fp8racecheck": ["-DFA8_EXTRA_BARRIER=1"],
}
# variants of a source other than the forward
VARIANT_SOURCE = {"bwdracecheck": "fa_bwd.hip", "fp8racecheck": "fa_fp8.hip"}
TEST_VARIANTS = ("exactmax", "racecheck", "g2", "g2racecheck", "bwdracecheck", "fp8racecheck")


def lib_path(variant: str | None = None) -> str:
    if variant is None:
        return os.path.join(PKG, LIB_NAME)
    return os.path.join(PKG, LIB_NAME.replace(".so", f"_{variant}.so"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def _obj(name: str, variant: str | None) -> str:
    stem = name.replace(".hip", "")
    return os.path.join(OBJ_DIR, f"{stem}{'_' + variant if variant else ''}.o")


def _compile(src: str, obj: str, extra, verbose):
    tmp = obj + ".tmp"
    _run([HIPCC, *FLAGS, *extra, "-c", src, "-o", tmp], verbose)
    os.replace(tmp, obj)


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)


def build_all(verbose: bool = False, variants=()) -> list[str]:
    """Compile every source (and each variant's source once more) in
    parallel, then link the default library and one library per variant."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = [(src, _obj(name, None), []) for name, src in zip(SOURCE_NAMES, SOURCES)]
    for v in variants:
        name = VARIANT_SOURCE.get(v, FWD_SOURCE)
        jobs.append((SOURCES[SOURCE_NAMES.index(name)], _obj(name, v), TILE_VARIANTS[v]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_compile, s, o, e, verbose) for s, o, e in jobs]:
            f.result()
    outs = [lib_path()]
    _link([_obj(n, None) for n in SOURCE_NAMES], outs[0], verbose)
    for v in variants:
        name = VARIANT_SOURCE.get(v, FWD_SOURCE)
        outs.append(lib_path(v))
        _link([_obj(n, v if n == name else None) for n in SOURCE_NAMES], outs[-1], verbose)
    return outs


def build_library(verbose: bool = False, variant: str | None = None) -> str:
    """Build the default library, or the default plus one variant's library;
    returns the path of the one asked for."""
    outs = build_all(verbose, () if variant is None else (variant,))
    return outs[-1]


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--tile-variant", choices=sorted(TILE_VARIANTS), default=None,
                    help="also build a variant of the forward into its own library")
    ap.add_argument("--all-variants", action="store_true", help="build every variant")
    a = ap.parse_args()
    if a.all_variants:
        print("\n".join(build_all(verbose=True, variants=tuple(TILE_VARIANTS))))
    elif a.tile_variant:
        print(build_library(verbose=True, variant=a.tile_variant))
    else:
        print("\n".join(build_all(verbose=True, variants=TEST_VARIANTS)))
