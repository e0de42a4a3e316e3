"""Compile the HIP library for gfx950 in-tree (hipcc cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_NAME = "libfa_mi355x.so"
SOURCES = [os.path.join(PKG, "csrc", name) for name in ("fa_fwd.hip", "fa_bwd.hip", "fa_fa1.hip", "fa_fp8.hip", "fa_quant8.hip")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-I" + os.path.join(ROOT, "include"),
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Tile candidates of the bf16 forward, for measurement only: each overrides
# compile-time constants of fa_fwd.hip (the default build overrides none).
TILE_VARIANTS = {
    "w4d128": ["-DFA_WAVES_D128=4"],       # 4 waves (128 query rows) per workgroup at d = 128
    "w8d64": ["-DFA_WAVES_D64=8"],         # 8 waves (256 query rows) per workgroup at d = 64
    "ahead1": ["-DFA_OPERAND_AHEAD=1"],    # MFMA operands requested one step pair ahead
    "ahead3": ["-DFA_OPERAND_AHEAD=3"],    # three step pairs ahead
}


def lib_path(variant: str | None = None) -> str:
    if variant is None:
        return os.path.join(PKG, LIB_NAME)
    return os.path.join(PKG, LIB_NAME.replace(".so", f"_{variant}.so"))


def build_library(verbose: bool = False, variant: str | None = None) -> str:
    out = lib_path(variant)
    tmp = out + ".tmp"
    extra = TILE_VARIANTS[variant] if variant is not None else []
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
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
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--tile-variant", choices=sorted(TILE_VARIANTS), default=None,
                    help="build a tile candidate of the forward into its own library (measurement only)")
    a = ap.parse_args()
    print(build_library(verbose=True, variant=a.tile_variant))
