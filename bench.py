"""Benchmark of the fused attention forward on one MI355X.

One step is one fa_fwd call over the 16K-token causal workload
(B=1, H=32, N=16384, d=128, bf16, inputs resident in HBM).  Prints ONE JSON
line: throughput in TFLOP/s (4*B*H*N^2*d, halved under the causal mask), the
roofline fraction of the dominant (only) kernel against the bf16 dense MFMA
peak, and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--all] [--shape B,H,N,d,causal] [--warm-s S]
                       [--input-bits normal|coarse|const] [--lib PATH]

--input-bits is a power diagnostic: the same launch on inputs whose low
mantissa bits are cleared (coarse) or that are all 0.5 (const); the line's
"data" field says so, and its value is not the workload's throughput.
--lib times another build of the library: a tile candidate of the forward
made by `python -m io_aware_exact_13_amd.build --tile-variant NAME`.
--splitkv S measures fa_fwd_splitkv with S key ranges per query block (-1:
the library's plan) instead of fa_fwd.
--fa1order measures the K/V-outer loop-order ablation fa_fwd_fa1order.
--fp8 measures the FP8 forward fa_fwd_fp8 on E4M3 operands that fa_quant_fp8
made beforehand (Q and K with the Hadamard rotation), against the FP8 dense
MFMA peak; the quantisation pass is timed separately and reported beside it.
--bwd measures fa_bwd (dQ, dK, dV from the forward's O and LSE; the two
kernels of one call) instead of the forward, against 2.5x the forward FLOPs.
--all also times every named workload, forward and backward, and a non-causal N=16384, d=128 run
(diagnostic: separates the causal overheads) on stderr.  --shape times an
ad-hoc shape instead of a named workload (used for the growth of the HBM
traffic with N: the same shape at N = 8192, 16384, 32768 and 65536).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS & % of MI355X bf16 MFMA peak at N=16K,d=128 (1 GPU)"
METRIC_BWD = "attention bwd TFLOPS (5 products, 2.5x fwd FLOPs) & % of MI355X bf16 MFMA peak (1 GPU)"
METRIC_FP8 = "attention fwd FP8 (E4M3) TFLOPS & % of MI355X fp8 MFMA peak at N=16K,d=128 (1 GPU)"

# --all: each extra workload is timed over ALL_STEPS calls after ALL_WARM_S
# seconds of untimed calls (its inputs are made on the host first, during
# which the GPU idles and its clock drops)
ALL_STEPS = 20
ALL_WARM_S = 0.3

KERNEL_SOURCES = {"fwd": "fa_fwd.hip", "fwd_fp8": "fa_fp8.hip"}

# HBM traffic per launch comes from rocprofv3 counter runs summarised under
# profiles/ (io_aware_exact_13_amd.profsum traffic): FETCH_SIZE and
# WRITE_SIZE of the kernel, each scaled by what the counter reads for a plain
# device copy of known size.  Each summary ends in a `traffic-record:` line
# naming the workload, the pass and the sha256 of the kernel source the
# counters were taken on; the figure is reported only while that source is
# unchanged (otherwise traffic is null).
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_sha256(pass_="fwd"):
    import hashlib
    path = os.path.join(ROOT, "io_aware_exact_13_amd", "csrc", KERNEL_SOURCES[pass_])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_records():
    """Every `traffic-record:` line under profiles/ as (file name, fields)."""
    import glob
    out = []
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.txt"))):
        with open(path, encoding="utf-8") as f:
            for ln in f:
                if ln.startswith("traffic-record:"):
                    fields = dict(kv.split("=", 1) for kv in ln.split(":", 1)[1].split())
                    out.append((os.path.basename(path), fields))
    return out


def measured_traffic(name, pass_="fwd"):
    """(bytes per launch, source description) from the newest matching record
    taken on the current kernel source, or (None, reason)."""
    sha = kernel_source_sha256(pass_)
    stale = None
    for fname, f in reversed(traffic_records()):
        if f.get("workload") != name or f.get("pass") != pass_:
            continue
        if f.get("source_sha256") != sha:
            stale = fname
            continue
        total = float(f["read_bytes"]) + float(f["write_bytes"])
        return round(total), f"profiles/{fname} (counters on source sha256 {sha[:16]})"
    return None, (f"not measured on this source (profiles/{stale} holds an older one)" if stale
                  else "not measured")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def usable_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def log_sclk(when):
    """Log the GPU shader clock level the amdgpu kernel module reports (stderr; best effort).

    Reads the amdgpu sysfs table (the current level carries a '*'); no other
    program is started, since a process that has touched the GPU must not
    exec one.
    """
    import glob
    try:
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            with open(path) as f:
                cur = [ln.strip() for ln in f if "*" in ln]
            if cur:
                log(f"[bench] sclk {when}: {cur[0]} ({path.split('/')[4]})")
                return
        log(f"[bench] sclk {when}: not reported")
    except OSError as e:
        log(f"[bench] sclk {when}: unreadable ({e.strerror})")


def diagnostic_inputs(tensors, bits):
    """Power diagnostic: the workload's bf16 inputs with their low 5 mantissa
    bits cleared ("coarse") or every element 0.5 ("const"); "normal" leaves
    them unchanged.  Same shapes, launch and instruction stream; only the bits
    the datapaths move change."""
    import torch
    if bits == "coarse":
        return [(t.view(torch.int16) & ~0x1F).view(torch.bfloat16) for t in tensors]
    if bits == "const":
        return [torch.full_like(t, 0.5) for t in tensors]
    return list(tensors)


def time_workload(w, steps, warmup, backward=False, n_splits=0, fa1order=False, fp8=False, warm_s=0.0,
                  input_bits="normal"):
    """Time `steps` calls of the forward (or, with backward, of fa_bwd on the
    forward's outputs) with HIP events on the launch stream: returns the total
    of the timed region, the sorted per-call durations, in ms, and the
    SHA-256 of the bf16 inputs' bytes (q, k, v).  After the
    `warmup` calls, untimed calls continue until `warm_s` seconds have passed
    (0: none), so that the shader clock has left its idle level before a
    short workload is timed."""
    import torch
    import io_aware_exact_13_amd as fa
    import workloads

    dev = torch.device("cuda:0")
    host = diagnostic_inputs(workloads.make_inputs(w), input_bits)
    shas = {name: workloads.sha256_of(t) for name, t in zip("qkv", host)}
    q, k, v = (t.to(dev) for t in host)
    del host
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if backward:
        do = workloads.make_grad(w).to(dev)
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta = torch.empty_like(lse)

        def call():
            fa.bwd(q, k, v, o, lse, do, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv, delta=delta,
                   stream=stream)
    elif fa1order:
        f32 = dict(dtype=torch.float32, device=dev)
        o_acc = torch.empty((w.B, w.H, w.N, w.d), **f32)
        m_ws, l_ws = torch.empty_like(lse), torch.empty_like(lse)

        def call():
            fa.fwd_fa1order(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, o_acc=o_acc, m=m_ws, l=l_ws,
                            stream=stream)
    elif fp8:
        signs = workloads.make_fp8_signs(w.seed, w.d)
        q8, qd = fa.quant_fp8(q, rotate=True, sign_bits=signs)
        k8, kd = fa.quant_fp8(k, rotate=True, sign_bits=signs)
        v8, vd = fa.quant_fp8(v, rotate=False)

        def call():
            fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
    elif n_splits:
        o_part = torch.empty((n_splits, w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        lse_part = torch.empty((n_splits, w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def call():
            fa.fwd_splitkv(q, k, v, scale=w.scale, causal=w.causal, n_splits=n_splits, out=o, lse=lse,
                           o_part=o_part, lse_part=lse_part, stream=stream)
    else:
        def call():
            fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < warm_s:
        for _ in range(4):
            call()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return total_ms, per, shas


def time_quant_fp8(w, steps, warmup):
    """Average time of one fa_quant_fp8 call (rotated) on the workload's Q, in ms,
    and its algorithmic bytes (bf16 read twice, E4M3 written once)."""
    import torch
    import io_aware_exact_13_amd as fa
    import workloads
    dev = torch.device("cuda:0")
    q = workloads.make_inputs(w)[0].to(dev)
    x8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    desc = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    signs = workloads.make_fp8_signs(w.seed, w.d)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        fa.quant_fp8(q, rotate=True, sign_bits=signs, out=x8, descale=desc, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        fa.quant_fp8(q, rotate=True, sign_bits=signs, out=x8, descale=desc, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, 5 * q.numel()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=os.cpu_count())
    except Exception:  # noqa: BLE001
        return os.cpu_count()


def cpu_baseline_fp8(w):
    """Time the oracle's FP8 forward (quantisation of one head's Q, K, V, then
    the online softmax with P rounded to E4M3) on one whole head."""
    import numpy as np
    from oracle import fp8 as ofp8
    import workloads
    q, k, v = workloads.make_inputs(w)
    signs = workloads.make_fp8_signs(w.seed, w.d)
    t0 = time.perf_counter()
    cq, _, dq = ofp8.quantize_heads(q[:1, :1].float().numpy(), True, signs)
    ck, _, dk = ofp8.quantize_heads(k[:1, :1].float().numpy(), True, signs)
    cv, _, dv = ofp8.quantize_heads(v[:1, :1].float().numpy(), False, 0)
    deq = [ofp8.dequantize_heads(c, s) for c, s in ((cq, dq), (ck, dk), (cv, dv))]
    ofp8.attention_fp8(*deq, w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.N * w.N * w.d / (2.0 if w.causal else 1.0)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "cpu_model": cpu_model(), "usable_cores": usable_cores(), "blas_threads": int(blas_threads()),
            "sample": f"1 of {w.B * w.H} heads of {w.name} (all {w.N} query rows), FP8 oracle "
                      f"(quantisation + online softmax with E4M3 P, fp64 numpy), {dt:.1f} s"}


def cpu_baseline(w, n_heads=32, backward=False):
    """Time the oracle on `n_heads` whole heads of the workload (every query
    row): the forward, or with backward the gradients."""
    import numpy as np
    import oracle
    import workloads
    threads = blas_threads()
    n_heads = min(n_heads, w.B * w.H)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w) if backward else None
    t0 = time.perf_counter()
    for i in range(n_heads):
        b, h = divmod(i, w.H)
        args = (q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy())
        if backward:
            oracle.attention_bwd_head(*args, do[b, h].double().numpy(), w.scale, w.causal)
        else:
            oracle.attention_head_rows(*args, w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.N * w.N * w.d * n_heads / (2.0 if w.causal else 1.0) * (2.5 if backward else 1.0)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "usable_cores": usable_cores(), "blas_threads": int(threads),
            "seconds": round(dt, 2),
            "sample": f"{n_heads} of {w.B * w.H} heads of {w.name} (all {w.N} query rows each), "
                      f"{'gradients, ' if backward else ''}fp64 numpy, {dt:.1f} s"}


def oracle_table():
    """Time the oracle as it stands (fp64 numpy, heads one after another, the
    host's BLAS threads) over every head of every named workload; one JSON
    line per workload."""
    import workloads
    for name in workloads.WORKLOAD_ORDER:
        w = workloads.WORKLOADS[name]
        r = cpu_baseline(w, n_heads=w.B * w.H)
        print(json.dumps({"workload": name, **r}), flush=True)


def gemm_calibration(m, steps, warmup, warm_s):
    """Time torch.matmul on bf16 [m, m] x [m, m] N(0,1) inputs (contiguous, no
    transposed view) on the launch stream and print one JSON line: the rate a
    library GEMM reaches on this GPU under the same power limit, a measured
    ceiling beside the published peak."""
    import torch
    from io_aware_exact_13_amd import accounting as acc
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(11)
    a = torch.randn((m, m), generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    b = torch.randn((m, m), generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    c = torch.empty((m, m), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record(stream)
        torch.matmul(a, b, out=c)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    mean = sum(per) / len(per)
    flops = 2.0 * m ** 3
    tf = flops / (mean * 1e-3) / 1e12
    log(f"[bench] bf16 GEMM {m}^3: mean {mean:.4f} ms, median {per[len(per) // 2]:.4f} ms -> {tf:.1f} TFLOP/s "
        f"({100 * tf / acc.PEAK_BF16_DENSE_TFLOPS:.1f}% of the bf16 dense peak)")
    print(json.dumps({"metric": "bf16 GEMM TFLOP/s (torch.matmul, N(0,1) inputs)", "value": round(tf, 2),
                      "unit": "TFLOP/s", "M": m, "steps": steps, "warmup": warmup,
                      "launch_ms": {"mean": round(mean, 5), "median": round(per[len(per) // 2], 5),
                                    "min": round(per[0], 5)},
                      "frac_of_peak": round(tf / acc.PEAK_BF16_DENSE_TFLOPS, 4)}), flush=True)


def ab_compare(w, variants, steps, reps, warm_s):
    """Time fa_fwd of several builds of the library on the same inputs in one
    process: each build is loaded through its own handle, and the builds take
    turns, `reps` rounds of (warm_s seconds of untimed calls, then `steps`
    timed calls on HIP events).  Prints one JSON line with TFLOP/s per build
    and round."""
    import ctypes
    import torch
    import workloads
    from io_aware_exact_13_amd import accounting as acc
    from io_aware_exact_13_amd.build import lib_path
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    libs = {}
    for name in variants:
        lib = ctypes.CDLL(lib_path(None if name == "default" else name))
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, ci, vp]
        lib.fa_fwd.restype = ci
        libs[name] = lib
    flops = acc.attention_flops(w.B, w.H, w.N, w.d, w.causal)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
            ctypes.c_float(w.scale), int(w.causal), stream.cuda_stream)
    res = {name: [] for name in libs}
    for r in range(reps):
        for name, lib in libs.items():
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < warm_s:
                for _ in range(4):
                    if lib.fa_fwd(*args) != 0:
                        raise RuntimeError(f"{name}: fa_fwd failed")
                torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(steps):
                lib.fa_fwd(*args)
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / steps
            res[name].append(round(flops / (ms * 1e-3) / 1e12, 1))
            log(f"[ab] {w.name} round {r} {name:10s} {ms * 1e3:9.1f} us  {res[name][-1]:7.1f} TFLOP/s")
    print(json.dumps({"metric": "fa_fwd TFLOP/s per build (same inputs, interleaved)", "workload": w.name,
                      "steps": steps, "warm_s": warm_s, "results": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lib", default=None,
                    help="time this build of the library (a tile candidate from build.py --tile-variant)")
    ap.add_argument("--input-bits", choices=("normal", "coarse", "const"), default="normal",
                    help="power diagnostic: clear the inputs' low mantissa bits or make them constant")
    ap.add_argument("--warm-s", type=float, default=0.0,
                    help="after the warmup calls, keep calling (untimed) for this many seconds")
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr table)")
    ap.add_argument("--shape", default=None, help="B,H,N,d,causal instead of a named workload")
    ap.add_argument("--bwd", action="store_true", help="measure fa_bwd (the gradients) instead of the forward")
    ap.add_argument("--fa1order", action="store_true",
                    help="measure the K/V-outer loop order ablation (fa_fwd_fa1order) instead of fa_fwd")
    ap.add_argument("--splitkv", type=int, default=0,
                    help="measure fa_fwd_splitkv with this many key ranges (-1: the library's plan)")
    ap.add_argument("--fp8", action="store_true", help="measure the FP8 forward fa_fwd_fp8 instead of fa_fwd")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy 3 times (counter calibration)")
    ap.add_argument("--ab", default=None, metavar="V1,V2,...",
                    help="only compare builds of the forward (names from build.py TILE_VARIANTS, or 'default') "
                         "on the same inputs in one process, interleaved over --reps rounds")
    ap.add_argument("--reps", type=int, default=2, help="rounds of --ab")
    ap.add_argument("--oracle-table", action="store_true",
                    help="only time the CPU oracle over every head of every named workload (no GPU work)")
    ap.add_argument("--gemm-calibration", type=int, default=0, metavar="M",
                    help="only time a plain bf16 M x M x M matrix product (torch.matmul, the vendor GEMM "
                         "library) on N(0,1) inputs: the MFMA rate this GPU sustains on a dense contraction")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: only --gpus 1 is supported: the kernel and its measurement cover one GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    import io_aware_exact_13_amd as fa
    import workloads
    from io_aware_exact_13_amd import accounting as acc

    if args.oracle_table:            # CPU only
        oracle_table()
        return
    if args.lib:
        fa.use_library(args.lib)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.load_library()   # fail loudly if the HIP library is missing
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device="cuda:0")   # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 512 MiB three times")
        return
    if args.gemm_calibration:
        gemm_calibration(args.gemm_calibration, args.steps, args.warmup, args.warm_s)
        return
    if args.ab:
        if args.shape:
            B, H, N, d, causal = (int(x) for x in args.shape.split(","))
            w = workloads.custom(B, H, N, d, bool(causal), seed=3)
        else:
            w = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
        ab_compare(w, args.ab.split(","), args.steps, args.reps, max(args.warm_s, 0.3))
        return

    if args.shape:
        B, H, N, d, causal = (int(x) for x in args.shape.split(","))
        w = workloads.custom(B, H, N, d, bool(causal), seed=3)
        name = w.name
    else:
        name = args.workload or workloads.HEADLINE
        w = workloads.WORKLOADS[name]
    flop_fn = acc.attention_bwd_flops if args.bwd else acc.attention_flops
    flops = flop_fn(w.B, w.H, w.N, w.d, w.causal)
    log(f"[bench] {name}{' backward' if args.bwd else ''}: warmup {args.warmup}, steps {args.steps}")
    log_sclk("before")
    if args.splitkv < 0:
        args.splitkv = fa.fa_fwd_splitkv_plan(w.B, w.H, w.N, w.d, int(w.causal))[0]
    total_ms, per, shas = time_workload(w, args.steps, args.warmup, backward=args.bwd,
                                  n_splits=0 if args.bwd else args.splitkv, fa1order=args.fa1order, fp8=args.fp8,
                                  warm_s=args.warm_s, input_bits=args.input_bits)
    log_sclk("after")
    ms_step = total_ms / args.steps
    avg_launch_ms = sum(per) / len(per)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = acc.PEAK_FP8_DENSE_TFLOPS if args.fp8 else acc.PEAK_BF16_DENSE_TFLOPS
    tile_fn = fa.fa_fwd_fp8_tile if args.fp8 else fa.fa_fwd_tile
    rows, keys, waves, blocks = tile_fn(w.B, w.H, w.N, w.d, int(w.causal))
    log(f"[bench] {ms_step:.4f} ms/step, median launch {per[len(per) // 2]:.4f} ms, "
        f"min {per[0]:.4f} ms -> {value:.1f} TFLOP/s ({100 * value / peak:.1f}% of peak)")
    quant = None
    if args.fp8:
        qms, qbytes = time_quant_fp8(w, max(5, args.steps // 2), 3)
        quant = {"ms_per_tensor": round(qms, 5), "GB/s": round(qbytes / (qms * 1e-3) / 1e9, 1),
                 "bytes": qbytes}
        log(f"[bench] fa_quant_fp8 (rotated) {qms * 1e3:.1f} us per tensor, {quant['GB/s']} GB/s "
            f"(bf16 read twice + E4M3 written)")

    if args.all:
        extra = workloads.custom(1, 32, 16384, 128, False, seed=3)
        for ow in [workloads.WORKLOADS[o] for o in workloads.WORKLOAD_ORDER] + [extra]:
            other = ow.name
            for mode in ("fwd", "bwd", "fp8"):
                bw = mode == "bwd"
                tms, p, _ = time_workload(ow, ALL_STEPS, 3, backward=bw, fp8=mode == "fp8", warm_s=ALL_WARM_S)
                f = (acc.attention_bwd_flops if bw else acc.attention_flops)(ow.B, ow.H, ow.N, ow.d, ow.causal)
                t = tms / ALL_STEPS
                pk = acc.PEAK_FP8_DENSE_TFLOPS if mode == "fp8" else acc.PEAK_BF16_DENSE_TFLOPS
                log(f"[bench-all] {other:32s} {mode} {t * 1e3:9.1f} us  "
                    f"{f / (t * 1e-3) / 1e12:7.1f} TFLOP/s "
                    f"{100 * f / (t * 1e-3) / 1e12 / pk:5.1f}% of its peak")
        # split-KV forward where the query blocks under-fill the GPU: one GPU's
        # share of the 16K causal workload over 8 GPUs (4 heads) and the tiny one
        for sw in (workloads.custom(1, 4, 16384, 128, True, seed=3), workloads.WORKLOADS["tiny_b1h1_n256_d64"]):
            plan = fa.fa_fwd_splitkv_plan(sw.B, sw.H, sw.N, sw.d, int(sw.causal))[0]
            f = acc.attention_flops(sw.B, sw.H, sw.N, sw.d, sw.causal)
            for ns in sorted({0, 2, plan, 8}):
                tms, p, _ = time_workload(sw, ALL_STEPS, 3, n_splits=ns, warm_s=ALL_WARM_S)
                t = tms / ALL_STEPS
                log(f"[bench-all] {sw.name:32s} {'fwd' if ns == 0 else f'split{ns}':>7s} {t * 1e3:9.1f} us  "
                    f"{f / (t * 1e-3) / 1e12:7.1f} TFLOP/s{'  (plan)' if ns == plan else ''}")

    if args.bwd or args.splitkv or args.fa1order or args.lib:
        traffic, traffic_source = None, "not measured for this pass or library"
    else:
        traffic, traffic_source = measured_traffic(name, "fwd_fp8" if args.fp8 else "fwd")
    result = {
        "metric": METRIC_BWD if args.bwd else (METRIC_FP8 if args.fp8 else METRIC),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.fp8 else "bf16",
        "data": ("synthetic" if args.input_bits == "normal" else
                 f"synthetic, power diagnostic: inputs '{args.input_bits}' (not the workload's values)"),
        "config": {"workload": name,
                   "pass": "bwd" if args.bwd else ("fwd_fa1order" if args.fa1order else "fwd_fp8" if args.fp8 else
                                                   (f"fwd_splitkv{args.splitkv}" if args.splitkv else "fwd")), "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "inputs_sha256": shas,
                   **({"untimed_warm_s": args.warm_s} if args.warm_s else {}),
                   **({"library": os.path.basename(args.lib)} if args.lib else {}),
                   "pct_of_bf16_peak": round(100 * value / acc.PEAK_BF16_DENSE_TFLOPS, 2),
                   **({"pct_of_fp8_peak": round(100 * value / peak, 2), "quantisation": quant} if args.fp8 else {}),
                   "launch": {"rows_per_block": rows, "keys_per_tile": keys, "waves": waves,
                              "blocks": blocks},
                   "launch_ms": {"mean": round(avg_launch_ms, 5), "median": round(per[len(per) // 2], 5),
                                 "min": round(per[0], 5)},
                   "tflops_at_median_launch": round(flops / (per[len(per) // 2] * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic, "traffic_source": traffic_source},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = (cpu_baseline_fp8(w) if args.fp8 else
                                  cpu_baseline(w, n_heads=8 if args.bwd else 32, backward=args.bwd))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
