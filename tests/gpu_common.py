"""Shared helpers of the GPU parity tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import io_aware_exact_13_amd as fa
import oracle
import workloads

# Required agreement between the GPU output and the fp64 oracle (bf16 inputs).
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


def device():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    if not os.path.exists(fa.lib_path()):
        raise RuntimeError("HIP library not built")
    return torch.device("cuda:0")


def announce(msg):
    print(msg, file=sys.stderr, flush=True)


def run_gpu(q, k, v, scale, causal, stream=None):
    dev = device()
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def to64(t):
    return t.double().cpu().numpy()


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place of |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8.0)


def compare_full(q, k, v, scale, causal, o, lse, with_rounding=False):
    """max|dO|, mean|dO|, max|dLSE| against the oracle.  With with_rounding, the
    first value is max(|dO| - half a bf16 ulp of the oracle's O): the part of
    the error not explained by O being stored in bf16."""
    ro, rl = oracle.attention(to64(q), to64(k), to64(v), scale, causal)
    do = np.abs(to64(o) - ro)
    dl = np.abs(to64(lse) - rl)
    if with_rounding:
        return float((do - bf16_half_ulp(ro)).max()), do.mean(), dl.max(), do.max()
    return do.max(), do.mean(), dl.max()


def oracle_cores():
    """Cores the oracle's thread pools may use: this process's CPU set, at
    most 16."""
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(cores, 16))


class oracle_threads:
    """Context for running the oracle on a thread pool: yields a worker count
    (one per usable core, at most 16) and holds the BLAS library to one thread
    meanwhile.  The pool's workers call BLAS at the same time, and OpenBLAS's
    own thread pool must not be driven from several threads at once: with
    four workers of two BLAS threads each, the oracle's gradient of one
    64K-token head came out wrong by a quarter of its largest element, while
    the same call alone, or with one BLAS thread per worker, agreed to 2e-16."""

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        self._limit = threadpool_limits(limits=1) if threadpool_limits else None
        return oracle_cores()

    def __exit__(self, *exc):
        if self._limit is not None:
            self._limit.restore_original_limits()
        return False


def row_spans(n, causal, parts, align=256):
    """Split query rows [0, n) into at most `parts` spans of similar oracle
    work, cut at multiples of `align`.  Under the mask a row's work grows with
    its index (rows [0, r) cost about r^2), so the cuts sit at n sqrt(i /
    parts) there and at n i / parts without it."""
    cuts = {0, n}
    for i in range(1, parts):
        f = (i / parts) ** 0.5 if causal else i / parts
        c = int(round(n * f / align)) * align
        if 0 < c < n:
            cuts.add(c)
    b = sorted(cuts)
    return list(zip(b[:-1], b[1:]))


def spans_per_head(n_heads, n, workers):
    """Spans per head so that a pool of `workers` gets about two tasks each,
    none under 256 rows."""
    return max(1, min(-(-2 * workers // max(1, n_heads)), n // 256))


def compare_all_heads(q, k, v, scale, causal, o, lse, workers=None):
    """Every element of every (b, h) against the oracle, one span of a head's
    query rows per task on a thread pool (the oracle's BLAS calls and ufuncs
    release the GIL).
    q, k, v: CPU bf16 [B, H, N, d]; o (bf16), lse (fp32): the GPU results on
    the CPU.  Returns max|dO|, mean|dO| over the whole tensor, max|dLSE| and
    max(|dO| - half a bf16 ulp of the oracle's O)."""
    from concurrent.futures import ThreadPoolExecutor
    B, H = q.shape[:2]

    N = q.shape[2]

    def part(task):
        bh, r0, r1 = task
        b, h = divmod(bh, H)
        kmax = r1 if causal else N
        ro, rl = oracle.attention_head_rows(q[b, h].double().numpy(), k[b, h, :kmax].double().numpy(),
                                            v[b, h, :kmax].double().numpy(), scale, causal,
                                            rows=np.arange(r0, r1))
        d = np.abs(o[b, h, r0:r1].double().numpy() - ro)
        dl = np.abs(lse[b, h, r0:r1].double().numpy() - rl)
        return float(d.max()), float(d.sum()), d.size, float(dl.max()), float((d - bf16_half_ulp(ro)).max())

    with oracle_threads() as cores:
        workers = workers or cores
        spans = row_spans(N, causal, spans_per_head(B * H, N, workers))
        tasks = [(bh, r0, r1) for bh in range(B * H) for r0, r1 in spans]
        with ThreadPoolExecutor(workers) as ex:
            res = list(ex.map(part, tasks))
    mo = max(r[0] for r in res)
    me = sum(r[1] for r in res) / sum(r[2] for r in res)
    ml = max(r[3] for r in res)
    beyond = max(r[4] for r in res)
    return mo, me, ml, beyond


_variant_libs = {}


def variant_lib(variant):
    """A variant build of the library (build.py TEST_VARIANTS), loaded beside
    the default one through its own handle, with the argument types of the
    entry points the tests call on it."""
    import ctypes
    from io_aware_exact_13_amd.build import lib_path
    lib = _variant_libs.get(variant)
    if lib is None:
        path = lib_path(variant)
        if not os.path.exists(path):
            raise RuntimeError(f"variant library {path} is not built")
        lib = ctypes.CDLL(path)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [vp] * 5 + [ci, ci, ci, ci, cf, ci, vp]
        lib.fa_fwd_splitkv.argtypes = [vp] * 5 + [ci, ci, ci, ci, cf, ci, ci, vp, vp, vp]
        lib.fa_bwd.argtypes = [vp] * 10 + [ci, ci, ci, ci, cf, ci, vp]
        lib.fa_fwd_fp8.argtypes = [vp] * 8 + [ci, ci, ci, ci, cf, ci, vp]
        for f in (lib.fa_fwd, lib.fa_fwd_splitkv, lib.fa_bwd, lib.fa_fwd_fp8):
            f.restype = ci
        _variant_libs[variant] = lib
    return lib


def _variant_call(variant, name, st):
    if st != 0:
        raise RuntimeError(f"{variant} {name} returned {st}")
    torch.cuda.synchronize()


def variant_fwd(variant, q, k, v, scale, causal):
    """fa_fwd of a variant build; q, k, v on the GPU.  Returns (o, lse)
    after a synchronisation."""
    lib = variant_lib(variant)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device)
    _variant_call(variant, "fa_fwd", lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                 lse.data_ptr(), B, H, N, d, scale, int(bool(causal)),
                                                 stream.cuda_stream))
    return o, lse


def variant_fwd_splitkv(variant, q, k, v, scale, causal, n_splits):
    """fa_fwd_splitkv of a variant build with its own workspaces; q, k, v on
    the GPU.  Returns (o, lse) after a synchronisation."""
    lib = variant_lib(variant)
    B, H, N, d = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), **f32)
    o_part = torch.empty((n_splits, B, H, N, d), **f32)
    lse_part = torch.empty((n_splits, B, H, N), **f32)
    stream = torch.cuda.current_stream(q.device)
    _variant_call(variant, "fa_fwd_splitkv",
                  lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, scale, int(bool(causal)), n_splits, o_part.data_ptr(),
                                     lse_part.data_ptr(), stream.cuda_stream))
    return o, lse


def variant_bwd(variant, q, k, v, o, lse, dout, scale, causal):
    """fa_bwd of a variant build; every tensor on the GPU.  Returns
    (dq, dk, dv) after a synchronisation."""
    lib = variant_lib(variant)
    B, H, N, d = q.shape
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device)
    ptrs = [t.data_ptr() for t in (q, k, v, o, lse, dout, dq, dk, dv, delta)]
    _variant_call(variant, "fa_bwd", lib.fa_bwd(*ptrs, B, H, N, d, scale, int(bool(causal)), stream.cuda_stream))
    return dq, dk, dv


def variant_fwd_fp8(variant, q8, k8, v8, qd, kd, vd, scale, causal):
    """fa_fwd_fp8 of a variant build; every tensor on the GPU.  Returns
    (o, lse) after a synchronisation."""
    lib = variant_lib(variant)
    B, H, N, d = q8.shape
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    stream = torch.cuda.current_stream(q8.device)
    ptrs = [t.data_ptr() for t in (q8, k8, v8, qd, kd, vd, o, lse)]
    _variant_call(variant, "fa_fwd_fp8",
                  lib.fa_fwd_fp8(*ptrs, B, H, N, d, scale, int(bool(causal)), stream.cuda_stream))
    return o, lse


def compare_rows(q, k, v, scale, causal, o, lse, picks):
    """picks: list of (b, h, rows).  Returns max|dO|, mean|dO|, max|dLSE| over them."""
    worst_o, worst_l, tot, cnt = 0.0, 0.0, 0.0, 0
    q64 = k64 = v64 = None
    for b, h, rows in picks:
        q64 = q[b, h].double().numpy()
        k64 = k[b, h].double().numpy()
        v64 = v[b, h].double().numpy()
        ro, rl = oracle.attention_head_rows(q64, k64, v64, scale, causal, rows)
        go = o[b, h, torch.as_tensor(rows)].double().cpu().numpy()
        gl = lse[b, h, torch.as_tensor(rows)].double().cpu().numpy()
        d = np.abs(go - ro)
        worst_o = max(worst_o, float(d.max()))
        worst_l = max(worst_l, float(np.abs(gl - rl).max()))
        tot += float(d.sum())
        cnt += d.size
    return worst_o, tot / cnt, worst_l


def sample_picks(w: workloads.Workload, n_heads=3, n_rand=48, seed=0):
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    while len(heads) < min(n_heads, w.B * w.H):
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    picks = []
    for b, h in sorted(heads):
        rows = set(range(min(40, w.N)))
        rows |= set(range(max(0, w.N - 40), w.N))
        rows |= set(int(x) for x in rng.integers(0, w.N, size=n_rand))
        # rows at query-block and key-tile boundaries
        for edge in (63, 64, 127, 128, 129, w.N // 2 - 1, w.N // 2):
            if 0 <= edge < w.N:
                rows.add(edge)
        picks.append((b, h, np.array(sorted(rows))))
    return picks


def fp8_flip_allowance(q, k, v, scale, causal, rows):
    """Per element of the given rows of one head (dequantised fp64 operands):
    how far O_ic moves when one E4M3 rounding of P lands on the other side of
    a midpoint, which fp32 (GPU) and fp64 (oracle) evaluations of P may do
    when P lies within rounding noise of it.  One code step is at most 2^-3
    of a normal P and 2^-9 in the subnormal range; a term's P is its final
    softmax weight w_ij times l_i e^{m_t - m_i} <= l_i, so the move is at most
    2^-3 max_j w_ij |v_jc| + 2^-9 max_j |v_jc| / l_i
    (l_i = sum_j e^{s_ij - m_i} over the visible keys)."""
    rows = np.asarray(rows, dtype=np.int64)
    n = k.shape[0]
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > rows[:, None], -np.inf, s)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    l = e.sum(axis=1, keepdims=True)
    w = e / l
    av = np.abs(v)
    top = np.zeros((rows.size, v.shape[1]))
    for c0 in range(0, n, 512):
        top = np.maximum(top, (w[:, c0:c0 + 512, None] * av[None, c0:c0 + 512, :]).max(axis=1))
    return 2.0 ** -3 * top + 2.0 ** -9 * av.max(axis=0)[None, :] / l


def e4m3_p_bounds(q, k, v, scale, causal, rows):
    """What rounding P to E4M3 before P V can move O, from the plain
    definition alone (no key blocking): for the given rows of one head
    (fp64 operands [N, d]), returns (the exact O, the exact LSE, a per-element
    bound on |O_fp8 - O|, the per-element variance of that difference under
    independent round-to-nearest errors).

    Whatever reference a blocked softmax rounds P against, that reference is
    at most the row's final maximum, so key j's rounded weight P_j and the
    factor alpha_j its block is later rescaled by satisfy alpha_j P_j =
    w_j l (w_j its final softmax weight, l = sum_j exp(s_j - max_j s_j)) with
    alpha_j <= 1.  E4M3 rounds a normal P (>= 2^-6) with error at most 2^-4 P
    and a smaller one with error at most 2^-10, so key j moves O_c by at most
    max(2^-4 w_j, 2^-10 / l) |v_jc|; the bound sums that over the keys, and
    the variance takes each error uniform over its range (variance a^2 / 3
    for error at most a)."""
    rows = np.asarray(rows, dtype=np.int64)
    n = k.shape[0]
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > rows[:, None], -np.inf, s)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    l = e.sum(axis=1, keepdims=True)
    w = e / l
    o = w @ v
    lse = mx[:, 0] + np.log(l[:, 0])
    visible = np.isfinite(s).astype(np.float64)
    a = np.maximum(2.0 ** -4 * w, visible * (2.0 ** -10) / l)
    bound = a @ np.abs(v)
    var = (a * a) @ (v * v) / 3.0
    return o, lse, bound, var
