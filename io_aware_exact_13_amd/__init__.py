"""MI355X-native fused exact attention, forward and gradients (HIP, gfx950).

Thin ctypes binding over the C ABI in include/fa.h.  Every step of the
computation runs in the HIP library; this module only marshals arguments.
If the library has not been built, calls fail loudly: there is no fallback
path.
"""
from __future__ import annotations

import ctypes
import math
import os

from .build import lib_path

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEAD_DIM = -3
FA_ERR_SCALE = -4
FA_ERR_ALIGN = -5
FA_ERR_LAUNCH = -6
FA_ERR_FLAG = -7
FA_ERR_ALIAS = -8
FA_ERR_SPLITS = -9
FA_ERR_SCRATCH = -10
FA_ERR_DEVICE = -11
NOALLOC_ROWS = 1 << 21     # rows (B*H*N) fa_bwd_noalloc's own workspace holds

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, call: str = "fa_fwd"):
        super().__init__(f"{call} failed with status {status}: {fa_status_str(status)}")
        self.status = status


_lib_override = None


def use_library(path: str) -> None:
    """Load the HIP library from `path` instead of the default build (for
    timing a tile candidate built by build.py --tile-variant).  Must be called
    before the first call into the library."""
    global _lib_override
    if _lib is not None:
        raise RuntimeError("the HIP library is already loaded")
    _lib_override = os.path.abspath(path)


def load_library():
    """Load the built HIP library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_override or lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                           "or python -m io_aware_exact_13_amd.build")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_fwd.restype = ci
    lib.fa_status_str.argtypes = [ci]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_fwd_tile.argtypes = [ci, ci, ci, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci),
                                ctypes.POINTER(ci), ctypes.POINTER(ctypes.c_longlong)]
    lib.fa_fwd_tile.restype = ci
    lib.fa_bwd.argtypes = [vp] * 10 + [ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_bwd.restype = ci
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_bwd_noalloc.restype = ci
    lib.fa_fwd_splitkv.argtypes = [vp] * 5 + [ci, ci, ci, ci, ctypes.c_float, ci, ci, vp, vp, vp]
    lib.fa_fwd_splitkv.restype = ci
    lib.fa_fwd_splitkv_plan.argtypes = [ci, ci, ci, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_fwd_splitkv_plan.restype = ci
    lib.fa_fwd_splitkv_ranges.argtypes = [ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci)]
    lib.fa_fwd_splitkv_ranges.restype = ci
    lib.fa_fwd_fa1order.argtypes = [vp] * 5 + [ci, ci, ci, ci, ctypes.c_float, ci, vp, vp, vp, vp]
    lib.fa_fwd_fa1order.restype = ci
    u64 = ctypes.c_uint64
    lib.fa_quant_fp8.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, u64, u64, vp]
    lib.fa_quant_fp8.restype = ci
    lib.fa_fwd_fp8.argtypes = [vp] * 8 + [ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_fwd_fp8_tile.argtypes = [ci, ci, ci, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci),
                                    ctypes.POINTER(ci), ctypes.POINTER(ctypes.c_longlong)]
    lib.fa_fwd_fp8_tile.restype = ci
    _lib = lib
    return lib


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int:
    """C-ABI fa_fwd with raw device addresses (ints); returns the status code."""
    return load_library().fa_fwd(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale),
                                 int(causal), stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream) -> int:
    """C-ABI fa_bwd with raw device addresses (ints); returns the status code."""
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d,
                                 ctypes.c_float(scale), int(causal), stream)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream) -> int:
    """C-ABI fa_bwd_noalloc with raw device addresses (ints); returns the status code."""
    return load_library().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d,
                                         ctypes.c_float(scale), int(causal), stream)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, n_splits, o_part, lse_part, stream) -> int:
    """C-ABI fa_fwd_splitkv with raw device addresses (ints); returns the status code."""
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), int(causal),
                                         int(n_splits), o_part, lse_part, stream)


def fa_fwd_splitkv_plan(B, H, N, d, causal):
    """(n_splits, o_part_bytes, lse_part_bytes) the library suggests for this shape."""
    n = ctypes.c_int()
    ob, lb = ctypes.c_size_t(), ctypes.c_size_t()
    st = load_library().fa_fwd_splitkv_plan(B, H, N, d, int(causal), ctypes.byref(n), ctypes.byref(ob),
                                            ctypes.byref(lb))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv_plan")
    return n.value, ob.value, lb.value


def fa_fwd_splitkv_ranges(B, H, N, d, causal, n_splits):
    """The range rule fa_fwd_splitkv uses: 0 (n_splits ranges per query block)
    or r > 0 (under the causal mask, ceil((b + 1) / r) ranges for block b)."""
    r = ctypes.c_int()
    st = load_library().fa_fwd_splitkv_ranges(B, H, N, d, int(causal), int(n_splits), ctypes.byref(r))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv_ranges")
    return r.value


def fa_fwd_fa1order(q, k, v, o, lse, B, H, N, d, scale, causal, o_acc, m, l, stream) -> int:
    """C-ABI fa_fwd_fa1order with raw device addresses (ints); returns the status code."""
    return load_library().fa_fwd_fa1order(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), int(causal),
                                          o_acc, m, l, stream)


def fa_quant_fp8(x, x8, descale, B, H, N, d, rotate, sign_lo, sign_hi, stream) -> int:
    """C-ABI fa_quant_fp8 with raw device addresses (ints); returns the status code."""
    return load_library().fa_quant_fp8(x, x8, descale, B, H, N, d, int(rotate), ctypes.c_uint64(sign_lo),
                                       ctypes.c_uint64(sign_hi), stream)


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, B, H, N, d, scale, causal, stream) -> int:
    """C-ABI fa_fwd_fp8 with raw device addresses (ints); returns the status code."""
    return load_library().fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o, lse, B, H, N, d,
                                     ctypes.c_float(scale), int(causal), stream)


def fa_fwd_fp8_tile(B, H, N, d, causal):
    """(rows_per_block, keys_per_tile, waves, blocks) of the launch fa_fwd_fp8 makes."""
    r, c, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    g = ctypes.c_longlong()
    st = load_library().fa_fwd_fp8_tile(B, H, N, d, int(causal), ctypes.byref(r), ctypes.byref(c),
                                        ctypes.byref(w), ctypes.byref(g))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8_tile")
    return r.value, c.value, w.value, g.value


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def fa_fwd_tile(B, H, N, d, causal):
    """(rows_per_block, keys_per_tile, waves, blocks) of the launch fa_fwd makes."""
    r, c, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    g = ctypes.c_longlong()
    st = load_library().fa_fwd_tile(B, H, N, d, int(causal), ctypes.byref(r), ctypes.byref(c),
                                    ctypes.byref(w), ctypes.byref(g))
    if st != FA_OK:
        raise FaError(st)
    return r.value, c.value, w.value, g.value


def _check_inputs(ts, names, device):
    """Every input on `device` (the first input's) and contiguous."""
    for t, name in zip(ts, names):
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a GPU tensor on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_buffer(t, name, dtype, shape, device):
    """A caller-provided output or workspace: the library writes it through a
    raw pointer, so its dtype, exact shape, device and layout are checked
    here before any launch."""
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _launch_stream(stream, device):
    """The stream a call runs on: torch's current stream of the tensors'
    device unless one is given, and then it must belong to that device.  The
    calls below also make that device current while they launch, as the C ABI
    asks (fa_bwd_noalloc finds its workspace through the current device)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if stream.device != device:
        raise ValueError(f"stream belongs to {stream.device}, the tensors to {device}")
    return stream


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """Attention forward on torch tensors: returns (o, lse).

    q, k, v: bf16 CUDA (HIP) tensors [B, H, N, d], contiguous.  o (bf16) and
    lse (fp32, [B, H, N]) are allocated with torch unless given.  The kernel
    runs on `stream` (default: torch's current stream of q's device).
    """
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    _check_inputs((q, k, v), ("q", "k", "v"), q.device)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(lse, "lse", torch.float32, (B, H, N), q.device)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, d, float(scale), int(bool(causal)), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def bwd(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None, delta=None,
        stream=None):
    """Gradients of fwd's output: returns (dq, dk, dv).

    q, k, v, o, dout: bf16 GPU tensors [B, H, N, d], contiguous; lse: the
    forward's fp32 [B, H, N].  dq, dk, dv (bf16) and the fp32 [B, H, N]
    workspace delta are allocated with torch unless given.
    """
    import torch
    ts = (q, k, v, o, dout)
    if any(t.dtype != torch.bfloat16 for t in ts) or lse.dtype != torch.float32:
        raise TypeError("q, k, v, o, dout must be bfloat16 and lse float32")
    if not all(t.is_cuda for t in ts + (lse,)):
        raise ValueError("all tensors must be GPU tensors")
    if q.dim() != 4 or any(t.shape != q.shape for t in ts) or lse.shape != q.shape[:3]:
        raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape and lse be [B, H, N]")
    _check_inputs(ts + (lse,), ("q", "k", "v", "o", "dout", "lse"), q.device)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _check_buffer(torch.empty_like(q) if dq is None else dq, "dq", torch.bfloat16, q.shape, q.device)
    dk = _check_buffer(torch.empty_like(q) if dk is None else dk, "dk", torch.bfloat16, q.shape, q.device)
    dv = _check_buffer(torch.empty_like(q) if dv is None else dv, "dv", torch.bfloat16, q.shape, q.device)
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(delta, "delta", torch.float32, (B, H, N), q.device)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, float(scale),
                    int(bool(causal)), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale=None, causal=False, stream=None):
    """fa_bwd through the entry point that allocates nothing (its D workspace
    is the library's own device array): the caller passes every output.
    B*H*N must not exceed NOALLOC_ROWS; calls that overlap in time on one GPU
    race on that array."""
    import torch
    ts = (q, k, v, o, dout)
    if any(t.dtype != torch.bfloat16 for t in ts) or lse.dtype != torch.float32:
        raise TypeError("q, k, v, o, dout must be bfloat16 and lse float32")
    if q.dim() != 4 or any(t.shape != q.shape for t in ts) or lse.shape != q.shape[:3]:
        raise ValueError("q, k, v, o, dout must share one [B, H, N, d] shape and lse be [B, H, N]")
    _check_inputs(ts + (lse,), ("q", "k", "v", "o", "dout", "lse"), q.device)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_buffer(t, name, torch.bfloat16, q.shape, q.device)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                            stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def fwd_splitkv(q, k, v, scale=None, causal=False, n_splits=None, out=None, lse=None, o_part=None,
                lse_part=None, stream=None):
    """Split-KV attention forward on torch tensors: returns (o, lse).

    Same inputs and results as fwd; n_splits defaults to the library's plan.
    The fp32 workspaces o_part [n_splits, B, H, N, d] and lse_part
    [n_splits, B, H, N] are allocated with torch unless given.
    """
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    _check_inputs((q, k, v), ("q", "k", "v"), q.device)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = fa_fwd_splitkv_plan(B, H, N, d, causal)[0]
    f32 = dict(dtype=torch.float32, device=q.device)
    out = _check_buffer(torch.empty_like(q) if out is None else out, "out", torch.bfloat16, q.shape, q.device)
    lse = _check_buffer(torch.empty((B, H, N), **f32) if lse is None else lse, "lse", torch.float32,
                        (B, H, N), q.device)
    o_part = _check_buffer(torch.empty((n_splits, B, H, N, d), **f32) if o_part is None else o_part, "o_part",
                           torch.float32, (n_splits, B, H, N, d), q.device)
    lse_part = _check_buffer(torch.empty((n_splits, B, H, N), **f32) if lse_part is None else lse_part,
                             "lse_part", torch.float32, (n_splits, B, H, N), q.device)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                            float(scale), int(bool(causal)), int(n_splits), o_part.data_ptr(), lse_part.data_ptr(),
                            stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv")
    return out, lse


def fwd_fa1order(q, k, v, scale=None, causal=False, out=None, lse=None, o_acc=None, m=None, l=None, stream=None):
    """The forward in the K/V-outer (FA1) loop order, an ablation: returns (o, lse).
    The fp32 workspaces o_acc [B, H, N, d], m and l [B, H, N] are allocated
    with torch unless given."""
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    _check_inputs((q, k, v), ("q", "k", "v"), q.device)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = _check_buffer(torch.empty_like(q) if out is None else out, "out", torch.bfloat16, q.shape, q.device)
    lse = _check_buffer(torch.empty((B, H, N), **f32) if lse is None else lse, "lse", torch.float32,
                        (B, H, N), q.device)
    o_acc = _check_buffer(torch.empty((B, H, N, d), **f32) if o_acc is None else o_acc, "o_acc", torch.float32,
                          (B, H, N, d), q.device)
    m = _check_buffer(torch.empty((B, H, N), **f32) if m is None else m, "m", torch.float32, (B, H, N), q.device)
    l = _check_buffer(torch.empty((B, H, N), **f32) if l is None else l, "l", torch.float32, (B, H, N), q.device)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_fwd_fa1order(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                             float(scale), int(bool(causal)), o_acc.data_ptr(), m.data_ptr(), l.data_ptr(),
                             stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fa1order")
    return out, lse


def quant_fp8(x, rotate=False, sign_bits=0, out=None, descale=None, stream=None):
    """Per-head E4M3 quantisation of a bf16 [B, H, N, d] tensor: returns
    (codes uint8 [B, H, N, d], descale fp32 [B, H]).  With `rotate`, rows get
    the random-sign Hadamard rotation whose signs are the bits of the
    128-bit integer `sign_bits` (bit c set: channel c negated)."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 GPU tensor [B, H, N, d]")
    B, H, N, d = x.shape
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    _check_buffer(out, "out", torch.uint8, x.shape, x.device)
    descale = torch.empty((B, H), dtype=torch.float32, device=x.device) if descale is None else descale
    _check_buffer(descale, "descale", torch.float32, (B, H), x.device)
    stream = _launch_stream(stream, x.device)
    bits = int(sign_bits)
    with torch.cuda.device(x.device):
        st = fa_quant_fp8(x.data_ptr(), out.data_ptr(), descale.data_ptr(), B, H, N, d, int(bool(rotate)),
                          bits & 0xFFFFFFFFFFFFFFFF, (bits >> 64) & 0xFFFFFFFFFFFFFFFF, stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_quant_fp8")
    return out, descale


def fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale=None, causal=False, out=None, lse=None,
            stream=None):
    """Attention forward on E4M3 operands (uint8 or float8_e4m3fn [B, H, N, d])
    with fp32 [B, H] dequantisation factors: returns (o bf16, lse fp32)."""
    import torch
    t8 = [t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in (q8, k8, v8)]
    if any(t.dtype != torch.uint8 for t in t8):
        raise TypeError("q8, k8, v8 must be uint8 or float8_e4m3fn")
    q8, k8, v8 = t8
    if q8.dim() != 4 or q8.shape != k8.shape or q8.shape != v8.shape:
        raise ValueError("q8, k8, v8 must share one [B, H, N, d] shape")
    _check_inputs((q8, k8, v8, q_descale, k_descale, v_descale),
                  ("q8", "k8", "v8", "q_descale", "k_descale", "v_descale"), q8.device)
    B, H, N, d = q8.shape
    for t in (q_descale, k_descale, v_descale):
        if t.dtype != torch.float32 or t.numel() != B * H:
            raise ValueError("descale factors must be contiguous fp32 [B, H]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device) if out is None else out
    _check_buffer(out, "out", torch.bfloat16, q8.shape, q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None else lse
    _check_buffer(lse, "lse", torch.float32, (B, H, N), q8.device)
    stream = _launch_stream(stream, q8.device)
    with torch.cuda.device(q8.device):
        st = fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(),
                        v_descale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, float(scale),
                        int(bool(causal)), stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse


_attention_fn = None


def _attention_function():
    """The torch.autograd.Function behind attention(), made on first use (the
    module imports torch only inside its calls)."""
    global _attention_fn
    if _attention_fn is None:
        import torch

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal):
                o, lse = fwd(q, k, v, scale=scale, causal=causal)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.scale, ctx.causal = scale, causal
                ctx.mark_non_differentiable(lse)
                return o, lse

            @staticmethod
            def backward(ctx, dout, _dlse):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = bwd(q, k, v, o, lse, dout.contiguous(), scale=ctx.scale, causal=ctx.causal)
                return dq, dk, dv, None, None

        _attention_fn = _Attention
    return _attention_fn


def attention(q, k, v, scale=None, causal=False, return_lse=False):
    """Attention with autograd: O = softmax(scale Q K^T [lower-triangular]) V
    through fa_fwd, and on backward dQ, dK, dV through fa_bwd (the gradient of
    O only; the logsumexp, returned with return_lse, carries none).  Same
    tensor rules as fwd: bf16 GPU tensors [B, H, N, d], contiguous."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o, lse = _attention_function().apply(q, k, v, float(scale), bool(causal))
    return (o, lse) if return_lse else o
