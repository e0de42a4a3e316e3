"""The C-ABI library: it loads, exports what include/fa.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed, no compute)."""
import os
import re

import pytest

import io_aware_exact_13_amd as fa
from io_aware_exact_13_amd.build import ROOT, build_library

HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        build_library()
    return fa.load_library()


def declared_functions():
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_noalloc", "fa_fwd", "fa_fwd_fa1order", "fa_fwd_fp8", "fa_fwd_fp8_tile",
                                    "fa_fwd_splitkv", "fa_fwd_splitkv_plan", "fa_fwd_splitkv_ranges", "fa_fwd_tile", "fa_quant_fp8",
                                    "fa_status_str"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    codes = [fa.FA_OK, fa.FA_ERR_NULL, fa.FA_ERR_SHAPE, fa.FA_ERR_HEAD_DIM, fa.FA_ERR_SCALE,
             fa.FA_ERR_ALIGN, fa.FA_ERR_LAUNCH, fa.FA_ERR_FLAG, fa.FA_ERR_ALIAS, fa.FA_ERR_SPLITS,
             fa.FA_ERR_SCRATCH, fa.FA_ERR_DEVICE]
    names = [fa.fa_status_str(c) for c in codes]
    assert names[0] == "ok"
    assert len(set(names)) == len(names)
    assert fa.fa_status_str(-99) == "unknown status"


# Fake, well-separated, 16-byte-aligned "device" addresses: every call below is
# invalid in some way, so the library returns before touching HIP.
Q, K, V, O, L = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40


def call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(k=0), fa.FA_ERR_NULL), (dict(v=0), fa.FA_ERR_NULL),
    (dict(o=0), fa.FA_ERR_NULL), (dict(lse=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=-1), fa.FA_ERR_SHAPE), (dict(N=0), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 20, N=1 << 20), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_HEAD_DIM), (dict(d=96), fa.FA_ERR_HEAD_DIM), (dict(d=256), fa.FA_ERR_HEAD_DIM),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE), (dict(scale=float("inf")), fa.FA_ERR_SCALE),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(scale=-0.1), fa.FA_ERR_SCALE),
    (dict(causal=2), fa.FA_ERR_FLAG), (dict(causal=-1), fa.FA_ERR_FLAG),
    (dict(q=Q + 8), fa.FA_ERR_ALIGN), (dict(o=O + 2), fa.FA_ERR_ALIGN), (dict(lse=L + 2), fa.FA_ERR_ALIGN),
    (dict(o=Q), fa.FA_ERR_ALIAS), (dict(o=V + 16), fa.FA_ERR_ALIAS), (dict(lse=O + 64), fa.FA_ERR_ALIAS),
    (dict(lse=K), fa.FA_ERR_ALIAS),
])
def test_bad_arguments_are_rejected_on_the_host(lib, kw, code):
    assert call(**kw) == code


def test_launch_shape_query(lib):
    rows, keys, waves, blocks = fa.fa_fwd_tile(1, 32, 16384, 128, 1)
    assert rows % (32 * waves) == 0 and keys in (32, 64, 128)
    assert blocks == 32 * (16384 // rows)
    assert fa.fa_fwd_tile(1, 1, 1, 64, 0)[3] == 1
    r = fa.fa_fwd_tile(2, 3, 129, 64, 0)[0]
    assert fa.fa_fwd_tile(2, 3, 129, 64, 0)[3] == 6 * (-(-129 // r))
    with pytest.raises(fa.FaError):
        fa.fa_fwd_tile(1, 1, 10, 80, 0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import io_aware_exact_13_amd
    monkeypatch.setattr(io_aware_exact_13_amd, "_lib", None)
    monkeypatch.setattr(io_aware_exact_13_amd, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        io_aware_exact_13_amd.load_library()


# fa_bwd: fake addresses again; every call is rejected on the host.
DO, DQ, DK, DV, DL = 6 << 40, 7 << 40, 8 << 40, 9 << 40, 10 << 40


def call_bwd(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=1, N=16, d=64,
             scale=0.125, causal=0):
    return fa.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(lse=0), fa.FA_ERR_NULL), (dict(dout=0), fa.FA_ERR_NULL),
    (dict(dq=0), fa.FA_ERR_NULL), (dict(dk=0), fa.FA_ERR_NULL), (dict(dv=0), fa.FA_ERR_NULL),
    (dict(delta=0), fa.FA_ERR_NULL),
    (dict(N=0), fa.FA_ERR_SHAPE), (dict(B=1 << 20, H=1 << 20, N=1 << 20), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_HEAD_DIM), (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(causal=3), fa.FA_ERR_FLAG),
    (dict(dout=DO + 8), fa.FA_ERR_ALIGN), (dict(dk=DK + 4), fa.FA_ERR_ALIGN), (dict(delta=DL + 1), fa.FA_ERR_ALIGN),
    (dict(dq=Q), fa.FA_ERR_ALIAS), (dict(dv=DO + 32), fa.FA_ERR_ALIAS), (dict(delta=L), fa.FA_ERR_ALIAS),
    (dict(dk=DQ + 16), fa.FA_ERR_ALIAS), (dict(delta=DV), fa.FA_ERR_ALIAS),
])
def test_bad_bwd_arguments_are_rejected_on_the_host(lib, kw, code):
    assert call_bwd(**kw) == code


def call_bwd_noalloc(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, B=1, H=1, N=16, d=64,
                    scale=0.125, causal=0):
    return fa.fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(dv=0), fa.FA_ERR_NULL), (dict(N=0), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_HEAD_DIM), (dict(scale=float("inf")), fa.FA_ERR_SCALE), (dict(causal=2), fa.FA_ERR_FLAG),
    (dict(dq=DQ + 8), fa.FA_ERR_ALIGN), (dict(dq=Q), fa.FA_ERR_ALIAS), (dict(dk=DQ + 16), fa.FA_ERR_ALIAS),
    (dict(N=fa.NOALLOC_ROWS + 1), fa.FA_ERR_SCRATCH), (dict(B=2, H=3, N=fa.NOALLOC_ROWS // 4), fa.FA_ERR_SCRATCH),
])
def test_bad_bwd_noalloc_arguments_are_rejected_on_the_host(lib, kw, code):
    """The no-allocation backward checks what fa_bwd checks, and refuses
    B*H*N beyond its own workspace, before any HIP call."""
    assert call_bwd_noalloc(**kw) == code


# fa_fwd_splitkv: fake addresses; every call is rejected on the host.
OP, LP = 11 << 40, 12 << 40


def call_split(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=16, d=64, scale=0.125, causal=0, n_splits=2, o_part=OP,
               lse_part=LP):
    return fa.fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, n_splits, o_part, lse_part, None)


@pytest.mark.parametrize("kw,code", [
    (dict(o_part=0), fa.FA_ERR_NULL), (dict(lse_part=0), fa.FA_ERR_NULL), (dict(q=0), fa.FA_ERR_NULL),
    (dict(n_splits=0), fa.FA_ERR_SPLITS), (dict(n_splits=65), fa.FA_ERR_SPLITS), (dict(n_splits=-3), fa.FA_ERR_SPLITS),
    (dict(N=0), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_HEAD_DIM), (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(causal=5), fa.FA_ERR_FLAG), (dict(o_part=OP + 4), fa.FA_ERR_ALIGN), (dict(lse_part=LP + 2), fa.FA_ERR_ALIGN),
    (dict(o_part=Q), fa.FA_ERR_ALIAS), (dict(lse_part=O), fa.FA_ERR_ALIAS), (dict(lse_part=OP + 64), fa.FA_ERR_ALIAS),
])
def test_bad_splitkv_arguments_are_rejected_on_the_host(lib, kw, code):
    assert call_split(**kw) == code


def test_splitkv_plan(lib):
    # one GPU's share of the 16K causal workload split over 8 GPUs: 4 heads, 256 query blocks, one
    # round of the CUs with causal lengths from 4 to 256 key tiles: the plan splits it
    n, ob, lb = fa.fa_fwd_splitkv_plan(1, 4, 16384, 128, 1)
    assert 2 <= n <= 16 and ob == n * 4 * 16384 * 128 * 4 and lb == n * 4 * 16384 * 4
    assert fa.fa_fwd_splitkv_plan(1, 32, 16384, 128, 1)[0] == 1      # 2048 blocks fill the GPU
    assert fa.fa_fwd_splitkv_plan(1, 1, 256, 64, 0)[0] == 1          # four 64-key tiles: too short to split
    assert fa.fa_fwd_splitkv_plan(1, 8, 65536, 128, 1)[0] == 1       # 2048 blocks
    assert 2 <= fa.fa_fwd_splitkv_plan(1, 1, 4096, 64, 0)[0] <= 8     # 64 tiles: ranges of at least 8
    assert fa.fa_fwd_splitkv_plan(1, 2, 16384, 128, 1)[0] >= 2       # 128 blocks, half the CUs
    with pytest.raises(fa.FaError):
        fa.fa_fwd_splitkv_plan(1, 1, 16, 96, 0)


def test_splitkv_range_rule(lib):
    """Without the mask every block has n_splits ranges; under it the rule is
    either that or ceil((b + 1) / r) ranges with r = ceil(blocks / n_splits)."""
    for shp in [(1, 4, 16384, 128), (1, 2, 16384, 128), (1, 8, 8192, 128), (1, 4, 16384, 64), (1, 1, 300, 128)]:
        br = fa.fa_fwd_tile(*shp, 1)[0]
        nqb = -(-shp[2] // br)
        for n in (1, 2, 3, 4, 6, 8):
            assert fa.fa_fwd_splitkv_ranges(*shp, 0, n) == 0
            r = fa.fa_fwd_splitkv_ranges(*shp, 1, n)
            assert r in (0, -(-nqb // n)) and (n > 1 or r == 0)
    assert fa.fa_fwd_splitkv_ranges(1, 2, 16384, 128, 1, 3) > 0       # measured: proportional is faster here
    with pytest.raises(fa.FaError):
        fa.fa_fwd_splitkv_ranges(1, 1, 16, 128, 1, 0)


# fa_fwd_fa1order: fake addresses; every call is rejected on the host.
OA, MW, LW = 13 << 40, 14 << 40, 15 << 40


def call_fa1(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=16, d=64, scale=0.125, causal=0, o_acc=OA, m=MW, l=LW):
    return fa.fa_fwd_fa1order(q, k, v, o, lse, B, H, N, d, scale, causal, o_acc, m, l, None)


@pytest.mark.parametrize("kw,code", [
    (dict(o_acc=0), fa.FA_ERR_NULL), (dict(m=0), fa.FA_ERR_NULL), (dict(l=0), fa.FA_ERR_NULL),
    (dict(N=0), fa.FA_ERR_SHAPE), (dict(d=80), fa.FA_ERR_HEAD_DIM), (dict(scale=-1.0), fa.FA_ERR_SCALE),
    (dict(causal=2), fa.FA_ERR_FLAG), (dict(o_acc=OA + 8), fa.FA_ERR_ALIGN), (dict(m=MW + 1), fa.FA_ERR_ALIGN),
    (dict(o_acc=K), fa.FA_ERR_ALIAS), (dict(l=MW), fa.FA_ERR_ALIAS), (dict(m=O + 64), fa.FA_ERR_ALIAS),
])
def test_bad_fa1order_arguments_are_rejected_on_the_host(lib, kw, code):
    assert call_fa1(**kw) == code


# fa_quant_fp8 / fa_fwd_fp8: fake addresses; every call is rejected on the host.
X8, DS, DQ, DK, DV = 16 << 40, 17 << 40, 18 << 40, 19 << 40, 20 << 40


def call_quant(x=Q, x8=X8, descale=DS, B=1, H=1, N=16, d=64, rotate=0):
    return fa.fa_quant_fp8(x, x8, descale, B, H, N, d, rotate, 0x1234, 0x5678, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), fa.FA_ERR_NULL), (dict(x8=0), fa.FA_ERR_NULL), (dict(descale=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N=-3), fa.FA_ERR_SHAPE), (dict(B=1 << 20, H=1 << 20), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_HEAD_DIM), (dict(rotate=2), fa.FA_ERR_FLAG),
    (dict(x=Q + 8), fa.FA_ERR_ALIGN), (dict(x8=X8 + 4), fa.FA_ERR_ALIGN), (dict(x8=X8 + 8), fa.FA_ERR_ALIGN),
    (dict(descale=DS + 2), fa.FA_ERR_ALIGN),
    (dict(x8=Q + 512), fa.FA_ERR_ALIAS), (dict(descale=X8 + 8), fa.FA_ERR_ALIAS), (dict(descale=Q), fa.FA_ERR_ALIAS),
])
def test_bad_quant_fp8_arguments_are_rejected_on_the_host(lib, kw, code):
    assert call_quant(**kw) == code


def call_fp8(q=Q, k=K, v=V, qd=DQ, kd=DK, vd=DV, o=O, lse=L, B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return fa.fa_fwd_fp8(q, k, v, qd, kd, vd, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(kd=0), fa.FA_ERR_NULL), (dict(lse=0), fa.FA_ERR_NULL),
    (dict(H=0), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_HEAD_DIM), (dict(causal=3), fa.FA_ERR_FLAG),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE), (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(v=V + 8), fa.FA_ERR_ALIGN), (dict(vd=DV + 1), fa.FA_ERR_ALIGN), (dict(o=O + 4), fa.FA_ERR_ALIGN),
    (dict(o=K), fa.FA_ERR_ALIAS), (dict(lse=DQ), fa.FA_ERR_ALIAS), (dict(lse=O + 64), fa.FA_ERR_ALIAS),
    (dict(o=V - 1024), fa.FA_ERR_ALIAS),
])
def test_bad_fwd_fp8_arguments_are_rejected_on_the_host(lib, kw, code):
    assert call_fp8(**kw) == code


def test_fp8_launch_shape_query(lib):
    rows, keys, waves, blocks = fa.fa_fwd_fp8_tile(1, 32, 16384, 128, 1)
    assert (rows, keys, waves) == (128, 64, 4) and blocks == 32 * 16384 // 128
    assert fa.fa_fwd_fp8_tile(2, 3, 1000, 64, 0)[3] == 6 * 8
    with pytest.raises(fa.FaError):
        fa.fa_fwd_fp8_tile(1, 1, 16, 96, 0)



def test_library_override_is_refused_once_loaded(lib):
    with pytest.raises(RuntimeError):
        fa.use_library("/nonexistent/libfa_mi355x_other.so")


def test_tile_variant_libraries_are_named_apart():
    from io_aware_exact_13_amd import build
    names = {build.lib_path()} | {build.lib_path(v) for v in build.TILE_VARIANTS}
    assert len(names) == 1 + len(build.TILE_VARIANTS)
    assert all(flag.startswith(("-DFA_", "-DFA8_")) for fl in build.TILE_VARIANTS.values() for flag in fl)
    assert set(build.VARIANT_SOURCE) <= set(build.TILE_VARIANTS)
    assert set(build.VARIANT_SOURCE.values()) <= set(build.SOURCE_NAMES)
    assert set(build.TEST_VARIANTS) <= set(build.TILE_VARIANTS)


def test_a_stream_of_another_device_is_rejected_before_any_call():
    """The Python calls launch on the tensors' device; a given stream must
    belong to it (host logic only: a stand-in stream object, no GPU)."""
    import types
    import torch
    other = types.SimpleNamespace(device=torch.device("cuda", 1), cuda_stream=0)
    with pytest.raises(ValueError, match="stream belongs to cuda:1"):
        fa._launch_stream(other, torch.device("cuda", 0))
    same = types.SimpleNamespace(device=torch.device("cuda", 0), cuda_stream=0)
    assert fa._launch_stream(same, torch.device("cuda", 0)) is same
