"""Host-side helpers of bench.py (no GPU): the power-diagnostic inputs and the
traffic figures' tie to the kernel source they were measured on."""
import torch

import bench


def _inputs():
    g = torch.Generator().manual_seed(5)
    return [torch.randn(2, 3, 17, 64, generator=g).to(torch.bfloat16) for _ in range(3)]


def test_normal_inputs_are_left_unchanged():
    ts = _inputs()
    out = bench.diagnostic_inputs(ts, "normal")
    assert all(torch.equal(a, b) for a, b in zip(ts, out))


def test_coarse_inputs_clear_exactly_the_low_five_mantissa_bits():
    ts = _inputs()
    out = bench.diagnostic_inputs(ts, "coarse")
    for a, b in zip(ts, out):
        ai, bi = a.view(torch.int16), b.view(torch.int16)
        assert int((bi & 0x1F).abs().max()) == 0
        assert torch.equal(ai & ~0x1F, bi)            # sign, exponent and top two mantissa bits kept
        assert b.shape == a.shape and b.dtype == torch.bfloat16


def test_const_inputs_are_one_half_everywhere():
    out = bench.diagnostic_inputs(_inputs(), "const")
    assert all(bool((t == 0.5).all()) and t.dtype == torch.bfloat16 for t in out)


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(monkeypatch):
    name, pass_ = next(iter(bench.MEASURED_TRAFFIC))
    sha, fetch_kib, write_kib = bench.MEASURED_TRAFFIC[(name, pass_)]
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda p="fwd": sha)
    assert bench.measured_traffic(name, pass_) == round(
        fetch_kib * 1024 * bench.FETCH_SCALE + write_kib * 1024 * bench.WRITE_SCALE)
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda p="fwd": "0" * 64)
    assert bench.measured_traffic(name, pass_) is None
    assert bench.measured_traffic("no_such_workload", pass_) is None
