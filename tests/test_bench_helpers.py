"""Host-side helpers of bench.py (no GPU): the power-diagnostic inputs, the
traffic figures' tie to the kernel source they were measured on, and the
refusal of more than one GPU."""
import os

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


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(monkeypatch, tmp_path):
    sha = "ab" * 32
    (tmp_path / "k_counters.txt").write_text(
        "summary text\n"
        f"traffic-record: workload=w1 pass=fwd source=fa_fwd.hip source_sha256={sha} "
        "read_bytes=6.0e8 write_bytes=1.5e8\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda p="fwd": sha)
    traffic, src = bench.measured_traffic("w1", "fwd")
    assert traffic == 750000000 and "k_counters.txt" in src and sha[:16] in src
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda p="fwd": "0" * 64)
    traffic, src = bench.measured_traffic("w1", "fwd")
    assert traffic is None and "older" in src
    assert bench.measured_traffic("no_such_workload", "fwd")[0] is None
    assert bench.measured_traffic("w1", "fwd_fp8")[0] is None


def test_committed_traffic_records_parse():
    for fname, fields in bench.traffic_records():
        assert {"workload", "pass", "source_sha256", "read_bytes", "write_bytes"} <= set(fields), fname
        assert float(fields["read_bytes"]) > 0 and float(fields["write_bytes"]) > 0


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py covers one GPU; --gpus 2 exits non-zero before touching a GPU
    and says why."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=root)
    assert res.returncode == 2
    assert "only --gpus 1 is supported" in res.stderr
    assert res.stdout.strip() == ""
