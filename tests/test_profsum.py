"""The rocprofv3 summary tool on synthetic CSV files (CPU only)."""
import csv

from io_aware_exact_13_amd import profsum

NAME = "void (anonymous namespace)::fa_fwd_kernel<128, true, false>(bf16 const*)"


def _trace(folder, durations_ns):
    path = folder / "p_kernel_trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        # written out of order: the tool sorts by dispatch id
        rows = [dict(Dispatch_Id=i + 1, Kernel_Name=NAME, Start_Timestamp=t + 10 * i * 10**6,
                     End_Timestamp=t + 10 * i * 10**6 + d) for i, d in enumerate(durations_ns)]
        w.writerows(reversed(rows))
        w.writerow(dict(Dispatch_Id=99, Kernel_Name="copyBuffer", Start_Timestamp=0, End_Timestamp=5))


def test_trace_durations_in_dispatch_order(tmp_path):
    _trace(tmp_path, [3e6, 2e6, 1e6, 1e6])
    got = profsum.kernel_durations(str(tmp_path), "fa_fwd")
    assert list(got) == ["fa_fwd_kernel<128, true, false>"]
    assert got["fa_fwd_kernel<128, true, false>"] == [3e6, 2e6, 1e6, 1e6]


def test_trace_skip_and_last_select_the_dispatches(tmp_path, capsys):
    _trace(tmp_path, [5e6, 4e6, 2e6, 1e6, 3e6])
    profsum.main(["trace", str(tmp_path), "--kernel", "fa_fwd", "--skip", "2", "--flops", "2e12"])
    out = capsys.readouterr().out
    assert "5 dispatches (first 2 left out" in out and "mean 2.0000 ms" in out and "median 2.0000 ms" in out
    assert "-> 1000.0 TFLOP/s" in out
    profsum.main(["trace", str(tmp_path), "--kernel", "fa_fwd", "--last", "2"])
    out = capsys.readouterr().out
    assert "(the last 2 in the figures below)" in out and "mean 2.0000 ms" in out and "max 3.0000 ms" in out
    profsum.main(["trace", str(tmp_path), "--kernel", "fa_fwd", "--last", "9"])
    out = capsys.readouterr().out
    assert "(the last 5 in" in out and "mean 3.0000 ms" in out
