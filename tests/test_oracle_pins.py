"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import json
import os

import pytest

import oracle
import pins
from io_aware_exact_13_amd import accounting

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_worked_example_value_is_the_printed_one():
    diff = pins.check_worked_example(oracle)
    assert diff == pytest.approx(1.11e-16, rel=0.01)


def test_io_accounting_matches_the_pages():
    with open(os.path.join(pins.GOLDEN, "io_accounting.json")) as f:
        cases = json.load(f)["cases"]
    mib = accounting.MIB
    c0, c1, c2 = cases
    assert accounting.score_matrix_bytes(c0["N"], c0["elem_bytes"]) == c0["resident_MiB"] * mib
    assert accounting.score_round_trip_bytes(c0["N"], c0["elem_bytes"]) == c0["round_trip_MiB"] * mib
    assert c1["N"] * c1["N"] == c1["elements"]
    assert accounting.score_matrix_bytes(c1["N"], c1["elem_bytes"]) == c1["resident_bytes"]
    assert accounting.score_matrix_bytes(c2["N"], c2["elem_bytes"]) == c2["resident_bytes"]


def test_flop_and_byte_formulas():
    # headline: B=1, H=32, N=16384, d=128, causal
    assert accounting.attention_flops(1, 32, 16384, 128, True) == 4 * 32 * 16384 ** 2 * 128 / 2
    assert accounting.attention_flops(1, 32, 16384, 128, True) == pytest.approx(2.1990e12, rel=1e-4)
    assert accounting.compulsory_bytes(1, 32, 16384, 128) == 538968064
    assert accounting.compulsory_bytes(4, 16, 4096, 128) == 269484032
    assert accounting.compulsory_bytes(16, 32, 2048, 64) == 541065216
    assert accounting.compulsory_bytes(1, 1, 256, 64) == 132096
    assert accounting.attention_flops(1, 1, 256, 64, False) == 16777216
    # 2.5 PFLOP/s-class peak: 256 CUs x 4096 FLOP/clk x 2.4 GHz
    assert accounting.PEAK_BF16_DENSE_TFLOPS == pytest.approx(256 * 4096 * 2.4e9 / 1e12, rel=1e-4)
