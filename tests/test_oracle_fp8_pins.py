"""The FP8 part of the oracle against the E4M3 format's definition, Hadamard
algebra, exact identities and a hand-computed example (no GPU)."""
import pytest

import pins_fp8
from oracle import fp8

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("check", pins_fp8.ALL_CHECKS, ids=lambda c: c.__name__)
def test_fp8_oracle_pin(check):
    check(fp8)
