"""Plant plausible slips in a copy of the FP8 oracle (on the CPU) and show that
the FP8 pins catch every one of them.  The real oracle is never modified."""
import os
import types

import pytest

import pins_fp8

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")

MUTATIONS = {
    "exponent_bias": ("(1.0 + m / 8.0) * np.ldexp(1.0, e - 7)", "(1.0 + m / 8.0) * np.ldexp(1.0, e - 8)"),
    "subnormal_with_hidden_bit": ("np.where(e == 0, m * E4M3_MIN_SUBNORMAL,",
                                  "np.where(e == 0, (8 + m) * E4M3_MIN_SUBNORMAL,"),
    "truncation": ("q = np.rint(a[nrm] / np.ldexp(1.0, e - 3))", "q = np.floor(a[nrm] / np.ldexp(1.0, e - 3))"),
    "ties_away": ("q = np.rint(a[nrm] / np.ldexp(1.0, e - 3))", "q = np.floor(a[nrm] / np.ldexp(1.0, e - 3) + 0.5)"),
    "subnormal_ties_away": ("np.rint(a[sub] / E4M3_MIN_SUBNORMAL)", "np.floor(a[sub] / E4M3_MIN_SUBNORMAL + 0.5)"),
    "no_binade_carry": ("carry = q == 16", "carry = q == 17"),
    "sign_dropped": ("code = code | np.where(np.signbit(x), 128, 0)", "code = code"),
    "overflow_accepted": ("(biased == 15) & (q - 8 == 7)", "(biased == 16) & (q - 8 == 7)"),
    "butterfly_sign": ("v[..., 1, :] = a - b", "v[..., 1, :] = b - a"),
    "butterfly_in_fp64": ("y = np.array(x, dtype=dtype, copy=True)", "y = np.array(x, dtype=np.float64, copy=True)"),
    "signs_ignored": ("return np.array([-1.0 if (sign_bits >> c) & 1 else 1.0",
                      "return np.array([1.0 if (sign_bits >> c) & 1 else 1.0"),
    "amax_without_abs": ("amax = np.abs(y).reshape(B, H, N * d)", "amax = y.reshape(B, H, N * d)"),
    "multiplier_inverted": ("np.float32(E4M3_MAX) / np.where(amax > 0, amax, np.float32(1))",
                            "np.where(amax > 0, amax, np.float32(1)) / np.float32(E4M3_MAX)"),
    "no_amax_floor": ("np.maximum(amax, np.float32(AMAX_MIN))", "amax"),
    "descale_without_sqrt": ("descale * np.float32(1.0 / np.sqrt(d))", "descale * np.float32(1.0)"),
    "p_not_rounded": ("pr = e4m3_round(p) if round_p else p", "pr = p"),
    "sum_of_rounded_p": ("l = alpha * l + p.sum(axis=1)", "l = alpha * l + pr.sum(axis=1)"),
    "acc_not_rescaled": ("acc = alpha[:, None] * acc + pr @ v", "acc = acc + pr @ v"),
    "mask_strict": ("keys[None, :] > rows[:, None], -np.inf, s)", "keys[None, :] >= rows[:, None], -np.inf, s)"),
    "max_not_running": ("m_new = np.maximum(m, bmax)", "m_new = np.where(np.isfinite(m), m, bmax)"),
}


def _mutated_oracle(old, new):
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_fp8_mutant")
    exec(compile(src.replace(old, new), "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_every_planted_fp8_slip_is_caught(name):
    mutant = _mutated_oracle(*MUTATIONS[name])
    caught = []
    for check in pins_fp8.ALL_CHECKS:
        try:
            check(mutant)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted slip {name}"
