"""Plant plausible slips in a copy of the oracle (on the CPU) and show that the
pins catch every one of them.  The real oracle is never modified."""
import os
import types

import pytest

import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention.py")

MUTATIONS = {
    "dropped_scale": ("s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)"),
    "transposed_scores": ("s = scale * (q_rows @ k.T)", "s = scale * (k @ q_rows.T)"),
    "mask_flipped": ("key_ids[None, :] <= row_ids[:, None]", "key_ids[None, :] >= row_ids[:, None]"),
    "mask_strict": ("key_ids[None, :] <= row_ids[:, None]", "key_ids[None, :] < row_ids[:, None]"),
    "causal_keys_off_by_one": ("n_keys = int(row_ids.max()) + 1", "n_keys = int(row_ids.max())"),
    "no_normalisation": ("p = e / l[:, None]", "p = e"),
    "lse_without_max": ("lse = m + np.log(l)", "lse = np.log(l)"),
    "lse_log2": ("lse = m + np.log(l)", "lse = m + np.log2(l)"),
    "max_not_subtracted": ("e = np.exp(s - m[:, None])", "e = np.exp(s)"),
    "online_no_rescale": ("out = out * shrink[:, None]", "out = out"),
    "online_sum_not_rescaled": ("l = shrink * l + weights.sum(axis=1)", "l = l + weights.sum(axis=1)"),
    "online_shrink_sign": ("shrink = np.exp(m - m_new)", "shrink = np.exp(m_new - m)"),
}


def _mutated_oracle(old, new):
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_every_planted_slip_is_caught(name):
    mutant = _mutated_oracle(*MUTATIONS[name])
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mutant)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted slip {name}"
