"""Plant plausible slips in a copy of the gradient oracle (on the CPU) and show
that the gradient pins catch every one of them.  The real oracle is never
modified."""
import os
import types

import pytest

import pins_bwd

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention_bwd.py")

MUTATIONS = {
    "no_softmax_jacobian_term": ("ds = p * (dp - d_row[:, None])", "ds = p * dp"),
    "row_term_from_plain_sum": ("d_row = (p * dp).sum(axis=1)", "d_row = dp.sum(axis=1)"),
    "dq_without_scale": ("dq[row_ids - r0] = scale * (ds @ kk)", "dq[row_ids - r0] = (ds @ kk)"),
    "dk_without_scale": ("dk[:n_keys] += scale * (ds.T @ q[row_ids])", "dk[:n_keys] += (ds.T @ q[row_ids])"),
    "dk_from_do": ("dk[:n_keys] += scale * (ds.T @ q[row_ids])", "dk[:n_keys] += scale * (ds.T @ do[row_ids])"),
    "dv_from_ds": ("dv[:n_keys] += p.T @ do[row_ids]", "dv[:n_keys] += ds.T @ do[row_ids]"),
    "dp_from_k": ("dp = do[row_ids] @ v[:n_keys].T", "dp = do[row_ids] @ k[:n_keys].T"),
    "mask_dropped": ("s = np.where(key_ids[None, :] <= row_ids[:, None], s, -np.inf)", "s = s"),
    "mask_strict": ("key_ids[None, :] <= row_ids[:, None]", "key_ids[None, :] < row_ids[:, None]"),
    "unnormalised_p": ("p = e / e.sum(axis=1)[:, None]", "p = e"),
}


def _mutated(old, new):
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_every_planted_gradient_slip_is_caught(name):
    mutant = _mutated(*MUTATIONS[name])
    caught = []
    for check in pins_bwd.ALL_BWD_CHECKS:
        try:
            check(mutant)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted slip {name}"
