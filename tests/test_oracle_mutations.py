"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

The copy is made from the oracle's source text, edited in memory and executed
as a throw-away module; the real oracle is never touched.
"""

import inspect
import types

import pytest

from oracle import attention as orc
from tests import test_oracle_pins as pins

MUTATIONS = {
    "dq_drops_scale": ("dq[b, sl, h, :] = scale * (ds @ kh)", "dq[b, sl, h, :] = (ds @ kh)"),
    "dk_drops_scale": ("dk_h += scale * (ds.T @ qb)", "dk_h += (ds.T @ qb)"),
    "ds_wrong_sign": ("ds = p * (dp - dl[:, None])", "ds = p * (dp + dl[:, None])"),
    "dv_uses_o": ("dv_h += p.T @ dob", "dv_h += p.T @ ob"),
    "dp_transposed_v": ("dp = dob @ vh.T", "dp = dob @ vh[:, ::-1].T"),
    "delta_uses_do_only": ("dl = np.sum(dob * ob, axis=1)", "dl = np.sum(dob, axis=1)"),
    "gqa_modulo_map": ("kv = h // groups\n    s = _scores", "kv = h % (k.shape[2])\n    s = _scores"),
    "fwd_gqa_modulo_map": ("            kv = h // groups\n            kh, vh = k[b, :, kv, :], v[b, :, kv, :]\n            for r0",
                           "            kv = h % k.shape[2]\n            kh, vh = k[b, :, kv, :], v[b, :, kv, :]\n            for r0"),
    "causal_off_by_one": ("s = np.where(cols > rows, -np.inf, s)", "s = np.where(cols >= rows + 1 + (rows > 0), -np.inf, s)"),
    "causal_masks_diagonal": ("s = np.where(cols > rows, -np.inf, s)", "s = np.where(cols >= rows, np.where(cols == 0, s, -np.inf), s)"),
    "lse_drops_max": ("return e / z, (m + np.log(z))[:, 0]", "return e / z, (np.log(z))[:, 0]"),
    "softmax_unnormalised": ("return e / z, (m + np.log(z))[:, 0]", "return e, (m + np.log(z))[:, 0]"),
    "scores_drop_scale": ("s = scale * (qb @ kh.T)", "s = (qb @ kh.T)"),
    "group_sum_last_head_only": ("dk_sum += dk_h", "dk_sum = dk_h"),
}


def _mutant(old, new):
    src = inspect.getsource(orc)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _any_pin_fails(mod):
    checks = [
        lambda: pins.check_finite_differences(mod, 4, 2, 5, 4, True) < 1e-6,
        lambda: pins.check_finite_differences(mod, 2, 2, 5, 4, False) < 1e-6,
        lambda: pins.check_against_sdpa(mod, 1, 4, 2, 9, 4, True)[0] < 1e-10,
        lambda: pins.check_against_sdpa(mod, 1, 4, 2, 9, 4, False)[0] < 1e-10,
        lambda: pins.check_closed_forms(mod, True) < 1e-12,
        lambda: pins.check_two_key_sigmoid(mod) < 1e-12,
        lambda: pins.check_softmax_and_mask(mod, True) < 1e-12,
        lambda: pins.check_dv_is_pt_do_and_delta(mod, True) < 1e-12,
        lambda: pins.check_gqa_is_sum_of_mha(mod, True) < 1e-12,
        lambda: pins.check_shift_invariance(mod, False) < 1e-11,
        lambda: pins.check_rows_cols(mod, True) < 1e-11,
    ]
    failed = []
    for i, c in enumerate(checks):
        try:
            ok = c()
        except Exception:  # a crash is also a detection
            ok = False
        if not ok:
            failed.append(i)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTATIONS[name]
    failed = _any_pin_fails(_mutant(old, new))
    assert failed, f"no pin caught mutation {name}"


def test_unmutated_copy_passes_every_pin():
    mod = _mutant("ROW_BLOCK = 512", "ROW_BLOCK = 512")
    assert _any_pin_fails(mod) == []
