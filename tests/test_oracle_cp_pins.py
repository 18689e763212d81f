"""Pins of the context-parallel oracle (``oracle.cp``) against other things.

The ring decomposition must reproduce the whole-sequence attention oracle
(itself pinned to torch's fp64 SDPA, finite differences and closed forms) for
the forward and the backward, causal or not, MHA or grouped; the merge has
closed-form special cases.  Planted mistakes in a copy of the module must be
caught.
"""

import inspect
import math
import types

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import cp

RNG = np.random.default_rng(77)


def _inputs(b, s, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, s, hq, d))
    k = rng.standard_normal((b, s, hkv, d))
    v = rng.standard_normal((b, s, hkv, d))
    do = rng.standard_normal((b, s, hq, d))
    return q, k, v, do


# ---------------------------------------------------------------- checks

def check_ring_fwd_is_full(mod, causal, hq=4, hkv=2, s=12, d=5, n_chunks=3, seed=1):
    q, k, v, _ = _inputs(2, s, hq, hkv, d, seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = mod.ring_fwd(q, k, v, scale, causal, hq // hkv, n_chunks)
    ro, rl = att.attention_fwd(q, k, v, scale, causal, hq // hkv)
    return max(np.abs(o - ro).max(), np.abs(lse - rl).max())


def check_ring_bwd_is_full(mod, causal, hq=4, hkv=2, s=12, d=5, n_chunks=4, seed=2):
    q, k, v, do = _inputs(1, s, hq, hkv, d, seed)
    scale = 1.0 / math.sqrt(d)
    got = mod.ring_bwd(q, k, v, do, scale, causal, hq // hkv, n_chunks)
    ref = att.attention_bwd(q, k, v, do, scale, causal, hq // hkv)
    return max(np.abs(got[n] - ref[n]).max() for n in ("dq", "dk", "dv", "o", "lse", "delta"))


def check_merge_special_cases(mod):
    """One part is the identity; an empty part (LSE = -inf) is ignored; rows
    empty in every part give O = 0 and LSE = -inf; the order of the parts does
    not matter; the LSE is torch's logsumexp."""
    o = RNG.standard_normal((3, 1, 4, 2, 3))
    l = RNG.standard_normal((3, 1, 2, 4))
    err = 0.0
    m1o, m1l = mod.merge_partials(o[:1], l[:1])
    err = max(err, np.abs(m1o - o[0]).max(), np.abs(m1l - l[0]).max())
    le = l.copy()
    le[2] = -np.inf
    a_o, a_l = mod.merge_partials(o, le)
    b_o, b_l = mod.merge_partials(o[:2], l[:2])
    err = max(err, np.abs(a_o - b_o).max(), np.abs(a_l - b_l).max())
    la = l.copy()
    la[:, 0, 1, 2] = -np.inf
    e_o, e_l = mod.merge_partials(o, la)
    if not (np.isneginf(e_l[0, 1, 2]) and np.all(e_o[0, 2, 1] == 0.0)):
        err = max(err, 1.0)
    p_o, p_l = mod.merge_partials(o[::-1], l[::-1])
    f_o, f_l = mod.merge_partials(o, l)
    err = max(err, np.abs(p_o - f_o).max(), np.abs(p_l - f_l).max())
    tl = torch.logsumexp(torch.from_numpy(l), dim=0).numpy()
    err = max(err, np.abs(f_l - tl).max())
    return err


def check_merge_two_halves(mod):
    """Closed form with two keys, one per part: p = sigmoid(s1 - s2)."""
    s1, s2 = 0.7, -1.3
    v1, v2 = np.array([2.0, -1.0]), np.array([0.5, 3.0])
    o, l = mod.merge_partials(np.stack([v1, v2])[:, None, None, None, :],
                              np.array([s1, s2])[:, None, None, None])
    p = 1.0 / (1.0 + math.exp(s2 - s1))
    want_o = p * v1 + (1 - p) * v2
    want_l = math.log(math.exp(s1) + math.exp(s2))
    return max(np.abs(o[0, 0, 0] - want_o).max(), abs(l[0, 0, 0] - want_l))


def test_ring_fwd_is_full_attention():
    for causal in (False, True):
        assert check_ring_fwd_is_full(cp, causal) < 1e-12


def test_ring_bwd_is_full_backward():
    for causal in (False, True):
        assert check_ring_bwd_is_full(cp, causal) < 1e-11


def test_merge_special_cases():
    assert check_merge_special_cases(cp) < 1e-12


def test_merge_two_keys_closed_form():
    assert check_merge_two_halves(cp) < 1e-14


def test_chunk_pairs():
    assert cp.chunk_pairs(3, True) == [(0, 0, True), (1, 0, False), (1, 1, True), (2, 0, False), (2, 1, False),
                                       (2, 2, True)]
    assert len(cp.chunk_pairs(3, False)) == 9 and not any(c for _, _, c in cp.chunk_pairs(3, False))


# ---------------------------------------------------------------- planted mistakes

MUTATIONS = {
    "merge_weights_without_lse": ("w = np.exp(lse_parts - m_safe[None])", "w = np.exp(lse_parts * 0.0)"),
    "merge_lse_is_max": ("lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, z)))",
                         "lse = np.where(empty, -np.inf, m_safe)"),
    "merge_unnormalised": ("coef = np.where(empty[None], 0.0, w / np.where(empty, 1.0, z)[None])",
                           "coef = np.where(empty[None], 0.0, w)"),
    "pair_uses_local_max": ("p = np.exp(s - lse_c[b, h][:, None])", "p = np.exp(s - np.max(s, axis=1, keepdims=True))"),
    "pair_drops_delta": ("ds = p * (dp - delta_c[b, h][:, None])", "ds = p * dp"),
    "diagonal_not_causal": ("pairs.append((i, j, causal and i == j))", "pairs.append((i, j, False))"),
    "future_chunks_visible": ("if causal and j > i:\n                continue", "if causal and j > i + 1:\n                continue"),
    "dk_overwritten": ("dk[:, j * c:(j + 1) * c] += tk", "dk[:, j * c:(j + 1) * c] = tk"),
}


def _mutant(old, new):
    src = inspect.getsource(cp)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("cp_mutant")
    exec(compile(src.replace(old, new), "cp_mutant", "exec"), mod.__dict__)
    return mod


def _any_pin_fails(mod):
    checks = [
        lambda: check_ring_fwd_is_full(mod, True) < 1e-12,
        lambda: check_ring_fwd_is_full(mod, False) < 1e-12,
        lambda: check_ring_bwd_is_full(mod, True) < 1e-11,
        lambda: check_ring_bwd_is_full(mod, False) < 1e-11,
        lambda: check_merge_special_cases(mod) < 1e-12,
        lambda: check_merge_two_halves(mod) < 1e-14,
    ]
    failed = []
    for i, c in enumerate(checks):
        try:
            ok = c()
        except Exception:
            ok = False
        if not ok:
            failed.append(i)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    assert _any_pin_fails(_mutant(*MUTATIONS[name])), f"no pin caught {name}"


def test_unmutated_copy_passes():
    assert _any_pin_fails(_mutant("import numpy as np", "import numpy as np")) == []
