"""Pins of the packed-sequence oracle (``oracle.varlen``).

Independent references: torch's fp64 SDPA over all T tokens with a
block-diagonal (optionally causal-within-block) mask and autograd for the
gradients; equal-length packing against the dense batched oracle; and the
padding / empty-sequence conventions.  Planted mistakes must be caught.
"""

import inspect
import math
import types

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import varlen as vl


def _inputs(t, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((t, hq, d)), rng.standard_normal((t, hkv, d)), rng.standard_normal((t, hkv, d)),
            rng.standard_normal((t, hq, d)))


def _mask(cu, t, causal):
    """[T, T] boolean 'may attend' mask: same sequence (and j <= i if causal)."""
    seg = np.full(t, -1)
    for b in range(len(cu) - 1):
        seg[cu[b]:cu[b + 1]] = b
    m = (seg[:, None] == seg[None, :]) & (seg[:, None] >= 0)
    if causal:
        m &= np.arange(t)[None, :] <= np.arange(t)[:, None]
    return m


def _sdpa_reference(q, k, v, do, cu, scale, causal, groups):
    """torch fp64: masked softmax attention over all tokens, autograd VJP."""
    t = q.shape[0]
    allowed = torch.from_numpy(_mask(cu, t, causal))
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    kr, vr = kt.repeat_interleave(groups, dim=1), vt.repeat_interleave(groups, dim=1)
    s = torch.einsum("ihd,jhd->hij", qt, kr) * scale
    s = s.masked_fill(~allowed[None], float("-inf"))
    lse = torch.logsumexp(s, dim=2)                         # [H, T]
    p = torch.where(allowed[None], torch.exp(s - lse[..., None]), torch.zeros(()))
    o = torch.einsum("hij,jhd->ihd", p, vr)
    o.backward(torch.from_numpy(do))
    return {"o": o.detach().numpy(), "lse": lse.detach().numpy(), "dq": qt.grad.numpy(), "dk": kt.grad.numpy(),
            "dv": vt.grad.numpy()}


CU = [0, 5, 5, 12, 13, 20]      # an empty sequence, a single-token one; T = 23 leaves 3 padding rows


def check_against_sdpa(mod, causal, hq=4, hkv=2, d=6, t=23, seed=3):
    q, k, v, do = _inputs(t, hq, hkv, d, seed)
    scale = 1.0 / math.sqrt(d)
    got = mod.varlen_bwd(q, k, v, do, CU, scale, causal, hq // hkv)
    ref = _sdpa_reference(q, k, v, do, CU, scale, causal, hq // hkv)
    err = 0.0
    for n in ("o", "dq", "dk", "dv"):
        err = max(err, np.abs(got[n] - ref[n]).max())
    fin = np.isfinite(ref["lse"])
    if not np.array_equal(np.isneginf(got["lse"]), ~fin):
        return float("inf")
    err = max(err, np.abs(got["lse"][fin] - ref["lse"][fin]).max())
    fo, fl = mod.varlen_fwd(q, k, v, CU, scale, causal, hq // hkv)
    if not np.array_equal(np.isneginf(fl), ~fin):
        return float("inf")
    err = max(err, np.abs(fo - ref["o"]).max(), np.abs(np.where(fin, fl, 0.0) - np.where(fin, ref["lse"], 0.0)).max())
    return err


def check_equal_lengths_is_dense(mod, causal, b=3, s=7, hq=2, hkv=1, d=4, seed=4):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal(sh) for sh in ((b, s, hq, d), (b, s, hkv, d), (b, s, hkv, d), (b, s, hq, d)))
    scale = 0.3
    cu = [i * s for i in range(b + 1)]
    got = mod.varlen_bwd(q.reshape(b * s, hq, d), k.reshape(b * s, hkv, d), v.reshape(b * s, hkv, d),
                         do.reshape(b * s, hq, d), cu, scale, causal, hq // hkv)
    ref = att.attention_bwd(q, k, v, do, scale, causal, hq // hkv)
    err = max(np.abs(got[n] - ref[n].reshape(got[n].shape)).max() for n in ("dq", "dk", "dv", "o"))
    # [Hq, T] against [B, Hq, S]
    for n in ("lse", "delta"):
        err = max(err, np.abs(got[n] - np.transpose(ref[n], (1, 0, 2)).reshape(hq, b * s)).max())
    return err


def check_padding_and_empty(mod):
    q, k, v, do = _inputs(23, 2, 2, 3, 9)
    got = mod.varlen_bwd(q, k, v, do, CU, 0.5, True, 1)
    pad = slice(20, 23)
    ok = (np.all(got["o"][pad] == 0) and np.all(np.isneginf(got["lse"][:, pad])) and
          all(np.all(got[n][pad] == 0) for n in ("dq", "dk", "dv")) and np.all(got["delta"][:, pad] == 0))
    # the single-token sequence: O = V row, dQ = dK = 0
    ok = ok and np.allclose(got["o"][12], v[12]) and np.all(np.abs(got["dq"][12]) < 1e-15)
    return 0.0 if ok else 1.0


@pytest.mark.parametrize("causal", [False, True])
def test_against_masked_sdpa(causal):
    assert check_against_sdpa(vl, causal) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_is_dense(causal):
    assert check_equal_lengths_is_dense(vl, causal) < 1e-12


def test_padding_and_empty_sequences():
    assert check_padding_and_empty(vl) == 0.0


MUTATIONS = {
    "lse_not_per_sequence": ("lse[:, a:e] = lb[0]", "lse[:, a:e] = lb[0] + 1e-3"),
    "crosses_sequences": ("        ob, lb = att.attention_fwd(_seq(q, a, e), _seq(k, a, e), _seq(v, a, e), scale, causal, groups)",
                          "        ob, lb = att.attention_fwd(_seq(q, a, e), _seq(k, a - 1 if a else a, e - 1 if a else e), _seq(v, a - 1 if a else a, e - 1 if a else e), scale, causal, groups)"),
    "bwd_off_by_one_segment": ("        r = att.attention_bwd(_seq(q, a, e), _seq(k, a, e), _seq(v, a, e), _seq(do, a, e), scale, causal, groups)",
                               "        r = att.attention_bwd(_seq(q, a, e), _seq(k, a, e), _seq(v, a, e), _seq(do, a, e), scale, not causal, groups)"),
    "padding_lse_zero": ("lse = np.full((hq, t), -np.inf)", "lse = np.zeros((hq, t))"),
}


def _mutant(old, new):
    src = inspect.getsource(vl)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("varlen_mutant")
    exec(compile(src.replace(old, new), "varlen_mutant", "exec"), mod.__dict__)
    return mod


def _any_fails(mod):
    checks = [lambda: check_against_sdpa(mod, True) < 1e-12, lambda: check_against_sdpa(mod, False) < 1e-12,
              lambda: check_equal_lengths_is_dense(mod, True) < 1e-12, lambda: check_padding_and_empty(mod) == 0.0]
    out = []
    for i, c in enumerate(checks):
        try:
            ok = c()
        except Exception:
            ok = False
        if not ok:
            out.append(i)
    return out


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    assert _any_fails(_mutant(*MUTATIONS[name])), name


def test_unmutated_copy_passes():
    assert _any_fails(_mutant("import numpy as np", "import numpy as np")) == []
