"""Pins of the sparse MLA oracle (``oracle.sparse_mla``).

Independent references: torch fp64 attention over all keys with a mask built
from the index lists (each selected key once; the latent rows serve as keys
and, cut to d_v channels, as values) and autograd for dq and the latent
gradient, which then sums both uses of a row; a listed-twice key equals a
key whose logit is raised by log 2; sentinel and out-of-range entries change
nothing; a token without valid entries has O = 0, LSE = -inf and no
gradient.  Planted mistakes in a copy of the module must be caught.
"""

import inspect
import math
import types

import numpy as np
import pytest
import torch

from oracle import sparse_mla as sm


def _problem(t=7, h=3, tk=11, k=5, dqk=6, dv=4, seed=0, dup=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((t, h, dqk))
    kv = rng.standard_normal((tk, dqk))
    do = rng.standard_normal((t, h, dv))
    idx = np.full((t, k), -1, dtype=np.int64)
    for i in range(t):
        n = int(rng.integers(0, k + 1)) if i else k          # token 0 uses every slot
        idx[i, :n] = rng.choice(tk, size=n, replace=False)
    idx[1] = -1                                               # a token with no valid entry
    if dup:
        idx[2, 1] = idx[2, 0]
    return q, kv, idx, do


def _dense_reference(q, kv, idx, do, scale, dv, counts=False):
    """torch fp64: softmax over all keys, masked to the selected ones (logit
    + log(multiplicity) when ``counts``), autograd VJP of sum(O * dO)."""
    t_, h_, _ = q.shape
    tk = kv.shape[0]
    mult = np.zeros((t_, tk))
    for t in range(t_):
        for j in idx[t]:
            if 0 <= j < tk:
                mult[t, j] += 1
    if not counts:
        mult = np.minimum(mult, 1)
    qt = torch.from_numpy(q).clone().requires_grad_(True)
    kvt = torch.from_numpy(kv).clone().requires_grad_(True)
    s = scale * torch.einsum("thd,jd->thj", qt, kvt)
    mt = torch.from_numpy(mult)[:, None, :]
    s = torch.where(mt > 0, s + torch.log(torch.clamp(mt, min=1.0)), torch.full_like(s, -math.inf))
    lse = torch.logsumexp(s, dim=2)
    lse_safe = torch.where(torch.isinf(lse), torch.zeros(()), lse)
    p = torch.where(mt > 0, torch.exp(s - lse_safe[..., None]), torch.zeros(()))
    o = torch.einsum("thj,jd->thd", p, kvt[:, :dv])
    (o * torch.from_numpy(do)).sum().backward()
    return {"o": o.detach().numpy(), "lse": lse.detach().numpy(), "dq": qt.grad.numpy(), "dkv": kvt.grad.numpy()}


def _err(got, ref):
    fin = np.isfinite(ref["lse"])
    if not np.array_equal(np.isneginf(got["lse"]), ~fin):
        return float("inf")
    e = max(np.abs(got[n] - ref[n]).max() for n in ("o", "dq", "dkv"))
    return max(e, np.abs(got["lse"][fin] - ref["lse"][fin]).max())


def check_against_dense(mod, seed=1):
    q, kv, idx, do = _problem(seed=seed)
    scale = 0.6
    got = mod.sparse_mla_bwd(q, kv, idx, do, scale, d_v=4)
    err = _err(got, _dense_reference(q, kv, idx, do, scale, 4))
    fo, fl = mod.sparse_mla_fwd(q, kv, idx, scale, d_v=4)
    return max(err, _err({"o": fo, "lse": fl, "dq": got["dq"], "dkv": got["dkv"]},
                         _dense_reference(q, kv, idx, do, scale, 4)))


def check_duplicates(mod, seed=2):
    q, kv, idx, do = _problem(seed=seed, dup=True)
    got = mod.sparse_mla_bwd(q, kv, idx, do, 0.4, d_v=4)
    return _err(got, _dense_reference(q, kv, idx, do, 0.4, 4, counts=True))


def check_sentinels_and_empty(mod, seed=3):
    q, kv, idx, do = _problem(seed=seed)
    base = mod.sparse_mla_bwd(q, kv, idx, do, 0.5, d_v=4)
    noisy = idx.copy()
    noisy[noisy < 0] = np.array([-7, kv.shape[0], kv.shape[0] + 3, -1])[np.arange((noisy < 0).sum()) % 4]
    alt = mod.sparse_mla_bwd(q, kv, noisy, do, 0.5, d_v=4)
    err = max(np.abs(base[n] - alt[n]).max() for n in ("o", "dq", "dkv"))
    ok = np.all(base["o"][1] == 0) and np.all(np.isneginf(base["lse"][1])) and np.all(base["dq"][1] == 0)
    return err if ok else float("inf")


def check_real_dims(mod, seed=4):
    """The supported dims (576 / 512) against the dense reference."""
    q, kv, idx, do = _problem(t=3, h=2, tk=9, k=4, dqk=576, dv=512, seed=seed)
    got = mod.sparse_mla_bwd(q, kv, idx, do, 1.0 / math.sqrt(576))
    return _err(got, _dense_reference(q, kv, idx, do, 1.0 / math.sqrt(576), 512))


def test_against_masked_dense_autograd():
    assert check_against_dense(sm) < 1e-12


def test_listed_twice_is_double_weight():
    assert check_duplicates(sm) < 1e-12


def test_sentinels_and_empty_rows():
    assert check_sentinels_and_empty(sm) == 0.0


def test_real_dims():
    assert check_real_dims(sm) < 1e-10


MUTATIONS = {
    "values_all_channels": ("o = p @ kj[:, :d_v]", "o = p @ kj[:, -d_v:]"),
    "no_delta": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "dkv_overwrite": ("np.add.at(out[\"dkv\"], j, scale * (ds.T @ q[t]))", "out[\"dkv\"][j] = scale * (ds.T @ q[t])"),
    "dkv_no_value_part": ("np.add.at(out[\"dkv\"][:, :d_v], j, p.T @ do[t])", "pass"),
    "dq_unscaled": ("out[\"dq\"][t] = scale * (ds @ kj)", "out[\"dq\"][t] = ds @ kj"),
    "sentinel_as_last_row": ("return idx_t[(idx_t >= 0) & (idx_t < tk)]", "return idx_t[idx_t < tk]"),
    "lse_without_max": ("out[\"lse\"][t] = (m + np.log(z))[:, 0]", "out[\"lse\"][t] = np.log(z)[:, 0]"),
}


def _mutant(old, new):
    src = inspect.getsource(sm)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("smla_mutant")
    exec(compile(src.replace(old, new), "smla_mutant", "exec"), mod.__dict__)
    return mod


def _any_fails(mod):
    checks = [lambda: check_against_dense(mod) < 1e-12, lambda: check_duplicates(mod) < 1e-12,
              lambda: check_sentinels_and_empty(mod) == 0.0, lambda: check_real_dims(mod) < 1e-10]
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
