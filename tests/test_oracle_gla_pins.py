"""Pins of the simple gated linear attention oracle (``oracle.linear_attn``).

Independent references: the recurrent (state) form written in torch fp64 with
autograd for every gradient including the gate's; central finite
differences; closed forms (no decay: causal linear attention by running sums
of outer products; a very strong decay: only the diagonal term survives; one
token); the identity dL/dG_t = q_t . dq_t - k_t . dk_t.  Planted mistakes in a
copy of the module must be caught.
"""

import inspect
import types

import numpy as np
import pytest
import torch

from oracle import linear_attn as la


def _inputs(b, t, h, dk, dv, seed, g_scale=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, t, h, dk))
    k = rng.standard_normal((b, t, h, dk))
    v = rng.standard_normal((b, t, h, dv))
    g = -g_scale * np.abs(rng.standard_normal((b, t, h)))
    do = rng.standard_normal((b, t, h, dv))
    return q, k, v, g, do


def _recurrent_torch(q, k, v, g, do, scale):
    """State recurrence S_t = exp(g_t) S_{t-1} + k_t^T v_t, o_t = scale q_t S_t,
    step by step in torch fp64; gradients by autograd."""
    qt, kt, vt, gt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v, g))
    b_, t_, h_, dk = q.shape
    dv = v.shape[3]
    outs = []
    for b in range(b_):
        for h in range(h_):
            s = torch.zeros((dk, dv), dtype=torch.float64)
            rows = []
            for t in range(t_):
                s = torch.exp(gt[b, t, h]) * s + torch.outer(kt[b, t, h], vt[b, t, h])
                rows.append(scale * (qt[b, t, h] @ s))
            outs.append(torch.stack(rows))
    o = torch.stack(outs).reshape(b_, h_, t_, dv).permute(0, 2, 1, 3)
    (o * torch.from_numpy(do)).sum().backward()
    return {"o": o.detach().numpy(), "dq": qt.grad.numpy(), "dk": kt.grad.numpy(), "dv": vt.grad.numpy(),
            "dg": gt.grad.numpy()}


def check_against_recurrent(mod, seed=1):
    q, k, v, g, do = _inputs(2, 13, 2, 3, 4, seed)
    got = mod.gla_bwd(q, k, v, g, do, 0.7)
    ref = _recurrent_torch(q, k, v, g, do, 0.7)
    fo = mod.gla_fwd(q, k, v, g, 0.7)
    err = max(np.abs(got[n] - ref[n]).max() for n in ("o", "dq", "dk", "dv", "dg"))
    return max(err, np.abs(fo - ref["o"]).max())


def check_finite_differences(mod, seed=2, eps=1e-6):
    q, k, v, g, do = _inputs(1, 6, 1, 2, 3, seed)
    scale = 0.9
    got = mod.gla_bwd(q, k, v, g, do, scale)

    def loss(q_, k_, v_, g_):
        return float(np.sum(mod.gla_fwd(q_, k_, v_, g_, scale) * do))

    worst = 0.0
    args = [q, k, v, g]
    for idx, name in enumerate(("dq", "dk", "dv", "dg")):
        x = args[idx]
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            ap, am = list(args), list(args)
            ap[idx], am[idx] = xp, xm
            fd = (loss(*ap) - loss(*am)) / (2 * eps)
            worst = max(worst, abs(fd - got[name][pos]) / max(1.0, abs(fd)))
    return worst


def check_closed_forms(mod, seed=3):
    q, k, v, _, do = _inputs(1, 7, 1, 3, 2, seed)
    err = 0.0
    # no decay: o_t = scale * q_t . sum_{s<=t} k_s^T v_s
    z = np.zeros((1, 7, 1))
    o = mod.gla_fwd(q, k, v, z, 0.5)
    run = np.cumsum(np.einsum("tk,tv->tkv", k[0, :, 0], v[0, :, 0]), axis=0)
    want = 0.5 * np.einsum("tk,tkv->tv", q[0, :, 0], run)
    err = max(err, np.abs(o[0, :, 0] - want).max())
    # strong decay: only s = t survives
    o = mod.gla_fwd(q, k, v, np.full((1, 7, 1), -80.0), 0.5)
    want = 0.5 * np.sum(q[0, :, 0] * k[0, :, 0], axis=1)[:, None] * v[0, :, 0]
    err = max(err, np.abs(o[0, :, 0] - want).max())
    # one token: o = scale (q.k) v, dq = scale (do.v) k, dg = 0 (the gate of the
    # first token multiplies the zero initial state)
    r = mod.gla_bwd(q[:, :1], k[:, :1], v[:, :1], np.full((1, 1, 1), -0.4), do[:, :1], 0.5)
    qk, dov = float(q[0, 0, 0] @ k[0, 0, 0]), float(do[0, 0, 0] @ v[0, 0, 0])
    err = max(err, np.abs(r["o"][0, 0, 0] - 0.5 * qk * v[0, 0, 0]).max(),
              np.abs(r["dq"][0, 0, 0] - 0.5 * dov * k[0, 0, 0]).max(), abs(r["dg"][0, 0, 0]))
    return err


def check_gate_identity(mod, seed=4):
    """dL/dG_t = dg_t - dg_{t+1} equals q_t . dq_t - k_t . dk_t."""
    q, k, v, g, do = _inputs(2, 9, 2, 3, 3, seed)
    r = mod.gla_bwd(q, k, v, g, do, 1.3)
    dG = r["dg"] - np.concatenate([r["dg"][:, 1:], np.zeros_like(r["dg"][:, :1])], axis=1)
    want = np.sum(q * r["dq"], axis=3) - np.sum(k * r["dk"], axis=3)
    return np.abs(dG - want).max()


def test_against_recurrent_autograd():
    assert check_against_recurrent(la) < 1e-12


def test_finite_differences():
    assert check_finite_differences(la) < 1e-7


def test_closed_forms():
    assert check_closed_forms(la) < 1e-12


def test_gate_identity():
    assert check_gate_identity(la) < 1e-12


def test_heads_subset():
    q, k, v, g, do = _inputs(2, 5, 3, 2, 2, 6)
    full = la.gla_bwd(q, k, v, g, do, 0.4)
    part = la.gla_bwd(q, k, v, g, do, 0.4, heads=[(1, 2)])
    for n in ("dq", "dk", "dv", "dg", "o"):
        assert np.array_equal(part[n][1, :, 2], full[n][1, :, 2])
        assert np.all(np.isnan(part[n][0, :, 0]))


MUTATIONS = {
    "decay_sign": ("diff = G[:, None] - G[None, :]", "diff = G[None, :] - G[:, None]"),
    "decay_strict": ("lower = np.tril(np.ones((t, t), dtype=bool))", "lower = np.tril(np.ones((t, t), dtype=bool), -1)"),
    "dk_not_transposed": ('out["dk"][b, :, h] = a_dov.T @ qb', 'out["dk"][b, :, h] = a_dov @ qb'),
    "dv_from_dov": ('out["dv"][b, :, h] = a_qk.T @ dob', 'out["dv"][b, :, h] = a_dov.T @ dob'),
    "dg_forward_cumsum": ('out["dg"][b, :, h] = np.cumsum(d_g_cum[::-1])[::-1]', 'out["dg"][b, :, h] = np.cumsum(d_g_cum)'),
    "dg_sign": ("d_g_cum = np.sum(w, axis=1) - np.sum(w, axis=0)", "d_g_cum = np.sum(w, axis=0) - np.sum(w, axis=1)"),
    "dq_unscaled": ("a_dov = scale * (dob @ vb.T) * dm", "a_dov = (dob @ vb.T) * dm"),
    "gate_not_cumulative": ("G = np.cumsum(g_bh)", "G = np.asarray(g_bh)"),
}


def _mutant(old, new):
    src = inspect.getsource(la)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("gla_mutant")
    exec(compile(src.replace(old, new), "gla_mutant", "exec"), mod.__dict__)
    return mod


def _any_fails(mod):
    checks = [lambda: check_against_recurrent(mod) < 1e-12, lambda: check_finite_differences(mod) < 1e-7,
              lambda: check_closed_forms(mod) < 1e-12, lambda: check_gate_identity(mod) < 1e-12]
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
