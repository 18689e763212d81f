"""Pins of the fp64 oracle against things other than itself.

Each check below would fail for a plausible mistake in the oracle: a dropped
``scale``, a wrong sign in dS, a transposed product, a wrong GQA head map, an
off-by-one causal mask, a missing max term in the LSE.  ``test_oracle_mutations``
plants exactly such mistakes in a copy of the oracle and confirms that.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as orc

RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _loss(mod, q, k, v, do, scale, causal, groups):
    o, _ = mod.attention_fwd(q, k, v, scale, causal, groups)
    return float(np.sum(o * do))


# ---------------------------------------------------------------- checks
# They take the oracle module as an argument so that the mutation tests can
# run them against planted mistakes.

def check_finite_differences(mod, hq, hkv, s, d, causal, step=1e-5, seed=0):
    """Central differences of L = sum(O * dO) against the analytic VJP."""
    rng = np.random.default_rng(seed)
    g = hq // hkv
    q, k, v = _rand(1, s, hq, d, rng=rng), _rand(1, s, hkv, d, rng=rng), _rand(1, s, hkv, d, rng=rng)
    do = _rand(1, s, hq, d, rng=rng)
    scale = 1.0 / math.sqrt(d)
    res = mod.attention_bwd(q, k, v, do, scale, causal, g)
    worst = 0.0
    for name, x, grad in (("q", q, res["dq"]), ("k", k, res["dk"]), ("v", v, res["dv"])):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + step
            lp = _loss(mod, q, k, v, do, scale, causal, g)
            x[idx] = old - step
            lm = _loss(mod, q, k, v, do, scale, causal, g)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * step)
        err = np.max(np.abs(num - grad)) / max(np.max(np.abs(num)), 1e-30)
        worst = max(worst, err)
    return worst


def _sdpa_ref(q, k, v, do, scale, causal, groups):
    """torch CPU fp64 scaled_dot_product_attention (math path) with autograd."""
    t = lambda a: torch.tensor(np.ascontiguousarray(np.transpose(a, (0, 2, 1, 3))), dtype=torch.float64, requires_grad=True)
    tq, tk, tv = t(q), t(k), t(v)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=groups > 1)
    o.backward(torch.tensor(np.transpose(do, (0, 2, 1, 3)), dtype=torch.float64))
    back = lambda a: np.transpose(a.detach().numpy(), (0, 2, 1, 3))
    # LSE from the library's own logsumexp over the same scores
    kk = tk.repeat_interleave(groups, dim=1) if groups > 1 else tk
    sc = scale * (tq @ kk.transpose(-1, -2))
    if causal:
        s = q.shape[1]
        sc = sc.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(sc, dim=-1).detach().numpy()
    return {"o": back(o), "dq": back(tq.grad), "dk": back(tk.grad), "dv": back(tv.grad), "lse": lse}


def check_against_sdpa(mod, b, hq, hkv, s, d, causal, seed=0):
    rng = np.random.default_rng(seed)
    g = hq // hkv
    q, k, v = _rand(b, s, hq, d, rng=rng), _rand(b, s, hkv, d, rng=rng), _rand(b, s, hkv, d, rng=rng)
    do = _rand(b, s, hq, d, rng=rng)
    scale = 0.7 / math.sqrt(d)
    ref = _sdpa_ref(q, k, v, do, scale, causal, g)
    o, lse = mod.attention_fwd(q, k, v, scale, causal, g)
    res = mod.attention_bwd(q, k, v, do, scale, causal, g)
    errs = {
        "o": np.max(np.abs(o - ref["o"])),
        "lse": np.max(np.abs(lse - ref["lse"])),
        "dq": np.max(np.abs(res["dq"] - ref["dq"])),
        "dk": np.max(np.abs(res["dk"] - ref["dk"])),
        "dv": np.max(np.abs(res["dv"] - ref["dv"])),
        "bwd_o": np.max(np.abs(res["o"] - ref["o"])),
        "bwd_lse": np.max(np.abs(res["lse"] - ref["lse"])),
    }
    return max(errs.values()), errs


def check_closed_forms(mod, causal, s=7, d=5, hq=2, hkv=1):
    """Q = 0 gives uniform attention; S = 1 gives O = V."""
    rng = np.random.default_rng(7)
    g = hq // hkv
    k, v = _rand(1, s, hkv, d, rng=rng), _rand(1, s, hkv, d, rng=rng)
    do = _rand(1, s, hq, d, rng=rng)
    q = np.zeros((1, s, hq, d))
    o, lse = mod.attention_fwd(q, k, v, 0.5, causal, g)
    res = mod.attention_bwd(q, k, v, do, 0.5, causal, g)
    errs = []
    for h in range(hq):
        for i in range(s):
            n = i + 1 if causal else s
            errs.append(np.max(np.abs(o[0, i, h] - v[0, :n, h // g].mean(axis=0))))
            errs.append(abs(lse[0, h, i] - math.log(n)))
    errs.append(np.max(np.abs(res["dk"])))  # dK = scale * dS^T Q = 0
    # S = 1: O = V, LSE = scale q.k, dQ = dK = 0, dV = sum of the group's dO
    q1, k1, v1, do1 = _rand(1, 1, hq, d, rng=rng), _rand(1, 1, hkv, d, rng=rng), _rand(1, 1, hkv, d, rng=rng), _rand(1, 1, hq, d, rng=rng)
    o1, lse1 = mod.attention_fwd(q1, k1, v1, 0.3, causal, g)
    r1 = mod.attention_bwd(q1, k1, v1, do1, 0.3, causal, g)
    for h in range(hq):
        errs.append(np.max(np.abs(o1[0, 0, h] - v1[0, 0, h // g])))
        errs.append(abs(lse1[0, h, 0] - 0.3 * float(q1[0, 0, h] @ k1[0, 0, h // g])))
    errs.append(np.max(np.abs(r1["dq"])))
    errs.append(np.max(np.abs(r1["dk"])))
    dv_expect = do1[0, 0].reshape(hkv, g, d).sum(axis=1)
    errs.append(np.max(np.abs(r1["dv"][0, 0] - dv_expect)))
    return max(errs)


def check_two_key_sigmoid(mod):
    """S = 2, D = 1, non-causal: row i attends keys with weight sigmoid(scale*q_i*(k0-k1))."""
    q = np.array([0.8, -1.3]).reshape(1, 2, 1, 1)
    k = np.array([0.5, -0.25]).reshape(1, 2, 1, 1)
    v = np.array([2.0, -1.0]).reshape(1, 2, 1, 1)
    scale = 0.9
    o, lse = mod.attention_fwd(q, k, v, scale, False, 1)
    errs = []
    for i in range(2):
        a = scale * q[0, i, 0, 0] * (k[0, 0, 0, 0] - k[0, 1, 0, 0])
        w0 = 1.0 / (1.0 + math.exp(-a))
        errs.append(abs(o[0, i, 0, 0] - (w0 * 2.0 + (1 - w0) * -1.0)))
        e0 = math.exp(scale * q[0, i, 0, 0] * 0.5)
        e1 = math.exp(scale * q[0, i, 0, 0] * -0.25)
        errs.append(abs(lse[0, 0, i] - math.log(e0 + e1)))
    # causal: row 0 sees key 0 only
    oc, lsec = mod.attention_fwd(q, k, v, scale, True, 1)
    errs.append(abs(oc[0, 0, 0, 0] - 2.0))
    errs.append(abs(lsec[0, 0, 0] - scale * 0.8 * 0.5))
    errs.append(abs(oc[0, 1, 0, 0] - o[0, 1, 0, 0]))
    return max(errs)


def check_softmax_and_mask(mod, causal, s=9, d=4):
    rng = np.random.default_rng(3)
    q, k = _rand(1, s, 2, d, rng=rng), _rand(1, s, 1, d, rng=rng)
    errs = []
    for h in range(2):
        p = mod.softmax_probs(q, k, 0.6, causal, 2, b=0, h=h)
        errs.append(np.max(np.abs(p.sum(axis=1) - 1.0)))
        if np.min(p) < 0:
            errs.append(1.0)
        if causal:
            errs.append(np.max(np.abs(np.triu(p, 1))))  # zero above the diagonal
            if np.min(np.diag(p)) <= 0:
                errs.append(1.0)
        # P_ij = exp(scale q_i.k_j - LSE_i)
        v = _rand(1, s, 1, d, rng=rng)
        _, lse = mod.attention_fwd(q, k, v, 0.6, causal, 2)
        sc = 0.6 * q[0, :, h, :] @ k[0, :, 0, :].T
        pe = np.exp(sc - lse[0, h][:, None])
        if causal:
            pe = np.tril(pe)
        errs.append(np.max(np.abs(pe - p)))
    return max(errs)


def check_dv_is_pt_do_and_delta(mod, causal, s=11, d=6, hq=4, hkv=2):
    rng = np.random.default_rng(5)
    g = hq // hkv
    q, k, v = _rand(1, s, hq, d, rng=rng), _rand(1, s, hkv, d, rng=rng), _rand(1, s, hkv, d, rng=rng)
    do = _rand(1, s, hq, d, rng=rng)
    res = mod.attention_bwd(q, k, v, do, 0.4, causal, g)
    o, _ = mod.attention_fwd(q, k, v, 0.4, causal, g)
    errs = [np.max(np.abs(res["delta"][0] - np.sum(do[0] * o[0], axis=-1).T))]
    for kv in range(hkv):
        acc = np.zeros((s, d))
        for r in range(g):
            h = kv * g + r
            p = mod.softmax_probs(q, k, 0.4, causal, g, b=0, h=h)
            acc += p.T @ do[0, :, h, :]
        errs.append(np.max(np.abs(acc - res["dv"][0, :, kv, :])))
    return max(errs)


def check_gqa_is_sum_of_mha(mod, causal, s=10, d=4, hq=6, hkv=2):
    rng = np.random.default_rng(11)
    g = hq // hkv
    q, k, v = _rand(2, s, hq, d, rng=rng), _rand(2, s, hkv, d, rng=rng), _rand(2, s, hkv, d, rng=rng)
    do = _rand(2, s, hq, d, rng=rng)
    gq = mod.attention_bwd(q, k, v, do, 0.5, causal, g)
    kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
    mh = mod.attention_bwd(q, kr, vr, do, 0.5, causal, 1)
    errs = [np.max(np.abs(gq["dq"] - mh["dq"])), np.max(np.abs(gq["o"] - mh["o"]))]
    errs.append(np.max(np.abs(gq["dk"] - mh["dk"].reshape(2, s, hkv, g, d).sum(axis=3))))
    errs.append(np.max(np.abs(gq["dv"] - mh["dv"].reshape(2, s, hkv, g, d).sum(axis=3))))
    return max(errs)


def check_shift_invariance(mod, causal, s=12, d=5):
    rng = np.random.default_rng(13)
    q, k, v = _rand(1, s, 2, d, rng=rng), _rand(1, s, 2, d, rng=rng), _rand(1, s, 2, d, rng=rng)
    do = _rand(1, s, 2, d, rng=rng)
    u = _rand(d, rng=rng)
    o, lse = mod.attention_fwd(q, k, v, 0.45, causal, 1)
    o2, lse2 = mod.attention_fwd(q, k + u, v, 0.45, causal, 1)
    shift = 0.45 * np.einsum("bshd,d->bhs", q, u)
    res = mod.attention_bwd(q, k, v, do, 0.45, causal, 1)
    return max(np.max(np.abs(o - o2)), np.max(np.abs(lse2 - lse - shift)), np.max(np.abs(res["dk"].sum(axis=1))))


def check_rows_cols(mod, causal, s=37, d=8, hq=4, hkv=2):
    """The per-row / per-key helpers against torch's autograd."""
    rng = np.random.default_rng(17)
    g = hq // hkv
    q, k, v = _rand(1, s, hq, d, rng=rng), _rand(1, s, hkv, d, rng=rng), _rand(1, s, hkv, d, rng=rng)
    do = _rand(1, s, hq, d, rng=rng)
    ref = _sdpa_ref(q, k, v, do, 0.35, causal, g)
    rows = [0, 5, 17, 36]
    r = mod.attention_rows(q, k, v, do, 0.35, causal, g, 0, 3, rows)
    errs = [np.max(np.abs(r["o"] - ref["o"][0, rows, 3])), np.max(np.abs(r["dq"] - ref["dq"][0, rows, 3])),
            np.max(np.abs(r["lse"] - ref["lse"][0, 3, rows]))]
    cols = [2, 20, 36]
    c = mod.attention_cols(q, k, v, do, 0.35, causal, g, 0, 1, cols)
    errs += [np.max(np.abs(c["dk"] - ref["dk"][0, cols, 1])), np.max(np.abs(c["dv"] - ref["dv"][0, cols, 1]))]
    return max(errs)


# ---------------------------------------------------------------- tests

FD_CASES = [(2, 2, 1, 4), (2, 2, 5, 4), (4, 2, 16, 4), (4, 2, 17, 8), (2, 2, 5, 8)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv,s,d", FD_CASES)
def test_finite_differences(hq, hkv, s, d, causal):
    assert check_finite_differences(orc, hq, hkv, s, d, causal) < 1e-6


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,hq,hkv,s,d", [(1, 2, 2, 33, 16), (2, 4, 2, 65, 8), (1, 8, 1, 20, 12), (1, 2, 2, 600, 8)])
def test_against_torch_sdpa_fp64(b, hq, hkv, s, d, causal):
    worst, errs = check_against_sdpa(orc, b, hq, hkv, s, d, causal)
    assert worst < 1e-10, errs


@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(causal):
    assert check_closed_forms(orc, causal) < 1e-12


def test_two_key_sigmoid():
    assert check_two_key_sigmoid(orc) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_and_causal_mask(causal):
    assert check_softmax_and_mask(orc, causal) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_dv_is_pt_do_and_delta(causal):
    assert check_dv_is_pt_do_and_delta(orc, causal) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_is_group_sum_of_mha(causal):
    assert check_gqa_is_sum_of_mha(orc, causal) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    assert check_shift_invariance(orc, causal) < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_row_and_key_helpers(causal):
    assert check_rows_cols(orc, causal) < 1e-11


def test_causal_first_row_sees_only_first_key():
    rng = np.random.default_rng(2)
    q, k, v = _rand(1, 6, 2, 4, rng=rng), _rand(1, 6, 2, 4, rng=rng), _rand(1, 6, 2, 4, rng=rng)
    o, lse = orc.attention_fwd(q, k, v, 0.5, True, 1)
    assert np.max(np.abs(o[0, 0] - v[0, 0])) == 0.0
    assert np.allclose(lse[0, :, 0], 0.5 * np.sum(q[0, 0] * k[0, 0], axis=-1), atol=1e-14)


def test_large_rows_blocked_matches_unblocked():
    """Row blocking (S > block) agrees with torch at S spanning several blocks."""
    worst, errs = check_against_sdpa(orc, 1, 2, 1, 1100, 4, True, seed=3)
    assert worst < 1e-10, errs
