"""Pins of the packed-sequence oracle (``oracle.varlen``).

Independent references: torch's fp64 SDPA over all tokens with a mask built
element by element (same sequence; causal with the last query aligned to the
last key) and autograd for the gradients, for equal and for different query
and key lengths; equal-length packing against the dense batched oracle;
different lengths against the square causal oracle (a query prefix with
dO = 0, or empty leading rows); a single query equals non-causal attention;
and the padding / empty-sequence conventions.  Planted mistakes must be
caught.
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


def _mask(cu, t, causal, cu_k=None, tk=None):
    """[Tq, Tk] boolean 'may attend' mask built element by element: same
    sequence, and under causal masking key position <= query position +
    (keys - queries of that sequence)."""
    cu_k = cu if cu_k is None else cu_k
    tk = t if tk is None else tk
    m = np.zeros((t, tk), dtype=bool)
    for b in range(len(cu) - 1):
        lq, lk = cu[b + 1] - cu[b], cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            for j in range(lk):
                m[cu[b] + i, cu_k[b] + j] = (not causal) or j <= i + lk - lq
    return m


def _sdpa_reference(q, k, v, do, cu, scale, causal, groups, cu_k=None):
    """torch fp64: masked softmax attention over all tokens, autograd VJP.
    Rows that see no key get LSE = -inf and P = 0."""
    t, tk = q.shape[0], k.shape[0]
    allowed = torch.from_numpy(_mask(cu, t, causal, cu_k, tk))
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    kr, vr = kt.repeat_interleave(groups, dim=1), vt.repeat_interleave(groups, dim=1)
    s = torch.einsum("ihd,jhd->hij", qt, kr) * scale
    s = s.masked_fill(~allowed[None], float("-inf"))
    lse = torch.logsumexp(s, dim=2)                         # [H, T]
    lse_safe = torch.where(torch.isinf(lse), torch.zeros(()), lse)
    p = torch.where(allowed[None], torch.exp(s - lse_safe[..., None]), torch.zeros(()))
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


CU_Q = [0, 5, 5, 12, 13, 20, 23]    # query lengths 5, 0, 7, 1, 7, 3; Tq = 26 (3 padding rows)
CU_K = [0, 9, 11, 14, 14, 25, 26]   # key lengths 9, 2, 3, 0, 11, 1; Tk = 29 (3 padding rows)


def check_rect_against_sdpa(mod, causal, hq=4, hkv=2, d=5, seed=8):
    rng = np.random.default_rng(seed)
    q, do = rng.standard_normal((26, hq, d)), rng.standard_normal((26, hq, d))
    k, v = rng.standard_normal((29, hkv, d)), rng.standard_normal((29, hkv, d))
    scale = 0.4
    got = mod.varlen_bwd(q, k, v, do, CU_Q, scale, causal, hq // hkv, CU_K)
    ref = _sdpa_reference(q, k, v, do, CU_Q, scale, causal, hq // hkv, CU_K)
    err = max(np.abs(got[n] - ref[n]).max() for n in ("o", "dq", "dk", "dv"))
    fin = np.isfinite(ref["lse"])
    if not np.array_equal(np.isneginf(got["lse"]), ~fin):
        return float("inf")
    err = max(err, np.abs(got["lse"][fin] - ref["lse"][fin]).max())
    fo, fl = mod.varlen_fwd(q, k, v, CU_Q, scale, causal, hq // hkv, CU_K)
    if not np.array_equal(np.isneginf(fl), ~fin):
        return float("inf")
    return max(err, np.abs(fo - ref["o"]).max())


def check_rect_reduces_to_square(mod, seed=12):
    """Bottom-right alignment against the (independently pinned) square
    causal oracle.  More keys than queries (lk > lq): the queries are the
    last lq rows of a square causal problem whose first lk - lq queries carry
    dO = 0 (so they add nothing to dK, dV).  More queries than keys: the
    first lq - lk rows see nothing; the last lk rows are the square problem."""
    rng = np.random.default_rng(seed)
    hq, d, scale = 2, 4, 0.7
    err = 0.0
    for lq, lk in ((3, 8), (8, 3), (1, 6)):
        q, do = rng.standard_normal((lq, hq, d)), rng.standard_normal((lq, hq, d))
        k, v = rng.standard_normal((lk, 1, d)), rng.standard_normal((lk, 1, d))
        got = mod.varlen_bwd(q, k, v, do, [0, lq], scale, True, hq, [0, lk])
        if lk >= lq:
            pre = rng.standard_normal((lk - lq, hq, d))
            qs = np.concatenate([pre, q])[None]
            dos = np.concatenate([np.zeros_like(pre), do])[None]
            ref = att.attention_bwd(qs, k[None], v[None], dos, scale, True, hq)
            rows = slice(lk - lq, lk)
            err = max(err, np.abs(got["o"] - ref["o"][0, rows]).max(), np.abs(got["dq"] - ref["dq"][0, rows]).max(),
                      np.abs(got["lse"] - ref["lse"][0][:, rows]).max(),
                      np.abs(got["dk"] - ref["dk"][0]).max(), np.abs(got["dv"] - ref["dv"][0]).max())
        else:
            e = lq - lk
            ref = att.attention_bwd(q[e:][None], k[None], v[None], do[e:][None], scale, True, hq)
            if not (np.all(got["o"][:e] == 0) and np.all(got["dq"][:e] == 0) and np.all(np.isneginf(got["lse"][:, :e]))):
                return float("inf")
            err = max(err, np.abs(got["o"][e:] - ref["o"][0]).max(), np.abs(got["dq"][e:] - ref["dq"][0]).max(),
                      np.abs(got["lse"][:, e:] - ref["lse"][0]).max(),
                      np.abs(got["dk"] - ref["dk"][0]).max(), np.abs(got["dv"] - ref["dv"][0]).max())
        if lq == 1:  # one query aligned with the last key sees every key: non-causal attention
            qs = np.concatenate([rng.standard_normal((lk - 1, hq, d)), q])[None]
            nc_o, _ = att.attention_fwd(qs, k[None], v[None], scale, False, hq)
            err = max(err, np.abs(got["o"] - nc_o[0, -1:]).max())
    return err


@pytest.mark.parametrize("causal", [False, True])
def test_rectangular_against_masked_sdpa(causal):
    assert check_rect_against_sdpa(vl, causal) < 1e-12


def test_rectangular_reduces_to_square_causal():
    assert check_rect_reduces_to_square(vl) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_against_masked_sdpa(causal):
    assert check_against_sdpa(vl, causal) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_is_dense(causal):
    assert check_equal_lengths_is_dense(vl, causal) < 1e-12


def test_padding_and_empty_sequences():
    assert check_padding_and_empty(vl) == 0.0


MUTATIONS = {
    "offset_sign_flipped": ("return j <= i + (lk - lq)", "return j <= i + (lq - lk)"),
    "causal_top_left": ("return j <= i + (lk - lq)", "return j <= i"),
    "empty_rows_lse_zero": ('out["lse"][h] = np.where(has, m + np.log(np.where(has, z, 1.0)), -np.inf)',
                            'out["lse"][h] = np.where(has, m + np.log(np.where(has, z, 1.0)), 0.0)'),
    "dv_not_summed_over_group": ('out["dv"][:, kv] += p.T @ do[:, h]', 'out["dv"][:, kv] = p.T @ do[:, h]'),
    "delta_missing": ("ds = p * (do[:, h] @ v[:, kv].T - delta[:, None])", "ds = p * (do[:, h] @ v[:, kv].T)"),
    "dk_unscaled": ('out["dk"][:, kv] += scale * (ds.T @ q[:, h])', 'out["dk"][:, kv] += ds.T @ q[:, h]'),
    "keys_use_query_offsets": ("for (a, e), (ka, ke) in zip(_segments(cu), _segments(cu_k)):",
                               "for (a, e), (ka, ke) in zip(_segments(cu), _segments(cu)):"),
    "padding_lse_zero": ('"o": np.zeros((tq, hq, d)), "lse": np.full((hq, tq), -np.inf)',
                         '"o": np.zeros((tq, hq, d)), "lse": np.zeros((hq, tq))'),
    "softmax_over_all_keys": ("e = np.where(vis, np.exp(s - m[:, None]), 0.0)",
                              "e = np.exp(np.where(vis, s, 0.0) - m[:, None])"),
}


def _mutant(old, new):
    src = inspect.getsource(vl)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("varlen_mutant")
    exec(compile(src.replace(old, new), "varlen_mutant", "exec"), mod.__dict__)
    return mod


def _any_fails(mod):
    checks = [lambda: check_against_sdpa(mod, True) < 1e-12, lambda: check_against_sdpa(mod, False) < 1e-12,
              lambda: check_equal_lengths_is_dense(mod, True) < 1e-12, lambda: check_padding_and_empty(mod) == 0.0,
              lambda: check_rect_against_sdpa(mod, True) < 1e-12, lambda: check_rect_against_sdpa(mod, False) < 1e-12,
              lambda: check_rect_reduces_to_square(mod) < 1e-12]
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
