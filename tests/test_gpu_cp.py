"""GPU parity of the context-parallel pieces: attn_merge against the oracle's
merge, and a one-GPU ring (every visible (query chunk, key chunk) pair as an
ordinary attn_fwd / attn_bwd call, then attn_merge) against the
whole-sequence oracle, forward and backward."""

import math

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd import binding as bd
from attention_backward_fwd_amd.synthetic import make_inputs
from oracle import attention as orc
from oracle import cp
from tests.gpu_helpers import TOL, err_ratio, np64, say

pytestmark = pytest.mark.gpu


def _partials(n, b, s, h, d, seed, empty_rows):
    """Seeded synthetic partial results; some rows see no key in some parts,
    `empty_rows` rows in no part at all."""
    g = torch.Generator().manual_seed(seed)
    o = torch.randn((n, b, s, h, d), generator=g).to(torch.bfloat16)
    lse = (3.0 * torch.randn((n, b, h, s), generator=g) + 1.0).float()
    mask = torch.rand((n, b, h, s), generator=g) < 0.25
    lse[mask] = -math.inf
    for r in range(empty_rows):
        lse[:, r % b, (3 * r) % h, (7 * r + 1) % s] = -math.inf
    return o, lse


def _check_lse(got, ref, case):
    got, ref = np64(got), np.asarray(ref)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), (case, "-inf pattern")
    fin = ~inf_ref
    assert np.all(np.isfinite(got[fin])), case
    err = np.max(np.abs(got[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin])), initial=0.0)
    assert err <= 1e-5, (case, "lse", err)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 2, 5])
def test_merge_against_oracle(n, d):
    o_p, l_p = _partials(n, 2, 77, 3, d, seed=10 * n + d, empty_rows=4)
    ref_o, ref_l = cp.merge_partials(o_p.double().numpy(), l_p.double().numpy())
    o, lse = bd.merge(o_p.cuda(), l_p.cuda())
    torch.cuda.synchronize()
    r = err_ratio(np64(o), ref_o)
    say(f"merge n={n} d={d}: o={r:.2e}")
    assert r <= TOL
    _check_lse(lse, ref_l, f"merge n={n} d={d}")
    empty = np.isneginf(ref_l)  # [B, H, S]; O of such rows must be exactly 0
    oo = np64(o).transpose(0, 2, 1, 3)  # [B, H, S, D]
    assert np.all(oo[empty] == 0.0)


def _chunk(t, i, c):
    return t[:, i * c:(i + 1) * c].contiguous()


def _ring_fwd(q, k, v, scale, causal, n_chunks):
    """Per query chunk: attn_fwd over each visible key chunk into a stack of
    partials, then attn_merge."""
    b, s, hq, d = q.shape
    c = s // n_chunks
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, s), dtype=torch.float32, device=q.device)
    merged = []
    for i in range(n_chunks):
        pairs = [(j, cz) for (qi, j, cz) in cp.chunk_pairs(n_chunks, causal) if qi == i]
        o_p = torch.full((len(pairs), b, c, hq, d), float("nan"), dtype=torch.bfloat16, device=q.device)
        l_p = torch.full((len(pairs), b, hq, c), float("nan"), dtype=torch.float32, device=q.device)
        qi_ = _chunk(q, i, c)
        for n, (j, cz) in enumerate(pairs):
            kj, vj = _chunk(k, j, c), _chunk(v, j, c)
            bd.attn_fwd(qi_, kj, vj, o_p[n], l_p[n], bd.shape_of(qi_, kj), scale, cz)
        oi, li = bd.merge(o_p, l_p)
        o[:, i * c:(i + 1) * c] = oi
        lse[:, :, i * c:(i + 1) * c] = li
        merged.append((oi, li))
    return o, lse, merged


CASES = [(1, 3, 80, 4, 2, 128, True), (1, 3, 80, 4, 2, 128, False), (2, 4, 64, 2, 2, 64, True),
         (1, 2, 200, 8, 8, 128, True)]


@pytest.mark.parametrize("b,n_chunks,c,hq,hkv,d,causal", CASES)
def test_ring_forward(b, n_chunks, c, hq, hkv, d, causal):
    inp = make_inputs(b, n_chunks * c, hq, hkv, d, seed=300 + c + d)
    scale = 1.0 / math.sqrt(d)
    f = {n: t.to(torch.float64).numpy() for n, t in inp.items()}
    ref_o, ref_l = orc.attention_fwd(f["q"], f["k"], f["v"], scale, causal, hq // hkv)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse, _ = _ring_fwd(q, k, v, scale, causal, n_chunks)
    torch.cuda.synchronize()
    case = f"ring fwd b{b} P{n_chunks} C{c} hq{hq} hkv{hkv} d{d} causal={causal}"
    r = err_ratio(np64(o), ref_o)
    say(f"{case}: o={r:.2e}")
    assert r <= TOL, case
    _check_lse(lse, ref_l, case)


@pytest.mark.parametrize("b,n_chunks,c,hq,hkv,d,causal", CASES)
def test_ring_backward(b, n_chunks, c, hq, hkv, d, causal):
    """dQ of a query chunk accumulates over its key chunks in one fp32
    accumulator (atomic path); each pair's dK/dV terms are summed in fp32
    by the test."""
    inp = make_inputs(b, n_chunks * c, hq, hkv, d, seed=500 + c + d)
    scale = 1.0 / math.sqrt(d)
    g = hq // hkv
    f = {n: t.to(torch.float64).numpy() for n, t in inp.items()}
    ref = orc.attention_bwd(f["q"], f["k"], f["v"], f["do"], scale, causal, g)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse, merged = _ring_fwd(q, k, v, scale, causal, n_chunks)
    dq = torch.empty_like(q)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    for i in range(n_chunks):
        oi, li = merged[i]
        qi_, doi = _chunk(q, i, c), _chunk(do, i, c)
        sh = bd.shape_of(qi_, _chunk(k, 0, c))
        delta = torch.empty((b, hq, c), dtype=torch.float32, device=q.device)
        acc = torch.empty((b, hq, c, d), dtype=torch.float32, device=q.device)
        bd.attn_bwd_preprocess(oi, doi, delta, acc, sh)
        dq_i = torch.empty_like(qi_)
        for (qi, j, cz) in cp.chunk_pairs(n_chunks, causal):
            if qi != i:
                continue
            kj, vj = _chunk(k, j, c), _chunk(v, j, c)
            dk_ij, dv_ij = torch.empty_like(kj), torch.empty_like(vj)
            nb = bd.attn_bwd_workspace_bytes(sh, cz, 1)
            ws = torch.empty(max(nb, 4) // 4, dtype=torch.float32, device=q.device)
            bd.attn_bwd(qi_, kj, vj, doi, li, delta, acc, dk_ij, dv_ij, ws if nb else None, sh, scale, cz, 1)
            if g > 1:  # reduce the pair's per-query-head dK/dV partials
                bd.attn_bwd_postprocess(acc, ws, dq_i, dk_ij, dv_ij, sh)
            dk[:, j * c:(j + 1) * c] += dk_ij.float()
            dv[:, j * c:(j + 1) * c] += dv_ij.float()
        bd.attn_bwd_postprocess(acc, None, dq_i, None, None, bd.shape_of(qi_, qi_))
        dq[:, i * c:(i + 1) * c] = dq_i
    torch.cuda.synchronize()
    case = f"ring bwd b{b} P{n_chunks} C{c} hq{hq} hkv{hkv} d{d} causal={causal}"
    ratios = {n: err_ratio(np64(t), ref[n]) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    say(f"{case}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (case, n, r)
