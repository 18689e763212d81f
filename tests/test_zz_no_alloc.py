"""attn_bwd_noalloc, the backward that runs on the library's own scratch
array instead of a caller workspace, against attn_bwd (use_atomic = 0, with
a caller workspace) and the fp64 oracle.

Each test makes two calls in a row on one GPU, the second on a smaller
problem, so the second call runs on scratch that still holds the first
call's partials.  Outputs start as NaN: an element the call fails to write
shows up.
"""

import math

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd import binding as bd
from attention_backward_fwd_amd.synthetic import make_inputs
from oracle import attention as orc
from tests.gpu_helpers import TOL, err_ratio, gqa_parts, np64, run_path, say, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _scratch_need(b, s, hq, g, d):
    nq = b * s * hq * d
    bn = 512 if d == 64 else 256  # key-block height of the backward kernel
    return ((2 * nq // g * gqa_parts(b, s, hq, g, d) * 4) if g > 1 else 0) + math.ceil(s / bn) * nq * 4


def _noalloc(d, causal, scale):
    """fwd -> preprocess -> attn_bwd_noalloc -> postprocess (dQ cast only)."""
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    sh = bd.shape_of(q, k)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    nan = float("nan")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    bd.attn_fwd(q, k, v, o, lse, sh, scale, causal)
    delta = torch.full((B, Hq, S), nan, dtype=torch.float32, device=q.device)
    dq_accum = torch.full((B, Hq, S, D), nan, dtype=torch.float32, device=q.device)
    dq = torch.full_like(q, nan)
    dk = torch.full((B, S, Hkv, D), nan, dtype=torch.bfloat16, device=q.device)
    dv = torch.full_like(dk, nan)
    bd.attn_bwd_preprocess(o, do, delta, None, sh)
    bd.attn_bwd_noalloc(q, k, v, do, lse, delta, dq_accum, dk, dv, sh, scale, causal)
    sh1 = bd.make_shape(B, S, Hq, 1, D)
    bd.attn_bwd_postprocess(dq_accum, None, dq, None, None, sh1)
    torch.cuda.synchronize()
    return {"dq_accum": dq_accum, "dq": dq, "dk": dk, "dv": dv}


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def _check_one(case, b, s, hq, hkv, d, causal, seed, with_oracle):
    g = hq // hkv
    assert _scratch_need(b, s, hq, g, d) <= SCRATCH_BYTES, case
    say(f"noalloc {case}: b{b} s{s} hq{hq} hkv{hkv} d{d} causal={causal} "
        f"scratch={_scratch_need(b, s, hq, g, d) / 2**20:.1f} MiB")
    inp = make_inputs(b, s, hq, hkv, d, seed=seed)
    dev = to_dev(inp)
    scale = 1.0 / math.sqrt(d)
    got = _noalloc(dev, causal, scale)
    want = run_path(dev, causal, scale, use_atomic=0)
    # The same kernels in the same order: bit for bit equal.
    for n in ("dq_accum", "dq", "dk", "dv"):
        assert torch.equal(_bits(got[n]), _bits(want[n])), (case, n)
    if with_oracle:
        f = {n: t.to(torch.float64).numpy() for n, t in inp.items()}
        ref = orc.attention_bwd(f["q"], f["k"], f["v"], f["do"], scale, causal, g)
        zs = float(np.max(np.abs(ref["dv"])))
        for n in ("dq", "dk", "dv"):
            r = err_ratio(np64(got[n]), ref[n], zero_scale=zs)
            say(f"  {n}: {r:.2e}")
            assert r <= TOL, (case, n, r)


def test_noalloc_mha_largest_then_small():
    # B1 S2048 Hq32 D64: 4 key blocks of 512 x 4 Mi floats x 4 B = exactly 64 MiB.
    _check_one("mha max", 1, 2048, 32, 32, 64, True, seed=5, with_oracle=False)
    _check_one("mha small", 2, 300, 4, 4, 128, False, seed=6, with_oracle=True)


def test_noalloc_gqa_then_smaller():
    _check_one("gqa", 2, 520, 8, 2, 128, True, seed=7, with_oracle=True)
    _check_one("gqa smaller", 1, 77, 4, 2, 64, False, seed=8, with_oracle=True)


def test_noalloc_rejects_oversize_without_launch():
    inp = to_dev(make_inputs(1, 4096, 8, 8, 128, seed=1))
    q, k = inp["q"], inp["k"]
    sh = bd.shape_of(q, k)
    dq_accum = torch.zeros((1, 8, 4096, 128), dtype=torch.float32, device=q.device)
    lse = torch.zeros((1, 8, 4096), dtype=torch.float32, device=q.device)
    dk = torch.zeros_like(k)
    with pytest.raises(bd.AttnError) as ei:
        bd.attn_bwd_noalloc(q, k, inp["v"], inp["do"], lse, lse, dq_accum, dk, dk, sh, 0.1, 1)
    assert ei.value.status == -9
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq_accum).item() == 0
