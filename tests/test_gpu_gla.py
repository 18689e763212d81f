"""GPU parity of the simple gated linear attention chunk backward
(gla_chunk_bwd) against the fp64 oracle: element by element on small
problems (one and several chunks, ragged last chunks, a single token, no
decay, strong decay), on whole heads of the benchmark workload, and bitwise
run-to-run reproducibility."""

import math

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd import binding as bd
from attention_backward_fwd_amd.synthetic import GLA_WORKLOAD, gla_inputs
from oracle import linear_attn as la
from tests.gpu_helpers import TOL, err_ratio, np64, say

pytestmark = pytest.mark.gpu

NAN = float("nan")


def run_gla(inp, scale):
    """gla_chunk_bwd with every output and the workspace poisoned first."""
    d = {n: x.cuda() for n, x in inp.items()}
    bb = bd.GlaBuffers(d["q"])
    for t in (bb.dq, bb.dk, bb.dv, bb.dg, bb.workspace):
        t.fill_(NAN)
    bd.gla_backward(d["q"], d["k"], d["v"], d["g"], d["do"], scale, buffers=bb)
    torch.cuda.synchronize()
    return {"dq": bb.dq, "dk": bb.dk, "dv": bb.dv, "dg": bb.dg}


def _dg_scale(inp, ref):
    """Error scale of dg.  dg_r sums the per-token terms q_t.dq_t - k_t.dk_t
    over t >= r; each term carries rounding error relative to |q.dq| + |k.dk|
    (not to their difference), and independent errors add up like a random
    walk.  So the scale is sqrt(sum_{t>=r} (|q_t.dq_t| + |k_t.dk_t|)^2), fp64
    from the oracle's gradients.  It matters where the terms cancel (strong
    decay: q.dq = k.dk on every token, exact dg ~0); elsewhere it is of the
    order of max|dg|."""
    q, k = inp["q"].double().numpy(), inp["k"].double().numpy()
    terms = np.abs(np.sum(q * ref["dq"], axis=3)) + np.abs(np.sum(k * ref["dk"], axis=3))
    return np.sqrt(np.cumsum((terms ** 2)[:, ::-1], axis=1)[:, ::-1])


def _compare(gpu, ref, case, heads=None, inp=None):
    ratios = {}
    for n in ("dq", "dk", "dv", "dg"):
        g_, r_ = np64(gpu[n]), ref[n]
        if heads is not None:
            g_ = np.stack([g_[b, :, h] for b, h in heads])
            r_ = np.stack([r_[b, :, h] for b, h in heads])
        if n == "dg" and inp is not None:
            sc = _dg_scale(inp, ref)
            if heads is not None:
                sc = np.stack([sc[b, :, h] for b, h in heads])
            bound = max(np.max(np.abs(r_)), np.max(sc))
            ratios[n] = float(np.max(np.abs(g_ - r_)) / bound) if np.all(np.isfinite(g_)) else float("inf")
            continue
        ratios[n] = err_ratio(g_, r_)
    say(f"{case}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (case, n, r)


# The last two span several 1024-token segments of the gate's running sum
# (T % 4 == 0: vector loads; T % 4 == 2: element loads) and a partial group of
# four heads.
CASES = [(1, 64, 1), (2, 100, 3), (1, 1, 2), (1, 200, 2), (2, 333, 1), (1, 129, 2), (1, 2500, 5), (1, 1030, 2)]


@pytest.mark.parametrize("b,t,h", CASES)
def test_gla_against_oracle(b, t, h):
    inp = gla_inputs(b, t, h, 128, seed=t + 10 * h)
    scale = 1.0 / math.sqrt(128)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = la.gla_bwd(f["q"], f["k"], f["v"], f["g"], f["do"], scale)
    _compare(run_gla(inp, scale), ref, f"gla B{b} T{t} H{h}", inp=inp)


@pytest.mark.parametrize("g_value", [0.0, -30.0])
def test_gla_decay_extremes(g_value):
    """No decay (plain causal linear attention: the states carry everything)
    and a decay so strong that only the diagonal term survives."""
    inp = gla_inputs(1, 150, 2, 128, seed=77)
    inp["g"] = torch.full_like(inp["g"], g_value)
    scale = 0.05
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = la.gla_bwd(f["q"], f["k"], f["v"], f["g"], f["do"], scale)
    _compare(run_gla(inp, scale), ref, f"gla decay g={g_value}", inp=inp)


def test_gla_is_deterministic():
    inp = gla_inputs(2, 300, 3, 128, seed=5)
    a = run_gla(inp, 0.1)
    b = run_gla(inp, 0.1)
    for n in ("dq", "dk", "dv"):
        assert torch.equal(a[n].view(torch.int16), b[n].view(torch.int16)), n
    assert torch.equal(a["dg"], b["dg"])


def test_gla_full_size_heads():
    """The benchmark workload; whole (batch, head) slices checked against the
    oracle (which computes those heads only)."""
    w = GLA_WORKLOAD
    inp = gla_inputs(w["batch"], w["seqlen"], w["heads"], w["head_dim"], seed=0)
    scale = 1.0 / math.sqrt(w["head_dim"])
    say(f"[gla full] {w['name']}: gpu")
    gpu = run_gla(inp, scale)
    heads = [(0, 0), (w["batch"] - 1, w["heads"] - 1), (1, 17)]
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = la.gla_bwd(f["q"], f["k"], f["v"], f["g"], f["do"], scale, heads=heads)
    ref_full = {n: np.nan_to_num(x) for n, x in ref.items()}
    _compare(gpu, ref_full, f"[gla full] {w['name']}", heads, inp=inp)
    for n in ("dq", "dk", "dv", "dg"):
        assert torch.all(torch.isfinite(gpu[n].float())), n
