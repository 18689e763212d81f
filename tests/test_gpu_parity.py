"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small problems, compared element by element on every output tensor; sizes
span several tiles and ragged tails (S not a multiple of 64/128), both head
dims, causal and not, MHA and grouped-query heads, both dQ paths.
"""

import math

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd.synthetic import WORKLOADS, make_inputs, workload_inputs
from oracle import attention as orc
from tests.gpu_helpers import TOL, err_ratio, gqa_parts, np64, run_path, say, to_dev

pytestmark = pytest.mark.gpu


def _oracle(inp, causal, scale, groups):
    f = {n: t.to(torch.float64).numpy() for n, t in inp.items()}
    return orc.attention_bwd(f["q"], f["k"], f["v"], f["do"], scale, causal, groups)


def _compare(case, gpu, ref, tol=TOL):
    zs = float(np.max(np.abs(ref["dv"])))
    ratios = {n: err_ratio(np64(gpu[n]), ref[n], zero_scale=zs) for n in ("o", "lse", "delta", "dq", "dk", "dv")}
    say(f"{case}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert ratios[n] <= tol, (case, n, ratios[n])
    return ratios


@pytest.mark.parametrize("use_atomic", [1, 0])
def test_small_workload_against_oracle(use_atomic):
    w = WORKLOADS["mha_s128_d64"]
    inp = workload_inputs(w)
    ref = _oracle(inp, False, w.scale, w.groups)
    gpu = run_path(to_dev(inp), False, w.scale, use_atomic)
    _compare(f"{w.name} atomic={use_atomic}", gpu, ref)


CASES = []
for s in (1, 17, 127, 129, 300):
    for d in (64, 128):
        for causal in (False, True):
            for hq, hkv in ((2, 2), (4, 2)):
                CASES.append((2 if s < 200 else 1, s, hq, hkv, d, causal))


@pytest.mark.parametrize("use_atomic", [1, 0])
@pytest.mark.parametrize("b,s,hq,hkv,d,causal", CASES)
def test_ragged_shapes(b, s, hq, hkv, d, causal, use_atomic):
    inp = make_inputs(b, s, hq, hkv, d, seed=s * 7 + d)
    scale = 1.0 / math.sqrt(d)
    ref = _oracle(inp, causal, scale, hq // hkv)
    gpu = run_path(to_dev(inp), causal, scale, use_atomic)
    _compare(f"b{b} s{s} hq{hq} hkv{hkv} d{d} causal={causal} atomic={use_atomic}", gpu, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_block_gqa(d, causal):
    """Several key blocks and query blocks, group of 4, two batches."""
    inp = make_inputs(2, 520, 8, 2, d, seed=99, qk_mult=1.5)
    scale = 1.0 / math.sqrt(d)
    ref = _oracle(inp, causal, scale, 4)
    for use_atomic in (1, 0):
        gpu = run_path(to_dev(inp), causal, scale, use_atomic)
        _compare(f"gqa4 s520 d{d} causal={causal} atomic={use_atomic}", gpu, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_long_sweep(d, causal):
    """Five key blocks (the last one ragged) and up to 35 query blocks per
    sweep, one query head per KV head (bf16 dK/dV written by the kernel)."""
    inp = make_inputs(1, 1100, 2, 2, d, seed=1100 + d)
    scale = 1.0 / math.sqrt(d)
    ref = _oracle(inp, causal, scale, 1)
    for use_atomic in (1, 0):
        gpu = run_path(to_dev(inp), causal, scale, use_atomic)
        _compare(f"s1100 d{d} causal={causal} atomic={use_atomic}", gpu, ref)


# (batch, heads_q, heads_kv, seqlen, head_dim): enough (batch, KV head) groups
# (a multiple of 8) that each XCD's share of the grid is walked a few groups
# at a time with their blocks interleaved, compared element by element.
INTERLEAVED = [
    (2, 8, 8, 300, 128),   # 16 groups: 2 per XCD
    (4, 16, 8, 520, 64),   # 32 groups: 4 per XCD, GQA-2
    (8, 8, 8, 257, 64),    # 64 groups: 8 per XCD, ragged tail
    (16, 8, 8, 130, 64),   # 128 groups: 16 per XCD, all 16 interleaved
    (32, 8, 8, 130, 64),   # 256 groups: 32 per XCD, all 32 interleaved (as at B8 H32 S1024 D64)
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,hq,hkv,s,d", INTERLEAVED)
def test_interleaved_group_order(b, hq, hkv, s, d, causal):
    inp = make_inputs(b, s, hq, hkv, d, seed=b * 100 + s)
    scale = 1.0 / math.sqrt(d)
    ref = _oracle(inp, causal, scale, hq // hkv)
    for use_atomic in (1, 0):
        gpu = run_path(to_dev(inp), causal, scale, use_atomic)
        _compare(f"b{b} hq{hq} hkv{hkv} s{s} d{d} causal={causal} atomic={use_atomic}", gpu, ref)


# (batch, heads_q, heads_kv, seqlen, head_dim, partials per KV head): grids
# large enough that one workgroup sweeps several query heads of its group
# (groups / partials of them), the dK/dV of those heads adding up in its
# accumulators; the steps cross from one head to the next mid-pipeline.
HEAD_CHUNKS = [
    (32, 16, 8, 300, 128, 1),   # groups of 2, both heads in one workgroup, ragged second key block
    (32, 16, 4, 600, 64, 2),    # groups of 4 as two chunks of 2, two 512-key blocks
    (22, 32, 4, 520, 128, 2),   # groups of 8 as two chunks of 4, 11 groups per XCD
    (6, 96, 16, 300, 128, 3),   # groups of 6 as three chunks of 2
    (37, 14, 7, 300, 128, 1),   # 259 (batch, KV head) groups: not a multiple of 8, grid in plain order
    (256, 4, 2, 17, 128, 1),    # one ragged query block per head: the sweep changes head at every step
    (512, 2, 1, 1, 64, 1),      # a single query and key per sequence
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,hq,hkv,s,d,parts", HEAD_CHUNKS)
def test_head_chunks(b, hq, hkv, s, d, parts, causal):
    assert gqa_parts(b, s, hq, hq // hkv, d) == parts
    inp = make_inputs(b, s, hq, hkv, d, seed=b * 1000 + s + d)
    scale = 1.0 / math.sqrt(d)
    ref = _oracle(inp, causal, scale, hq // hkv)
    for use_atomic in (1, 0):
        gpu = run_path(to_dev(inp), causal, scale, use_atomic)
        _compare(f"b{b} hq{hq} hkv{hkv} s{s} d{d} parts={parts} causal={causal} atomic={use_atomic}", gpu, ref)


def test_group_of_eight_odd_length():
    inp = make_inputs(1, 333, 16, 2, 128, seed=5, qk_mult=1.5)
    scale = 1.0 / math.sqrt(128)
    for causal in (False, True):
        ref = _oracle(inp, causal, scale, 8)
        gpu = run_path(to_dev(inp), causal, scale, 1)
        _compare(f"gqa8 s333 causal={causal}", gpu, ref)


def test_non_default_scale():
    inp = make_inputs(1, 200, 2, 1, 64, seed=3)
    for scale in (0.05, 0.4):
        ref = _oracle(inp, True, scale, 2)
        gpu = run_path(to_dev(inp), True, scale, 0)
        _compare(f"scale={scale}", gpu, ref)


@pytest.mark.parametrize("d", [64, 128])
def test_split_path_bitwise_deterministic(d):
    inp = to_dev(make_inputs(2, 700, 4, 2, d, seed=11))
    scale = 1.0 / math.sqrt(d)
    runs = [run_path(inp, True, scale, 0) for _ in range(3)]

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)

    for n in ("dq", "dk", "dv", "o", "lse", "dq_accum"):
        for r in runs[1:]:
            assert torch.equal(bits(runs[0][n]), bits(r[n])), n


@pytest.mark.parametrize("causal", [False, True])
def test_dq_sum_alone_repeats_the_split_sum(causal):
    """attn_bwd_dq_sum over the partials attn_bwd(use_atomic = 0) left in the
    workspace rewrites dq_accum with the same bits."""
    from attention_backward_fwd_amd import binding as bd
    inp = to_dev(make_inputs(2, 700, 4, 2, 128, seed=13))
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    scale = 1.0 / math.sqrt(128)
    sh = bd.shape_of(q, k)
    o, lse = bd.forward(q, k, v, causal, scale)
    bb = bd.BwdBuffers(q, k, causal, 0)
    bd.attn_bwd_preprocess(o, do, bb.delta, None, sh)
    bd.attn_bwd(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, sh, scale, causal, 0)
    torch.cuda.synchronize()
    first = bb.dq_accum.clone()
    assert torch.isfinite(first).all()
    bb.dq_accum.fill_(float("nan"))
    bd.attn_bwd_dq_sum(bb.workspace, bb.dq_accum, sh, causal)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int32), bb.dq_accum.view(torch.int32))


def test_atomic_and_split_agree():
    inp = to_dev(make_inputs(1, 1000, 4, 4, 128, seed=12))
    scale = 1.0 / math.sqrt(128)
    a = run_path(inp, True, scale, 1)
    s = run_path(inp, True, scale, 0)
    # same dK/dV bits (no atomics there); dQ equal up to fp32 summation order
    assert torch.equal(a["dk"], s["dk"]) and torch.equal(a["dv"], s["dv"])
    diff = (a["dq_accum"] - s["dq_accum"]).abs().max().item()
    assert diff <= 1e-5 * a["dq_accum"].abs().max().item()


def test_outputs_untouched_outside_shape():
    """Writes stay inside the tensors: guard bands around every output survive."""
    b, s, hq, hkv, d = 1, 77, 4, 2, 64
    inp = to_dev(make_inputs(b, s, hq, hkv, d, seed=4))
    from attention_backward_fwd_amd import binding as bd
    sh = bd.shape_of(inp["q"], inp["k"])
    pad = 4096
    sentinel = 1024.0  # exact in bf16 and fp32
    n_q, n_kv = b * s * hq * d, b * s * hkv * d

    def guarded(n, dtype):
        t = torch.full((n + 2 * pad,), sentinel, dtype=dtype, device="cuda")
        return t, t[pad:pad + n]

    og, o = guarded(n_q, torch.bfloat16)
    lg, lse = guarded(b * hq * s, torch.float32)
    bd.attn_fwd(inp["q"], inp["k"], inp["v"], o, lse, sh, 0.125, 1)
    dg, delta = guarded(b * hq * s, torch.float32)
    ag, acc = guarded(n_q, torch.float32)
    qg, dq = guarded(n_q, torch.bfloat16)
    kg, dk = guarded(n_kv, torch.bfloat16)
    vg, dv = guarded(n_kv, torch.bfloat16)
    for use_atomic in (1, 0):
        nbytes = bd.attn_bwd_workspace_bytes(sh, 1, use_atomic)
        wg, ws = guarded(nbytes // 4, torch.float32)
        bd.attn_bwd_preprocess(o, inp["do"], delta, acc if use_atomic else None, sh)
        bd.attn_bwd(inp["q"], inp["k"], inp["v"], inp["do"], lse, delta, acc, dk, dv, ws, sh, 0.125, 1, use_atomic)
        bd.attn_bwd_postprocess(acc, ws, dq, dk, dv, sh)
        torch.cuda.synchronize()
        for g in (og, lg, dg, ag, qg, kg, vg, wg):
            head, tail = g[:pad].float(), g[-pad:].float()
            assert torch.all(head == sentinel) and torch.all(tail == sentinel)
