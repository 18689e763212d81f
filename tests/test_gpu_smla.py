"""GPU parity of sparse MLA (attn_sparse_mla_fwd) against the fp64 oracle:
element by element on small problems (ragged head tiles and entry tiles,
unused slots, out-of-range entries, keys listed twice, tokens without a valid
entry) and on sampled tokens of the benchmark workload."""

import math

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd import binding as bd
from attention_backward_fwd_amd.synthetic import SMLA_WORKLOAD, smla_indices, smla_inputs
from oracle import sparse_mla as sm
from tests.gpu_helpers import TOL, err_ratio, np64, say

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(576)


def _indices(t, tk, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((t, k), -1, dtype=np.int32)
    for i in range(t):
        n = int(rng.integers(1, k + 1))
        idx[i, :n] = rng.choice(tk, size=min(n, tk), replace=False)[:n] if n <= tk else rng.integers(0, tk, n)
    idx[min(1, t - 1)] = -1                                   # a token without any valid entry
    if t > 2 and k > 3:
        idx[2, 0] = tk + 5                                    # out of range: unused
        idx[2, 1] = idx[2, 2] if idx[2, 2] >= 0 else 0       # a key listed twice
    return idx


def _check(o, lse, ro, rl, case):
    r = err_ratio(np64(o), ro)
    lse, rl = np64(lse), np.asarray(rl)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl)), (case, "LSE -inf pattern")
    fin = np.isfinite(rl)
    le = np.max(np.abs(lse[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin])), initial=0.0)
    say(f"{case}: o={r:.2e} lse={le:.2e}")
    assert r <= TOL, (case, r)
    assert le <= 1e-3, (case, le)
    empty = np.isneginf(rl)
    assert np.all(np64(o)[empty] == 0.0), case


CASES = [(5, 40, 3, 37), (17, 100, 32, 64), (9, 300, 40, 100), (3, 7, 1, 1), (6, 70, 64, 33)]


@pytest.mark.parametrize("t,tk,h,k", CASES)
def test_smla_fwd_against_oracle(t, tk, h, k):
    inp = smla_inputs(t, tk, h, seed=t + k)
    idx = _indices(t, tk, k, seed=h)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ro, rl = sm.sparse_mla_fwd(f["q"], f["kv"], idx, SCALE)
    o, lse = bd.sparse_mla_forward(inp["q"].cuda(), inp["kv"].cuda(), torch.from_numpy(idx).cuda(), SCALE)
    torch.cuda.synchronize()
    _check(o, lse, ro, rl, f"smla fwd T{t} Tk{tk} H{h} K{k}")


def test_smla_fwd_full_size_sampled():
    w = SMLA_WORKLOAD
    t, h, k = w["tokens"], w["heads"], w["topk"]
    inp = smla_inputs(t, t, h, seed=0)
    idx = smla_indices(t, t, k, seed=0)
    say(f"[smla full] {w['name']}: gpu")
    o, lse = bd.sparse_mla_forward(inp["q"].cuda(), inp["kv"].cuda(), idx.cuda(), SCALE)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 2047, 2048, 3000, t - 1]
    qf = inp["q"][rows].double().numpy()
    ro, rl = sm.sparse_mla_fwd(qf, inp["kv"].double().numpy(), idx[rows].numpy(), SCALE)
    _check(o[rows], lse[rows], ro, rl, f"[smla full] {w['name']} tokens {rows}")


def _run_bwd(inp, idx, use_atomic=True, fill=float("nan")):
    """Forward, then the backward on the atomic (use_atomic) or the
    deterministic path, with every output poisoned (NaN) and the
    deterministic path's workspace filled with the fp32 value `fill` (which
    its integer regions then read as garbage)."""
    q, kv, do = inp["q"].cuda(), inp["kv"].cuda(), inp["do"].cuda()
    ix = idx.cuda() if isinstance(idx, torch.Tensor) else torch.from_numpy(idx).cuda()
    o, lse = bd.sparse_mla_forward(q, kv, ix, SCALE)
    bb = bd.SmlaBwdBuffers(q, kv, use_atomic, ix)
    for x in (bb.delta, bb.dq, bb.dkv_accum, bb.dkv):
        if x is not None:
            x.fill_(float("nan"))
    if bb.workspace is not None:
        bb.workspace.view(torch.float32)[: bb.workspace.numel() // 4].fill_(fill)
    dq, dkv = bd.sparse_mla_backward(q, kv, ix, o, lse, do, SCALE, buffers=bb)
    torch.cuda.synchronize()
    return {"dq": dq, "dkv": dkv, "delta": bb.delta, "o": o}


@pytest.mark.parametrize("t,tk,h,k", CASES)
def test_smla_bwd_against_oracle(t, tk, h, k):
    inp = smla_inputs(t, tk, h, seed=t + k)
    idx = _indices(t, tk, k, seed=h)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx, f["do"], SCALE)
    gpu = _run_bwd(inp, idx)
    case = f"smla bwd T{t} Tk{tk} H{h} K{k}"
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv", "delta")}
    say(f"{case}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (case, n, r)
    # keys nobody selected get exact zeros; tokens without entries get dq = 0
    unused = np.all(ref["dkv"] == 0.0, axis=1)
    assert np.all(np64(gpu["dkv"])[unused] == 0.0), case
    assert np.all(np64(gpu["dq"])[1] == 0.0), case


def test_smla_bwd_full_size():
    """The benchmark workload: dq of sampled tokens against the oracle, and
    over all keys the sums sum_j dkv[j, :512] = sum_{t,h} dO[t,h] and
    sum_j dkv[j, 512:] = 0 (softmax rows sum to one; dS rows sum to zero)."""
    w = SMLA_WORKLOAD
    t, h, k = w["tokens"], w["heads"], w["topk"]
    inp = smla_inputs(t, t, h, seed=0)
    idx = smla_indices(t, t, k, seed=0)
    say(f"[smla full bwd] {w['name']}: gpu")
    gpu = _run_bwd(inp, idx)
    rows = [0, 5, 2047, 2048, 3001, t - 1]
    sub = sm.sparse_mla_bwd(inp["q"][rows].double().numpy(), inp["kv"].double().numpy(), idx[rows].numpy(),
                            inp["do"][rows].double().numpy(), SCALE)
    r = err_ratio(np64(gpu["dq"][rows]), sub["dq"])
    dkv = gpu["dkv"].double()
    want_v = inp["do"].cuda().double().sum(dim=(0, 1))
    err_v = (dkv[:, :512].sum(dim=0) - want_v).abs().max().item() / dkv[:, :512].abs().sum(dim=0).max().item()
    err_k = dkv[:, 512:].sum(dim=0).abs().max().item() / dkv[:, 512:].abs().sum(dim=0).max().item()
    say(f"[smla full bwd] dq(sampled)={r:.2e} sum dkv[:, :512] err={err_v:.2e} sum dkv[:, 512:] err={err_k:.2e}")
    assert r <= TOL
    assert err_v <= 2e-2 and err_k <= 2e-2
    assert torch.all(torch.isfinite(gpu["dkv"].float())) and torch.all(torch.isfinite(gpu["dq"].float()))


def test_smla_bwd_mid_size_elementwise():
    """The benchmark workload's structure (32 heads, causal index lists in
    random order) at 1024 tokens and top-512: dq, dkv and Delta of every
    token and key against the oracle."""
    t, h, k = 1024, 32, 512
    inp = smla_inputs(t, t, h, seed=4)
    idx = smla_indices(t, t, k, seed=4)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx.numpy(), f["do"], SCALE)
    gpu = _run_bwd(inp, idx)
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv", "delta")}
    say(f"smla bwd T{t} H{h} K{k}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (n, r)


def _gappy_indices(t, tk, k, seed):
    """Lists whose second 32-entry tile holds no valid entry, with unused and
    out-of-range entries scattered through the other tiles and valid entries
    after the gap."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(tk, size=k, replace=False) for _ in range(t)]).astype(np.int32)
    idx[:, 32:64] = -1                                        # a whole tile of unused slots
    mask = rng.random((t, k)) < 0.2
    idx[mask] = -1                                            # scattered unused slots
    idx[:, 5] = tk + 11                                       # out of range
    idx[:, 70] = -3                                           # another negative sentinel
    return idx


def test_smla_gaps_and_scattered_sentinels():
    t, tk, h, k = 6, 400, 40, 130
    inp = smla_inputs(t, tk, h, seed=21)
    idx = _gappy_indices(t, tk, k, seed=22)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ro, rl = sm.sparse_mla_fwd(f["q"], f["kv"], idx, SCALE)
    o, lse = bd.sparse_mla_forward(inp["q"].cuda(), inp["kv"].cuda(), torch.from_numpy(idx).cuda(), SCALE)
    torch.cuda.synchronize()
    _check(o, lse, ro, rl, "smla fwd gaps")
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx, f["do"], SCALE)
    gpu = _run_bwd(inp, idx)
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv")}
    say("smla bwd gaps: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (n, r)
    unused = np.all(ref["dkv"] == 0.0, axis=1)
    assert np.all(np64(gpu["dkv"])[unused] == 0.0)


# ------------------------------------------------------------ deterministic dKV path

SPLIT_CASES = CASES + [(64, 3000, 32, 256), (40, 5000, 8, 700)]   # the last two: two sort passes, several tiles


@pytest.mark.parametrize("t,tk,h,k", SPLIT_CASES)
def test_smla_bwd_split_against_oracle(t, tk, h, k):
    """use_atomic=False: dq and dkv against the oracle element by element;
    dq identical to the atomic path's (the same kernel code computes it);
    dkv bitwise identical over two runs with different workspace garbage."""
    inp = smla_inputs(t, tk, h, seed=t + k)
    idx = _indices(t, tk, k, seed=h)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx, f["do"], SCALE)
    gpu = _run_bwd(inp, idx, use_atomic=False)
    case = f"smla bwd split T{t} Tk{tk} H{h} K{k}"
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv", "delta")}
    say(f"{case}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (case, n, r)
    unused = np.all(ref["dkv"] == 0.0, axis=1)
    assert np.all(np64(gpu["dkv"])[unused] == 0.0), case
    atomic = _run_bwd(inp, idx, use_atomic=True)
    assert torch.equal(gpu["dq"], atomic["dq"]), case
    again = _run_bwd(inp, idx, use_atomic=False, fill=-7.5)
    assert torch.equal(gpu["dkv"], again["dkv"]) and torch.equal(gpu["dq"], again["dq"]), case


def test_smla_bwd_split_wide_key_range():
    """Key rows 0 .. 299999 (19-bit keys: two radix passes of 10 and 9 bits,
    1024-digit counts), most of them selected by no token (their dkv rows
    must be exact zeros), and 128 heads (four 32-head tiles per token, so
    four partial rows per entry)."""
    t, tk, h, k = 6, 300000, 128, 300
    rng = np.random.default_rng(31)
    idx = np.stack([rng.choice(tk, size=k, replace=False) for _ in range(t)]).astype(np.int32)
    idx[0, :5] = [0, 1, tk - 1, tk - 2, 150000]                 # both ends of the key range
    idx[1, 7] = idx[1, 8]                                       # a key listed twice
    idx[2, 100:] = -1
    inp = smla_inputs(t, tk, h, seed=32)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx, f["do"], SCALE)
    gpu = _run_bwd(inp, idx, use_atomic=False)
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv")}
    say("smla bwd split wide keys: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (n, r)
    unused = np.all(ref["dkv"] == 0.0, axis=1)
    assert unused.sum() > tk - t * k
    assert np.all(np64(gpu["dkv"])[unused] == 0.0)


def test_smla_bwd_split_gaps_and_scattered_sentinels():
    t, tk, h, k = 6, 400, 40, 130
    inp = smla_inputs(t, tk, h, seed=21)
    idx = _gappy_indices(t, tk, k, seed=22)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx, f["do"], SCALE)
    gpu = _run_bwd(inp, idx, use_atomic=False)
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv")}
    say("smla bwd split gaps: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (n, r)
    unused = np.all(ref["dkv"] == 0.0, axis=1)
    assert np.all(np64(gpu["dkv"])[unused] == 0.0)


def test_smla_bwd_split_mid_size_elementwise():
    """As test_smla_bwd_mid_size_elementwise, on the deterministic path
    (1024 tokens x 512 entries: 128 sort tiles, two radix passes)."""
    t, h, k = 1024, 32, 512
    inp = smla_inputs(t, t, h, seed=4)
    idx = smla_indices(t, t, k, seed=4)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = sm.sparse_mla_bwd(f["q"], f["kv"], idx.numpy(), f["do"], SCALE)
    gpu = _run_bwd(inp, idx, use_atomic=False)
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("dq", "dkv", "delta")}
    say(f"smla bwd split T{t} H{h} K{k}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (n, r)


def test_smla_bwd_split_full_size():
    """The benchmark workload on the deterministic path: dq of sampled tokens
    against the oracle, dkv of sampled keys against the oracle (each key's
    gradient summed over the tokens that select it), the whole dkv against
    the atomic path's element by element, and bitwise repeatability."""
    w = SMLA_WORKLOAD
    t, h, k = w["tokens"], w["heads"], w["topk"]
    inp = smla_inputs(t, t, h, seed=0)
    idx = smla_indices(t, t, k, seed=0)
    say(f"[smla full bwd split] {w['name']}: gpu")
    gpu = _run_bwd(inp, idx, use_atomic=False)
    atomic = _run_bwd(inp, idx, use_atomic=True)
    assert torch.equal(gpu["dq"], atomic["dq"])
    r_atomic = err_ratio(np64(gpu["dkv"]), np64(atomic["dkv"]))
    again = _run_bwd(inp, idx, use_atomic=False, fill=3.25)
    assert torch.equal(gpu["dkv"], again["dkv"])
    # Keys 3800, 4000, 4095 (selected by ~150, ~50 and 1 of the later tokens):
    # the oracle over those tokens, whole (all their entries).
    keys = [3800, 4000, 4095]
    idx_np = idx.numpy()
    toks = sorted(set(np.nonzero(np.isin(idx_np, keys))[0].tolist()))
    sub = sm.sparse_mla_bwd(inp["q"][toks].double().numpy(), inp["kv"].double().numpy(), idx_np[toks],
                            inp["do"][toks].double().numpy(), SCALE)
    r_keys = err_ratio(np64(gpu["dkv"][keys]), sub["dkv"][keys])
    r_dq = err_ratio(np64(gpu["dq"][toks[:8]]), sub["dq"][:8])
    say(f"[smla full bwd split] dkv vs atomic={r_atomic:.2e} dkv(keys {keys}, {len(toks)} tokens)={r_keys:.2e} "
        f"dq(sampled)={r_dq:.2e}")
    assert r_atomic <= TOL and r_keys <= TOL and r_dq <= TOL
