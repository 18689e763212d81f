"""GPU parity of packed variable-length sequences (attn_fwd_varlen,
attn_bwd_varlen, with the dense preprocess/postprocess on the batch-1 view)
against the packed-sequence oracle: element by element on small packs with
empty, single-token, ragged and multi-block sequences and capacity padding,
and on samples of the full-size pack the benchmark times."""

import math

import numpy as np
import pytest
import torch

from attention_backward_fwd_amd import binding as bd
from attention_backward_fwd_amd.synthetic import (VARLEN_PACK, cu_seqlens, make_inputs,
                                                  varlen_pack_inputs)
from oracle import attention as orc
from oracle import varlen as vl
from tests.gpu_helpers import TOL, err_ratio, np64, say

pytestmark = pytest.mark.gpu

NAN = float("nan")


def _pack(lengths, pad, hq, hkv, d, seed):
    t = sum(lengths) + pad
    inp = make_inputs(1, t, hq, hkv, d, seed=seed)
    return {n: x[0] for n, x in inp.items()}


def run_varlen(dev, cu, max_seqlen, causal, scale, use_atomic, cu_k=None, max_seqlen_k=None):
    """fwd -> preprocess -> bwd (-> sum) -> postprocess; every output and
    scratch buffer starts as NaN, so an element left unwritten shows up."""
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    cu_k = cu if cu_k is None else cu_k
    n_seqs = cu.numel() - 1
    sh = bd.varlen_shape_of(q, k, n_seqs, max_seqlen, max_seqlen_k)
    o = torch.full_like(q, NAN)
    lse = torch.full((q.shape[1], q.shape[0]), NAN, dtype=torch.float32, device=q.device)
    bd.attn_fwd_varlen(q, k, v, o, lse, cu, cu_k, sh, scale, causal)
    bb = bd.VarlenBwdBuffers(q, k, n_seqs, max_seqlen, causal, use_atomic, max_seqlen_k)
    for t in (bb.delta, bb.dq_accum, bb.dq, bb.dk, bb.dv) + ((bb.workspace,) if bb.workspace is not None else ()):
        t.fill_(NAN)
    bd.backward_varlen(q, k, v, o, lse, do, cu, max_seqlen, causal, scale, use_atomic, buffers=bb, cu_seqlens_k=cu_k,
                       max_seqlen_k=max_seqlen_k)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "delta": bb.delta, "dq": bb.dq, "dk": bb.dk, "dv": bb.dv}


def _padding_rows(cu_list, t, max_seqlen):
    inside = np.zeros(t, dtype=bool)
    for a, e in zip(cu_list[:-1], cu_list[1:]):
        inside[a:min(e, a + max_seqlen)] = True
    return ~inside


def _unseen_keys(cu, cu_k, tk, mq, mk):
    """Key rows of sequences without queries: no query sees them (with at
    least one query, the last query sees every key of its sequence)."""
    out = np.zeros(tk, dtype=bool)
    for b in range(len(cu) - 1):
        if min(cu[b + 1] - cu[b], mq) == 0:
            out[cu_k[b]:cu_k[b] + min(cu_k[b + 1] - cu_k[b], mk)] = True
    return out


def _check(gpu, ref, pad, case, pad_k=None, unseen=None):
    ratios = {n: err_ratio(np64(gpu[n]), ref[n]) for n in ("o", "dq", "dk", "dv", "delta")}
    say(f"{case}: " + " ".join(f"{n}={r:.2e}" for n, r in ratios.items()))
    for n, r in ratios.items():
        assert r <= TOL, (case, n, r)
    lse, rl = np64(gpu["lse"]), ref["lse"]
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl)), (case, "LSE -inf pattern")
    fin = np.isfinite(rl)
    err = np.max(np.abs(lse[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin])), initial=0.0)
    assert err <= 1e-3, (case, "lse", err)
    # capacity padding and rows that see no key: exact zeros
    pad_k = pad if pad_k is None else pad_k
    empty = np.isneginf(rl).all(axis=0)
    for n in ("o", "dq"):
        assert np.all(np64(gpu[n])[pad | empty] == 0.0), (case, n, "padding / empty rows not zero")
    for n in ("dk", "dv"):
        assert np.all(np64(gpu[n])[pad_k] == 0.0), (case, n, "padding rows not zero")
    if unseen is not None:
        for n in ("dk", "dv"):  # keys no query sees: exact zeros too
            assert np.all(np64(gpu[n])[unseen] == 0.0), (case, n, "unseen keys not zero")


SMALL = [
    # lengths, pad, hq, hkv, d, causal
    ([5, 0, 7, 1, 7], 3, 4, 2, 64, True),
    ([5, 0, 7, 1, 7], 3, 4, 2, 64, False),
    ([300, 1, 0, 257, 520, 33], 40, 4, 1, 128, True),
    ([600, 256, 700], 0, 2, 2, 64, False),
    ([64, 511, 96, 1], 17, 2, 2, 128, True),
    # 4 sequences x 4 KV heads = 16 groups: two per XCD, interleaved
    ([300, 1, 257, 40], 5, 8, 4, 64, True),
    ([300, 1, 257, 40], 5, 8, 4, 128, False),
]


@pytest.mark.parametrize("use_atomic", [1, 0])
@pytest.mark.parametrize("lengths,pad,hq,hkv,d,causal", SMALL)
def test_varlen_against_oracle(lengths, pad, hq, hkv, d, causal, use_atomic):
    inp = _pack(lengths, pad, hq, hkv, d, seed=sum(lengths) + d)
    cu = cu_seqlens(lengths)
    t = inp["q"].shape[0]
    scale = 1.0 / math.sqrt(d)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = vl.varlen_bwd(f["q"], f["k"], f["v"], f["do"], cu.tolist(), scale, causal, hq // hkv)
    case = f"varlen L={lengths} pad={pad} hq{hq} hkv{hkv} d{d} causal={causal} atomic={use_atomic}"
    say(case)
    gpu = run_varlen({n: x.cuda() for n, x in inp.items()}, cu.cuda(), max(lengths), causal, scale, use_atomic)
    _check(gpu, ref, _padding_rows(cu.tolist(), t, max(lengths)), case)


def test_varlen_split_is_deterministic():
    lengths = [300, 1, 257, 520, 33]
    inp = _pack(lengths, 9, 4, 2, 128, seed=11)
    cu = cu_seqlens(lengths).cuda()
    dev = {n: x.cuda() for n, x in inp.items()}
    a = run_varlen(dev, cu, 520, True, 0.125, 0)
    b = run_varlen(dev, cu, 520, True, 0.125, 0)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n]), n


def test_varlen_all_padding():
    """No sequence at all (cu = [0]) and a pack of only empty sequences:
    every row is padding."""
    inp = _pack([], 40, 2, 2, 64, seed=5)
    dev = {n: x.cuda() for n, x in inp.items()}
    for cu_list, m in (([0], 0), ([0, 0, 0], 16)):
        gpu = run_varlen(dev, torch.tensor(cu_list, dtype=torch.int32).cuda(), m, True, 0.125, 1)
        assert torch.all(gpu["o"] == 0) and torch.all(gpu["dq"] == 0)
        assert torch.all(gpu["dk"] == 0) and torch.all(gpu["dv"] == 0)
        assert torch.all(torch.isneginf(gpu["lse"]))


def test_varlen_equal_lengths_match_dense():
    """A pack of equal-length sequences is the dense batched problem: the
    packed path's results equal the dense path's bit for bit (same kernels,
    same per-sequence arithmetic)."""
    b, s, hq, hkv, d = 3, 200, 4, 2, 128
    inp = make_inputs(b, s, hq, hkv, d, seed=21)
    dev = {n: x.cuda() for n, x in inp.items()}
    o_d, lse_d = bd.forward(dev["q"], dev["k"], dev["v"], True, 0.09)
    dq_d, dk_d, dv_d = bd.backward(dev["q"], dev["k"], dev["v"], o_d, lse_d, dev["do"], True, 0.09, use_atomic=False)
    packed = {n: x.reshape(b * s, x.shape[2], d) for n, x in dev.items()}
    cu = cu_seqlens([s] * b).cuda()
    gpu = run_varlen(packed, cu, s, True, 0.09, 0)
    assert torch.equal(gpu["o"].view(b, s, hq, d), o_d)
    assert torch.equal(gpu["lse"].view(hq, b, s).permute(1, 0, 2), lse_d)
    assert torch.equal(gpu["dq"].view(b, s, hq, d), dq_d)
    assert torch.equal(gpu["dk"].view(b, s, hkv, d), dk_d)
    assert torch.equal(gpu["dv"].view(b, s, hkv, d), dv_d)


def test_varlen_sequence_cut_at_max_seqlen():
    """A sequence longer than max_seqlen is cut to its first max_seqlen rows;
    the rest count as padding (the oracle sees the cut pack)."""
    inp = _pack([100, 300], 0, 2, 1, 64, seed=31)
    f = {n: x.double().numpy() for n, x in inp.items()}
    # Oracle: sequences [0,100) and [100,300); rows 300..399 padding.
    ref = vl.varlen_bwd(f["q"], f["k"], f["v"], f["do"], [0, 100, 300], 0.125, True, 2)
    gpu = run_varlen({n: x.cuda() for n, x in inp.items()}, torch.tensor([0, 100, 400], dtype=torch.int32).cuda(),
                     200, True, 0.125, 0)
    _check(gpu, ref, _padding_rows([0, 100, 400], 400, 200), "varlen cut at max_seqlen")


# Different query and key lengths per sequence: (query lengths, key lengths,
# query padding, key padding, hq, hkv, d, causal).  Causal alignment puts the
# last query on the last key: lq < lk gives every query a key prefix, lq > lk
# leaves the first lq - lk queries without keys; lk = 0 and lq = 0 sequences.
RECT = [
    ([5, 64, 300, 1], [9, 64, 520, 700], 4, 6, 4, 2, 128, True),
    ([5, 64, 300, 1], [9, 64, 520, 700], 4, 6, 4, 2, 128, False),
    ([40, 300, 10, 0], [7, 100, 0, 30], 3, 0, 2, 2, 64, True),
    ([40, 300, 10, 0], [7, 100, 0, 30], 3, 0, 2, 1, 64, False),
    ([600, 33], [257, 290], 0, 11, 2, 2, 128, True),
]


@pytest.mark.parametrize("use_atomic", [1, 0])
@pytest.mark.parametrize("lq,lk,pq,pk,hq,hkv,d,causal", RECT)
def test_varlen_rectangular_against_oracle(lq, lk, pq, pk, hq, hkv, d, causal, use_atomic):
    tq, tk = sum(lq) + pq, sum(lk) + pk
    g = torch.Generator().manual_seed(sum(lq) + 7 * sum(lk) + d)
    inp = {"q": torch.randn((tq, hq, d), generator=g), "k": torch.randn((tk, hkv, d), generator=g),
           "v": torch.randn((tk, hkv, d), generator=g), "do": torch.randn((tq, hq, d), generator=g)}
    inp = {n: x.to(torch.bfloat16) for n, x in inp.items()}
    cu, cu_k = cu_seqlens(lq), cu_seqlens(lk)
    scale = 1.0 / math.sqrt(d)
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = vl.varlen_bwd(f["q"], f["k"], f["v"], f["do"], cu.tolist(), scale, causal, hq // hkv, cu_k.tolist())
    case = f"varlen rect Lq={lq} Lk={lk} pad={pq},{pk} hq{hq} hkv{hkv} d{d} causal={causal} atomic={use_atomic}"
    say(case)
    gpu = run_varlen({n: x.cuda() for n, x in inp.items()}, cu.cuda(), max(lq), causal, scale, use_atomic,
                     cu_k.cuda(), max(lk))
    _check(gpu, ref, _padding_rows(cu.tolist(), tq, max(lq)), case, _padding_rows(cu_k.tolist(), tk, max(lk)),
           _unseen_keys(cu.tolist(), cu_k.tolist(), tk, max(lq), max(lk)))


@pytest.mark.parametrize("use_atomic", [1, 0])
def test_varlen_leading_padding(use_atomic):
    """Offsets that do not start at row 0: rows before the first sequence
    are padding too."""
    cu_l, cuk_l = [5, 30, 60], [3, 40, 41]
    g = torch.Generator().manual_seed(41)
    inp = {"q": torch.randn((70, 4, 64), generator=g), "k": torch.randn((50, 2, 64), generator=g),
           "v": torch.randn((50, 2, 64), generator=g), "do": torch.randn((70, 4, 64), generator=g)}
    inp = {n: x.to(torch.bfloat16) for n, x in inp.items()}
    f = {n: x.double().numpy() for n, x in inp.items()}
    ref = vl.varlen_bwd(f["q"], f["k"], f["v"], f["do"], cu_l, 0.125, True, 2, cuk_l)
    cu, cuk = torch.tensor(cu_l, dtype=torch.int32), torch.tensor(cuk_l, dtype=torch.int32)
    gpu = run_varlen({n: x.cuda() for n, x in inp.items()}, cu.cuda(), 30, True, 0.125, use_atomic, cuk.cuda(), 37)
    _check(gpu, ref, _padding_rows(cu_l, 70, 30), f"leading padding atomic={use_atomic}",
           _padding_rows(cuk_l, 50, 37), _unseen_keys(cu_l, cuk_l, 50, 30, 37))


def test_varlen_no_keys_at_all():
    """Queries but no key rows anywhere (total_k = 0), and keys but no query
    rows: O = 0, LSE = -inf, dQ = 0, and dK = dV = 0."""
    g = torch.Generator().manual_seed(3)
    q = torch.randn((20, 2, 64), generator=g).to(torch.bfloat16).cuda()
    kv = torch.randn((24, 2, 64), generator=g).to(torch.bfloat16).cuda()
    cu = torch.tensor([0, 12, 20], dtype=torch.int32).cuda()
    cz = torch.tensor([0, 0, 0], dtype=torch.int32).cuda()
    gpu = run_varlen({"q": q, "k": kv[:0], "v": kv[:0], "do": q.clone()}, cu, 12, True, 0.125, 0, cz, 0)
    assert torch.all(gpu["o"] == 0) and torch.all(gpu["dq"] == 0) and torch.all(torch.isneginf(gpu["lse"]))
    cuk = torch.tensor([0, 10, 24], dtype=torch.int32).cuda()
    gpu = run_varlen({"q": q[:0], "k": kv, "v": kv, "do": q[:0]}, cz, 0, True, 0.125, 1, cuk, 14)
    assert torch.all(gpu["dk"] == 0) and torch.all(gpu["dv"] == 0)


@pytest.mark.parametrize("use_atomic", [1, 0])
def test_varlen_full_pack_sampled(use_atomic):
    """The benchmark's pack, sampled: O, LSE, dQ of chosen rows and dK, dV
    of chosen keys of every sequence, each from the oracle on that sequence
    alone; padding rows exactly zero."""
    spec = VARLEN_PACK
    inp, lengths, cu = varlen_pack_inputs(spec)
    say(f"[varlen full] lengths={lengths} atomic={use_atomic}")
    scale = 1.0 / math.sqrt(spec["head_dim"])
    g = spec["heads_q"] // spec["heads_kv"]
    gpu = run_varlen({n: x.cuda() for n, x in inp.items()}, cu.cuda(), max(lengths), True, scale, use_atomic)
    f = {n: x.double().numpy() for n, x in inp.items()}
    rng = np.random.default_rng(1)
    worst = {}
    cul = cu.tolist()
    for i, (a, e) in enumerate(zip(cul[:-1], cul[1:])):
        n = e - a
        sl = {k: v[a:e][None] for k, v in f.items()}
        h = int(rng.integers(0, spec["heads_q"]))
        rows = sorted({0, 1, n // 2, n - 1, int(rng.integers(0, n))})
        ref = orc.attention_rows(sl["q"], sl["k"], sl["v"], sl["do"], scale, True, g, 0, h, rows)
        got = {"o": np64(gpu["o"][[a + r for r in rows], h]), "lse": np64(gpu["lse"][h, [a + r for r in rows]]),
               "dq": np64(gpu["dq"][[a + r for r in rows], h])}
        kv = h // g
        cols = sorted({0, n // 3, n - 1})
        refc = orc.attention_cols(sl["q"], sl["k"], sl["v"], sl["do"], scale, True, g, 0, kv, cols)
        got["dk"] = np64(gpu["dk"][[a + c for c in cols], kv])
        got["dv"] = np64(gpu["dv"][[a + c for c in cols], kv])
        refc.update(ref)
        for nme in got:
            worst[nme] = max(worst.get(nme, 0.0), err_ratio(got[nme], refc[nme]))
    say("[varlen full] " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for nme in ("o", "lse", "dq", "dk", "dv"):
        assert worst[nme] <= TOL, (nme, worst[nme])
    pad = slice(cul[-1], None)
    for nme in ("o", "dq", "dk", "dv"):
        assert torch.all(gpu[nme][pad] == 0), nme
    assert torch.all(torch.isneginf(gpu["lse"][:, pad]))
