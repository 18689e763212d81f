"""Seeded synthetic inputs for attention forward/backward.

This module only draws random numbers and names the workload shapes; it holds
none of the attention arithmetic.  Both the fp64 oracle (through the tests) and
the GPU path consume what it produces, so the two sides always see identical
bf16 inputs.

Recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws standard-normal
fp32 tensors in [batch, seq, heads, dim] order Q, K, V, dO; Q and K are then
multiplied by ``qk_mult`` (1.5 gives sharper softmax rows); finally every
tensor is rounded to bf16 (round-to-nearest-even).

Packed sequences: ``length_mix`` draws sequence lengths uniformly from
[lo, hi] with its own seeded generator until the next one would overflow the
token budget, and gives the last sequence the tokens left; ``cu_seqlens`` is
the running sum of the lengths.  The packed tensors are ``make_inputs`` with
batch 1 and seq = total rows (capacity), viewed as [T, heads, dim].
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    causal: tuple  # the causal settings the workload is run with
    qk_mult: float = 1.0
    paths: tuple = ("atomic", "split")

    @property
    def groups(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five seeded synthetic workloads (sizes only).
WORKLOADS = {
    "mha_s128_d64": Workload("mha_s128_d64", 1, 2, 2, 128, 64, (False,)),
    "mha_causal_b8_h32_s1024_d64": Workload("mha_causal_b8_h32_s1024_d64", 8, 32, 32, 1024, 64, (True,), paths=("atomic",)),
    "gqa4_causal_b8_h32_s2048_d128": Workload("gqa4_causal_b8_h32_s2048_d128", 8, 32, 8, 2048, 128, (True,)),
    "mha_causal_b4_h32_s4096_d128": Workload("mha_causal_b4_h32_s4096_d128", 4, 32, 32, 4096, 128, (True,)),
    "gqa8_b1_h64_s8192_d128": Workload("gqa8_b1_h64_s8192_d128", 1, 64, 8, 8192, 128, (False, True), qk_mult=1.5),
}


def make_inputs(batch, seqlen, heads_q, heads_kv, head_dim, seed=0, qk_mult=1.0):
    """Return dict q, k, v, do of bf16 CPU tensors in BSHD layout."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((batch, seqlen, heads_q, head_dim), generator=g, dtype=torch.float32)
    k = torch.randn((batch, seqlen, heads_kv, head_dim), generator=g, dtype=torch.float32)
    v = torch.randn((batch, seqlen, heads_kv, head_dim), generator=g, dtype=torch.float32)
    do = torch.randn((batch, seqlen, heads_q, head_dim), generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    return {n: t.to(torch.bfloat16) for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}


def workload_inputs(w: Workload, seed=0):
    return make_inputs(w.batch, w.seqlen, w.heads_q, w.heads_kv, w.head_dim, seed=seed, qk_mult=w.qk_mult)


def length_mix(budget, lo, hi, seed=0):
    """Seeded sequence lengths in [lo, hi] summing to ``budget`` (the last one
    takes the remainder, so it may be shorter than ``lo``)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    out, used = [], 0
    while used < budget:
        n = int(torch.randint(lo, hi + 1, (1,), generator=g))
        n = min(n, budget - used)
        out.append(n)
        used += n
    return out


def cu_seqlens(lengths):
    """int32 cumulative offsets [0, l0, l0+l1, ...] as a CPU tensor."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


# Packed causal workload: 16384 tokens (the token count of four 4096-token
# sequences) in a seeded mix of 256 .. 4096-token sequences, 32 heads of 128,
# plus 512 rows of capacity padding.
VARLEN_PACK = {"name": "varlen_causal_h32_t16384_d128", "tokens": 16384, "lo": 256, "hi": 4096, "pad": 512,
               "heads_q": 32, "heads_kv": 32, "head_dim": 128, "seed": 7}


def varlen_pack_inputs(spec=VARLEN_PACK, seed=0):
    """(inputs dict of [T, H, D] bf16 tensors, lengths, cu_seqlens) of a pack."""
    lengths = length_mix(spec["tokens"], spec["lo"], spec["hi"], spec["seed"])
    t = spec["tokens"] + spec["pad"]
    inp = make_inputs(1, t, spec["heads_q"], spec["heads_kv"], spec["head_dim"], seed=seed)
    return {n: x[0] for n, x in inp.items()}, lengths, cu_seqlens(lengths)


# Simple gated linear attention: q, k, v, do standard normal (bf16 RNE) in
# [batch, seq, heads, dim] order, and the per-token log decay
# g = log(sigmoid(x)) / 16 with x standard normal (fp32; always < 0, mean
# about -0.05), drawn after the four tensors from the same generator.
GLA_WORKLOAD = {"name": "gla_b4_h32_t4096_d128", "batch": 4, "seqlen": 4096, "heads": 32, "head_dim": 128}


def gla_inputs(batch, seqlen, heads, head_dim, seed=0):
    """dict q, k, v, do (bf16) and g (fp32) as CPU tensors."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    shp = (batch, seqlen, heads, head_dim)
    out = {n: torch.randn(shp, generator=gen, dtype=torch.float32).to(torch.bfloat16) for n in ("q", "k", "v", "do")}
    x = torch.randn((batch, seqlen, heads), generator=gen, dtype=torch.float32)
    out["g"] = torch.nn.functional.logsigmoid(x) / 16.0
    return out


# Sparse MLA: q [T, H, 576], kv [Tk, 576], do [T, H, 512] standard normal
# (bf16 RNE, drawn in that order); each token's index list holds
# min(K, t + 1) distinct keys drawn uniformly from 0 .. t (keys are the same
# tokens, causal), in random order, then -1 in the unused slots.
# Workload: 4096 tokens, 32 heads (a 128-head model split four ways), 2048
# entries per token.
SMLA_WORKLOAD = {"name": "smla_t4096_h32_k2048", "tokens": 4096, "heads": 32, "topk": 2048}


def smla_indices(tokens, kv_tokens, topk, seed=0):
    """int32 [tokens, topk] causal index lists (see above) as a CPU tensor."""
    gen = torch.Generator(device="cpu").manual_seed(seed + 1)
    out = torch.full((tokens, topk), -1, dtype=torch.int32)
    for t in range(tokens):
        n_keys = min(t + 1, kv_tokens)
        n = min(topk, n_keys)
        out[t, :n] = torch.randperm(n_keys, generator=gen)[:n].to(torch.int32)
    return out


def smla_inputs(tokens, kv_tokens, heads, seed=0):
    """dict q, kv, do (bf16 CPU tensors)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((tokens, heads, 576), generator=gen, dtype=torch.float32)
    kv = torch.randn((kv_tokens, 576), generator=gen, dtype=torch.float32)
    do = torch.randn((tokens, heads, 512), generator=gen, dtype=torch.float32)
    return {n: x.to(torch.bfloat16) for n, x in (("q", q), ("kv", kv), ("do", do))}
