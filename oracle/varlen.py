"""fp64 CPU oracle of attention over variable-length packed sequences.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only the test-suite, the
package smoke check and the benchmark's CPU leg may use it, and it shares
nothing with the GPU library.

Packed "THD" input, the way the cuDNN frontend pull request "CSA: add
fused Compressor forward+backward CuTe-DSL kernels (ported from Megatron-LM)"
(NVIDIA cudnn-frontend #427, description) passes sequences through int32
``cu_seqlens``: the T tokens of all sequences are stored back to back,
Q [T, Hq, D], K and V [T, Hkv, D], and sequence b holds tokens
cu_seqlens[b] .. cu_seqlens[b+1]-1; tokens at or past cu_seqlens[-1] are
capacity padding, whose gradients that page makes exact zeros.

Readings used here (and by the kernels): attention never crosses sequences;
within a sequence it is the ordinary (optionally causal) attention with the
causal mask in the sequence's own positions; queries and keys have the same
lengths; a sequence of length 0 contributes nothing; a padding row sees no
key, so its O is 0 and its LSE is -inf (the forward's convention for rows
without visible keys), and its dQ, dK, dV are 0.

Row-indexed values (LSE, Delta) are stored head-major over all tokens,
[Hq, T], as the packed layout's row index suggests.
"""

from __future__ import annotations

import numpy as np

from oracle import attention as att


def _segments(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]


def _seq(x, a, e):
    return np.asarray(x, dtype=np.float64)[a:e][None]   # [1, len, H, D]


def varlen_fwd(q, k, v, cu, scale, causal=False, groups=1):
    """Returns (O [T, Hq, D], LSE [Hq, T]), fp64; padding rows O = 0, LSE = -inf."""
    t, hq, d = np.shape(q)
    o = np.zeros((t, hq, d))
    lse = np.full((hq, t), -np.inf)
    for a, e in _segments(cu):
        if e == a:
            continue
        ob, lb = att.attention_fwd(_seq(q, a, e), _seq(k, a, e), _seq(v, a, e), scale, causal, groups)
        o[a:e] = ob[0]
        lse[:, a:e] = lb[0]
    return o, lse


def varlen_bwd(q, k, v, do, cu, scale, causal=False, groups=1):
    """Returns a dict with dq, dk, dv ([T, H, D]), o ([T, Hq, D]), lse and
    delta ([Hq, T]), fp64; padding rows get zero gradients, O = 0, LSE = -inf
    and Delta = 0."""
    t, hq, d = np.shape(q)
    hkv = np.shape(k)[1]
    out = {"dq": np.zeros((t, hq, d)), "dk": np.zeros((t, hkv, d)), "dv": np.zeros((t, hkv, d)),
           "o": np.zeros((t, hq, d)), "lse": np.full((hq, t), -np.inf), "delta": np.zeros((hq, t))}
    for a, e in _segments(cu):
        if e == a:
            continue
        r = att.attention_bwd(_seq(q, a, e), _seq(k, a, e), _seq(v, a, e), _seq(do, a, e), scale, causal, groups)
        for n in ("dq", "dk", "dv", "o"):
            out[n][a:e] = r[n][0]
        for n in ("lse", "delta"):
            out[n][:, a:e] = r[n][0]
    return out
