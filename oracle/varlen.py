"""fp64 CPU oracle of attention over variable-length packed sequences.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only the test-suite, the
package smoke check and the benchmark's CPU leg may use it, and it shares
nothing with the GPU library.

Packed "THD" input, the way the cuDNN frontend pull request "CSA: add
fused Compressor forward+backward CuTe-DSL kernels (ported from Megatron-LM)"
(NVIDIA cudnn-frontend #427, description) passes sequences through int32
``cu_seqlens``: the tokens of all sequences are stored back to back,
Q [Tq, Hq, D], K and V [Tk, Hkv, D], and sequence b holds query rows
cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1 (cu_k = cu_q when
queries and keys are the same tokens); rows at or past the last offset are
capacity padding, whose gradients that page makes exact zeros.

Readings used here (and by the kernels): attention never crosses sequences;
within a sequence of lq queries and lk keys it is the ordinary softmax
attention of the textbook definition (the one ``oracle.attention`` spells
out), and under causal masking query i (0-based, in the sequence) sees key j
iff j <= i + (lk - lq), i.e. the last query is aligned with the last key
(for lq == lk this is the usual j <= i).  A query that sees no key (i <
lq - lk, or lk == 0) and every padding row has O = 0 and LSE = -inf, and
contributes nothing to any gradient; its dQ is 0.  A sequence with no
queries or no keys contributes nothing.

Row-indexed values (LSE, Delta) are stored head-major over all query rows,
[Hq, Tq].
"""

from __future__ import annotations

import numpy as np


def _segments(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]


def visible_keys(lq, lk, causal):
    """[lq, lk] boolean: may query i see key j (bottom-right causal alignment)."""
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    return j <= i + (lk - lq)


def seq_attention(q, k, v, do, scale, causal, groups):
    """One sequence: q, do [lq, Hq, D]; k, v [lk, Hkv, D].

    Returns a dict with o, dq [lq, Hq, D], dk, dv [lk, Hkv, D], lse and delta
    [Hq, lq], all fp64, from the definition: S = scale Q K^T with invisible
    entries removed, P = softmax over the visible keys, O = P V,
    Delta = rowsum(dO * O), dS = P * (dO V^T - Delta), dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO (dK, dV summed over each group's heads).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    lq, hq, d = q.shape
    lk = k.shape[0]
    out = {"o": np.zeros((lq, hq, d)), "dq": np.zeros((lq, hq, d)), "dk": np.zeros(k.shape),
           "dv": np.zeros(v.shape), "lse": np.full((hq, lq), -np.inf), "delta": np.zeros((hq, lq))}
    if lq == 0 or lk == 0:
        return out
    vis = visible_keys(lq, lk, causal)
    has = vis.any(axis=1)                      # rows that see at least one key
    for h in range(hq):
        kv = h // groups
        s = np.where(vis, scale * (q[:, h] @ k[:, kv].T), -np.inf)
        m = np.where(has, np.max(s, axis=1), 0.0)
        e = np.where(vis, np.exp(s - m[:, None]), 0.0)
        z = np.sum(e, axis=1)
        p = e / np.where(has, z, 1.0)[:, None]
        o = p @ v[:, kv]
        delta = np.sum(do[:, h] * o, axis=1)
        ds = p * (do[:, h] @ v[:, kv].T - delta[:, None])
        out["o"][:, h] = o
        out["lse"][h] = np.where(has, m + np.log(np.where(has, z, 1.0)), -np.inf)
        out["delta"][h] = delta
        out["dq"][:, h] = scale * (ds @ k[:, kv])
        out["dk"][:, kv] += scale * (ds.T @ q[:, h])
        out["dv"][:, kv] += p.T @ do[:, h]
    return out


def varlen_bwd(q, k, v, do, cu, scale, causal=False, groups=1, cu_k=None):
    """Packed sequences: returns a dict with dq, o ([Tq, Hq, D]), dk, dv
    ([Tk, Hkv, D]), lse and delta ([Hq, Tq]), fp64.  ``cu`` holds the query
    offsets, ``cu_k`` the key offsets (default: the same).  Padding rows get
    zero gradients, O = 0, LSE = -inf and Delta = 0."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    tq, hq, d = q.shape
    cu_k = cu if cu_k is None else cu_k
    if len(cu_k) != len(cu):
        raise ValueError("cu and cu_k must describe the same number of sequences")
    out = {"dq": np.zeros((tq, hq, d)), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
           "o": np.zeros((tq, hq, d)), "lse": np.full((hq, tq), -np.inf), "delta": np.zeros((hq, tq))}
    for (a, e), (ka, ke) in zip(_segments(cu), _segments(cu_k)):
        r = seq_attention(q[a:e], k[ka:ke], v[ka:ke], do[a:e], scale, causal, groups)
        for n in ("dq", "o"):
            out[n][a:e] = r[n]
        for n in ("dk", "dv"):
            out[n][ka:ke] = r[n]
        for n in ("lse", "delta"):
            out[n][:, a:e] = r[n]
    return out


def varlen_fwd(q, k, v, cu, scale, causal=False, groups=1, cu_k=None):
    """Returns (O [Tq, Hq, D], LSE [Hq, Tq]), fp64; padding rows O = 0,
    LSE = -inf.  The forward part of ``varlen_bwd`` (dO is not needed)."""
    r = varlen_bwd(q, k, v, np.zeros(np.shape(q)), cu, scale, causal, groups, cu_k)
    return r["o"], r["lse"]
