"""fp64 CPU oracle of the context-parallel (ring) building blocks.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only the test-suite, the
package smoke check and the benchmark's CPU leg may use it, and it shares
nothing with the GPU library.

Context parallelism splits the sequence into chunks.  The Megatron-LM pull
request "TileLang implementation of the fused DSA operations" (NVIDIA
Megatron-LM #5049, description, "Packed THD and CP behavior") routes such
context-parallel cases through a common path; the pages do not write the
arithmetic down.  The plain definitions used here:

* Attention of a query row over a key set that is the disjoint union of
  chunks K_1 .. K_P.  With LSE_k the log-sum-exp of the row's scores over
  chunk k and O_k the softmax-weighted values over chunk k alone,

      LSE = log sum_k exp(LSE_k),      O = sum_k exp(LSE_k - LSE) O_k,

  because exp(LSE_k) is chunk k's share of the softmax denominator.  A chunk
  the row cannot see (all scores -inf) has LSE_k = -inf and weight 0; a row
  that sees no key at all gets LSE = -inf and O = 0 (the forward kernel's
  convention for such rows).

* The backward of one (query chunk, key chunk) pair with the *global* LSE and
  Delta of the query rows: P = exp(S - LSE) are then the entries of the full
  softmax, so dS = P o (dP - Delta) and the pair's dQ, dK, dV terms are the
  full gradients' terms for that pair; dQ sums over key chunks, dK and dV
  over query chunks.

Chunks have equal length C, so every pair is either fully visible (key chunk
before the query chunk), diagonal (same chunk: causal within the chunk) or
invisible (key chunk after the query chunk, under causal masking).
"""

from __future__ import annotations

import numpy as np

from oracle import attention as att


def merge_partials(o_parts, lse_parts):
    """Merge P partial results of the same query rows.

    o_parts: [P, B, S, H, D]; lse_parts: [P, B, H, S] (natural log, -inf for
    rows that saw no key of that part).  Returns (O [B,S,H,D], LSE [B,H,S])
    in fp64.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    n_parts = lse_parts.shape[0]
    if o_parts.shape[0] != n_parts or n_parts < 1:
        raise ValueError("o_parts and lse_parts need the same number (>= 1) of parts")
    m = np.max(lse_parts, axis=0)                       # [B, H, S]
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])                # exp(-inf) = 0 for empty parts
    z = np.sum(w, axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, z)))
    coef = np.where(empty[None], 0.0, w / np.where(empty, 1.0, z)[None])   # [P, B, H, S]
    o = np.einsum("pbhs,pbshd->bshd", coef, o_parts)
    return o, lse


def chunk_pairs(n_chunks, causal):
    """(query chunk, key chunk, causal-within-pair) for every visible pair."""
    pairs = []
    for i in range(n_chunks):
        for j in range(n_chunks):
            if causal and j > i:
                continue
            pairs.append((i, j, causal and i == j))
    return pairs


def _chunk(x, i, c):
    return x[:, i * c:(i + 1) * c]


def ring_fwd(q, k, v, scale, causal, groups, n_chunks):
    """Forward as the ring computes it: per visible chunk pair the ordinary
    attention of the query chunk over the key chunk, then one merge per query
    chunk.  Returns (O, LSE) over the whole sequence, fp64."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b, s, hq, d = q.shape
    if s % n_chunks:
        raise ValueError("sequence length must split into equal chunks")
    c = s // n_chunks
    o = np.empty((b, s, hq, d))
    lse = np.empty((b, hq, s))
    for i in range(n_chunks):
        parts_o, parts_l = [], []
        for qi, kj, cz in chunk_pairs(n_chunks, causal):
            if qi != i:
                continue
            po, pl = att.attention_fwd(_chunk(q, i, c), _chunk(k, kj, c), _chunk(v, kj, c), scale, cz, groups)
            parts_o.append(po)
            parts_l.append(pl)
        mo, ml = merge_partials(np.stack(parts_o), np.stack(parts_l))
        o[:, i * c:(i + 1) * c] = mo
        lse[:, :, i * c:(i + 1) * c] = ml
    return o, lse


def pair_bwd(qc, kc, vc, doc, lse_c, delta_c, scale, causal, groups):
    """Gradient terms of one chunk pair given the query rows' global LSE and
    Delta ([B, Hq, C] each).  Returns (dq, dk, dv) terms, fp64; dk/dv summed
    over the query heads of each group."""
    qc, kc, vc, doc = (np.asarray(x, dtype=np.float64) for x in (qc, kc, vc, doc))
    b_, c, hq, d = qc.shape
    hkv = hq // groups
    dq = np.zeros(qc.shape)
    dk = np.zeros(kc.shape)
    dv = np.zeros(vc.shape)
    rows = np.arange(c)[:, None]
    cols = np.arange(c)[None, :]
    for b in range(b_):
        for h in range(hq):
            kv = h // groups
            s = scale * (qc[b, :, h, :] @ kc[b, :, kv, :].T)
            if causal:
                s = np.where(cols > rows, -np.inf, s)
            p = np.exp(s - lse_c[b, h][:, None])
            dp = doc[b, :, h, :] @ vc[b, :, kv, :].T
            ds = p * (dp - delta_c[b, h][:, None])
            dq[b, :, h, :] = scale * (ds @ kc[b, :, kv, :])
            dk[b, :, kv, :] += scale * (ds.T @ qc[b, :, h, :])
            dv[b, :, kv, :] += p.T @ doc[b, :, h, :]
    return dq, dk, dv


def ring_bwd(q, k, v, do, scale, causal, groups, n_chunks):
    """Backward as the ring computes it: global O and LSE from ``ring_fwd``,
    Delta = rowsum(dO o O), then the pair terms summed.  Returns a dict with
    dq, dk, dv, o, lse, delta (fp64)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = q.shape[1]
    c = s // n_chunks
    o, lse = ring_fwd(q, k, v, scale, causal, groups, n_chunks)
    delta = np.transpose(np.sum(do * o, axis=3), (0, 2, 1))   # [B, H, S]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for i, j, cz in chunk_pairs(n_chunks, causal):
        tq, tk, tv = pair_bwd(_chunk(q, i, c), _chunk(k, j, c), _chunk(v, j, c), _chunk(do, i, c),
                              lse[:, :, i * c:(i + 1) * c], delta[:, :, i * c:(i + 1) * c], scale, cz, groups)
        dq[:, i * c:(i + 1) * c] += tq
        dk[:, j * c:(j + 1) * c] += tk
        dv[:, j * c:(j + 1) * c] += tv
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "delta": delta}
