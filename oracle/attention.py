"""Plain fp64 CPU oracle of exact softmax attention and its gradients.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark use it. It shares no code with the GPU
library (no kernels, headers, tables or helpers) and imports only numpy.

What it computes
----------------
The operation is the one the TileLang pull request "[Example] Introduce
split+sum template, and optimize atomic_add performance for bwd examples"
(tile-ai/tilelang #940) exercises in its FlashAttention examples: the
sequence diagram calls ``attention(Q, K, V, causal, groups, use_atomic)``
and autograd's backward returns ``(dq, dk, dv)``.  The pages never write the
equations down, so this module is the textbook definition, materialised:

  S   = scale * Q_h K_kv^T                   (S x S scores, kv = h // groups)
  S_ij = -inf for j > i                       (causal)
  P   = softmax_j(S)                          (row-wise, max-subtracted)
  O_h = P V_kv,     LSE_i = m_i + ln sum_j exp(S_ij - m_i)

and the backward is the vector-Jacobian product of L = sum(O * dO):

  dV_h  = P^T dO               dP = dO V_kv^T
  Delta = rowsum(dO * O)       dS = P * (dP - Delta)
  dQ_h  = scale * dS K_kv      dK_h = scale * dS^T Q_h

with the grouped-query reduction dK_kv = sum over the query heads h of the
group (h = kv*groups + r, r < groups), and likewise dV.  The head mapping
``kv = h // groups`` and the [batch, seq, head, dim] index order are the ones
the review comments on ``example_gqa_bwd.py`` in that pull request show for
the dK accumulation (index ``[bz, by*block_M + i, bx // groups, j]``).

Readings where the pages are silent (each is also listed in the design notes):
  * LSE is the natural logarithm and includes ``scale``.
  * Causal means query i sees key j iff j <= i, with S_q == S_k.
  * Layout is BSHD for Q, K, V, O, dO, dQ, dK, dV; [B, H, S] for LSE, Delta.

The oracle works one (batch, query head) at a time and in blocks of query
rows, so the S x S matrix never exists whole; the blocking is over rows only
(each row's softmax is computed complete), which changes nothing in the
arithmetic the definition prescribes.  Matrix products use numpy's matmul.
"""

from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check(q, k, v, groups):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [batch, seq, heads, dim]")
    b, s, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[1] != s or k.shape[3] != d:
        raise ValueError("k, v must be [batch, seq, heads_kv, dim] matching q")
    if groups < 1 or hq % groups or hq // groups != k.shape[2]:
        raise ValueError("heads_q must equal heads_kv * groups")
    return b, s, hq, d


def _scores(qb, kh, scale, causal, row0):
    """scale * q k^T for query rows row0.. of one head, causal entries -inf."""
    s = scale * (qb @ kh.T)
    if causal:
        rows = np.arange(row0, row0 + qb.shape[0])[:, None]
        cols = np.arange(kh.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def _softmax_rows(s):
    """Row-wise softmax and log-sum-exp of a score block (natural log)."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def softmax_probs(q, k, scale, causal=False, groups=1, b=0, h=0):
    """The full S x S probability matrix P of one (batch, query head).

    Exposed for the invariant checks (rows sum to one, causal zeros); only
    meant for small S.
    """
    q, k = _as64(q), _as64(k)
    kv = h // groups
    s = _scores(q[b, :, h, :], k[b, :, kv, :], scale, causal, 0)
    p, _ = _softmax_rows(s)
    return p


def attention_fwd(q, k, v, scale, causal=False, groups=1):
    """Forward: returns (O [B,S,Hq,D], LSE [B,Hq,S]) in fp64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    b_, s_, hq, d = _check(q, k, v, groups)
    o = np.empty((b_, s_, hq, d))
    lse = np.empty((b_, hq, s_))
    for b in range(b_):
        for h in range(hq):
            kv = h // groups
            kh, vh = k[b, :, kv, :], v[b, :, kv, :]
            for r0 in range(0, s_, ROW_BLOCK):
                qb = q[b, r0:r0 + ROW_BLOCK, h, :]
                p, l = _softmax_rows(_scores(qb, kh, scale, causal, r0))
                o[b, r0:r0 + ROW_BLOCK, h, :] = p @ vh
                lse[b, h, r0:r0 + ROW_BLOCK] = l
    return o, lse


def attention_bwd(q, k, v, do, scale, causal=False, groups=1, heads=None):
    """Backward (VJP of sum(O * dO)): returns dict with dq, dk, dv, o, lse, delta.

    ``heads`` optionally restricts the work to a list of KV heads (all query
    heads of each listed group are processed); gradients of other heads are
    left as NaN.  This exists so that tests can check one group of a large
    problem at full sequence length.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    b_, s_, hq, d = _check(q, k, v, groups)
    hkv = hq // groups
    kv_list = range(hkv) if heads is None else list(heads)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    o = np.full(q.shape, np.nan)
    lse = np.full((b_, hq, s_), np.nan)
    delta = np.full((b_, hq, s_), np.nan)
    for b in range(b_):
        for kv in kv_list:
            kh, vh = k[b, :, kv, :], v[b, :, kv, :]
            dk_sum = np.zeros((s_, d))
            dv_sum = np.zeros((s_, d))
            for r in range(groups):
                h = kv * groups + r
                dk_h = np.zeros((s_, d))
                dv_h = np.zeros((s_, d))
                for r0 in range(0, s_, ROW_BLOCK):
                    sl = slice(r0, r0 + ROW_BLOCK)
                    qb, dob = q[b, sl, h, :], do[b, sl, h, :]
                    p, l = _softmax_rows(_scores(qb, kh, scale, causal, r0))
                    ob = p @ vh
                    dv_h += p.T @ dob
                    dp = dob @ vh.T
                    dl = np.sum(dob * ob, axis=1)
                    ds = p * (dp - dl[:, None])
                    dq[b, sl, h, :] = scale * (ds @ kh)
                    dk_h += scale * (ds.T @ qb)
                    o[b, sl, h, :] = ob
                    lse[b, h, sl] = l
                    delta[b, h, sl] = dl
                dk_sum += dk_h
                dv_sum += dv_h
            dk[b, :, kv, :] = dk_sum
            dv[b, :, kv, :] = dv_sum
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "delta": delta}


def attention_rows(q, k, v, do, scale, causal, groups, b, h, rows):
    """O, LSE, Delta and dQ of selected query rows of one (batch, query head).

    Each row needs only its own softmax row, so this is exact for any S at
    O(S*D) cost per row.  Same definition as ``attention_bwd``.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    kv = h // groups
    kh, vh = k[b, :, kv, :], v[b, :, kv, :]
    out = {"o": [], "lse": [], "delta": [], "dq": []}
    for i in rows:
        s = _scores(q[b, i:i + 1, h, :], kh, scale, causal, i)
        p, l = _softmax_rows(s)
        oi = p @ vh
        dl = np.sum(do[b, i:i + 1, h, :] * oi, axis=1)
        dp = do[b, i:i + 1, h, :] @ vh.T
        ds = p * (dp - dl[:, None])
        out["o"].append(oi[0])
        out["lse"].append(l[0])
        out["delta"].append(dl[0])
        out["dq"].append(scale * (ds @ kh)[0])
    return {key: np.array(val) for key, val in out.items()}


def attention_cols(q, k, v, do, scale, causal, groups, b, kv, cols):
    """dK and dV at selected key rows ``cols`` of one (batch, KV head).

    dK_j and dV_j sum over every query row i that sees key j, for every query
    head of the group, so each needs those rows' LSE and Delta; those come
    from the complete softmax rows (computed here block by block).  With
    causal masking only rows i >= min(cols) take part.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    s_ = q.shape[1]
    d = q.shape[3]
    cols = np.asarray(cols)
    kh, vh = k[b, :, kv, :], v[b, :, kv, :]
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    first = int(cols.min()) if causal else 0
    for r in range(groups):
        h = kv * groups + r
        for r0 in range(first, s_, ROW_BLOCK):
            sl = slice(r0, min(r0 + ROW_BLOCK, s_))
            qb, dob = q[b, sl, h, :], do[b, sl, h, :]
            p, _ = _softmax_rows(_scores(qb, kh, scale, causal, r0))
            ob = p @ vh
            dl = np.sum(dob * ob, axis=1)
            pc = p[:, cols]
            dpc = dob @ vh[cols].T
            dsc = pc * (dpc - dl[:, None])
            dv += pc.T @ dob
            dk += scale * (dsc.T @ qb)
    return {"dk": dk, "dv": dv}
