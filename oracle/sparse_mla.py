"""fp64 CPU oracle of sparse MLA attention (attention over top-k gathered
latent keys) and its gradients.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only the test-suite, the
package smoke check and the benchmark's CPU leg may use it, and it shares
nothing with the GPU library.

The Megatron-LM pull request "TileLang implementation of the fused DSA
operations" (NVIDIA Megatron-LM #5049, file table and review summary) adds a
sparse MLA forward and a backward with preprocess/postprocess kernels: each
query token attends to the keys its indexer selected (top-k, with -1 as the
sentinel of an unused slot), the latent key rows are 576 wide and the value
is their first 512 channels (the only supported dims, "dim=576 /
v_channels=512"), bf16 compute with fp32 accumulation.  The pages write no
equations; the readings used here (and by the kernels):

  For token t and head h, with J_t the valid entries of idx[t] (0 <= j < Tk;
  anything else, -1 in particular, is an unused slot):
    s_i  = scale * q[t,h] . kv[J_t[i]]            (one logit per entry)
    P    = softmax over the entries,  LSE = log sum_i exp(s_i)
    O    = sum_i P_i kv[J_t[i], :512]
  A key listed twice is two entries (it simply gets twice the weight).  A
  token with no valid entry has O = 0 and LSE = -inf.
  Backward (VJP of sum O . dO), Delta = O . dO:
    dP_i = dO . kv[J_t[i], :512],   dS_i = P_i (dP_i - Delta)
    dq[t,h]           = scale * sum_i dS_i kv[J_t[i]]
    dkv[J_t[i]]      += scale * dS_i q[t,h]           (all heads, all tokens)
    dkv[J_t[i], :512] += P_i dO[t,h]

Layouts: q [T, H, 576], kv [Tk, 576], idx [T, K] int, O and dO [T, H, 512],
LSE and Delta [T, H].
"""

from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512


def _valid(idx_t, tk):
    idx_t = np.asarray(idx_t, dtype=np.int64)
    return idx_t[(idx_t >= 0) & (idx_t < tk)]


def sparse_mla_fwd(q, kv, idx, scale, d_v=D_V):
    """(O [T, H, d_v], LSE [T, H]) in fp64."""
    q, kv = np.asarray(q, dtype=np.float64), np.asarray(kv, dtype=np.float64)
    t_, h_, _ = q.shape
    tk = kv.shape[0]
    o = np.zeros((t_, h_, d_v))
    lse = np.full((t_, h_), -np.inf)
    for t in range(t_):
        j = _valid(idx[t], tk)
        if len(j) == 0:
            continue
        s = scale * (q[t] @ kv[j].T)                      # [H, n]
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        z = np.sum(e, axis=1, keepdims=True)
        o[t] = (e / z) @ kv[j, :d_v]
        lse[t] = (m + np.log(z))[:, 0]
    return o, lse


def sparse_mla_bwd(q, kv, idx, do, scale, d_v=D_V):
    """dict with dq [T, H, 576], dkv [Tk, 576], o, lse, delta (fp64)."""
    q, kv, do = (np.asarray(x, dtype=np.float64) for x in (q, kv, do))
    t_, h_, _ = q.shape
    tk = kv.shape[0]
    out = {"dq": np.zeros(q.shape), "dkv": np.zeros(kv.shape), "o": np.zeros((t_, h_, d_v)),
           "lse": np.full((t_, h_), -np.inf), "delta": np.zeros((t_, h_))}
    for t in range(t_):
        j = _valid(idx[t], tk)
        if len(j) == 0:
            continue
        kj = kv[j]                                        # [n, 576]
        s = scale * (q[t] @ kj.T)                         # [H, n]
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        z = np.sum(e, axis=1, keepdims=True)
        p = e / z
        o = p @ kj[:, :d_v]
        delta = np.sum(do[t] * o, axis=1)                 # [H]
        dp = do[t] @ kj[:, :d_v].T                        # [H, n]
        ds = p * (dp - delta[:, None])
        out["dq"][t] = scale * (ds @ kj)
        np.add.at(out["dkv"], j, scale * (ds.T @ q[t]))
        np.add.at(out["dkv"][:, :d_v], j, p.T @ do[t])
        out["o"][t] = o
        out["lse"][t] = (m + np.log(z))[:, 0]
        out["delta"][t] = delta
    return out
