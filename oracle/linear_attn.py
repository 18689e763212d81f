"""fp64 CPU oracle of simple gated linear attention ("simple_gla") and its
gradients.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only the test-suite, the
package smoke check and the benchmark's CPU leg may use it, and it shares
nothing with the GPU library.

The flash-linear-attention pull request "[Perf] TileLang backends for
linear-attention chunk backward (simple_gla / gla / delta_rule / gdn)"
(fla-org/flash-linear-attention #1046, summary and "How") speeds up the chunk
backward of these kernels, simple_gla first in its list; it names the pieces
(the dq/dk/dv/dg stage and the chunk state recurrence) but writes no
equations.  Readings used here, the standard definition of simple gated linear
attention (one scalar gate per token and head):

  state   S_t = exp(g_t) S_{t-1} + k_t^T v_t,   S_0 = 0   (K x V per head)
  output  o_t = scale * q_t S_t

with g the per-token log decay (natural log; g <= 0 keeps the state from
growing), q, k [B, T, H, K], v [B, T, H, V], g [B, T, H].  Unrolled, with the
running sum G_t = g_1 + ... + g_t,

  o_t = scale * sum_{s <= t} exp(G_t - G_s) (q_t . k_s) v_s.

The backward is the vector-Jacobian product of L = sum_t do_t . o_t.  With
W_ts = scale exp(G_t - G_s) (q_t . k_s)(do_t . v_s) for s <= t:

  dq_t = scale sum_{s<=t} exp(G_t - G_s) (do_t . v_s) k_s
  dk_s = scale sum_{t>=s} exp(G_t - G_s) (do_t . v_s) q_t
  dv_s = scale sum_{t>=s} exp(G_t - G_s) (q_t . k_s) do_t
  dL/dG_t = sum_s W_ts - sum_t' W_t't  (= q_t . dq_t - k_t . dk_t)
  dg_r = sum_{t >= r} dL/dG_t          (G is the running sum of g)

This module materialises the T x T matrices of one (batch, head) at a time
(the quadratic form); no chunking.
"""

from __future__ import annotations

import numpy as np


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _decay(g_bh):
    """[T, T] matrix exp(G_t - G_s) for s <= t, else 0 (G = running sum)."""
    G = np.cumsum(g_bh)
    t = len(G)
    diff = G[:, None] - G[None, :]
    lower = np.tril(np.ones((t, t), dtype=bool))
    return np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)


def gla_fwd(q, k, v, g, scale):
    """o [B, T, H, V], fp64."""
    q, k, v, g = _as64(q), _as64(k), _as64(v), _as64(g)
    b_, t_, h_, _ = q.shape
    o = np.zeros(v.shape[:3] + (v.shape[3],))
    for b in range(b_):
        for h in range(h_):
            dm = _decay(g[b, :, h])
            a = scale * (q[b, :, h] @ k[b, :, h].T) * dm
            o[b, :, h] = a @ v[b, :, h]
    return o


def gla_bwd(q, k, v, g, do, scale, heads=None):
    """dict of dq, dk [B,T,H,K], dv [B,T,H,V], dg [B,T,H] and o, fp64.

    ``heads`` optionally restricts the work to a list of (batch, head) pairs
    (other entries are left NaN), for checks of single heads of a large
    problem.
    """
    q, k, v, g, do = _as64(q), _as64(k), _as64(v), _as64(g), _as64(do)
    b_, t_, h_, _ = q.shape
    out = {n: np.full(x.shape, np.nan) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("o", do))}
    pairs = [(b, h) for b in range(b_) for h in range(h_)] if heads is None else list(heads)
    for b, h in pairs:
        qb, kb, vb, dob = q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]
        dm = _decay(g[b, :, h])
        a_qk = scale * (qb @ kb.T) * dm          # [t, s]
        a_dov = scale * (dob @ vb.T) * dm        # [t, s]
        out["o"][b, :, h] = a_qk @ vb
        out["dq"][b, :, h] = a_dov @ kb
        out["dk"][b, :, h] = a_dov.T @ qb
        out["dv"][b, :, h] = a_qk.T @ dob
        w = a_qk * (dob @ vb.T)                  # W_ts
        d_g_cum = np.sum(w, axis=1) - np.sum(w, axis=0)
        out["dg"][b, :, h] = np.cumsum(d_g_cum[::-1])[::-1]
    return out
