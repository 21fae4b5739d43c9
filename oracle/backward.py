"""Gradients of grouped-query attention with respect to Q, K and V, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method's training half recomputes the probabilities from the saved row
statistics instead of storing P ([EffSeq] 在线 softmax: the forward keeps only
the running maximum and normalizer per row; [AttnVar] 3.5: tiles are recomputed
rather than the T x T matrices kept).  The result is still the gradient of the
plain attention, so this oracle is the chain rule applied to the materialized
definition of ``oracle.sdpa.attention``, written out per (sequence, query head):

    S = scale * Q_a K_g^T + M,   P = softmax_rows(S),   O_a = P V_g
    dV_g += P^T dO_a                      (every query head of the group adds in)
    dP    = dO_a V_g^T
    dS    = P * (dP - rowsum(dP * P))     (softmax Jacobian, row by row)
    dQ_a  = scale * dS K_g
    dK_g += scale * dS^T Q_a

Group heads: the K/V head g(a) = floor(a / r) serves r query heads
([EffSeq] 分组查询注意力), so its gradients are the sums over those r heads --
the same sums the expanded (repeated) K/V form would produce.

rowsum(dP * P) equals rowsum(dO_a * O_a), the form a kernel uses without P.
Rows with no visible key have no output and are rejected as in the forward.
"""

from __future__ import annotations

import numpy as np

from .sdpa import default_q_pos, default_scale, group_index, softmax_rows, visibility


def attention_backward(q, k, v, d_out, *, scale=None, causal=True, q_pos=None, kv_len=None):
    """Return (dq, dk, dv) float64 with the shapes of q, k, v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    B, h_q, S_q, d_h = q.shape
    _, h_kv, T_k, _ = k.shape
    if d_out.shape != q.shape or v.shape != k.shape:
        raise ValueError("shape mismatch")
    g = group_index(h_q, h_kv)
    if scale is None:
        scale = default_scale(d_h)
    kv_len = np.full(B, T_k, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    if q_pos is None:
        q_pos = default_q_pos(B, S_q, T_k, kv_len)
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(B, S_q)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        L = int(kv_len[b])
        vis = visibility(q_pos[b], L, L, causal)                  # (S_q, L)
        for a in range(h_q):
            kg, vg = k[b, g[a], :L], v[b, g[a], :L]
            s = (q[b, a] @ kg.T) * scale
            s = np.where(vis, s, -np.inf)
            p = softmax_rows(s)                                   # raises on a row with no visible key
            do = d_out[b, a]
            dv[b, g[a], :L] += p.T @ do
            dp = do @ vg.T
            ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
            dq[b, a] = scale * (ds @ kg)
            dk[b, g[a], :L] += scale * (ds.T @ q[b, a])
    return dq, dk, dv


def row_logsumexp(q, k, *, scale=None, causal=True, q_pos=None, kv_len=None):
    """L[b, a, i] = log sum_j exp(S_ij) over the visible keys (natural log), float64.

    The row statistic the training forward saves: with it, P = exp(S - L) is
    recomputed exactly ([EffSeq] 在线 softmax: m and l per row; L = m + log l).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, h_q, S_q, d_h = q.shape
    _, h_kv, T_k, _ = k.shape
    g = group_index(h_q, h_kv)
    if scale is None:
        scale = default_scale(d_h)
    kv_len = np.full(B, T_k, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    if q_pos is None:
        q_pos = default_q_pos(B, S_q, T_k, kv_len)
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(B, S_q)
    out = np.empty((B, h_q, S_q))
    for b in range(B):
        L = int(kv_len[b])
        vis = visibility(q_pos[b], L, L, causal)
        for a in range(h_q):
            s = (q[b, a] @ k[b, g[a], :L].T) * scale
            s = np.where(vis, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            out[b, a] = (m + np.log(np.sum(np.exp(s - m), axis=1, keepdims=True)))[:, 0]
    return out
