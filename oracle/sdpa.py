"""Materialized grouped-query scaled-dot-product attention in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method reaches exactly the plain softmax-attention result; tiling and the
online softmax only reorder floating-point work ([EffSeq] 资源变化: the blocks
accumulate the same softmax attention result; [AttnVar] 3.5: mathematically
equivalent to standard attention, not a sparse approximation).  So this oracle
is the definition written out, with the full score matrix S and probability
matrix P built for every (sequence, query head):

  [EffSeq] 分组查询注意力:  O_a = softmax(Q_a K_{g(a)}^T / sqrt(d_h) + M) V_{g(a)},
                            g(a) = floor(a / r),  r = h_q / h_kv
  [Ch09]  09.2:             the same formula, M_{t,j} = -inf for j > t, else 0
  [EffSeq] 分块注意力:      S = Q K^T / sqrt(d_h) + M,  P = softmax(S),  O = P V

Readings where the pages leave a step open (listed again in the design doc):
  * scale is an explicit argument; ``None`` means 1/sqrt(d_h) as the formula fixes;
  * the mask is exactly -inf, applied by selection, never a large finite value
    ([MhaMqaGqa] section 1: 0 where access is allowed, -inf at future positions);
  * the padding mask of [EffSeq] is read as per-sequence key lengths: key j of
    sequence b is visible only if j < kv_len[b];
  * positions are absolute: a cached decode query at position p sees keys j <= p
    ([Ch09] 09.2: the current position pointer fixes the query's absolute position;
    a zero-based triangular template on a 1 x T matrix would show only key 0);
  * a query row with no visible key has no defined output: this oracle raises
    ``ValueError`` (the online-softmax code on [EffSeq] 两块算例 does the same).
"""

from __future__ import annotations

import math

import numpy as np


def group_index(h_q: int, h_kv: int) -> list[int]:
    """K/V head read by each query head: g(a) = floor(a / r), r = h_q / h_kv.

    [EffSeq] 分组查询注意力 (h_q must be divisible by h_kv; zero-based head a reads
    group floor(a/r)); [MhaMqaGqa] section 6 (heads 0-3 -> KV 0, 4-7 -> KV 1);
    [Ch09] 09.2 (A,A,B,B order, never A,B,A,B).  Non-divisible counts are rejected,
    never rounded ([Ch09] 09.1 warns that estimator scripts round the head width up).
    """
    if h_q < 1 or h_kv < 1:
        raise ValueError("head counts must be >= 1")
    if h_q % h_kv != 0:
        raise ValueError(f"h_q={h_q} is not divisible by h_kv={h_kv}")
    r = h_q // h_kv
    return [a // r for a in range(h_q)]


def default_scale(d_h: int) -> float:
    """1/sqrt(d_h), the factor inside the softmax ([EffSeq] 分组查询注意力 formula)."""
    return 1.0 / math.sqrt(d_h)


def default_q_pos(B: int, S_q: int, T_k: int, kv_len: np.ndarray) -> np.ndarray:
    """Absolute position of every query row when the caller gives none.

    Prefill (S_q == T_k): query i sits at position i, whatever kv_len (the
    padding mask removes keys, not query positions).  Otherwise the S_q queries
    are the newest S_q positions of the visible history: kv_len[b] - S_q + i
    ([MhaMqaGqa] parameter table: T counts the visible history including the
    current position; [Ch09] 09.2: a cached query carries its absolute
    position, the current-position pointer, not its index in the chunk).
    """
    pos = np.empty((B, S_q), dtype=np.int64)
    for b in range(B):
        for i in range(S_q):
            pos[b, i] = i if S_q == T_k else int(kv_len[b]) - S_q + i
    return pos


def visibility(q_pos_b: np.ndarray, kv_len_b: int, T_k: int, causal: bool) -> np.ndarray:
    """Boolean (S_q, T_k) matrix: key j visible to query i.

    Visible iff j < kv_len_b (padding mask) and, when causal, j <= q_pos_b[i]
    ([EffSeq] 分组查询注意力: M is a causal or padding mask; [Ch09] 09.2: M is -inf
    for j > t).
    """
    j = np.arange(T_k)[None, :]
    vis = j < kv_len_b
    if causal:
        vis = vis & (j <= q_pos_b[:, None])
    return np.broadcast_to(vis, (q_pos_b.shape[0], T_k)).copy()


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row softmax of a score matrix whose masked entries are -inf.

    Subtracting the row maximum keeps every exponent argument <= 0; numerator
    and denominator are scaled by the same factor so the weights are unchanged
    ([EffSeq] 在线 softmax, paragraph on subtracting the maximum).
    """
    if not np.all(np.any(np.isfinite(S), axis=1)):
        raise ValueError("a query row sees no key, so its softmax is undefined")
    m = np.max(S, axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / np.sum(E, axis=1, keepdims=True)


def attention(q, k, v, *, scale=None, causal=True, q_pos=None, kv_len=None) -> np.ndarray:
    """Grouped-query attention, materialized, float64.

    Args:
      q: (B, h_q, S_q, d_h) queries (any real dtype; converted to float64).
      k, v: (B, h_kv, T_k, d_h) keys and values, cache layout (B, h_kv, T, d_h)
        ([EffSeq] 缓存字节: keep the cache as (B, h_kv, T, d_h) and read it through
        the group index).
      scale: multiplier of Q K^T; None -> 1/sqrt(d_h).
      causal: apply the causal mask (key j visible only if j <= query position).
      q_pos: (B, S_q) absolute query positions; None -> ``default_q_pos``.
      kv_len: (B,) number of valid keys per sequence; None -> T_k.

    Returns:
      (B, h_q, S_q, d_h) float64 output; O[b, a] is O_a of the formula.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (B, heads, seq, d_h)")
    B, h_q, S_q, d_h = q.shape
    Bk, h_kv, T_k, d_k = k.shape
    if (Bk, d_k) != (B, d_h) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    g = group_index(h_q, h_kv)
    if scale is None:
        scale = default_scale(d_h)
    kv_len = np.full(B, T_k, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    if kv_len.shape != (B,) or np.any(kv_len < 0) or np.any(kv_len > T_k):
        raise ValueError("kv_len must be (B,) with 0 <= kv_len <= T_k")
    if q_pos is None:
        q_pos = default_q_pos(B, S_q, T_k, kv_len)
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(B, S_q)
    if not np.all(np.isfinite(q)):
        raise ValueError("q holds non-finite values")

    out = np.empty((B, h_q, S_q, d_h), dtype=np.float64)
    for b in range(B):
        L = int(kv_len[b])
        # rows at or past kv_len[b] are never read (the padding mask removes them);
        # only the rows that are read must be finite
        kb, vb = k[b, :, :L], v[b, :, :L]
        if not (np.all(np.isfinite(kb)) and np.all(np.isfinite(vb))):
            raise ValueError("k or v holds non-finite values in a visible row")
        vis = visibility(q_pos[b], L, L, causal)
        for a in range(h_q):
            K = kb[g[a]]
            V = vb[g[a]]
            S = (q[b, a] @ K.T) * scale                      # (S_q, kv_len[b]), materialized
            S = np.where(vis, S, -np.inf)
            P = softmax_rows(S)                              # (S_q, T_k), materialized
            out[b, a] = P @ V
    return out
