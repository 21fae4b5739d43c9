"""Block-wise online softmax for one query row, and the merge of two partial states.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is the algorithm of [EffSeq] 在线 softmax, taken in the page's order and
notation and written from its description:

  state after the positions J already read:
      m = max_{j in J} s_j,   l = sum_{j in J} e^{s_j - m},   u = sum_{j in J} e^{s_j - m} v_j
  start from (m, l, u) = (-inf, 0, 0); a block whose keys are all masked is skipped,
  so that -inf - (-inf) never occurs;
  a new block I with maximum m_hat moves both sums to the common base m' = max(m, m_hat):
      l' = e^{m - m'} l + sum_{j in I} e^{s_j - m'}
      u' = e^{m - m'} u + sum_{j in I} e^{s_j - m'} v_j
  after the last block the output is o = u / l.

``merge_states`` is the combine rule of [AttnVar] 3.5 for two partial states
computed over disjoint key sets: m' = max(m, m_b), l' = e^{m - m'} l + e^{m_b - m'} l_b,
and the unnormalized weighted value sum rescaled the same way.

These functions are the oracle's own self-check of tiling (tiled result equals
the materialized one, [EffSeq] 两块算例) and the reference semantics of the
split-KV combine.  They are float64 throughout.
"""

from __future__ import annotations

import numpy as np


def _empty_state(d: int):
    return (-np.inf, 0.0, np.zeros(d, dtype=np.float64))


def online_states(scores, values, block: int):
    """Yield the state (m, l, u) after each block of ``block`` keys.

    scores: (T,) scaled and masked scores (masked entries are -inf).
    values: (T, d) value vectors.
    Blocks with no visible key leave the state unchanged (and still yield it).
    """
    s_all = np.asarray(scores, dtype=np.float64)
    v_all = np.asarray(values, dtype=np.float64)
    if s_all.ndim != 1 or v_all.ndim != 2 or v_all.shape[0] != s_all.shape[0]:
        raise ValueError("scores must be (T,) and values (T, d)")
    if block < 1:
        raise ValueError("block must be >= 1")
    if not np.all(np.isfinite(s_all) | np.isneginf(s_all)):
        raise ValueError("scores must be finite or -inf")
    if not np.all(np.isfinite(v_all)):
        raise ValueError("values must be finite")
    m, l, u = _empty_state(v_all.shape[1])
    for start in range(0, s_all.shape[0], block):
        s = s_all[start:start + block]
        v = v_all[start:start + block]
        seen = ~np.isneginf(s)
        if seen.any():
            s, v = s[seen], v[seen]
            m_new = max(m, float(np.max(s)))
            carry = np.exp(m - m_new)          # e^{m - m'}; 0 while nothing has been read
            w = np.exp(s - m_new)              # e^{s_j - m'} for j in the new block
            l = carry * l + float(np.sum(w))
            u = carry * u + w @ v
            m = m_new
        yield (m, l, u.copy())


def finish_state(state) -> np.ndarray:
    """o = u / l; a state that saw no visible key has no output."""
    m, l, u = state
    if l == 0.0:
        raise ValueError("query has no visible key")
    return u / l


def online_attention_row(scores, values, block: int = 2) -> np.ndarray:
    """Output of one query row computed block by block with the online state."""
    state = None
    for state in online_states(scores, values, block):
        pass
    if state is None:
        raise ValueError("query has no visible key")
    return finish_state(state)


def merge_states(a, b):
    """Combine two partial states over disjoint key sets ([AttnVar] 3.5)."""
    m_a, l_a, u_a = a
    m_b, l_b, u_b = b
    m_new = max(m_a, m_b)
    if np.isneginf(m_new):
        return (-np.inf, 0.0, np.zeros_like(np.asarray(u_a, dtype=np.float64)))
    c_a = np.exp(m_a - m_new)
    c_b = np.exp(m_b - m_new)
    return (m_new, c_a * l_a + c_b * l_b, c_a * np.asarray(u_a, np.float64) + c_b * np.asarray(u_b, np.float64))
