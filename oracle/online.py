"""Block-wise online softmax for one query row, and the merge of two partial states.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is the algorithm of [EffSeq] 在线 softmax in the page's notation, built
here as a fold: every block's own state is merged into the running one.  The
page's description:

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


def block_state(scores, values):
    """State (m, l, u) of one block of keys taken on its own.

    m is the largest visible score of the block, l = sum_j e^{s_j - m} and
    u = sum_j e^{s_j - m} v_j over its visible keys; a block whose keys are all
    masked is the empty state (-inf, 0, 0), so it leaves any state it is merged
    into unchanged ([EffSeq] 在线 softmax: fully masked blocks are skipped).
    """
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    live = np.isfinite(s)
    if not live.any():
        return _empty_state(v.shape[1])
    m = float(np.max(s[live]))
    w = np.exp(s[live] - m)
    return (m, float(np.sum(w)), w @ v[live])


def online_states(scores, values, block: int):
    """Yield the running state (m, l, u) after each block of ``block`` keys.

    scores: (T,) scaled and masked scores (masked entries are -inf).
    values: (T, d) value vectors.
    The running state starts empty and takes each block's own state through
    ``merge_states``: both move to the common base m' = max(m, m_hat), which is
    the page's update l' = e^{m - m'} l + sum_I e^{s_j - m'} (and the same for u),
    since sum_I e^{s_j - m'} = e^{m_hat - m'} sum_I e^{s_j - m_hat}.
    """
    s_all = np.asarray(scores, dtype=np.float64)
    v_all = np.asarray(values, dtype=np.float64)
    if s_all.ndim != 1 or v_all.ndim != 2 or v_all.shape[0] != s_all.shape[0]:
        raise ValueError("expected scores of shape (T,) and values of shape (T, d)")
    if block < 1:
        raise ValueError("the block length is at least one key")
    if np.any(np.isnan(s_all) | (s_all == np.inf)):
        raise ValueError("a score is NaN or +inf; masked keys carry -inf")
    if not np.all(np.isfinite(v_all)):
        raise ValueError("a value vector holds NaN or inf")
    state = _empty_state(v_all.shape[1])
    for start in range(0, s_all.shape[0], block):
        state = merge_states(state, block_state(s_all[start:start + block], v_all[start:start + block]))
        yield (state[0], state[1], np.array(state[2], dtype=np.float64))


def finish_state(state) -> np.ndarray:
    """o = u / l; a state built from no visible key has no output."""
    m, l, u = state
    if l == 0.0:
        raise ValueError("no key is visible to this query row, so its output is undefined")
    return u / l


def online_attention_row(scores, values, block: int = 2) -> np.ndarray:
    """Output of one query row computed block by block with the online state."""
    state = None
    for state in online_states(scores, values, block):
        pass
    if state is None:
        raise ValueError("no key is visible to this query row, so its output is undefined")
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
