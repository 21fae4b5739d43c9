"""Rotary position encoding of query and key rows, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:
  [EffSeq] 分组查询注意力: with shared K/V the position encoding still acts on
      the query and key that are compared; under rotary encoding every query
      head and every key head that is actually stored is rotated by its
      position (so a group's single K head is rotated once, not r times);
  [MhaMqaGqa] note under the parameter table: Q and K may be position-encoded
      first; the attention formulas then use the processed Q and K;
  [Ch09] 09.4: a cache shared between consumers is read-only to them -- rotating
      or changing a stored key in place would change what the other readers see.

What they leave open, and the reading taken here (listed again in the design doc):
  the rotation itself.  The pages give no formula, so the common rotary form is
  used: a head vector x of even width d is split into halves, element i paired
  with element i + d/2, and the pair at position p is rotated by the angle
  p * theta_i with theta_i = base ** (-2 i / d), base 10000 unless given:

      y[i]       = x[i] cos(p theta_i) - x[i + d/2] sin(p theta_i)
      y[i + d/2] = x[i + d/2] cos(p theta_i) + x[i] sin(p theta_i)

  i.e. pair i, read as the complex number x[i] + 1j * x[i + d/2], is multiplied
  by exp(1j * p * theta_i).  Positions are the same absolute positions the
  attention mask uses.
"""

from __future__ import annotations

import numpy as np


def inv_freq(d: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base ** (-2 i / d) for i = 0 .. d/2 - 1 (float64)."""
    if d < 2 or d % 2:
        raise ValueError("rotary encoding needs an even head width")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def rope(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of x (..., S, d) by the positions (..., S) (broadcast).

    Returns a new float64 array; x is not modified.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    theta = inv_freq(d, base)
    pos = np.asarray(positions, dtype=np.float64)[..., None]          # (..., S, 1)
    ang = pos * theta                                                 # (..., S, d/2)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
