"""Pins of the rotary position encoding in the oracle (oracle/rope.py).

The pages require the rotation of every query head and stored key head by
position ([EffSeq] 分组查询注意力) but print no formula; the rotation is the
stated reading (half-split pairs, theta_i = base^(-2i/d)).  These tests pin
that reading by a hand-worked d = 4 case and by properties every rotation
by position has, chosen so that a swapped pairing, a wrong sign or a wrong
frequency exponent fails at least one of them.
"""

import json
import os
import math

import numpy as np
import pytest

import oracle
import importlib

rope_mod = importlib.import_module("oracle.rope")


def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"cos": math.cos, "sin": math.sin}))


def test_worked_d4(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "rope_d4_worked.json")))
    x = np.array(fx["x"])
    for case in fx["cases"]:
        got = oracle.rope(x[None, :], np.array([case["position"]]), base=fx["base"])[0]
        want = np.array([_eval(e) for e in case["expected"]])
        assert np.allclose(got, want, rtol=0, atol=1e-12), (case["position"], got, want)


def test_inv_freq_closed_form():
    th = oracle.inv_freq(128)
    assert th[0] == 1.0
    assert math.isclose(th[32], 10000.0 ** -0.5, rel_tol=1e-15)          # i = d/4 -> base^(-1/2)
    assert math.isclose(th[-1], 10000.0 ** (-126 / 128), rel_tol=1e-15)
    with pytest.raises(ValueError):
        oracle.inv_freq(7)


def test_d2_is_complex_rotation():
    # d = 2: theta_0 = 1, so (x0 + i x1) * exp(i p)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 2))
    p = rng.integers(0, 5000, 10)
    got = oracle.rope(x, p)
    z = (x[:, 0] + 1j * x[:, 1]) * np.exp(1j * p)
    assert np.allclose(got[:, 0], z.real, atol=1e-9) and np.allclose(got[:, 1], z.imag, atol=1e-9)


def test_position_zero_identity_and_pair_norms():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 7, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(7)), x)
    y = oracle.rope(x, rng.integers(0, 32768, 7))
    nx = x[..., :32] ** 2 + x[..., 32:] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12)           # each pair keeps its length


def test_composition_and_inverse():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 128))
    a, b = rng.integers(0, 10000, 5), rng.integers(0, 10000, 5)
    assert np.allclose(oracle.rope(oracle.rope(x, a), b), oracle.rope(x, a + b), atol=1e-9)
    assert np.allclose(oracle.rope(oracle.rope(x, a), -a), x, atol=1e-9)


def test_scores_depend_on_relative_position_only():
    # <R_p q, R_s k> = <R_(p-s) q, k>: the property that makes the rotation a
    # relative position encoding inside the attention score
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for p, s in [(0, 0), (5, 3), (4096, 4000), (31999, 17)]:
        lhs = oracle.rope(q[None], np.array([p]))[0] @ oracle.rope(k[None], np.array([s]))[0]
        rhs = oracle.rope(q[None], np.array([p - s]))[0] @ k
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_then_attention_is_attention_of_rotated_rows():
    # [MhaMqaGqa]: the attention formula uses the position-processed Q and K.  With
    # K rotated once per stored head, every query head of a group sees the same keys.
    rng = np.random.default_rng(9)
    B, h_q, h_kv, T, d = 1, 4, 2, 6, 8
    q = rng.standard_normal((B, h_q, T, d))
    k = rng.standard_normal((B, h_kv, T, d))
    v = rng.standard_normal((B, h_kv, T, d))
    pos = np.arange(T)
    qr, kr = oracle.rope(q, pos), oracle.rope(k, pos)
    o = oracle.attention(qr, kr, v, causal=True)
    # expanded form: repeat the rotated K per query head; identical
    o2 = oracle.attention(qr, np.repeat(kr, 2, axis=1), np.repeat(v, 2, axis=1), causal=True)
    assert np.array_equal(o, o2)
    # a shift of all positions by the same amount leaves the causal output unchanged
    o3 = oracle.attention(oracle.rope(q, pos + 1000), oracle.rope(k, pos + 1000), v, causal=True)
    assert np.allclose(o, o3, atol=1e-9)


def _interleaved(x, positions, base=10000.0):
    # mutant: pairs (2i, 2i + 1) instead of (i, i + d/2)
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    th = rope_mod.inv_freq(d, base)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * th
    e, o = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = e * np.cos(ang) - o * np.sin(ang)
    y[..., 1::2] = o * np.cos(ang) + e * np.sin(ang)
    return y


@pytest.mark.parametrize("mutant", ["interleaved", "sign", "exponent"])
def test_mutants_fail_the_worked_case(golden_dir, mutant, monkeypatch):
    fx = json.load(open(os.path.join(golden_dir, "rope_d4_worked.json")))
    x = np.array(fx["x"])
    if mutant == "interleaved":
        f = _interleaved
    elif mutant == "sign":
        f = lambda xx, pp, base=10000.0: oracle.rope(xx, -np.asarray(pp), base)
    else:
        monkeypatch.setattr(rope_mod, "inv_freq",
                            lambda d, base=10000.0: np.power(float(base), -np.arange(d // 2) / d))
        f = rope_mod.rope
    bad = 0
    for case in fx["cases"]:
        got = f(x[None, :], np.array([case["position"]]), base=fx["base"])[0]
        want = np.array([_eval(e) for e in case["expected"]])
        bad += not np.allclose(got, want, rtol=0, atol=1e-12)
    assert bad > 0
