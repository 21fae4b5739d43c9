"""Pins of the CPU oracle against values the pages print and closed forms.

Each test names the passage it checks.  None of them re-types the oracle's
own formula: the expected values come from the pages (tests/golden/*.json)
or from closed forms worked out by hand.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import sdpa


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- [EffSeq] 头与投影, d_h = 1 worked case
def test_two_keys_d1_as_two_query_rows(golden_dir):
    g = _load(golden_dir, "worked_two_keys_d1.json")
    q = np.array(g["queries"], dtype=np.float64).reshape(1, 1, 2, 1)
    k = np.array(g["keys"], dtype=np.float64).reshape(1, 1, 2, 1)
    v = np.array(g["values"], dtype=np.float64).reshape(1, 1, 2, 1)
    # both queries read both cached keys: no causal mask; scale = 1/sqrt(1) = 1
    o = oracle.attention(q, k, v, causal=False)
    tol = 0.5 * 10 ** -g["printed_decimals"]
    assert o[0, 0, 0, 0] == pytest.approx(g["printed"]["query_0"]["output"], abs=tol)
    assert o[0, 0, 1, 0] == pytest.approx(g["printed"]["query_1"]["output"], abs=tol)
    # closed form of the second output: (10 + 20 e) / (1 + e)
    assert o[0, 0, 1, 0] == pytest.approx((10 + 20 * math.e) / (1 + math.e), abs=1e-13)


def test_two_keys_d1_as_two_mqa_heads_decode(golden_dir):
    g = _load(golden_dir, "worked_two_keys_d1.json")
    # two query heads sharing one K/V head (h_kv = 1): a decode step at position 1
    q = np.array(g["queries"], dtype=np.float64).reshape(1, 2, 1, 1)
    k = np.array(g["keys"], dtype=np.float64).reshape(1, 1, 2, 1)
    v = np.array(g["values"], dtype=np.float64).reshape(1, 1, 2, 1)
    o = oracle.attention(q, k, v, causal=True, q_pos=np.array([[1]]), kv_len=np.array([2]))
    tol = 0.5 * 10 ** -g["printed_decimals"]
    assert o[0, 0, 0, 0] == pytest.approx(15.0, abs=tol)
    assert o[0, 1, 0, 0] == pytest.approx(g["printed"]["query_1"]["output"], abs=tol)


def test_two_keys_d1_weights(golden_dir):
    g = _load(golden_dir, "worked_two_keys_d1.json")
    S = np.array([[0.0 * 1, 0.0 * 2], [1.0 * 1, 1.0 * 2]])   # query * key, scale 1
    P = sdpa.softmax_rows(S)
    tol = 0.5 * 10 ** -g["printed_decimals"]
    np.testing.assert_allclose(P[0], g["printed"]["query_0"]["weights"], atol=tol)
    np.testing.assert_allclose(P[1], g["printed"]["query_1"]["weights"], atol=tol)


# ---------------------------------------------------------------- [MhaMqaGqa] section 2, closed form
def test_same_kv_read_by_two_queries_closed_form():
    # scores [2, 0] and [0, 2] after scaling; one value channel [10, 20].  The page's
    # printed results were lost in extraction; the closed forms follow from softmax.
    q = np.array([[2.0, 0.0], [0.0, 2.0]]).reshape(1, 1, 2, 2)
    k = np.eye(2).reshape(1, 1, 2, 2)
    v = np.array([[10.0, 0.0], [20.0, 0.0]]).reshape(1, 1, 2, 2)
    o = oracle.attention(q, k, v, scale=1.0, causal=False)
    e2 = math.exp(2.0)
    assert o[0, 0, 0, 0] == pytest.approx((10 * e2 + 20) / (e2 + 1), abs=1e-12)
    assert o[0, 0, 1, 0] == pytest.approx((10 + 20 * e2) / (e2 + 1), abs=1e-12)
    assert o[0, 0, 0, 0] == pytest.approx(11.192029220221176, abs=1e-12)
    assert o[0, 0, 1, 0] == pytest.approx(18.807970779778827, abs=1e-12)


# ---------------------------------------------------------------- [EffSeq] 两块算例
def test_two_block_example_states(golden_dir):
    g = _load(golden_dir, "two_block_example.json")
    scores = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    values = np.array(g["values"])[:, None]
    states = list(oracle.online_states(scores, values, block=g["block"]))
    assert len(states) == 2
    m1, l1, u1 = states[0]
    assert m1 == pytest.approx(math.log(2), abs=1e-15)
    assert l1 == pytest.approx(g["after_block_1"]["l"], abs=1e-14)
    assert u1[0] == pytest.approx(g["after_block_1"]["u"], abs=1e-14)
    m2, l2, u2 = states[1]
    assert m2 == pytest.approx(math.log(4), abs=1e-15)
    assert l2 == pytest.approx(g["after_block_2"]["l"], abs=1e-14)
    assert u2[0] == pytest.approx(g["after_block_2"]["u"], abs=1e-14)
    assert oracle.finish_state(states[1])[0] == pytest.approx(g["after_block_2"]["output"], abs=1e-14)


def test_two_block_example_one_shot(golden_dir):
    g = _load(golden_dir, "two_block_example.json")
    # through the materialized attention: d_h = 1, q = 1, keys = log[1..4], scale 1
    q = np.ones((1, 1, 1, 1))
    k = np.log(np.array([1.0, 2.0, 3.0, 4.0])).reshape(1, 1, 4, 1)
    v = np.array(g["values"]).reshape(1, 1, 4, 1)
    o = oracle.attention(q, k, v, scale=1.0, causal=False)
    assert o[0, 0, 0, 0] == pytest.approx(g["one_shot"]["output"], abs=1e-14)
    w = sdpa.softmax_rows(np.log(np.array([[1.0, 2.0, 3.0, 4.0]])))
    np.testing.assert_allclose(w[0] * 10, g["one_shot"]["weights_times_10"], atol=1e-13)


def test_two_block_local_normalization_is_wrong(golden_dir):
    g = _load(golden_dir, "two_block_example.json")
    scores = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    values = np.array(g["values"])[:, None]
    o1 = oracle.online_attention_row(scores[:2], values[:2], block=2)[0]
    o2 = oracle.online_attention_row(scores[2:], values[2:], block=2)[0]
    assert o1 == pytest.approx(5 / 3, abs=1e-14)
    assert o2 == pytest.approx(25 / 7, abs=1e-14)
    tol = 0.5 * 10 ** -g["wrong_local_normalization"]["printed_decimals"]
    assert (o1 + o2) / 2 == pytest.approx(g["wrong_local_normalization"]["plain_average"], abs=tol)
    # and the merge of the two block states gives the right answer, 3
    s1 = list(oracle.online_states(scores[:2], values[:2], 2))[-1]
    s2 = list(oracle.online_states(scores[2:], values[2:], 2))[-1]
    assert oracle.finish_state(oracle.merge_states(s1, s2))[0] == pytest.approx(3.0, abs=1e-14)


# ---------------------------------------------------------------- group map
def test_group_maps(golden_dir):
    g = _load(golden_dir, "group_maps.json")
    for c in g["cases"]:
        m = oracle.group_index(c["h_q"], c["h_kv"])
        if "map" in c:
            assert m == c["map"], c["citation"]
        if "map_prefix" in c:
            assert m[: len(c["map_prefix"])] == c["map_prefix"], c["citation"]
        if "head" in c:
            assert m[c["head"]] == c["kv_head"], c["citation"]


def test_group_map_rejects_non_divisible():
    with pytest.raises(ValueError):
        oracle.group_index(12, 5)
    with pytest.raises(ValueError):
        oracle.group_index(4, 0)


def test_mha_and_mqa_maps():
    # [EffSeq] table: h_kv = h_q is MHA (identity map), h_kv = 1 is MQA (all read head 0)
    assert oracle.group_index(8, 8) == list(range(8))
    assert oracle.group_index(8, 1) == [0] * 8


def test_default_scale():
    assert oracle.default_scale(128) == pytest.approx(1 / math.sqrt(128), rel=1e-15)
    assert oracle.default_scale(1) == 1.0


# ---------------------------------------------------------------- the online algorithm equals the definition
@pytest.mark.parametrize("block", [1, 2, 3, 64, 200])
def test_online_equals_materialized(block):
    rng = np.random.default_rng(7)
    T, d = 200, 5
    for trial in range(5):
        s = rng.normal(size=T) * 3
        s[rng.random(T) < 0.3] = -np.inf
        s[rng.integers(T)] = 0.5                     # at least one visible key
        v = rng.normal(size=(T, d))
        got = oracle.online_attention_row(s, v, block)
        P = sdpa.softmax_rows(s[None, :])
        np.testing.assert_allclose(got, (P @ v)[0], rtol=0, atol=1e-12)


def test_online_all_masked_raises():
    with pytest.raises(ValueError):
        oracle.online_attention_row(np.full(6, -np.inf), np.ones((6, 2)), 2)
    with pytest.raises(ValueError):
        oracle.attention(np.ones((1, 1, 1, 2)), np.ones((1, 1, 3, 2)), np.ones((1, 1, 3, 2)),
                         kv_len=np.array([0]))


def test_online_skips_leading_masked_blocks_without_nan():
    s = np.array([-np.inf, -np.inf, 1.0, 2.0])
    v = np.array([[1.0], [2.0], [3.0], [4.0]])
    states = list(oracle.online_states(s, v, 2))
    assert np.isneginf(states[0][0]) and states[0][1] == 0.0
    out = oracle.finish_state(states[1])
    assert np.isfinite(out).all()
    assert out[0] == pytest.approx((3 + 4 * math.e) / (1 + math.e), abs=1e-14)


def test_merge_states_is_order_free_and_matches_whole():
    rng = np.random.default_rng(3)
    s = rng.normal(size=50) * 4
    v = rng.normal(size=(50, 3))
    parts = [list(oracle.online_states(s[i:i + 10], v[i:i + 10], 10))[-1] for i in range(0, 50, 10)]
    acc = (-np.inf, 0.0, np.zeros(3))
    for p in parts:
        acc = oracle.merge_states(acc, p)
    rev = (-np.inf, 0.0, np.zeros(3))
    for p in reversed(parts):
        rev = oracle.merge_states(p, rev)
    want = (sdpa.softmax_rows(s[None]) @ v)[0]
    np.testing.assert_allclose(oracle.finish_state(acc), want, atol=1e-12)
    np.testing.assert_allclose(oracle.finish_state(rev), want, atol=1e-12)
    # merging with an empty state is the identity
    e = oracle.merge_states(parts[0], (-np.inf, 0.0, np.zeros(3)))
    assert e[0] == parts[0][0] and e[1] == pytest.approx(parts[0][1], rel=1e-15)
