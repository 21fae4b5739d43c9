"""The oracle against brute force, a library routine, special cases and invariants."""

import math

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- brute force on the tiny workload
def _brute(q, k, v, scale, causal):
    """Scalar Python loops with math.exp: no numpy matmul, no vectorized softmax."""
    B, h_q, S, d = q.shape
    h_kv, T = k.shape[1], k.shape[2]
    r = h_q // h_kv
    out = np.zeros(q.shape)
    for b in range(B):
        for a in range(h_q):
            kv = a // r
            for i in range(S):
                sc = []
                for j in range(T):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for t in range(d):
                        dot += float(q[b, a, i, t]) * float(k[b, kv, j, t])
                    sc.append((j, dot * scale))
                mx = max(s for _, s in sc)
                den = sum(math.exp(s - mx) for _, s in sc)
                for t in range(d):
                    out[b, a, i, t] = sum(math.exp(s - mx) * float(v[b, kv, j, t]) for j, s in sc) / den
    return out


def test_brute_force_tiny_prefill_workload():
    w = inputs.WORKLOADS["tiny_prefill_f32"]
    x = inputs.make_workload(w)
    assert x["q"].shape == (1, 4, 3, 2) and x["k"].shape == (1, 2, 3, 2)
    scale = 1 / math.sqrt(2)
    want = _brute(x["q"], x["k"], x["v"], scale, True)
    got = oracle.attention(x["q"], x["k"], x["v"], causal=True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("h_q,h_kv", [(4, 4), (4, 2), (6, 3), (4, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_random_small(h_q, h_kv, causal):
    rng = np.random.default_rng(h_q * 10 + h_kv)
    q, k, v = _rand(rng, 2, h_q, 5, 3), _rand(rng, 2, h_kv, 5, 3), _rand(rng, 2, h_kv, 5, 3)
    want = _brute(q, k, v, 0.7, causal)
    got = oracle.attention(q, k, v, scale=0.7, causal=causal)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- the group map is checked, not just shapes
def test_gqa_equals_mha_on_expanded_kv_exactly():
    rng = np.random.default_rng(1949)
    h_q, h_kv = 8, 2
    q, k, v = _rand(rng, 2, h_q, 7, 4), _rand(rng, 2, h_kv, 7, 4), _rand(rng, 2, h_kv, 7, 4)
    r = h_q // h_kv
    got = oracle.attention(q, k, v)
    mha = oracle.attention(q, np.repeat(k, r, axis=1), np.repeat(v, r, axis=1))
    assert np.array_equal(got, mha)                  # same arithmetic, error exactly 0


def test_wrong_abab_map_is_detected():
    # tiling the K/V heads (A,B,A,B) instead of repeating them (A,A,B,B) keeps every
    # shape and must still change the result
    rng = np.random.default_rng(1949)
    h_q, h_kv = 4, 2
    q, k, v = _rand(rng, 1, h_q, 6, 4), _rand(rng, 1, h_kv, 6, 4), _rand(rng, 1, h_kv, 6, 4)
    good = oracle.attention(q, k, v)
    wrong = oracle.attention(q, np.tile(k, (1, 2, 1, 1)), np.tile(v, (1, 2, 1, 1)))
    assert wrong.shape == good.shape
    assert np.max(np.abs(wrong - good)) > 1e-3


def test_mha_special_case_per_head_loop():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 1, 3, 4, 2), _rand(rng, 1, 3, 4, 2), _rand(rng, 1, 3, 4, 2)
    got = oracle.attention(q, k, v)
    for a in range(3):
        one = oracle.attention(q[:, a:a + 1], k[:, a:a + 1], v[:, a:a + 1])
        np.testing.assert_array_equal(got[:, a:a + 1], one)


def test_mqa_special_case_every_head_reads_kv0():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 4, 4, 2), _rand(rng, 1, 1, 4, 2), _rand(rng, 1, 1, 4, 2)
    got = oracle.attention(q, k, v)
    for a in range(4):
        np.testing.assert_array_equal(got[:, a:a + 1], oracle.attention(q[:, a:a + 1], k, v))


# ---------------------------------------------------------------- a library routine as an independent check
def test_against_torch_sdpa_prefill_and_decode():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    rng = np.random.default_rng(5)
    B, h_q, h_kv, T, d = 2, 8, 2, 33, 16
    q, k, v = _rand(rng, B, h_q, T, d), _rand(rng, B, h_kv, T, d), _rand(rng, B, h_kv, T, d)
    r = h_q // h_kv
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk.repeat_interleave(r, 1), tv.repeat_interleave(r, 1),
                                         is_causal=True).numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v, causal=True), ref, atol=1e-12)
    # decode: one query at absolute position p, explicit boolean mask (not is_causal)
    p = 20
    qd = q[:, :, p:p + 1]
    mask = torch.zeros(1, T, dtype=torch.bool)
    mask[0, : p + 1] = True
    refd = F.scaled_dot_product_attention(torch.from_numpy(qd), tk.repeat_interleave(r, 1),
                                          tv.repeat_interleave(r, 1), attn_mask=mask).numpy()
    got = oracle.attention(qd, k, v, causal=True, q_pos=np.full((B, 1), p), kv_len=np.full(B, T))
    np.testing.assert_allclose(got, refd, atol=1e-12)


# ---------------------------------------------------------------- decode positions
def test_decode_at_last_position_equals_last_prefill_row():
    rng = np.random.default_rng(21)
    B, h_q, h_kv, T, d = 2, 4, 2, 9, 3
    q, k, v = _rand(rng, B, h_q, T, d), _rand(rng, B, h_kv, T, d), _rand(rng, B, h_kv, T, d)
    pre = oracle.attention(q, k, v, causal=True)
    dec = oracle.attention(q[:, :, T - 1:], k, v, causal=True)     # default q_pos = kv_len - 1
    np.testing.assert_allclose(dec[:, :, 0], pre[:, :, T - 1], atol=1e-14)
    # and at an interior position with the history cut at that position
    p = 4
    dec2 = oracle.attention(q[:, :, p:p + 1], k, v, causal=True, q_pos=np.full((B, 1), p))
    np.testing.assert_allclose(dec2[:, :, 0], pre[:, :, p], atol=1e-14)


def test_zero_based_triangular_template_is_wrong_for_decode():
    # a 1 x T causal template built as if the query were at position 0 shows only key 0
    rng = np.random.default_rng(22)
    T = 8
    q, k, v = _rand(rng, 1, 2, 1, 3), _rand(rng, 1, 1, T, 3), _rand(rng, 1, 1, T, 3)
    right = oracle.attention(q, k, v, causal=True, q_pos=np.array([[T - 1]]))
    zero_based = oracle.attention(q, k, v, causal=True, q_pos=np.array([[0]]))
    np.testing.assert_allclose(zero_based[0, :, 0], np.broadcast_to(v[0, 0, 0], (2, 3)), atol=1e-14)
    assert np.max(np.abs(right - zero_based)) > 1e-3


# ---------------------------------------------------------------- invariants
def test_output_in_convex_hull_of_visible_values():
    rng = np.random.default_rng(31)
    B, h_q, h_kv, T, d = 1, 4, 2, 12, 5
    q, k, v = _rand(rng, B, h_q, T, d) * 3, _rand(rng, B, h_kv, T, d), _rand(rng, B, h_kv, T, d)
    o = oracle.attention(q, k, v, causal=True)
    g = oracle.group_index(h_q, h_kv)
    for a in range(h_q):
        for i in range(T):
            vis = v[0, g[a], : i + 1]
            assert np.all(o[0, a, i] >= vis.min(axis=0) - 1e-12)
            assert np.all(o[0, a, i] <= vis.max(axis=0) + 1e-12)


def test_causal_prefix_independence():
    rng = np.random.default_rng(32)
    B, h_q, h_kv, T, d = 1, 4, 2, 10, 3
    q, k, v = _rand(rng, B, h_q, T, d), _rand(rng, B, h_kv, T, d), _rand(rng, B, h_kv, T, d)
    o = oracle.attention(q, k, v, causal=True)
    i = 5
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = _rand(rng, B, h_kv, T - i - 1, d)
    v2[:, :, i + 1:] = _rand(rng, B, h_kv, T - i - 1, d)
    o2 = oracle.attention(q, k2, v2, causal=True)
    np.testing.assert_array_equal(o[:, :, : i + 1], o2[:, :, : i + 1])
    assert np.max(np.abs(o[:, :, i + 1:] - o2[:, :, i + 1:])) > 1e-6


def test_causal_row0_is_first_value_exactly():
    rng = np.random.default_rng(33)
    q, k, v = _rand(rng, 2, 6, 5, 4), _rand(rng, 2, 3, 5, 4), _rand(rng, 2, 3, 5, 4)
    o = oracle.attention(q, k, v, causal=True)
    g = oracle.group_index(6, 3)
    for b in range(2):
        for a in range(6):
            np.testing.assert_array_equal(o[b, a, 0], v[b, g[a], 0])


def test_unmasked_joint_key_permutation_invariance():
    rng = np.random.default_rng(34)
    q, k, v = _rand(rng, 1, 4, 6, 3), _rand(rng, 1, 2, 6, 3), _rand(rng, 1, 2, 6, 3)
    perm = rng.permutation(6)
    a = oracle.attention(q, k, v, causal=False)
    b = oracle.attention(q, k[:, :, perm], v[:, :, perm], causal=False)
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_equal_scores_give_mean_of_visible_values():
    rng = np.random.default_rng(35)
    T, d = 7, 3
    q = np.zeros((1, 2, T, d))
    k, v = _rand(rng, 1, 1, T, d), _rand(rng, 1, 1, T, d)
    o = oracle.attention(q, k, v, causal=True)
    for i in range(T):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, : i + 1].mean(axis=0), atol=1e-14)


def test_padding_mask_equals_truncated_keys():
    rng = np.random.default_rng(36)
    B, h_q, h_kv, T, d = 3, 4, 2, 9, 3
    q, k, v = _rand(rng, B, h_q, 1, d), _rand(rng, B, h_kv, T, d), _rand(rng, B, h_kv, T, d)
    lens = np.array([9, 4, 1])
    o = oracle.attention(q, k, v, causal=False, q_pos=np.zeros((B, 1)), kv_len=lens)
    for b in range(B):
        t = oracle.attention(q[b:b + 1], k[b:b + 1, :, : lens[b]], v[b:b + 1, :, : lens[b]], causal=False)
        np.testing.assert_allclose(o[b], t[0], atol=1e-14)


def test_scale_enters_as_multiplier():
    # scale c on Q K^T equals unscaled attention of c * q (a closed form, not the oracle's code)
    rng = np.random.default_rng(37)
    q, k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 4, 3)
    np.testing.assert_allclose(oracle.attention(q, k, v, scale=0.3),
                               oracle.attention(0.3 * q, k, v, scale=1.0), atol=1e-13)
    np.testing.assert_allclose(oracle.attention(q, k, v),
                               oracle.attention(q / math.sqrt(3), k, v, scale=1.0), atol=1e-13)


def test_rejects_non_finite_inputs():
    q = np.ones((1, 1, 2, 2))
    k = np.ones((1, 1, 2, 2))
    k[0, 0, 1, 0] = np.nan
    with pytest.raises(ValueError):
        oracle.attention(q, k, np.ones((1, 1, 2, 2)))
