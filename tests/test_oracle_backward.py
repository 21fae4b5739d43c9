"""Pins of the attention gradients in the oracle (oracle/backward.py).

The gradient formulas are pinned against things other than themselves:
central finite differences of the (already pinned) forward oracle, torch's
autograd on a float64 CPU attention written with repeat_interleave'd K/V,
closed-form special cases and invariants of the softmax Jacobian.  Planted
mistakes in the oracle (a dropped term, an unsummed group, a missing scale,
a transposed product) must each fail one of them.
"""


import numpy as np
import pytest

import oracle



def _inputs(seed, B=1, h_q=4, h_kv=2, T=5, d=3, S_q=None):
    rng = np.random.default_rng(seed)
    S_q = T if S_q is None else S_q
    return (rng.standard_normal((B, h_q, S_q, d)), rng.standard_normal((B, h_kv, T, d)),
            rng.standard_normal((B, h_kv, T, d)), rng.standard_normal((B, h_q, S_q, d)))


def _finite_diff(q, k, v, do, eps=1e-6, **kw):
    def loss(qq, kk, vv):
        return float(np.sum(do * oracle.attention(qq, kk, vv, **kw)))
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("kw", [{"causal": True}, {"causal": False}, {"causal": True, "kv_len": np.array([4])},
                                {"causal": True, "scale": 0.7}])
def test_matches_finite_differences(kw):
    q, k, v, do = _inputs(1)
    got = oracle.attention_backward(q, k, v, do, **kw)
    want = _finite_diff(q, k, v, do, **kw)
    for g, w in zip(got, want):
        assert np.allclose(g, w, rtol=0, atol=1e-7), np.max(np.abs(g - w))


def test_decode_shape_finite_differences():
    # one query per sequence at its absolute position against a longer cache
    q, k, v, do = _inputs(2, B=2, h_q=2, h_kv=1, T=6, d=2, S_q=1)
    kw = {"causal": True, "q_pos": np.array([[5], [3]]), "kv_len": np.array([6, 4])}
    got = oracle.attention_backward(q, k, v, do, **kw)
    want = _finite_diff(q, k, v, do, **kw)
    for g, w in zip(got, want):
        assert np.allclose(g, w, rtol=0, atol=1e-7)


def test_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    q, k, v, do = _inputs(3, B=2, h_q=8, h_kv=2, T=33, d=16)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    r = 4
    ke, ve = tk.repeat_interleave(r, dim=1), tv.repeat_interleave(r, dim=1)
    s = (tq @ ke.transpose(-1, -2)) / np.sqrt(16)
    mask = torch.ones(33, 33, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ ve
    gq, gk, gv = torch.autograd.grad(o, (tq, tk, tv), grad_outputs=torch.tensor(do))
    got = oracle.attention_backward(q, k, v, do, causal=True)
    for g, w in zip(got, (gq, gk, gv)):
        assert np.allclose(g, w.numpy(), rtol=0, atol=1e-12)


def test_invariants():
    q, k, v, do = _inputs(4, B=1, h_q=4, h_kv=1, T=9, d=5)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=True)
    # rows of dS sum to zero, so the key gradients of a head sum to zero
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # causal row 0 sees one key with weight 1: no query gradient there
    assert np.allclose(dq[:, :, 0], 0.0, atol=1e-15)
    # the last key is seen only by the last query (weight p): dV = sum over heads of p * dO
    def p_last_of(a):
        s = q[0, a, -1] @ k[0, 0].T / np.sqrt(5)
        e = np.exp(s - s.max())
        return e[-1] / e.sum()
    p_last = np.array([p_last_of(a) for a in range(4)])
    assert np.allclose(dv[0, 0, -1], (p_last[:, None] * do[0, :, -1]).sum(axis=0), atol=1e-12)
    # all keys equal: scores are constant per row, softmax is flat, dS = 0 -> dQ = 0
    k_eq = np.repeat(k[:, :, :1], 9, axis=2)
    dq2, _, _ = oracle.attention_backward(q, k_eq, v, do, causal=True)
    assert np.allclose(dq2, 0.0, atol=1e-12)


def test_logsumexp():
    from scipy.special import logsumexp

    q, k, _, _ = _inputs(5, B=1, h_q=4, h_kv=2, T=7, d=4)
    L = oracle.row_logsumexp(q, k, causal=True)
    for a in range(4):
        s = q[0, a] @ k[0, a // 2].T / 2.0
        for i in range(7):
            assert np.isclose(L[0, a, i], logsumexp(s[i, : i + 1]), rtol=0, atol=1e-12)
    # P recomputed from L is the forward's softmax
    s = q[0, 1] @ k[0, 0].T / 2.0
    p = np.where(np.tril(np.ones((7, 7), bool)), np.exp(s - L[0, 1][:, None]), 0.0)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)


# ---------------------------------------------------------------------------- mutants
def _mutant_backward(kind):
    def f(q, k, v, d_out, *, scale=None, causal=True, q_pos=None, kv_len=None):
        q, k, v, d_out = (np.asarray(a, np.float64) for a in (q, k, v, d_out))
        B, h_q, S_q, d_h = q.shape
        h_kv, T_k = k.shape[1], k.shape[2]
        g = oracle.group_index(h_q, h_kv)
        scale = oracle.default_scale(d_h) if scale is None else scale
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            vis = oracle.visibility(np.arange(S_q), T_k, T_k, causal)
            for a in range(h_q):
                s = np.where(vis, (q[b, a] @ k[b, g[a]].T) * scale, -np.inf)
                p = oracle.softmax_rows(s)
                do = d_out[b, a]
                dp = do @ v[b, g[a]].T
                if kind == "no_rowsum":
                    ds = p * dp
                else:
                    ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
                sc = 1.0 if kind == "no_scale" else scale
                dq[b, a] = sc * (ds @ k[b, g[a]])
                if kind == "first_head_only" and a % (h_q // h_kv) != 0:
                    continue
                dv[b, g[a]] += p.T @ do
                dk[b, g[a]] += sc * ((ds @ q[b, a]) if kind == "transposed" else (ds.T @ q[b, a]))
        return dq, dk, dv
    return f


@pytest.mark.parametrize("kind", ["no_rowsum", "no_scale", "first_head_only", "transposed"])
def test_mutants_fail_finite_differences(kind):
    q, k, v, do = _inputs(6)
    got = _mutant_backward(kind)(q, k, v, do, causal=True)
    want = _finite_diff(q, k, v, do, causal=True)
    assert any(not np.allclose(g, w, rtol=0, atol=1e-7) for g, w in zip(got, want))
    # and the unmutated rewrite passes, so the harness itself is sound
    ok = _mutant_backward("none")(q, k, v, do, causal=True)
    assert all(np.allclose(g, w, rtol=0, atol=1e-7) for g, w in zip(ok, want))
