"""Plant plausible mistakes in the oracle (CPU only) and check that the pins catch each one.

Every mutant replaces one helper of ``oracle.sdpa`` or ``oracle.online``; the
suite of pin checks below (worked values from the pages, closed forms, brute
force) must fail for each of them.  This is what makes the oracle trustworthy:
its pins are sensitive to a dropped term, a wrong sign or index, or a swapped
operand.
"""

import importlib
import json
import math
import os

import numpy as np
import pytest

import oracle

sdpa = importlib.import_module("oracle.sdpa")
online = importlib.import_module("oracle.online")


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _brute(q, k, v, scale):
    B, h_q, S, d = q.shape
    r = h_q // k.shape[1]
    out = np.zeros(q.shape)
    for b in range(B):
        for a in range(h_q):
            for i in range(S):
                sc = [sum(q[b, a, i, t] * k[b, a // r, j, t] for t in range(d)) * scale for j in range(i + 1)]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                for t in range(d):
                    out[b, a, i, t] = sum(w[j] * v[b, a // r, j, t] for j in range(i + 1)) / sum(w)
    return out


def pins_hold(golden_dir) -> bool:
    """True iff every pin holds.  Exceptions count as failures."""
    try:
        g = _golden(golden_dir, "worked_two_keys_d1.json")
        q = np.array(g["queries"]).reshape(1, 2, 1, 1)
        k = np.array(g["keys"]).reshape(1, 1, 2, 1)
        v = np.array(g["values"]).reshape(1, 1, 2, 1)
        o = oracle.attention(q, k, v, causal=True, q_pos=np.array([[1]]), kv_len=np.array([2]))
        if abs(o[0, 0, 0, 0] - 15.0) > 5e-7 or abs(o[0, 1, 0, 0] - 17.310586) > 5e-7:
            return False
        gm = _golden(golden_dir, "group_maps.json")
        for c in gm["cases"]:
            m = oracle.group_index(c["h_q"], c["h_kv"])
            if "map" in c and m != c["map"]:
                return False
            if "head" in c and m[c["head"]] != c["kv_head"]:
                return False
        rng = np.random.default_rng(1949)
        q, k, v = rng.standard_normal((1, 4, 3, 2)), rng.standard_normal((1, 2, 3, 2)), rng.standard_normal((1, 2, 3, 2))
        if np.max(np.abs(oracle.attention(q, k, v) - _brute(q, k, v, 1 / math.sqrt(2)))) > 1e-12:
            return False
        # padding: lengths cut the history
        qd = rng.standard_normal((2, 2, 1, 2))
        kd, vd = rng.standard_normal((2, 1, 5, 2)), rng.standard_normal((2, 1, 5, 2))
        od = oracle.attention(qd, kd, vd, causal=True, kv_len=np.array([5, 2]))
        ot = oracle.attention(qd[1:], kd[1:, :, :2], vd[1:, :, :2], causal=True)
        if np.max(np.abs(od[1] - ot[0])) > 1e-13:
            return False
        # a decode query at the default position equals the last causal prefill row
        qp, kp, vp = rng.standard_normal((1, 2, 4, 2)), rng.standard_normal((1, 1, 4, 2)), rng.standard_normal((1, 1, 4, 2))
        if np.max(np.abs(oracle.attention(qp[:, :, 3:], kp, vp)[:, :, 0] - oracle.attention(qp, kp, vp)[:, :, 3])) > 1e-13:
            return False
        tb = _golden(golden_dir, "two_block_example.json")
        st = list(oracle.online_states(np.log([1.0, 2.0, 3.0, 4.0]), np.array(tb["values"])[:, None], 2))
        if abs(st[0][1] - 1.5) > 1e-14 or abs(st[1][2][0] - 7.5) > 1e-14:
            return False
        s1, s2 = st[0], list(oracle.online_states(np.log([3.0, 4.0]), np.array([[3.0], [4.0]]), 2))[-1]
        if abs(oracle.finish_state(oracle.merge_states(s1, s2))[0] - 3.0) > 1e-14:
            return False
        return True
    except Exception:
        return False


def test_unmutated_oracle_passes_pins(golden_dir):
    assert pins_hold(golden_dir)


MUTANTS = {
    "abab_group_map": (sdpa, "group_index", lambda h_q, h_kv: [a % h_kv for a in range(h_q)]),
    "scale_one_over_d": (sdpa, "default_scale", lambda d: 1.0 / d),
    "no_scale": (sdpa, "default_scale", lambda d: 1.0),
    "causal_excludes_diagonal": (sdpa, "visibility",
                                 lambda qp, L, T, c: (np.arange(T)[None] < L) & ((np.arange(T)[None] < qp[:, None]) | (not c))),
    "causal_off_by_one_later": (sdpa, "visibility",
                                lambda qp, L, T, c: np.broadcast_to((np.arange(T)[None] < L) & ((np.arange(T)[None] <= qp[:, None] + 1) | (not c)), (qp.shape[0], T)).copy()),
    "zero_based_decode_position": (sdpa, "default_q_pos",
                                   lambda B, S_q, T_k, kv_len: np.tile(np.arange(S_q), (B, 1))),
    "softmax_over_queries": (sdpa, "softmax_rows",
                             lambda S: np.exp(S - S.max(0, keepdims=True)) / np.exp(S - S.max(0, keepdims=True)).sum(0, keepdims=True)),
    "softmax_missing_normalization": (sdpa, "softmax_rows", lambda S: np.exp(S - S.max(1, keepdims=True))),
    "merge_drops_rescale": (online, "merge_states",
                            lambda a, b: (max(a[0], b[0]), a[1] + b[1], np.asarray(a[2]) + np.asarray(b[2]))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch, golden_dir):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    if mod is online and attr == "merge_states":
        monkeypatch.setattr(oracle, "merge_states", fn)
    if mod is sdpa and attr == "group_index":
        monkeypatch.setattr(oracle, "group_index", fn)
    assert not pins_hold(golden_dir), f"mutant {name} slipped past every pin"


def test_online_mutant_without_carry_is_caught(monkeypatch, golden_dir):
    # an online update that forgets e^{m - m'} on the old sums
    def bad_states(scores, values, block):
        s_all, v_all = np.asarray(scores, float), np.asarray(values, float)
        m, l, u = -np.inf, 0.0, np.zeros(v_all.shape[1])
        for st in range(0, len(s_all), block):
            s, v = s_all[st:st + block], v_all[st:st + block]
            m2 = max(m, s.max())
            w = np.exp(s - m2)
            l, u, m = l + w.sum(), u + w @ v, m2
            yield (m, l, u.copy())
    monkeypatch.setattr(oracle, "online_states", bad_states)
    assert not pins_hold(golden_dir)
