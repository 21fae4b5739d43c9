"""GPU parity of the training path: the forward's row log-sum-exp and the
gradients dQ, dK, dV against the float64 oracle (oracle/backward.py).

Parity bar for the gradients (bf16 inputs, fp32 accumulation and outputs): the
kernel rounds P and dS to bf16 before the products that use them (relative
error up to 2^-9 per term, independent between terms), and O and the row
statistics it recomputes P from are fp32.  A gradient element sum_j t_j then
carries an error of about 2^-9 / sqrt(3) * sqrt(sum_j t_j^2); over a whole tensor
that is below 2^-9 of its norm unless the sums cancel heavily.  The bar is
  relative Frobenius error <= 4 * 2^-9 (7.8e-3) per tensor,
  and every element within 2e-2 * max|g| of the oracle,
with the oracle computed from the same bf16 inputs in float64.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu

REL_FRO = 4 * 2.0 ** -9
MAX_REL = 2e-2


def _check_grad(got, want, what):
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    nrm = np.linalg.norm(want)
    err = got - want
    if nrm == 0.0:
        # exact answer 0 (a one-key row: dP - delta cancels); fp32 rounding of O(1) terms remains
        assert np.max(np.abs(got)) <= 1e-5, f"{what}: expected zeros, got {np.max(np.abs(got)):.3g}"
        return
    rel = np.linalg.norm(err) / nrm
    mx = np.max(np.abs(err)) / np.max(np.abs(want))
    print(f"{what}: rel_fro {rel:.2e} max/max {mx:.2e}", flush=True)
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3g}"
    assert mx <= MAX_REL, f"{what}: max error {mx:.3g} of max |g|"


def _run(B, h_q, h_kv, T, d, causal, seed, kv_lens=None, out_dtype="f32"):
    import torch

    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", seed)
    d_out = inputs.normal(seed, "d_out", (B, h_q, T, d), "bf16")
    q, k, v, do = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(d_out, "bf16")
    lens = None if kv_lens is None else ints_dev(kv_lens)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o, lse = ops.gqa_prefill_lse(q, k, v, causal=causal, kv_lens=lens, out_dtype=od)
    dq, dk, dv = ops.gqa_prefill_backward(q, k, v, o, do, lse, causal=causal, kv_lens=lens)
    torch.cuda.synchronize()
    return x, d_out, to_host64(lse), (to_host64(dq), to_host64(dk), to_host64(dv))


def _oracle(x, d_out, causal, kv_lens=None):
    return oracle.attention_backward(f64(x["q"], "bf16"), f64(x["k"], "bf16"), f64(x["v"], "bf16"),
                                     f64(d_out, "bf16"), causal=causal,
                                     kv_len=None if kv_lens is None else np.asarray(kv_lens))


BWD_CASES = [
    # B, h_q, h_kv, T, d, causal, kv_lens
    (1, 4, 2, 70, 64, True, None),
    (2, 8, 2, 200, 128, True, [200, 131]),
    (1, 8, 1, 97, 128, False, None),            # MQA, no mask
    (1, 4, 4, 33, 128, True, None),             # MHA
    (1, 2, 1, 1, 64, True, None),               # one row
    (1, 16, 2, 300, 128, True, None),           # r = 8, several key blocks and ragged tail
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B%d_hq%d_hkv%d_T%d_d%d_causal%d" % c[:6])
def test_backward_parity(case):
    B, h_q, h_kv, T, d, causal, lens = case
    print(f"case backward {case}", flush=True)
    x, d_out, _, got = _run(B, h_q, h_kv, T, d, causal, 14000 + T, kv_lens=lens)
    want = _oracle(x, d_out, causal, lens)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        _check_grad(g, w, f"{case} {name}")


def test_backward_from_bf16_output():
    # O in bf16 only enters delta = rowsum(dO * O); the bar still holds
    x, d_out, _, got = _run(1, 8, 2, 150, 128, True, 14500, out_dtype="bf16")
    want = _oracle(x, d_out, True)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        _check_grad(g, w, f"bf16 O {name}")


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 40)])
def test_lse_parity(dt, d):
    import torch

    B, h_q, h_kv, T = 2, 4, 2, 150
    x = inputs.make_prefill(B, h_q, h_kv, d, T, dt, 14600 + d)
    lens = np.array([150, 77], np.int32)
    _, lse = ops.gqa_prefill_lse(to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt), kv_lens=ints_dev(lens))
    torch.cuda.synchronize()
    want = oracle.row_logsumexp(f64(x["q"], dt), f64(x["k"], dt), causal=True, kv_len=lens)
    got = to_host64(lse)
    # fp32 sums of exponentials: relative 1e-6 of the sum, so ~1e-6 absolute in the log
    assert np.max(np.abs(got - want)) <= (1e-5 if dt == "f32" else 2e-5)


def test_backward_deterministic_and_key_gradients_sum_to_zero():
    _, _, _, a = _run(1, 8, 2, 257, 128, True, 14700)
    _, _, _, b = _run(1, 8, 2, 257, 128, True, 14700)
    for ga, gb in zip(a, b):
        assert np.array_equal(ga, gb)
    # rows of dS sum to zero, so the key gradients of each K/V head sum to zero
    dk = a[1]
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-3 * np.max(np.abs(dk)) * np.sqrt(dk.shape[2])


def test_backward_prefill_workload_sampled():
    """The causal prefill workload at full size: dQ rows and the gradients of the
    last keys (seen by few rows) against the oracle; the key-gradient sum at all keys."""
    import torch

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    print(f"case {w.name} backward", flush=True)
    x = inputs.make_workload(w)
    d_out = inputs.normal(w.seed, "d_out", (w.B, w.h_q, w.T, w.d_h), "bf16")
    q, k, v, do = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(d_out, "bf16")
    o, lse = ops.gqa_prefill_lse(q, k, v)
    dq, dk, dv = ops.gqa_prefill_backward(q, k, v, o, do, lse)
    torch.cuda.synchronize()
    dq, dk, dv = to_host64(dq), to_host64(dk), to_host64(dv)
    r = w.h_q // w.h_kv
    Q, K, V, DO = (f64(a, "bf16") for a in (x["q"], x["k"], x["v"], d_out))
    # dQ of sampled rows: the oracle on one query row at its position against its K/V head
    for a in (0, 5, 31):
        g = a // r
        for i in (0, 1, 63, 64, 2047, 4095):
            want = oracle.attention_backward(Q[:, a:a + 1, i:i + 1], K[:, g:g + 1, : i + 1], V[:, g:g + 1, : i + 1],
                                             DO[:, a:a + 1, i:i + 1], causal=True, q_pos=np.array([[i]]))[0]
            got = dq[0, a, i]
            # + 1e-4: row 0 has one key, so dP - delta cancels to fp32 rounding (exact answer 0)
            assert np.linalg.norm(got - want[0, 0, 0]) <= REL_FRO * np.linalg.norm(want) + 1e-4, (a, i)
    # dK, dV of the last 64 keys of two K/V heads: only rows >= T - 64 see them, so the oracle
    # on those rows of the group's r heads gives their whole gradient
    lo = w.T - 64
    for g in (0, 7):
        _, dkw, dvw = oracle.attention_backward(Q[:, g * r:(g + 1) * r, lo:], K[:, g:g + 1], V[:, g:g + 1],
                                                DO[:, g * r:(g + 1) * r, lo:], causal=True,
                                                q_pos=np.arange(lo, w.T)[None, :])
        _check_grad(dk[0, g, lo:], dkw[0, 0, lo:], f"full-size dK tail g={g}")
        _check_grad(dv[0, g, lo:], dvw[0, 0, lo:], f"full-size dV tail g={g}")
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-3 * np.max(np.abs(dk)) * np.sqrt(w.T)


@pytest.mark.parametrize("o_dtype", ["f32", "bf16"])
def test_backward_with_o_not_16_byte_aligned(o_dtype):
    """delta = rowsum(dO * O) reads O with 16-byte loads when O is 16-byte aligned and
    element by element otherwise; an O that starts one element into a buffer takes the
    second path and gives gradients within the same bar of the oracle."""
    import torch

    B, h_q, h_kv, T, d = 1, 8, 2, 150, 128
    print(f"case backward misaligned O {o_dtype}", flush=True)
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 14800)
    d_out = inputs.normal(14800, "d_out", (B, h_q, T, d), "bf16")
    q, k, v, do = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(d_out, "bf16")
    od = torch.float32 if o_dtype == "f32" else torch.bfloat16
    o, lse = ops.gqa_prefill_lse(q, k, v, out_dtype=od)
    buf = torch.empty(o.numel() + 1, dtype=od, device=o.device)
    o_off = buf[1:].view(o.shape)
    o_off.copy_(o)
    assert o_off.data_ptr() % 16 != 0
    grads = ops.gqa_prefill_backward(q, k, v, o_off, do, lse)
    torch.cuda.synchronize()
    want = _oracle(x, d_out, True)
    for name, g, w in zip(("dq", "dk", "dv"), grads, want):
        _check_grad(to_host64(g), w, f"misaligned O {o_dtype} {name}")
