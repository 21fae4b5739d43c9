"""GPU parity of the training path: the forward's row log-sum-exp and the
gradients dQ, dK, dV against the float64 oracle (oracle/backward.py).

Parity bar for the gradients (bf16 inputs, fp32 accumulation and outputs): the
kernel rounds P and dS to bf16 before the products that use them (relative
error up to 2^-9 per term, independent between terms), and O and the row
statistics it recomputes P from are fp32.  A gradient element sum_j t_j then
carries an error of about 2^-9 / sqrt(3) * sqrt(sum_j t_j^2); over a whole tensor
that is below 2^-9 of its norm unless the sums cancel heavily.  The bar is
  relative Frobenius error <= 4 * 2^-9 (7.8e-3) per tensor,
  every element within 2e-2 * max|g| of the oracle,
  and, as for the forward output, max-abs <= 2e-2 and mean-abs <= 2e-3 for a
  gradient of unit scale (max|g|, mean|g| <= 1), scaled by max|g| and mean|g|
  above that,
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
ABS_MAX = 2e-2
ABS_MEAN = 2e-3


def _check_grad(got, want, what, absolute=True):
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
    abs_max, abs_mean = float(np.max(np.abs(err))), float(np.mean(np.abs(err)))
    g_max, g_mean = float(np.max(np.abs(want))), float(np.mean(np.abs(want)))
    print(f"{what}: rel_fro {rel:.2e} max/max {mx:.2e} | max-abs {abs_max:.2e} mean-abs {abs_mean:.2e} "
          f"(max|g| {g_max:.2e} mean|g| {g_mean:.2e})", flush=True)
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3g}"
    assert mx <= MAX_REL, f"{what}: max error {mx:.3g} of max |g|"
    # the forward's absolute bar (2e-2 max-abs, 2e-3 mean-abs) for gradients of unit
    # scale; larger gradients carry the same bar relative to their scale
    if absolute:
        assert abs_max <= ABS_MAX * max(1.0, g_max), f"{what}: max-abs {abs_max:.3g}"
        assert abs_mean <= ABS_MEAN * max(1.0, g_mean), f"{what}: mean-abs {abs_mean:.3g}"


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
    (1, 32, 1, 130, 128, True, None),           # MQA, causal: 32 heads share each key block's items
    (2, 8, 4, 180, 128, False, [180, 70]),      # no causal mask, padded second sequence
    (1, 8, 2, 161, 128, True, [100]),           # keys end inside a 64-key block; rows past them see 100 keys
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


def test_backward_prefill_workload_every_element():
    """The causal prefill workload at full size (B=1, h_q=32, h_kv=8, d_h=128, T=4096),
    in the launch configuration the benchmark times: every element of dQ, dK and dV
    against the float64 oracle, one K/V head's group of query heads per host thread,
    under the bar above for each gradient of each group; rows at tile edges on their own."""
    import torch

    from tests.gpu_util import parallel_map

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    print(f"case {w.name} backward, every element", flush=True)
    x = inputs.make_workload(w)
    d_out = inputs.normal(w.seed, "d_out", (w.B, w.h_q, w.T, w.d_h), "bf16")
    q, k, v, do = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(d_out, "bf16")
    o, lse = ops.gqa_prefill_lse(q, k, v)
    dq, dk, dv = ops.gqa_prefill_backward(q, k, v, o, do, lse)
    torch.cuda.synchronize()
    dq, dk, dv = to_host64(dq), to_host64(dk), to_host64(dv)
    del q, k, v, do, o, lse
    r = w.h_q // w.h_kv

    def group(g):
        hs = slice(g * r, (g + 1) * r)
        return oracle.attention_backward(f64(x["q"][:, hs], "bf16"), f64(x["k"][:, g:g + 1], "bf16"),
                                         f64(x["v"][:, g:g + 1], "bf16"), f64(d_out[:, hs], "bf16"), causal=True)

    wants = parallel_map(group, range(w.h_kv))
    for g, (wq, wk, wv) in enumerate(wants):
        hs = slice(g * r, (g + 1) * r)
        _check_grad(dq[:, hs], wq, f"full-size dQ g={g}")
        _check_grad(dk[:, g:g + 1], wk, f"full-size dK g={g}")
        _check_grad(dv[:, g:g + 1], wv, f"full-size dV g={g}")
        # tile edges of the query rows (dQ; row 0 sees one key, so its exact dQ is 0 and
        # the whole-tensor check above covers it) and of the keys (dK, dV: 16-, 32- and
        # 64-key blocks), each row under the relative bars: a row of an early key sums
        # ~16K rounded terms, so its error sits at the 2^-9-scale relative level and the
        # absolute mean bar, derived for whole tensors, does not apply to it
        for i in (1, 15, 16, 31, 32, 63, 64, 2047, 2048, 4095):
            _check_grad(dq[:, hs, i], wq[:, :, i], f"full-size dQ g={g} row {i}", absolute=False)
        for j in (0, 1, 15, 16, 31, 32, 63, 64, 2047, 2048, 4095):
            _check_grad(dk[:, g, j], wk[:, 0, j], f"full-size dK g={g} key {j}", absolute=False)
            _check_grad(dv[:, g, j], wv[:, 0, j], f"full-size dV g={g} key {j}", absolute=False)


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


def test_backward_empty_and_short_sequences():
    """A sequence with no keys has no visible pair: all of its gradients are 0.  The
    others (one shorter than a 64-key block) match the oracle one sequence at a time."""
    B, h_q, h_kv, T, d = 3, 8, 2, 200, 128
    lens = [200, 0, 45]
    print(f"case backward lengths {lens}", flush=True)
    x, d_out, _, got = _run(B, h_q, h_kv, T, d, True, 14900, kv_lens=lens)
    for b in range(B):
        if lens[b] == 0:
            for name, g in zip(("dq", "dk", "dv"), got):
                assert np.all(g[b] == 0.0), f"empty sequence {name}"
            continue
        sl = slice(b, b + 1)
        xb = {k_: x[k_][sl] for k_ in ("q", "k", "v")}
        want = _oracle(xb, d_out[sl], True, [lens[b]])
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            _check_grad(g[sl], w, f"lengths {lens} b={b} {name}")
