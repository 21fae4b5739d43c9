"""GPU parity at the named workloads' full sizes, in the launch configuration the
benchmark times, checked on sampled outputs the oracle computes one by one.

Sampled rows include the first and last positions and tile boundaries; for
decode, whole sequences (every query head) are checked, including the
shortest and longest ragged histories.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu


def test_prefill_causal_bf16_T4096_sampled():
    import torch

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    print(f"case {w.name}", flush=True)
    x = inputs.make_workload(w)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o = ops.gqa_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    got = to_host64(o)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(0)
    positions = sorted({0, 1, 31, 32, 63, 64, 127, 128, 2047, 2048, 4094, 4095, *rng.integers(0, 4096, 8).tolist()})
    heads = [0, 3, 4, 17, 31]
    r = w.h_q // w.h_kv
    for a in heads:
        g = a // r
        kk, vv = f64(x["k"][:, g:g + 1], "bf16"), f64(x["v"][:, g:g + 1], "bf16")
        for i in positions:
            want = oracle.attention(f64(x["q"][:, a:a + 1, i:i + 1], "bf16"), kk, vv, causal=True,
                                    q_pos=np.array([[i]]), kv_len=np.array([w.T]))
            check_parity(got[:, a:a + 1, i:i + 1], want, mode="bf16", what=f"head {a} pos {i}")


def _decode_sampled(w, batch_rows):
    import torch

    print(f"case {w.name}", flush=True)
    x = inputs.make_workload(w)
    o = ops.gqa_decode(to_dev(x["q"], "bf16"), to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16"),
                       ints_dev(x["seq_lens"]), q_pos=ints_dev(x["q_pos"]), max_seq_len=int(x["seq_lens"].max()))
    torch.cuda.synchronize()
    got = to_host64(o)
    assert np.all(np.isfinite(got))
    for b in batch_rows:
        L = int(x["seq_lens"][b])
        want = oracle.attention(f64(x["q"][b:b + 1], "bf16"), f64(x["k_cache"][b:b + 1, :, :L], "bf16"),
                                f64(x["v_cache"][b:b + 1, :, :L], "bf16"), causal=True,
                                q_pos=np.array([[x["q_pos"][b]]]), kv_len=np.array([L]))
        check_parity(got[b:b + 1], want, mode="bf16", what=f"{w.name} b={b}")


def test_decode_bf16_B64_T8192_sampled():
    _decode_sampled(inputs.WORKLOADS["decode_bf16_B64_T8192"], [0, 31, 63])


@pytest.mark.parametrize("name", ["decode_mha_B8_T32000", "decode_gqa_B8_T32000", "decode_mqa_B8_T32000"])
def test_decode_sweep_sampled(name):
    _decode_sampled(inputs.WORKLOADS[name], [0, 7])


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_ragged_append_decode_B32_sampled(fused):
    """The ragged step as kv_append then decode, and as the one fused call the
    benchmark times."""
    import torch

    w = inputs.WORKLOADS["ragged_append_decode_B32"]
    print(f"case {w.name} fused={fused}", flush=True)
    x = inputs.make_workload(w)
    kd, vd = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    kn, vn, wp = to_dev(x["k_new"], "bf16"), to_dev(x["v_new"], "bf16"), ints_dev(x["write_pos"])
    q, sl, qp, msl = to_dev(x["q"], "bf16"), ints_dev(x["seq_lens"]), ints_dev(x["q_pos"]), int(x["seq_lens"].max())
    if fused:
        o = ops.gqa_append_decode(q, kd, vd, kn, vn, wp, sl, q_pos=qp, max_seq_len=msl)
    else:
        ops.gqa_kv_append(kd, vd, kn, vn, wp)
        o = ops.gqa_decode(q, kd, vd, sl, q_pos=qp, max_seq_len=msl)
    torch.cuda.synchronize()
    got = to_host64(o)
    assert np.all(np.isfinite(got))
    hist = x["hist"]
    picks = sorted({int(np.argmin(hist)), int(np.argmax(hist)), 5})
    for b in picks:
        L = int(x["seq_lens"][b])
        k = x["k_cache"][b:b + 1, :, :L].copy()
        v = x["v_cache"][b:b + 1, :, :L].copy()
        k[0, :, hist[b]] = x["k_new"][b, :, 0]
        v[0, :, hist[b]] = x["v_new"][b, :, 0]
        want = oracle.attention(f64(x["q"][b:b + 1], "bf16"), f64(k, "bf16"), f64(v, "bf16"), causal=True,
                                q_pos=np.array([[hist[b]]]), kv_len=np.array([L]))
        check_parity(got[b:b + 1], want, mode="bf16", what=f"ragged b={b} hist={hist[b]}")
    # the appended rows themselves, bit for bit
    bi = torch.arange(w.B, device=kd.device)
    ti = torch.as_tensor(hist, dtype=torch.long, device=kd.device)
    rows = kd[bi, :, ti].cpu().view(torch.int16).numpy()
    assert np.array_equal(rows, x["k_new"][:, :, 0].view(np.int16))
