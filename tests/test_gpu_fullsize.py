"""GPU parity at the named workloads' full sizes, in the launch configuration the
benchmark times, over EVERY output element.

The float64 oracle runs on the host for every (sequence, K/V head) slice in
parallel threads; max-abs and mean-abs are taken over the whole output against
the bar for bf16 inputs with fp32 accumulation (2e-2 / 2e-3).  Rows at tile
edges (first and last positions, multiples of 32 and 64) are also asserted on
their own, so a fault confined to one tile edge cannot hide in the mean.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, check_parity, f64, ints_dev, parallel_map, to_dev, to_host64

pytestmark = pytest.mark.gpu

EDGE_POSITIONS = (0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 2047, 2048, 4094, 4095)


def _report(what, got, want):
    err = np.abs(got - want)
    print(f"{what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} over {err.size} values", flush=True)


def test_prefill_causal_bf16_T4096_every_element():
    import torch

    w = inputs.WORKLOADS["prefill_causal_bf16_T4096"]
    print(f"case {w.name}", flush=True)
    x = inputs.make_workload(w)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o = ops.gqa_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    got = to_host64(o)
    del q, k, v, o
    r = w.h_q // w.h_kv

    def head(a):
        g = a // r
        return oracle.attention(f64(x["q"][:, a:a + 1], "bf16"), f64(x["k"][:, g:g + 1], "bf16"),
                                f64(x["v"][:, g:g + 1], "bf16"), causal=True)

    want = np.concatenate(parallel_map(head, range(w.h_q)), axis=1)
    _report(w.name, got, want)
    check_parity(got, want, mode="bf16", what=w.name)
    for i in EDGE_POSITIONS:
        check_parity(got[:, :, i], want[:, :, i], mode="bf16", what=f"{w.name} position {i}")


def _decode_want(x, w, hist=None):
    """Oracle output of a decode workload, one (sequence, K/V head) slice at a time.
    With ``hist``, row hist[b] of every cache head holds the appended token."""
    r = w.h_q // w.h_kv

    def slice_(bg):
        b, g = divmod(bg, w.h_kv)
        L = int(x["seq_lens"][b])
        k = x["k_cache"][b:b + 1, g:g + 1, :L].copy()
        v = x["v_cache"][b:b + 1, g:g + 1, :L].copy()
        if hist is not None:
            k[0, 0, hist[b]] = x["k_new"][b, g, 0]
            v[0, 0, hist[b]] = x["v_new"][b, g, 0]
        return oracle.attention(f64(x["q"][b:b + 1, g * r:(g + 1) * r], "bf16"), f64(k, "bf16"), f64(v, "bf16"),
                                causal=True, q_pos=np.array([[x["q_pos"][b]]]), kv_len=np.array([L]))

    parts = parallel_map(slice_, range(w.B * w.h_kv))
    return np.stack([np.concatenate(parts[b * w.h_kv:(b + 1) * w.h_kv], axis=1)[0] for b in range(w.B)])


def _decode_every_element(w):
    import torch

    print(f"case {w.name}", flush=True)
    x = inputs.make_workload(w)
    kd, vd = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    o = ops.gqa_decode(to_dev(x["q"], "bf16"), kd, vd, ints_dev(x["seq_lens"]), q_pos=ints_dev(x["q_pos"]),
                       max_seq_len=int(x["seq_lens"].max()))
    torch.cuda.synchronize()
    got = to_host64(o)
    del kd, vd, o
    torch.cuda.empty_cache()
    want = _decode_want(x, w)
    _report(w.name, got, want)
    check_parity(got, want, mode="bf16", what=w.name)


def test_decode_bf16_B64_T8192_every_element():
    _decode_every_element(inputs.WORKLOADS["decode_bf16_B64_T8192"])


@pytest.mark.parametrize("name", ["decode_mha_B8_T32000", "decode_gqa_B8_T32000", "decode_mqa_B8_T32000"])
def test_decode_sweep_every_element(name):
    _decode_every_element(inputs.WORKLOADS[name])


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_ragged_append_decode_B32_every_element(fused):
    """The ragged step as kv_append then decode, and as the one fused call the
    benchmark times, on the 32 histories of the workload's draw (543,025 rows)."""
    import torch

    w = inputs.WORKLOADS["ragged_append_decode_B32"]
    print(f"case {w.name} fused={fused}", flush=True)
    x = inputs.make_workload(w)
    assert int(x["seq_lens"].sum()) == 543_025
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
    hist = x["hist"]
    # the appended rows themselves, bit for bit
    bi = torch.arange(w.B, device=kd.device)
    ti = torch.as_tensor(hist, dtype=torch.long, device=kd.device)
    rows_k = kd[bi, :, ti].cpu().view(torch.int16).numpy()
    rows_v = vd[bi, :, ti].cpu().view(torch.int16).numpy()
    assert np.array_equal(rows_k, x["k_new"][:, :, 0].view(np.int16))
    assert np.array_equal(rows_v, x["v_new"][:, :, 0].view(np.int16))
    del kd, vd, o
    torch.cuda.empty_cache()
    want = _decode_want(x, w, hist=hist)
    _report(f"{w.name} fused={fused}", got, want)
    check_parity(got, want, mode="bf16", what=f"{w.name} fused={fused}")
    assert BF16_MAX_ABS == 2e-2 and BF16_MEAN_ABS == 2e-3
