"""GPU parity of prefill (and chunked prefill) against the float64 oracle.

Every case goes through the C ABI (ctypes binding) on the same seeded inputs
the oracle reads.  Sizes span several 128-row blocks and 64-key tiles with
ragged tails so that every tiling boundary is crossed.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _run_prefill(x, dtype, *, causal=True, kv_lens=None, out_dtype=None, scale=None):
    import torch

    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    od = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o = ops.gqa_prefill(q, k, v, causal=causal, scale=scale,
                        kv_lens=None if kv_lens is None else ints_dev(kv_lens), out_dtype=od)
    torch.cuda.synchronize()
    return to_host64(o)


def _oracle(x, dtype, *, causal=True, kv_lens=None, scale=None):
    return oracle.attention(f64(x["q"], dtype), f64(x["k"], dtype), f64(x["v"], dtype),
                            causal=causal, kv_len=kv_lens, scale=scale)


def test_tiny_prefill_workload_fp32():
    w = inputs.WORKLOADS["tiny_prefill_f32"]
    x = inputs.make_workload(w)
    print(f"case {w.name}", flush=True)
    got = _run_prefill(x, "f32")
    check_parity(got, _oracle(x, "f32"), mode="f32", what=w.name)


def test_worked_two_keys_fp32(golden_dir):
    import torch

    g = json.load(open(os.path.join(golden_dir, "worked_two_keys_d1.json")))
    q = torch.tensor(g["queries"], dtype=torch.float32).reshape(1, 1, 2, 1).cuda()
    k = torch.tensor(g["keys"], dtype=torch.float32).reshape(1, 1, 2, 1).cuda()
    v = torch.tensor(g["values"], dtype=torch.float32).reshape(1, 1, 2, 1).cuda()
    o = ops.gqa_prefill(q, k, v, causal=False).cpu().numpy()
    assert abs(o[0, 0, 0, 0] - 15.0) <= 1e-5
    assert abs(o[0, 0, 1, 0] - (10 + 20 * math.e) / (1 + math.e)) <= 1e-5


def test_two_block_example_fp32():
    import torch

    q = torch.ones(1, 1, 1, 1).cuda()
    k = torch.log(torch.tensor([1.0, 2.0, 3.0, 4.0])).reshape(1, 1, 4, 1).cuda()
    v = torch.tensor([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 4, 1).cuda()
    # one query row against four keys: use the chunk entry point (S_q=1, positions from the end)
    o = ops.gqa_prefill_chunk(q, k, v, causal=True, scale=1.0).cpu().numpy()
    assert abs(o[0, 0, 0, 0] - 3.0) <= 1e-5


FP32_CASES = [
    # B, h_q, h_kv, T, d_h, causal
    (2, 6, 3, 37, 5, True),
    (1, 8, 1, 70, 256, True),
    (2, 4, 4, 45, 33, False),
    (1, 12, 4, 33, 128, True),
]


@pytest.mark.parametrize("case", FP32_CASES, ids=lambda c: "B%d_hq%d_hkv%d_T%d_d%d_c%d" % c)
def test_prefill_fp32_random(case):
    B, h_q, h_kv, T, d, causal = case
    print(f"case fp32 {case}", flush=True)
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "f32", 7000 + T)
    check_parity(_run_prefill(x, "f32", causal=causal), _oracle(x, "f32", causal=causal), mode="f32", what=str(case))


def test_prefill_fp32_padding():
    B, h_q, h_kv, T, d = 3, 4, 2, 40, 16
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "f32", 7100)
    lens = np.array([40, 17, 1], np.int32)
    for causal in (True, False):
        got = _run_prefill(x, "f32", causal=causal, kv_lens=lens)
        want = np.stack([oracle.attention(f64(x["q"][b:b + 1], "f32"), f64(x["k"][b:b + 1], "f32"),
                                          f64(x["v"][b:b + 1], "f32"), causal=causal,
                                          kv_len=lens[b:b + 1])[0] for b in range(B)])
        check_parity(got, want, mode="f32", what=f"padding causal={causal}")


BF16_CASES = [
    # B, h_q, h_kv, T, d_h, causal
    (2, 8, 2, 200, 128, True),     # r=4: 4 heads x 32 positions per workgroup
    (1, 4, 4, 130, 64, True),      # MHA, d_h 64
    (1, 8, 1, 150, 128, True),     # MQA r=8
    (1, 64, 2, 70, 128, True),     # r=32
    (1, 6, 2, 100, 64, True),      # r=3 (one head per workgroup)
    (2, 8, 2, 129, 128, False),    # no mask
    (1, 32, 8, 300, 128, True),    # the prefill workload's head layout, shorter
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "B%d_hq%d_hkv%d_T%d_d%d_c%d" % c)
def test_prefill_bf16_random(case):
    B, h_q, h_kv, T, d, causal = case
    print(f"case bf16 {case}", flush=True)
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 8000 + T)
    check_parity(_run_prefill(x, "bf16", causal=causal), _oracle(x, "bf16", causal=causal),
                 mode="bf16", what=str(case))


def test_prefill_bf16_out_bf16():
    x = inputs.make_prefill(1, 8, 2, 128, 150, "bf16", 8200)
    got = _run_prefill(x, "bf16", out_dtype="bf16")
    check_parity(got, _oracle(x, "bf16"), mode="bf16out", what="bf16 out")


# The output leaves each wave through LDS in parts of d_h bytes per row, several rows
# per store instruction; these shapes vary the rows' heads within a wave (r = 64, 128:
# 2-4 positions per head), the part count (fp32 / bf16 output, d_h 64 / 128) and the
# ragged last block.
LAYOUT_CASES = [
    # B, h_q, h_kv, T, d_h, output dtype
    (1, 128, 1, 37, 128, "f32"),    # r=128: 128 heads x 2 positions per workgroup
    (1, 64, 1, 45, 64, "bf16"),     # r=64, d_h 64, bf16 output
    (1, 4, 4, 130, 64, "bf16"),     # MHA, d_h 64, bf16 output
    (2, 8, 2, 97, 128, "bf16"),     # r=4, ragged last block, bf16 output
    (1, 16, 2, 75, 64, "f32"),      # r=8: 8 heads x 32 positions, d_h 64
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=lambda c: "B%d_hq%d_hkv%d_T%d_d%d_%s" % c)
def test_prefill_bf16_output_layouts(case):
    B, h_q, h_kv, T, d, od = case
    print(f"case layout {case}", flush=True)
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 8700 + T)
    got = _run_prefill(x, "bf16", out_dtype=od)
    check_parity(got, _oracle(x, "bf16"), mode="bf16out" if od == "bf16" else "bf16", what=str(case))


def test_prefill_bf16_padding_and_poison():
    # keys past kv_lens are NaN: they must never reach the output
    B, h_q, h_kv, T, d = 3, 8, 2, 200, 128
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 8300)
    lens = np.array([200, 77, 1], np.int32)
    for b in range(B):
        x["k"][b, :, lens[b]:] = inputs.BF16_QNAN
        x["v"][b, :, lens[b]:] = inputs.BF16_QNAN
    for causal in (True, False):
        got = _run_prefill(x, "bf16", causal=causal, kv_lens=lens)
        want = np.stack([oracle.attention(f64(x["q"][b:b + 1], "bf16"), f64(x["k"][b:b + 1], "bf16"),
                                          f64(x["v"][b:b + 1], "bf16"), causal=causal,
                                          kv_len=lens[b:b + 1])[0] for b in range(B)])
        check_parity(got, want, mode="bf16", what=f"poison causal={causal}")


def test_prefill_bf16_empty_rows_are_zero():
    import torch

    x = inputs.make_prefill(2, 4, 2, 64, 70, "bf16", 8400)
    got = _run_prefill(x, "bf16", kv_lens=np.array([0, 70], np.int32))
    assert np.all(got[0] == 0.0)
    check_parity(got[1:], _oracle({k: v[1:] for k, v in x.items()}, "bf16"), mode="bf16", what="len 0")


@pytest.mark.parametrize("d_h,T", [(128, 300), (128, 1500), (64, 1500)])
def test_prefill_bf16_deterministic(d_h, T):
    """Repeated launches give the same bits: a tile load racing with a read of its
    stage would show as run-to-run differences (many tiles per workgroup here)."""
    import torch

    x = inputs.make_prefill(1, 8, 2, d_h, T, "bf16", 8500 + d_h)
    a = _run_prefill(x, "bf16")
    for _ in range(4):
        assert np.array_equal(a, _run_prefill(x, "bf16"))


def test_prefill_does_not_write_outside_output():
    import torch

    x = inputs.make_prefill(1, 8, 2, 128, 100, "bf16", 8600)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    n = 8 * 100 * 128
    guard = torch.full((n + 2048,), 12345.0, device="cuda")
    out = guard[1024:1024 + n].view(1, 8, 100, 128)
    ops.gqa_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    g = guard.cpu().numpy()
    assert np.all(g[:1024] == 12345.0) and np.all(g[1024 + n:] == 12345.0)


def test_prefill_bf16_out_does_not_write_outside_output():
    import torch

    # 100 positions: the last 64-position block holds 36 rows, the rest must stay untouched
    x = inputs.make_prefill(1, 8, 2, 128, 100, "bf16", 8650)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    n = 8 * 100 * 128
    guard = torch.full((n + 2048,), 123.0, dtype=torch.bfloat16, device="cuda")
    out = guard[1024:1024 + n].view(1, 8, 100, 128)
    ops.gqa_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    g = guard.float().cpu().numpy()
    assert np.all(g[:1024] == 123.0) and np.all(g[1024 + n:] == 123.0)
    check_parity(out.float().cpu().numpy(), _oracle(x, "bf16"), mode="bf16out", what="guarded bf16 out")


# ---------------------------------------------------------------- chunked / offset prefill
CHUNK_CASES = [
    # dtype, B, h_q, h_kv, S_q, T_cap, d_h
    ("bf16", 2, 8, 2, 100, 400, 128),
    ("bf16", 1, 32, 8, 64, 1000, 64),
    ("f32", 2, 4, 2, 20, 90, 16),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "%s_B%d_hq%d_hkv%d_S%d_T%d_d%d" % c)
def test_prefill_chunk(case):
    import torch

    dt, B, h_q, h_kv, S_q, T_cap, d = case
    print(f"case chunk {case}", flush=True)
    rng = np.random.default_rng(S_q + T_cap)
    q = inputs.normal(9000 + T_cap, "q", (B, h_q, S_q, d), dt)
    k = inputs.normal(9000 + T_cap, "k", (B, h_kv, T_cap, d), dt)
    v = inputs.normal(9000 + T_cap, "v", (B, h_kv, T_cap, d), dt)
    lens = rng.integers(S_q, T_cap + 1, size=B).astype(np.int32)
    pos0 = (lens - S_q).astype(np.int32)
    pos0[0] = max(0, pos0[0] - 7)          # explicit offset that leaves keys past the chunk unseen
    mode = "f32" if dt == "f32" else "bf16"
    o = ops.gqa_prefill_chunk(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), kv_lens=ints_dev(lens),
                              q_pos0=ints_dev(pos0))
    torch.cuda.synchronize()
    got = to_host64(o)
    qp = pos0[:, None] + np.arange(S_q)[None]
    want = oracle.attention(f64(q, dt), f64(k, dt), f64(v, dt), causal=True, q_pos=qp, kv_len=lens)
    check_parity(got, want, mode=mode, what=str(case))
    # default positions: the newest S_q positions of each sequence
    o2 = ops.gqa_prefill_chunk(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), kv_lens=ints_dev(lens))
    torch.cuda.synchronize()
    want2 = oracle.attention(f64(q, dt), f64(k, dt), f64(v, dt), causal=True, kv_len=lens)
    check_parity(to_host64(o2), want2, mode=mode, what=str(case) + " default positions")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_chunk_full_capacity_default_positions(dt):
    """A chunk as long as the cache (S_q == T_cap) with shorter kv_lens and no
    explicit positions is a prefill: row i sits at position i and kv_lens masks
    keys only, as the oracle's default positions say ([Ch09] 09.2: positions are
    absolute).  Matches gqa_prefill with the same kv_lens."""
    import torch

    B, h_q, h_kv, T, d = 3, 8, 2, 300, 128 if dt == "bf16" else 24
    print(f"case chunk S_q == T_cap {dt}", flush=True)
    q = inputs.normal(9700, "q", (B, h_q, T, d), dt)
    k = inputs.normal(9700, "k", (B, h_kv, T, d), dt)
    v = inputs.normal(9700, "v", (B, h_kv, T, d), dt)
    lens = np.array([300, 173, 64], np.int32)
    o = ops.gqa_prefill_chunk(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), kv_lens=ints_dev(lens))
    p = ops.gqa_prefill(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), kv_lens=ints_dev(lens))
    torch.cuda.synchronize()
    got = to_host64(o)
    want = oracle.attention(f64(q, dt), f64(k, dt), f64(v, dt), causal=True, kv_len=lens)
    check_parity(got, want, mode="f32" if dt == "f32" else "bf16", what=f"chunk S_q == T_cap {dt}")
    assert np.array_equal(got, to_host64(p)), "the full-capacity chunk must equal gqa_prefill"
