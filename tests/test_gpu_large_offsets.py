"""GPU parity where tensor offsets pass 2^31 bytes: caches of 2^22 rows per head.

A (sequence, K/V head) slice of such a cache is 1 GiB at d_h 128, so the slices
of later sequences and heads start past 2^31 bytes and every address has to be
formed in 64 bits.  Only the visible rows hold seeded data; every other row is
NaN, so a read of an invisible row (or of the wrong slice) poisons the output.
The oracle reads the visible rows only, so the checks stay cheap.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu

T_BIG = 1 << 22   # rows per (sequence, head): 1 GiB of bf16 at d_h 128


def _nan_cache(B, h, d):
    import torch

    return torch.full((B, h, T_BIG, d), float("nan"), dtype=torch.bfloat16, device="cuda")


def _fill(cache, rows):
    """rows (B, h, L, d) bf16 bits -> the first L rows of every slice of `cache`."""
    cache[:, :, :rows.shape[2]] = to_dev(rows, "bf16")


@pytest.mark.parametrize("h_q", [8, 32], ids=["r8_16x16_kernel", "r32_wide_kernel"])
def test_decode_past_2gib(h_q):
    import torch

    B, h_kv, d = 3, 1, 128
    lens = np.array([1500, 3000, 2000], np.int32)
    print(f"case decode large offsets h_q={h_q}", flush=True)
    seed = 41000 + h_q
    q = inputs.normal(seed, "q", (B, h_q, 1, d), "bf16")
    k = inputs.normal(seed, "k", (B, h_kv, int(lens.max()), d), "bf16")
    v = inputs.normal(seed, "v", (B, h_kv, int(lens.max()), d), "bf16")
    kd, vd = _nan_cache(B, h_kv, d), _nan_cache(B, h_kv, d)
    for b in range(B):
        kd[b, :, :lens[b]] = to_dev(np.ascontiguousarray(k[b:b + 1, :, :lens[b]]), "bf16")[0]
        vd[b, :, :lens[b]] = to_dev(np.ascontiguousarray(v[b:b + 1, :, :lens[b]]), "bf16")[0]
    o = ops.gqa_decode(to_dev(q, "bf16"), kd, vd, ints_dev(lens))
    torch.cuda.synchronize()
    want = np.stack([oracle.attention(f64(q[b:b + 1], "bf16"), f64(k[b:b + 1, :, :lens[b]], "bf16"),
                                      f64(v[b:b + 1, :, :lens[b]], "bf16"), causal=False)[0] for b in range(B)])
    check_parity(to_host64(o), want, mode="bf16", what=f"decode h_q={h_q}")
    del kd, vd
    torch.cuda.empty_cache()


def test_chunked_prefill_past_2gib():
    import torch

    B, h_q, h_kv, d, S_q = 2, 8, 2, 128, 200
    lens = np.array([900, 1300], np.int32)
    print("case chunked prefill large offsets", flush=True)
    seed = 42000
    q = inputs.normal(seed, "q", (B, h_q, S_q, d), "bf16")
    k = inputs.normal(seed, "k", (B, h_kv, int(lens.max()), d), "bf16")
    v = inputs.normal(seed, "v", (B, h_kv, int(lens.max()), d), "bf16")
    kd, vd = _nan_cache(B, h_kv, d), _nan_cache(B, h_kv, d)
    for b in range(B):
        kd[b, :, :lens[b]] = to_dev(np.ascontiguousarray(k[b:b + 1, :, :lens[b]]), "bf16")[0]
        vd[b, :, :lens[b]] = to_dev(np.ascontiguousarray(v[b:b + 1, :, :lens[b]]), "bf16")[0]
    # default positions: the newest S_q positions of each history
    o = ops.gqa_prefill_chunk(to_dev(q, "bf16"), kd, vd, kv_lens=ints_dev(lens))
    torch.cuda.synchronize()
    want = np.stack([oracle.attention(f64(q[b:b + 1], "bf16"), f64(k[b:b + 1, :, :lens[b]], "bf16"),
                                      f64(v[b:b + 1, :, :lens[b]], "bf16"), causal=True,
                                      kv_len=lens[b:b + 1])[0] for b in range(B)])
    check_parity(to_host64(o), want, mode="bf16", what="chunked prefill")
    del kd, vd
    torch.cuda.empty_cache()


def test_kv_append_at_the_last_row_past_2gib():
    import torch

    B, h_kv, d = 3, 2, 128
    print("case kv_append large offsets", flush=True)
    kd, vd = _nan_cache(B, h_kv, d), _nan_cache(B, h_kv, d)
    k_new = inputs.normal(43000, "k_new", (B, h_kv, 1, d), "bf16")
    v_new = inputs.normal(43000, "v_new", (B, h_kv, 1, d), "bf16")
    wp = np.array([0, T_BIG // 2, T_BIG - 1], np.int32)
    ops.gqa_kv_append(kd, vd, to_dev(k_new, "bf16"), to_dev(v_new, "bf16"), ints_dev(wp))
    torch.cuda.synchronize()
    for b in range(B):
        got_k = kd[b, :, wp[b]].view(torch.int16).cpu().numpy().view(np.uint16)
        got_v = vd[b, :, wp[b]].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got_k, k_new[b, :, 0]), f"k row {wp[b]} of sequence {b}"
        assert np.array_equal(got_v, v_new[b, :, 0]), f"v row {wp[b]} of sequence {b}"
    # the rows around each written one are untouched
    for b in range(B):
        for j in (int(wp[b]) - 1, int(wp[b]) + 1):
            if 0 <= j < T_BIG:
                assert torch.isnan(kd[b, :, j].float()).all() and torch.isnan(vd[b, :, j].float()).all()
    del kd, vd
    torch.cuda.empty_cache()
