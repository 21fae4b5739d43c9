"""The allocation-free decode entry point (gqa_decode_noalloc), through the C ABI.

It runs the same kernels and split plan as gqa_decode, with the partial states in
the library's static device scratch instead of a caller's workspace, so its output
must equal gqa_decode's bit for bit -- and both match the oracle.  Two calls in a
row on one GPU share the scratch; the second, smaller one must not see the
first's partial states.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _oracle_decode(x):
    out = []
    for b in range(x["q"].shape[0]):
        L = int(x["seq_lens"][b])
        out.append(oracle.attention(f64(x["q"][b:b + 1], "bf16"), f64(x["k_cache"][b:b + 1, :, :L], "bf16"),
                                    f64(x["v_cache"][b:b + 1, :, :L], "bf16"), causal=True,
                                    q_pos=np.array([[L - 1]]), kv_len=np.array([L]))[0])
    return np.stack(out)


# (B, h_q, h_kv, T_cap, d_h, lens, out dtype): the first of each pair is the larger call
PAIRS = [
    ((6, 32, 8, 6000, 128, [6000, 5999, 4097, 3000, 64, 1], "f32"),
     (2, 16, 4, 900, 128, [900, 333], "f32")),
    ((2, 32, 1, 9000, 128, [9000, 8000], "bf16"),          # wide kernel, batched merge
     (1, 8, 1, 700, 64, [700], "bf16")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["16x16_then_smaller", "wide_then_smaller"])
def test_decode_noalloc_two_calls_match_decode(pair):
    import torch

    runs = []
    for i, (B, h_q, h_kv, T, d, lens, od) in enumerate(pair):
        print(f"case decode_noalloc call {i}: B={B} h_q={h_q} h_kv={h_kv} T={T} d={d} out={od}", flush=True)
        x = inputs.make_decode(B, h_q, h_kv, d, T, "bf16", 15000 + 10 * i + T, seq_lens=lens, poison=True)
        dev = (to_dev(x["q"], "bf16"), to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16"),
               ints_dev(x["seq_lens"]))
        dt = torch.float32 if od == "f32" else torch.bfloat16
        out = torch.empty((B, h_q, 1, d), dtype=dt, device="cuda")
        ops.gqa_decode_noalloc(*dev, max_seq_len=int(max(lens)), out=out)
        runs.append((x, dev, dt, out, od))
    torch.cuda.synchronize()
    for x, dev, dt, out, od in runs:
        ref = ops.gqa_decode(*dev, max_seq_len=int(x["seq_lens"].max()), out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "gqa_decode_noalloc differs from gqa_decode"
        check_parity(to_host64(out), _oracle_decode(x), mode="bf16" if od == "f32" else "bf16out",
                     what="decode_noalloc")
