"""GPU parity of KV-cached decode and kv_append against the float64 oracle."""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _decode(x, dtype, *, q_pos=None, max_seq_len=None, out_dtype=None):
    import torch

    od = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o = ops.gqa_decode(to_dev(x["q"], dtype), to_dev(x["k_cache"], dtype), to_dev(x["v_cache"], dtype),
                       ints_dev(x["seq_lens"]), q_pos=None if q_pos is None else ints_dev(q_pos),
                       max_seq_len=max_seq_len, out_dtype=od)
    torch.cuda.synchronize()
    return to_host64(o)


def _oracle_decode(x, dtype, q_pos=None):
    B = x["q"].shape[0]
    lens = np.asarray(x["seq_lens"])
    qp = (lens - 1) if q_pos is None else np.asarray(q_pos)
    out = []
    for b in range(B):
        L = int(min(lens[b], qp[b] + 1))
        out.append(oracle.attention(f64(x["q"][b:b + 1], dtype), f64(x["k_cache"][b:b + 1, :, :L], dtype),
                                    f64(x["v_cache"][b:b + 1, :, :L], dtype), causal=True,
                                    q_pos=np.array([[qp[b]]]), kv_len=np.array([L]))[0])
    return np.stack(out)


DECODE_CASES = [
    # dtype, B, h_q, h_kv, T_cap, d_h, lens
    ("bf16", 3, 8, 2, 1000, 128, [1000, 517, 1]),
    ("bf16", 2, 32, 1, 3000, 128, [3000, 2999]),      # MQA, r=32: a full 32-column tile
    ("bf16", 1, 64, 1, 700, 128, [700]),              # r=64: two head chunks
    ("bf16", 2, 4, 4, 2100, 64, [2100, 1300]),        # MHA, d_h 64
    ("bf16", 2, 12, 4, 257, 128, [257, 129]),         # r=3, lengths straddling tiles
    ("bf16", 4, 32, 8, 9000, 128, [9000, 8192, 4097, 33]),
    ("bf16", 1, 16, 1, 9000, 128, [9000]),            # r=16 on the 16x16 kernel, 36 splits
    ("bf16", 1, 8, 1, 6000, 64, [6000]),              # d_h 64, 24 splits (batched merge)
    ("f32", 3, 8, 2, 300, 40, [300, 151, 1]),
    ("f32", 1, 32, 1, 100, 128, [100]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "%s_B%d_hq%d_hkv%d_T%d_d%d" % c[:6])
def test_decode_parity(case):
    dt, B, h_q, h_kv, T_cap, d, lens = case
    print(f"case decode {case[:6]}", flush=True)
    x = inputs.make_decode(B, h_q, h_kv, d, T_cap, dt, 10000 + T_cap, seq_lens=lens, poison=True)
    got = _decode(x, dt)
    check_parity(got, _oracle_decode(x, dt), mode="f32" if dt == "f32" else "bf16", what=str(case[:6]))


def test_decode_explicit_positions_and_hint():
    # q_pos below seq_len - 1 hides the newer rows; max_seq_len sizes the grid
    x = inputs.make_decode(3, 16, 4, 128, 5000, "bf16", 11000, seq_lens=[5000, 4000, 3000], poison=True)
    qp = np.array([2500, 3999, 10], np.int32)
    got = _decode(x, "bf16", q_pos=qp, max_seq_len=5000)
    check_parity(got, _oracle_decode(x, "bf16", q_pos=qp), mode="bf16", what="q_pos")


def test_decode_out_bf16():
    x = inputs.make_decode(2, 8, 2, 128, 1500, "bf16", 11100, seq_lens=[1500, 700], poison=True)
    check_parity(_decode(x, "bf16", out_dtype="bf16"), _oracle_decode(x, "bf16"), mode="bf16out", what="bf16 out")


def test_decode_zero_length_writes_zeros():
    x = inputs.make_decode(2, 8, 2, 128, 600, "bf16", 11200, seq_lens=[0, 600])
    got = _decode(x, "bf16")
    assert np.all(got[0] == 0.0)
    xx = {k: (v[1:] if hasattr(v, "shape") and v.shape[:1] == (2,) else v) for k, v in x.items()}
    check_parity(got[1:], _oracle_decode(xx, "bf16"), mode="bf16", what="len 0")


@pytest.mark.parametrize("h_q,h_kv", [(16, 2), (64, 2)], ids=["r8_16x16", "r32_wide"])
def test_decode_longest_first_order(h_q, h_kv):
    """Workgroups take the sequences in order of visible length, longest first: a batch
    with equal lengths, a zero length and a spread of lengths matches the oracle on
    both kernels, and the zero-length sequence is written as zeros."""
    lens = [5000, 1, 0, 4096, 4096, 77, 2500, 5000, 640, 3333, 12, 4999]
    print(f"case decode longest-first h_q={h_q} h_kv={h_kv}", flush=True)
    x = inputs.make_decode(len(lens), h_q, h_kv, 128, 5000, "bf16", 11600 + h_q, seq_lens=lens, poison=True)
    got = _decode(x, "bf16")
    assert np.all(got[2] == 0.0)
    keep = [i for i, n in enumerate(lens) if n > 0]
    xx = {k: (v[keep] if hasattr(v, "shape") and v.shape[:1] == (len(lens),) else v) for k, v in x.items()}
    check_parity(got[keep], _oracle_decode(xx, "bf16"), mode="bf16", what="longest-first")


def test_decode_large_batch_natural_order():
    """More sequences than a workgroup has threads: grid order is kept (no ranking)."""
    rng = np.random.Generator(np.random.PCG64(11700))
    B = 300
    lens = rng.integers(1, 200, size=B, endpoint=True).astype(np.int32)
    print(f"case decode B={B} natural order", flush=True)
    x = inputs.make_decode(B, 8, 2, 64, 200, "bf16", 11700, seq_lens=lens, poison=True)
    check_parity(_decode(x, "bf16"), _oracle_decode(x, "bf16"), mode="bf16", what="B=300")


def test_decode_equals_last_prefill_row_bf16():
    import torch

    B, h_q, h_kv, T, d = 2, 8, 2, 700, 128
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 11300)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    pre = ops.gqa_prefill(q, k, v)
    dec = ops.gqa_decode(q[:, :, T - 1:].contiguous(), k, v, ints_dev([T, T]))
    torch.cuda.synchronize()
    a, b = to_host64(pre)[:, :, T - 1], to_host64(dec)[:, :, 0]
    assert np.max(np.abs(a - b)) <= 1e-2


def test_decode_deterministic():
    x = inputs.make_decode(2, 32, 8, 128, 4000, "bf16", 11400)
    assert np.array_equal(_decode(x, "bf16"), _decode(x, "bf16"))


def test_decode_reused_workspace():
    """One workspace reused by many calls, of two shapes in turn: the partial states of
    one call never leak into another (results bit-identical to the first call of each
    shape, which matches the oracle)."""
    import torch

    shapes = [(8, 32, 8, 8000, [8000, 7000, 6000, 5000, 4000, 3000, 2000, 1000]), (3, 16, 4, 5000, [5000, 64, 1])]
    ws_bytes = max(ops.gqa_decode_workspace_bytes(B, hq, hkv, T, 128, torch.bfloat16) for B, hq, hkv, T, _ in shapes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    runs = []
    for i, (B, hq, hkv, T, lens) in enumerate(shapes):
        x = inputs.make_decode(B, hq, hkv, 128, T, "bf16", 11500 + i, seq_lens=lens, poison=True)
        dev = (to_dev(x["q"], "bf16"), to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16"), ints_dev(x["seq_lens"]))
        runs.append((x, dev))
    first = [None, None]
    for it in range(40):
        for i, (x, (q, k, v, sl)) in enumerate(runs):
            o = ops.gqa_decode(q, k, v, sl, workspace=ws)
            torch.cuda.synchronize()
            got = to_host64(o)
            if first[i] is None:
                first[i] = got
                check_parity(got, _oracle_decode(x, "bf16"), mode="bf16", what=f"reused workspace shape {i}")
            else:
                assert np.array_equal(got, first[i]), (it, i)


# ---------------------------------------------------------------- kv_append
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 40), ("bf16", 3)])
def test_kv_append_bit_exact(dt, d):
    import torch

    B, h_kv, T_cap = 4, 3, 50
    k = inputs.normal(12000, "k", (B, h_kv, T_cap, d), dt)
    v = inputs.normal(12000, "v", (B, h_kv, T_cap, d), dt)
    kn = inputs.normal(12000, "k_new", (B, h_kv, 1, d), dt)
    vn = inputs.normal(12000, "v_new", (B, h_kv, 1, d), dt)
    wp = np.array([0, 49, 50, -1], np.int32)            # last two are out of range: skipped
    kd, vd = to_dev(k, dt), to_dev(v, dt)
    ops.gqa_kv_append(kd, vd, to_dev(kn, dt), to_dev(vn, dt), ints_dev(wp))
    torch.cuda.synchronize()
    view = np.int16 if dt == "bf16" else np.float32
    gk = kd.cpu().view(torch.int16).numpy() if dt == "bf16" else kd.cpu().numpy()
    gv = vd.cpu().view(torch.int16).numpy() if dt == "bf16" else vd.cpu().numpy()
    ek, ev = k.view(view).copy(), v.view(view).copy()
    for b in range(B):
        if 0 <= wp[b] < T_cap:
            ek[b, :, wp[b]] = kn.view(view)[b, :, 0]
            ev[b, :, wp[b]] = vn.view(view)[b, :, 0]
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


def test_append_then_decode_ragged_small():
    import torch

    B, h_q, h_kv, d = 6, 16, 2, 128
    T_cap = inputs.round_up(2000 + 1, 64)
    x = inputs.make_append_decode(B, h_q, h_kv, d, T_cap, "bf16", 12100, hist_hi=2000)
    kd, vd = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    ops.gqa_kv_append(kd, vd, to_dev(x["k_new"], "bf16"), to_dev(x["v_new"], "bf16"), ints_dev(x["write_pos"]))
    o = ops.gqa_decode(to_dev(x["q"], "bf16"), kd, vd, ints_dev(x["seq_lens"]), q_pos=ints_dev(x["q_pos"]),
                       max_seq_len=int(x["seq_lens"].max()))
    torch.cuda.synchronize()
    got = to_host64(o)
    k = x["k_cache"].copy()
    v = x["v_cache"].copy()
    for b in range(B):
        k[b, :, x["hist"][b]] = x["k_new"][b, :, 0]
        v[b, :, x["hist"][b]] = x["v_new"][b, :, 0]
    want = _oracle_decode({"q": x["q"], "k_cache": k, "v_cache": v, "seq_lens": x["seq_lens"]}, "bf16",
                          q_pos=x["q_pos"])
    check_parity(got, want, mode="bf16", what="append+decode")


# ---------------------------------------------------------------- fused append + decode
def _append_then_decode(x, kn, vn, wp, dt, fused):
    """One decode step on fresh device copies of the caches: kv_append then decode as two
    calls, or the fused call.  Returns (o, k_cache, v_cache) on the host, bit for bit."""
    import torch

    q, kd, vd = to_dev(x["q"], dt), to_dev(x["k_cache"], dt), to_dev(x["v_cache"], dt)
    knd, vnd, wpd, sl = to_dev(kn, dt), to_dev(vn, dt), ints_dev(wp), ints_dev(x["seq_lens"])
    if fused:
        o = ops.gqa_append_decode(q, kd, vd, knd, vnd, wpd, sl)
    else:
        ops.gqa_kv_append(kd, vd, knd, vnd, wpd)
        o = ops.gqa_decode(q, kd, vd, sl)
    torch.cuda.synchronize()
    bits = (lambda t: t.cpu().view(torch.int16).numpy()) if dt == "bf16" else (lambda t: t.cpu().view(torch.int32).numpy())
    return o.cpu().numpy(), bits(kd), bits(vd)


APPEND_CASES = [
    # dtype, B, h_q, h_kv, T_cap, d_h, seq_lens, write_pos
    ("bf16", 6, 16, 2, 2048, 128, [1000, 64, 65, 1, 2048, 700], [999, 63, 64, 0, 2047, 699]),   # the usual step
    ("bf16", 5, 16, 2, 2048, 128, [1000, 64, 500, 300, 9], [1005, -1, 2048, 127, 8]),   # invisible, skipped rows
    ("bf16", 3, 8, 8, 3000, 64, [3000, 1500, 2], [2999, 1499, 1]),      # MHA, d_h 64
    ("bf16", 3, 64, 2, 1500, 128, [1500, 700, 3], [1499, 699, 2]),      # r = 32: append and decode launched apart
    ("f32", 3, 8, 2, 300, 40, [300, 151, 1], [299, 150, 0]),            # fp32 path
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=lambda c: "%s_B%d_hq%d_hkv%d_T%d_d%d" % c[:6])
def test_append_decode_equals_two_calls(case):
    """The fused call leaves the same caches and writes the same output, bit for bit, as
    kv_append followed by decode: rows at and across tile edges, a write position past the
    visible keys (written, never read), positions outside the cache (skipped), and the
    shapes that keep two launches."""
    dt, B, h_q, h_kv, T_cap, d, lens, wp = case
    print(f"case append+decode {case[:6]}", flush=True)
    x = inputs.make_decode(B, h_q, h_kv, d, T_cap, dt, 12500 + T_cap, seq_lens=lens, poison=True)
    kn = inputs.normal(12500 + T_cap, "k_new", (B, h_kv, 1, d), dt)
    vn = inputs.normal(12500 + T_cap, "v_new", (B, h_kv, 1, d), dt)
    o2, k2, v2 = _append_then_decode(x, kn, vn, np.array(wp, np.int32), dt, fused=False)
    o1, k1, v1 = _append_then_decode(x, kn, vn, np.array(wp, np.int32), dt, fused=True)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert np.array_equal(o1, o2, equal_nan=True)


def test_append_decode_ragged_parity():
    """Fused step on a ragged batch against the oracle over the appended caches."""
    import torch

    B, h_q, h_kv, d = 8, 32, 4, 128
    T_cap = inputs.round_up(3000 + 1, 64)
    x = inputs.make_append_decode(B, h_q, h_kv, d, T_cap, "bf16", 12600, hist_hi=3000)
    kd, vd = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    o = ops.gqa_append_decode(to_dev(x["q"], "bf16"), kd, vd, to_dev(x["k_new"], "bf16"),
                              to_dev(x["v_new"], "bf16"), ints_dev(x["write_pos"]), ints_dev(x["seq_lens"]),
                              q_pos=ints_dev(x["q_pos"]), max_seq_len=int(x["seq_lens"].max()))
    torch.cuda.synchronize()
    k = x["k_cache"].copy()
    v = x["v_cache"].copy()
    for b in range(B):
        k[b, :, x["hist"][b]] = x["k_new"][b, :, 0]
        v[b, :, x["hist"][b]] = x["v_new"][b, :, 0]
    want = _oracle_decode({"q": x["q"], "k_cache": k, "v_cache": v, "seq_lens": x["seq_lens"]}, "bf16",
                          q_pos=x["q_pos"])
    check_parity(to_host64(o), want, mode="bf16", what="fused append+decode")
    assert np.array_equal(kd.cpu().view(torch.int16).numpy(), k.view(np.int16))


# Kernel paths the shapes below reach (split plan for the bf16 path):
#   r > 16, T_cap <= 256        -> wide kernel, one split, output written directly
#   r > 16, T_cap = 3000        -> wide kernel, 12 splits, batched merge
#   r = 16, T_cap = 9000        -> 16x16 kernel, 36 splits, batched merge
#   r = 4,  T_cap = 1500        -> 16x16 kernel, 6 splits, plain merge
PATH_CASES = [
    # B, h_q, h_kv, T_cap, d_h, lens
    (2, 32, 1, 200, 128, [200, 77]),
    (2, 32, 1, 200, 64, [200, 3]),
    (2, 64, 2, 3000, 64, [3000, 1999]),
    (2, 32, 1, 3000, 128, [3000, 2048]),
    (1, 16, 1, 9000, 128, [9000]),
    (2, 8, 2, 1500, 64, [1500, 700]),
]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: "B%d_hq%d_hkv%d_T%d_d%d" % c[:5])
def test_decode_kernel_paths_and_output_dtypes(case, out_dtype):
    """Every decode kernel path (wide kernel at d_h 64 and 128, direct write, plain
    and batched merge) with fp32 and bf16 output, against the oracle."""
    B, h_q, h_kv, T_cap, d, lens = case
    print(f"case decode path {case[:5]} out {out_dtype}", flush=True)
    x = inputs.make_decode(B, h_q, h_kv, d, T_cap, "bf16", 12000 + T_cap + d, seq_lens=lens, poison=True)
    got = _decode(x, "bf16", out_dtype=out_dtype)
    check_parity(got, _oracle_decode(x, "bf16"), mode="bf16out" if out_dtype == "bf16" else "bf16",
                 what=f"{case[:5]} {out_dtype}")


@pytest.mark.parametrize("h_q,h_kv", [(16, 4), (64, 2)], ids=["r4_16x16", "r32_wide"])
def test_decode_max_seq_len_truncates_visibility(h_q, h_kv):
    """max_seq_len below a sequence's length hides the keys at and past it: the
    visible keys are j < min(seq_lens[b], q_pos[b] + 1, max_seq_len), checked
    against the oracle with the history cut there."""
    lens = np.array([5000, 4000, 3000, 900], np.int32)
    msl = 3500
    print(f"case decode max_seq_len {msl} h_q={h_q} h_kv={h_kv}", flush=True)
    x = inputs.make_decode(len(lens), h_q, h_kv, 128, 5000, "bf16", 12500 + h_q, seq_lens=lens, poison=True)
    got = _decode(x, "bf16", max_seq_len=msl)
    want = []
    for b in range(len(lens)):
        L = int(min(lens[b], msl))
        want.append(oracle.attention(f64(x["q"][b:b + 1], "bf16"), f64(x["k_cache"][b:b + 1, :, :L], "bf16"),
                                     f64(x["v_cache"][b:b + 1, :, :L], "bf16"), causal=True,
                                     q_pos=np.array([[lens[b] - 1]]), kv_len=np.array([L]))[0])
    check_parity(got, np.stack(want), mode="bf16", what=f"max_seq_len {msl}")
