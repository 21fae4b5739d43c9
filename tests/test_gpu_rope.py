"""GPU parity of rotary position encoding against the float64 oracle.

gqa_rope and gqa_kv_append_rope are compared element by element with
``oracle.rope`` on the same seeded inputs (fp32: absolute 1e-5; bf16 output:
one bf16 unit in the last place of the expected value -- the output's rounding --
plus 1e-6 of the pair's magnitude for the fp32 arithmetic, with nearly all
elements within half a unit).  The end-to-end cases feed
the rotated rows to prefill and decode and compare with the oracle's attention
over the oracle's rotated rows, rounded to bf16 the way the kernel's inputs are.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import bf16_half_ulp, check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _bf16_round(x64):
    return inputs.f32_to_bf16_bits(np.asarray(x64, dtype=np.float32))


def _pair_mag(x):
    d = x.shape[-1]
    m = np.abs(x[..., : d // 2]) + np.abs(x[..., d // 2:])
    return np.concatenate([m, m], axis=-1)


def _check_rope(got, want, dtype, what, x=None):
    """fp32: absolute 1e-5.  bf16: within one bf16 ulp of the expected value plus the
    fp32 arithmetic's share, 1e-6 of the pair's magnitude (that share decides the
    rounding where the two terms of a rotated element cancel)."""
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - want)
    if dtype == "f32":
        assert err.max() <= 1e-5, f"{what}: max-abs {err.max():.3g}"
        return
    hu = bf16_half_ulp(want)
    slack = 1e-6 * _pair_mag(x) if x is not None else 0.0
    assert np.all(err <= 2 * hu + slack), f"{what}: {np.max((err - slack) / hu):.3f} half-ulps"
    assert np.mean(err <= hu + slack) > 0.999, f"{what}: too many results off the nearest bf16"


ROPE_CASES = [
    # dtype, B, H, S, d, pos0
    ("bf16", 2, 8, 300, 128, [0, 31000]),
    ("bf16", 1, 4, 64, 64, [12345]),
    ("f32", 2, 3, 50, 40, [0, 32767]),
    ("f32", 1, 2, 7, 2, None),
    ("f32", 3, 2, 33, 256, [5, 0, 20000]),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: "%s_B%d_H%d_S%d_d%d" % c[:5])
def test_rope_parity(case):
    import torch

    dt, B, H, S, d, pos0 = case
    print(f"case rope {case[:5]}", flush=True)
    x = inputs.normal(13000 + d, "q", (B, H, S, d), dt)
    p0 = np.zeros(B, np.int64) if pos0 is None else np.asarray(pos0)
    y = ops.gqa_rope(to_dev(x, dt), pos0=None if pos0 is None else ints_dev(pos0))
    torch.cuda.synchronize()
    want = oracle.rope(f64(x, dt), p0[:, None, None] + np.arange(S)[None, None, :])
    _check_rope(to_host64(y), want, dt, str(case[:5]), x=f64(x, dt))


def test_rope_in_place_equals_out_of_place():
    import torch

    x = inputs.normal(13100, "q", (2, 4, 100, 128), "bf16")
    a = to_dev(x, "bf16")
    b = ops.gqa_rope(a, pos0=ints_dev([7, 4000]))
    ops.gqa_rope(a, pos0=ints_dev([7, 4000]), out=a)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dt,h_q,h_kv,S,d,offset", [("bf16", 32, 8, 300, 128, 0), ("f32", 8, 2, 77, 64, 0),
                                                  ("bf16", 6, 3, 50, 64, 1), ("bf16", 4, 1, 33, 18, 0)],
                         ids=["bf16_vec8", "f32_vec4", "bf16_misaligned", "bf16_d18"])
def test_rope_qk_one_launch_equals_two_calls(dt, h_q, h_kv, S, d, offset):
    import torch

    print(f"case rope_qk {dt} {h_q} {h_kv} {S} {d} {offset}", flush=True)
    xq = inputs.normal(13300 + d, "q", (2, h_q, S, d), dt)
    xk = inputs.normal(13300 + d, "k", (2, h_kv, S, d), dt)
    q, k = to_dev(xq, dt), to_dev(xk, dt)
    if offset:   # one element into a larger buffer: not 16-byte aligned, so the element-wise path
        qb = torch.empty(q.numel() + offset, dtype=q.dtype, device="cuda")
        qb[offset:] = q.flatten()
        q = qb[offset:].view(q.shape)
    pos = ints_dev([5, 9000])
    qa, ka = ops.gqa_rope_qk(q, k, pos0=pos)
    qb_, kb_ = ops.gqa_rope(q, pos0=pos), ops.gqa_rope(k, pos0=pos)
    torch.cuda.synchronize()
    iv = (lambda t: t.view(torch.int16)) if dt == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(iv(qa), iv(qb_)) and torch.equal(iv(ka), iv(kb_))
    want = oracle.rope(f64(xk, dt), np.array([5, 9000])[:, None, None] + np.arange(S)[None, None, :])
    _check_rope(to_host64(ka), want, dt, "rope_qk k", x=f64(xk, dt))
    # in place
    ops.gqa_rope_qk(q, k, pos0=pos, q_out=q, k_out=k)
    torch.cuda.synchronize()
    assert torch.equal(iv(q), iv(qb_)) and torch.equal(iv(k), iv(kb_))


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_kv_append_rope(dt, d):
    import torch

    B, h_kv, T_cap = 4, 3, 40
    k = inputs.normal(13200, "k", (B, h_kv, T_cap, d), dt)
    v = inputs.normal(13200, "v", (B, h_kv, T_cap, d), dt)
    kn = inputs.normal(13200, "k_new", (B, h_kv, 1, d), dt)
    vn = inputs.normal(13200, "v_new", (B, h_kv, 1, d), dt)
    wp = np.array([0, 39, 40, 17], np.int32)                 # 40 is out of range: skipped
    kd, vd = to_dev(k, dt), to_dev(v, dt)
    knd = to_dev(kn, dt)
    ops.gqa_kv_append_rope(kd, vd, knd, to_dev(vn, dt), ints_dev(wp))
    # the same rotation through gqa_rope (one row per sequence at write_pos)
    ref = ops.gqa_rope(knd, pos0=ints_dev(wp))
    torch.cuda.synchronize()
    view = torch.int16 if dt == "bf16" else torch.int32
    gk = kd.cpu()
    gv = vd.cpu()
    for b in range(B):
        if not 0 <= wp[b] < T_cap:
            continue
        assert torch.equal(gk[b, :, wp[b]].view(view), ref.cpu()[b, :, 0].view(view))
        want = oracle.rope(f64(kn[b, :, 0], dt), np.full(h_kv, wp[b]))
        _check_rope(gk[b, :, wp[b]].float().numpy().astype(np.float64), want, dt, f"b={b}", x=f64(kn[b, :, 0], dt))
        assert torch.equal(gv[b, :, wp[b]].view(view), torch.from_numpy(np.ascontiguousarray(vn[b, :, 0])).view(view)
                           if dt == "f32" else torch.from_numpy(vn[b, :, 0].view(np.int16)))
    # every other row untouched
    mask = np.ones((B, T_cap), bool)
    for b in range(B):
        if 0 <= wp[b] < T_cap:
            mask[b, wp[b]] = False
    host_k = gk.view(view).numpy() if dt == "bf16" else gk.numpy().view(np.int32)
    orig_k = k.view(np.int16) if dt == "bf16" else k.view(np.int32)
    for b in range(B):
        assert np.array_equal(host_k[b][:, mask[b]], orig_k[b][:, mask[b]])


def test_rope_then_prefill():
    import torch

    B, h_q, h_kv, T, d = 1, 8, 2, 700, 128
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 13300)
    qd, kd, vd = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o = ops.gqa_prefill(ops.gqa_rope(qd), ops.gqa_rope(kd), vd)
    torch.cuda.synchronize()
    pos = np.arange(T)
    qr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["q"], "bf16"), pos))).astype(np.float64)
    kr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["k"], "bf16"), pos))).astype(np.float64)
    want = oracle.attention(qr, kr, f64(x["v"], "bf16"), causal=True)
    check_parity(to_host64(o), want, mode="bf16", what="rope+prefill")


def test_rope_append_decode():
    # prompt keys rotated at their positions, the new key rotated inside the append,
    # the query rotated at its absolute position, then decode
    import torch

    B, h_q, h_kv, d = 4, 16, 4, 128
    T_cap = inputs.round_up(3000 + 1, 64)
    x = inputs.make_append_decode(B, h_q, h_kv, d, T_cap, "bf16", 13400, hist_hi=3000)
    hist = x["hist"]
    k_hist = np.nan_to_num(f64(x["k_cache"], "bf16"))             # NaN rows beyond each history
    kd = ops.gqa_rope(to_dev(x["k_cache"], "bf16"))               # whole cache, positions 0..T_cap-1
    vd = to_dev(x["v_cache"], "bf16")
    ops.gqa_kv_append_rope(kd, vd, to_dev(x["k_new"], "bf16"), to_dev(x["v_new"], "bf16"), ints_dev(x["write_pos"]))
    qd = ops.gqa_rope(to_dev(x["q"], "bf16"), pos0=ints_dev(x["q_pos"]))
    o = ops.gqa_decode(qd, kd, vd, ints_dev(x["seq_lens"]), q_pos=ints_dev(x["q_pos"]),
                       max_seq_len=int(x["seq_lens"].max()))
    torch.cuda.synchronize()
    got = to_host64(o)
    for b in range(B):
        L = int(x["seq_lens"][b])
        k = k_hist[b:b + 1, :, :L].copy()
        k[0, :, hist[b]] = f64(x["k_new"][b, :, 0], "bf16")
        v = f64(x["v_cache"][b:b + 1, :, :L], "bf16").copy()
        v[0, :, hist[b]] = f64(x["v_new"][b, :, 0], "bf16")
        kr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(k, np.arange(L)))).astype(np.float64)
        qr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["q"][b:b + 1], "bf16"),
                                                             np.array([hist[b]])))).astype(np.float64)
        want = oracle.attention(qr, kr, v, causal=True, q_pos=np.array([[hist[b]]]), kv_len=np.array([L]))
        check_parity(got[b:b + 1], want, mode="bf16", what=f"rope decode b={b}")


# ---------------------------------------------------------------- rotation inside the attention kernels
@pytest.mark.parametrize("d,lens,out_dtype", [(128, None, None), (64, [700, 333], "bf16")],
                         ids=["d128", "d64_padded_bf16out"])
def test_prefill_rope_fused_equals_rope_then_prefill(d, lens, out_dtype):
    """Q rotated as the prefill kernel loads it: bit-identical to gqa_rope on Q then
    gqa_prefill, and within the bf16 bounds of the oracle over rotated rows."""
    import torch

    B, h_q, h_kv, T = 2, 8, 2, 700
    print(f"case prefill_rope d={d} lens={lens}", flush=True)
    x = inputs.make_prefill(B, h_q, h_kv, d, T, "bf16", 13500 + d)
    qd, kd, vd = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    od = None if out_dtype is None else torch.bfloat16
    kv = None if lens is None else ints_dev(lens)
    krot = ops.gqa_rope(kd)
    o_sep = ops.gqa_prefill(ops.gqa_rope(qd), krot, vd, kv_lens=kv, out_dtype=od)
    o_fused = ops.gqa_prefill_rope(qd, krot, vd, kv_lens=kv, out_dtype=od)
    torch.cuda.synchronize()
    assert torch.equal(o_fused, o_sep)
    if lens is None:
        pos = np.arange(T)
        qr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["q"], "bf16"), pos))).astype(np.float64)
        kr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["k"], "bf16"), pos))).astype(np.float64)
        want = oracle.attention(qr, kr, f64(x["v"], "bf16"), causal=True)
        check_parity(to_host64(o_fused), want, mode="bf16", what="fused rope prefill")


@pytest.mark.parametrize("h_q,h_kv,d,qpos", [(16, 4, 128, True), (8, 8, 64, False), (64, 2, 128, True)],
                         ids=["r4", "mha_d64_default_pos", "r32_two_launches"])
def test_append_decode_rope_equals_separate_calls(h_q, h_kv, d, qpos):
    """The decode step with rotary encoding in one call -- new key rotated at its write
    position, query at its position -- against gqa_kv_append_rope, gqa_rope on the
    query and gqa_decode: same caches and output, bit for bit."""
    import torch

    B = 5
    T_cap = inputs.round_up(2500 + 1, 64)
    print(f"case append_decode_rope h_q={h_q} h_kv={h_kv} d={d}", flush=True)
    x = inputs.make_append_decode(B, h_q, h_kv, d, T_cap, "bf16", 13600 + h_q + d, hist_hi=2500)
    kd0 = ops.gqa_rope(to_dev(x["k_cache"], "bf16"))          # prompt keys, rotated at their positions
    vd0 = to_dev(x["v_cache"], "bf16")
    q, kn, vn = to_dev(x["q"], "bf16"), to_dev(x["k_new"], "bf16"), to_dev(x["v_new"], "bf16")
    wp, sl, msl = ints_dev(x["write_pos"]), ints_dev(x["seq_lens"]), int(x["seq_lens"].max())
    qp = ints_dev(x["q_pos"]) if qpos else None
    k1, v1 = kd0.clone(), vd0.clone()
    ops.gqa_kv_append_rope(k1, v1, kn, vn, wp)
    o1 = ops.gqa_decode(ops.gqa_rope(q, pos0=ints_dev(x["q_pos"])), k1, v1, sl, q_pos=qp, max_seq_len=msl)
    k2, v2 = kd0.clone(), vd0.clone()
    o2 = ops.gqa_append_decode_rope(q, k2, v2, kn, vn, wp, sl, q_pos=qp, max_seq_len=msl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)) and torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert bool(torch.isfinite(o2).all())


@pytest.mark.parametrize("explicit_pos", [True, False], ids=["q_pos0", "newest_rows"])
def test_prefill_chunk_rope_equals_rope_then_chunk(explicit_pos):
    """Chunked prefill with Q rotated in the kernel at each row's absolute position:
    bit-identical to gqa_rope at those positions followed by gqa_prefill_chunk."""
    import torch

    B, h_q, h_kv, S_q, T_cap, d = 3, 16, 4, 100, 1000, 128
    print(f"case prefill_chunk_rope explicit={explicit_pos}", flush=True)
    x = inputs.make_decode(B, h_q, h_kv, d, T_cap, "bf16", 13700, seq_lens=[1000, 640, 101])
    q = to_dev(inputs.normal(13700, "q", (B, h_q, S_q, d), "bf16"), "bf16")
    kc = ops.gqa_rope(to_dev(x["k_cache"], "bf16"))
    vc = to_dev(x["v_cache"], "bf16")
    lens = np.array([1000, 640, 101], np.int32)
    pos0 = np.array([900, 200, 1], np.int32) if explicit_pos else lens - S_q
    qp = ints_dev(pos0) if explicit_pos else None
    q_host = inputs.normal(13700, "q", (B, h_q, S_q, d), "bf16")
    o_sep = ops.gqa_prefill_chunk(ops.gqa_rope(q, pos0=ints_dev(pos0)), kc, vc, kv_lens=ints_dev(lens), q_pos0=qp)
    o_fused = ops.gqa_prefill_chunk_rope(q, kc, vc, kv_lens=ints_dev(lens), q_pos0=qp)
    torch.cuda.synchronize()
    assert torch.equal(o_fused, o_sep)
    assert bool(torch.isfinite(o_fused).all())
    # and against the oracle: keys rotated at 0..T_cap-1, query row i at pos0[b] + i,
    # both rounded to bf16 as the kernels' operands are
    qpos = pos0[:, None].astype(np.int64) + np.arange(S_q)[None]
    kr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["k_cache"], "bf16"), np.arange(T_cap)))).astype(np.float64)
    qr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(q_host, "bf16"), qpos[:, None, :]))).astype(np.float64)
    want = oracle.attention(qr, kr, f64(x["v_cache"], "bf16"), causal=True, q_pos=qpos, kv_len=lens)
    check_parity(to_host64(o_fused), want, mode="bf16", what=f"chunk rope explicit={explicit_pos}")


@pytest.mark.parametrize("d", [128, 64])
def test_append_decode_rope_edge_positions(d):
    """Write positions on tile edges, past the visible keys (written rotated, never
    read) and outside the cache (skipped): the fused rotating step leaves the same
    caches and output as gqa_kv_append_rope, gqa_rope on the query and gqa_decode."""
    import torch

    B, h_q, h_kv, T_cap = 6, 16, 2, 1024
    lens = np.array([1000, 64, 65, 500, 300, 9], np.int32)
    wp = np.array([999, 63, 64, 505, -1, 1024], np.int32)
    print(f"case append_decode_rope edges d={d}", flush=True)
    x = inputs.make_decode(B, h_q, h_kv, d, T_cap, "bf16", 13800 + d, seq_lens=lens, poison=True)
    kn = to_dev(inputs.normal(13800 + d, "k_new", (B, h_kv, 1, d), "bf16"), "bf16")
    vn = to_dev(inputs.normal(13800 + d, "v_new", (B, h_kv, 1, d), "bf16"), "bf16")
    k0, v0 = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    q, sl, wpd = to_dev(x["q"], "bf16"), ints_dev(lens), ints_dev(wp)
    k1, v1 = k0.clone(), v0.clone()
    ops.gqa_kv_append_rope(k1, v1, kn, vn, wpd)
    o1 = ops.gqa_decode(ops.gqa_rope(q, pos0=ints_dev(lens - 1)), k1, v1, sl)
    k2, v2 = k0.clone(), v0.clone()
    o2 = ops.gqa_append_decode_rope(q, k2, v2, kn, vn, wpd, sl)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)) and torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert torch.equal(o1, o2)
    # and against the oracle: the cache rows as given, except an appended row inside the
    # visible range, which holds the new key rotated at its write position; the query
    # rotated at its position lens[b] - 1
    kn_h = inputs.normal(13800 + d, "k_new", (B, h_kv, 1, d), "bf16")
    vn_h = inputs.normal(13800 + d, "v_new", (B, h_kv, 1, d), "bf16")
    got = to_host64(o2)
    for b in range(B):
        L = int(lens[b])
        k = f64(x["k_cache"][b:b + 1, :, :L], "bf16").copy()
        v = f64(x["v_cache"][b:b + 1, :, :L], "bf16").copy()
        if 0 <= wp[b] < L:
            rot = oracle.rope(f64(kn_h[b:b + 1], "bf16"), np.array([[wp[b]]]))
            k[0, :, wp[b]] = inputs.bf16_bits_to_f32(_bf16_round(rot)).astype(np.float64)[0, :, 0]
            v[0, :, wp[b]] = f64(vn_h[b, :, 0], "bf16")
        qr = inputs.bf16_bits_to_f32(_bf16_round(oracle.rope(f64(x["q"][b:b + 1], "bf16"),
                                                             np.array([[L - 1]])))).astype(np.float64)
        want = oracle.attention(qr, k, v, causal=True, q_pos=np.array([[L - 1]]), kv_len=np.array([L]))
        check_parity(got[b:b + 1], want, mode="bf16", what=f"rope decode edges b={b} wp={wp[b]}")
