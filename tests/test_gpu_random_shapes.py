"""GPU parity on randomly drawn shapes: prefill, chunked prefill, decode and paged decode.

The shapes come from one seeded generator (printed in each case id), so a failure
names a reproducible configuration.  Each draw mixes what the named cases fix one
at a time: head ratios 1..64 (MHA, GQA, MQA), d_h 64 and 128, lengths that end
anywhere inside a tile (1 included), causal and full masks, explicit and default
positions, padded key lengths, fp32 and bf16 outputs, and page sizes 64 and 128.
Every output element is compared with the float64 oracle at the bf16 bar.
"""

import numpy as np
import pytest

import oracle
from grouped_query_attention_prefill_amd import inputs, ops
from tests.gpu_util import check_parity, f64, ints_dev, to_dev, to_host64

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


def _heads(rng):
    h_kv = int(rng.choice([1, 2, 4, 8]))
    r = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32, 64]))
    while h_kv * r > 128:
        r //= 2
    return h_kv * r, h_kv


def _draw(kind, i):
    rng = np.random.default_rng([20261204, ["prefill", "chunk", "decode", "paged"].index(kind), i])
    h_q, h_kv = _heads(rng)
    c = {"kind": kind, "seed": 30000 + 1000 * ["prefill", "chunk", "decode", "paged"].index(kind) + i,
         "h_q": h_q, "h_kv": h_kv,
         "d": int(rng.choice([64, 128])), "B": int(rng.integers(1, 4)),
         "out": str(rng.choice(["f32", "bf16"]))}
    if kind == "prefill":
        c["T"] = int(rng.integers(1, 600))
        c["causal"] = bool(rng.integers(0, 2))
        c["lens"] = rng.integers(1, c["T"] + 1, size=c["B"]).tolist() if rng.integers(0, 2) else None
    elif kind == "chunk":
        c["T_cap"] = int(rng.integers(2, 900))
        c["S_q"] = int(rng.integers(1, min(c["T_cap"], 300) + 1))
        c["lens"] = rng.integers(c["S_q"], c["T_cap"] + 1, size=c["B"]).tolist()
        c["pos0"] = [int(rng.integers(0, L - c["S_q"] + 1)) for L in c["lens"]] if rng.integers(0, 2) else None
        c["causal"] = bool(rng.integers(0, 2))
    else:
        c["B"] = int(rng.integers(1, 6))
        page = int(rng.choice([64, 128]))
        T_cap = int(rng.integers(1, 4000))
        if kind == "paged":
            T_cap = (T_cap + page - 1) // page * page
            c["page"] = page
        c["T_cap"] = T_cap
        c["lens"] = rng.integers(1, T_cap + 1, size=c["B"]).tolist()
        c["q_pos"] = [int(rng.integers(0, L)) for L in c["lens"]] if rng.integers(0, 2) else None
        c["clamp"] = int(rng.integers(1, max(c["lens"]) + 1)) if rng.integers(0, 4) == 0 else None
    return c


CASES = [_draw(k, i) for k in ("prefill", "chunk", "decode", "paged") for i in range(8)]


def _id(c):
    keys = [k for k in ("B", "h_q", "h_kv", "d", "T", "T_cap", "S_q") if k in c]
    return c["kind"] + "_" + "_".join(f"{k}{c[k]}" for k in keys) + f"_s{c['seed']}"


def _mode(c):
    return "bf16out" if c["out"] == "bf16" else "bf16"


def _out_dtype(c):
    import torch

    return torch.bfloat16 if c["out"] == "bf16" else torch.float32


def _prefill(c):
    import torch

    x = inputs.make_prefill(c["B"], c["h_q"], c["h_kv"], c["d"], c["T"], "bf16", c["seed"])
    lens = None if c["lens"] is None else np.asarray(c["lens"], np.int32)
    o = ops.gqa_prefill(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), causal=c["causal"],
                        kv_lens=None if lens is None else ints_dev(lens), out_dtype=_out_dtype(c))
    torch.cuda.synchronize()
    want = oracle.attention(f64(x["q"], "bf16"), f64(x["k"], "bf16"), f64(x["v"], "bf16"), causal=c["causal"],
                            kv_len=lens)
    return to_host64(o), want


def _chunk(c):
    import torch

    B, S_q, T_cap, d = c["B"], c["S_q"], c["T_cap"], c["d"]
    q = inputs.normal(c["seed"], "q", (B, c["h_q"], S_q, d), "bf16")
    k = inputs.normal(c["seed"], "k", (B, c["h_kv"], T_cap, d), "bf16")
    v = inputs.normal(c["seed"], "v", (B, c["h_kv"], T_cap, d), "bf16")
    lens = np.asarray(c["lens"], np.int32)
    pos0 = None if c["pos0"] is None else np.asarray(c["pos0"], np.int32)
    o = ops.gqa_prefill_chunk(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), kv_lens=ints_dev(lens),
                              q_pos0=None if pos0 is None else ints_dev(pos0), causal=c["causal"],
                              out_dtype=_out_dtype(c))
    torch.cuda.synchronize()
    qp = None if pos0 is None else pos0[:, None] + np.arange(S_q)[None]
    want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), causal=c["causal"], q_pos=qp,
                            kv_len=lens)
    return to_host64(o), want


def _paginate(cache, page, seed):
    B, h, T, d = cache.shape
    mp = T // page
    n_pages = B * mp + 2
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * mp].reshape(B, mp)
    pool = np.full((n_pages, h, page, d), NAN_BF16, dtype=cache.dtype)
    for b in range(B):
        for j in range(mp):
            pool[perm[b, j]] = cache[b, :, j * page:(j + 1) * page]
    return pool, perm.astype(np.int32)


def _decode(c):
    import torch

    x = inputs.make_decode(c["B"], c["h_q"], c["h_kv"], c["d"], c["T_cap"], "bf16", c["seed"], seq_lens=c["lens"],
                           poison=True)
    lens = np.asarray(c["lens"], np.int32)
    qp = None if c["q_pos"] is None else np.asarray(c["q_pos"], np.int32)
    args = dict(q_pos=None if qp is None else ints_dev(qp), max_seq_len=c["clamp"], out_dtype=_out_dtype(c))
    if c["kind"] == "paged":
        kp, bt = _paginate(x["k_cache"], c["page"], c["seed"])
        vp, _ = _paginate(x["v_cache"], c["page"], c["seed"])
        o = ops.gqa_decode_paged(to_dev(x["q"], "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"), ints_dev(bt),
                                 ints_dev(lens), **args)
    else:
        o = ops.gqa_decode(to_dev(x["q"], "bf16"), to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16"),
                           ints_dev(lens), **args)
    torch.cuda.synchronize()
    # keys visible to sequence b: j < min(len_b, q_pos_b + 1, max_seq_len)
    pos = lens - 1 if qp is None else qp
    out = []
    for b in range(c["B"]):
        n = int(min(lens[b], pos[b] + 1, c["clamp"] if c["clamp"] is not None else lens[b]))
        out.append(oracle.attention(f64(x["q"][b:b + 1], "bf16"), f64(x["k_cache"][b:b + 1, :, :n], "bf16"),
                                    f64(x["v_cache"][b:b + 1, :, :n], "bf16"), causal=False,
                                    kv_len=np.array([n]))[0])
    return to_host64(o), np.stack(out)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_random_shape_parity(case):
    print(f"case {case}", flush=True)
    run = {"prefill": _prefill, "chunk": _chunk, "decode": _decode, "paged": _decode}[case["kind"]]
    got, want = run(case)
    check_parity(got, want, mode=_mode(case), what=_id(case))
