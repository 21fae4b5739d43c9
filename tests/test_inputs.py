"""The seeded input generators: bf16 rounding, determinism, ragged lengths, poisoning."""

import numpy as np

from grouped_query_attention_prefill_amd import inputs


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.00390625, 1.01171875, 1.0078125 + 2 ** -9, -2.5, 3.0e38, np.inf], dtype=np.float32)
    b = inputs.f32_to_bf16_bits(f)
    back = inputs.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    assert back[0] == 1.0 and back[1] == 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: rounds to even (1 + 2^-6)
    assert back[2] == np.float32(1.015625)
    # above the tie rounds up
    assert back[3] == np.float32(1.0078125)
    assert back[4] == -2.5 and np.isinf(back[6])
    nan = inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(inputs.bf16_bits_to_f32(nan))[0]


def test_bf16_widening_is_exact():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000).astype(np.float32)
    b = inputs.f32_to_bf16_bits(x)
    w = inputs.bf16_bits_to_f32(b)
    assert np.all(inputs.f32_to_bf16_bits(w) == b)
    assert np.max(np.abs(w - x) / np.abs(x)) <= 2 ** -8


def test_determinism_and_stream_keys():
    a = inputs.make_prefill(1, 4, 2, 8, 5, "bf16", 1950)
    b = inputs.make_prefill(1, 4, 2, 8, 5, "bf16", 1950)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    q0 = inputs.rng_for(1950, inputs.TENSOR_IDS["q"], 0).standard_normal((4, 5, 8), dtype=np.float32)
    assert np.array_equal(inputs.bf16_bits_to_f32(a["q"][0]), inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(q0)))


def test_ragged_lengths_and_poison():
    x = inputs.make_append_decode(6, 4, 2, 8, 80, "bf16", 1953, hist_hi=64)
    h = x["hist"]
    assert h.min() >= 1 and h.max() <= 64
    assert np.array_equal(x["seq_lens"], h + 1) and np.array_equal(x["q_pos"], h)
    k = inputs.bf16_bits_to_f32(x["k_cache"])
    for b in range(6):
        assert np.all(np.isfinite(k[b, :, : h[b]]))
        assert np.all(np.isnan(k[b, :, h[b]:]))


def test_named_workloads():
    w = inputs.WORKLOADS
    assert w["prefill_causal_bf16_T4096"].T == 4096 and w["prefill_causal_bf16_T4096"].seed == 1950
    assert w["decode_mqa_B8_T32000"].h_kv == 1
    assert w["ragged_append_decode_B32"].T == 32832
    x = inputs.make_workload(w["tiny_prefill_f32"])
    assert x["q"].dtype == np.float32 and x["q"].shape == (1, 4, 3, 2)


def test_normal_row_matches_full_draw():
    full = inputs.normal(77, "k", (3, 2, 5, 4), "bf16")
    for b in range(3):
        assert np.array_equal(inputs.normal_row(77, "k", b, (2, 5, 4), "bf16"), full[b])


def test_ragged_workload_lengths_follow_the_plain_generator():
    """History lengths of the ragged workload: Generator(PCG64(1953)).integers(1, 32768,
    32, endpoint=True), drawn before any tensor; with the appended token the 32
    sequences hold 543,025 rows, i.e. 2,224,230,400 bytes of bf16 K and V at
    h_kv = 8, d_h = 128."""
    w = inputs.WORKLOADS["ragged_append_decode_B32"]
    h = inputs.ragged_lengths(w.seed, w.B, 1, w.hist_hi)
    want = np.random.Generator(np.random.PCG64(1953)).integers(1, 32768, 32, endpoint=True)
    assert np.array_equal(h, want)
    assert int((h + 1).sum()) == 543_025
    assert int((h + 1).sum()) * 2 * w.h_kv * w.d_h * 2 == 2_224_230_400
    assert int(h.max()) + 1 <= w.T
