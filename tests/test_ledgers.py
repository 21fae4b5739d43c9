"""The byte / FLOP ledgers against the values printed on the pages (tests/golden/ledgers.json)."""

import json
import os

import pytest

from oracle import ledgers

KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


@pytest.fixture(scope="module")
def g(golden_dir):
    with open(os.path.join(golden_dir, "ledgers.json")) as f:
        return json.load(f)


def test_cache_bytes_small(g):
    c = g["cache_bytes_small"]
    a = c["args"]
    assert ledgers.kv_cache_bytes(**a) == c["total"]
    assert ledgers.kv_cache_bytes(**{**a, "L": 1}) == c["per_layer"]
    assert ledgers.kv_cache_bytes(**{**a, "T": 4}) == c["total_at_T4"]
    assert ledgers.kv_cache_bytes(**{**a, "h_kv": 4}) == c["mha_h_kv4"]
    assert ledgers.kv_cache_bytes(**{**a, "h_kv": 1}) == c["mqa_h_kv1"]


def test_projection_params(g):
    c = g["projection_params"]
    a = c["args"]
    assert ledgers.projection_params(**a) == c["gqa"] == sum(c["parts"])
    assert ledgers.projection_params(**{**a, "h_kv": 4}) == c["mha"]
    assert ledgers.projection_params(**{**a, "h_kv": 1}) == c["mqa"]


def test_kv_bytes_long_context(g):
    c = g["kv_bytes_7b_32k"]
    a = c["args"]
    n = ledgers.kv_cache_bytes(L=a["L"], B=a["B"], T=a["N"], h_kv=a["H_KV"], d_h=a["d_h"], s=a["s"])
    assert n == c["bytes"]
    assert round(n / 1e9, 2) == c["approx_GB"]
    assert n / GiB == c["GiB"]
    n8 = ledgers.kv_cache_bytes(L=a["L"], B=a["B"], T=a["N"], h_kv=8, d_h=a["d_h"], s=a["s"])
    assert round(n8 / 1e9, 2) == c["approx_GB_8_kv_heads"]


def test_ch09_cache_example(g):
    c = g["ch09_cache_example"]
    a = c["args"]
    n = ledgers.kv_cache_bytes(L=a["L"], B=a["B"], T=a["T"], h_kv=a["H"], d_h=a["d"], s=a["s"])
    assert n == c["bytes"] and n == c["MiB"] * MiB


def test_per_token_layer_and_history(g):
    c = g["per_token_layer"]
    assert ledgers.kv_bytes_per_token_layer(32, 128, 2) == c["mha_bytes"] == c["mha_elements"] * 2
    assert ledgers.kv_bytes_per_token_layer(8, 128, 2) == c["gqa_bytes"]
    assert ledgers.kv_bytes_per_token_layer(1, 128, 2) == c["mqa_bytes"]
    for name, h_kv in (("mha", 32), ("gqa", 8), ("mqa", 1)):
        assert ledgers.kv_cache_bytes(1, 1, 8192, h_kv, 128, 2) == c["history_8k_per_layer_MiB"][name] * MiB
    assert ledgers.kv_cache_bytes(32, 1, 8192, 32, 128, 2) == c["mha_32_layers_GiB"] * GiB


def test_decode_flops_and_intensity(g):
    c = g["decode_flops"]
    a = c["args"]
    for h_kv in (32, 8, 1):   # the count does not depend on the number of KV heads
        assert ledgers.decode_flops(a["h_q"], a["d_h"], [a["T"]]) == c["flops"]
    for name, h_kv in (("mha", 32), ("gqa", 8), ("mqa", 1)):
        assert ledgers.kv_read_intensity(32, h_kv, 128, 2) == c["intensity_flop_per_byte"][name]
        # the same figure from the two ledgers: FLOPs over bytes of one layer's 8K history
        assert c["flops"] / ledgers.kv_cache_bytes(1, 1, 8192, h_kv, 128, 2) == c["intensity_flop_per_byte"][name]


def test_score_matrix_sizes(g):
    c = g["score_matrix"]
    assert 1 * 4 * 1024 * 1024 == c["full_elements"]
    assert c["full_elements"] * 4 == c["full_MiB_fp32"] * MiB
    assert 64 * 64 == c["tile_elements"] and c["tile_elements"] * 4 == c["tile_KiB_fp32"] * KiB
    assert 4096 * 4096 * 2 == c["fp16_N4096_MiB"] * MiB
    assert 32768 * 32768 * 2 == c["fp16_N32768_GiB"] * GiB


def test_kv_tile(g):
    c = g["kv_tile"]
    assert ledgers.kv_cache_bytes(1, 1, 256, 1, 128, 2) == c["bytes"] == c["KiB"] * KiB


def test_ragged_and_prefill_counts():
    assert ledgers.ragged_kv_bytes([3, 5], 2, 2, 2, 2) == ledgers.kv_cache_bytes(2, 1, 8, 2, 2, 2)
    # brute-force count of visible causal pairs
    T = 37
    pairs = sum(1 for i in range(T) for j in range(T) if j <= i)
    assert ledgers.prefill_flops(2, 3, 4, T) == 4 * 2 * 3 * 4 * pairs
    assert ledgers.prefill_flops(1, 32, 128, 4096) == 137_472_507_904
    assert ledgers.prefill_flops(1, 1, 1, 5, causal=False) == 4 * 25
