"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws numbers and lays them
out.  Both the HIP path and the CPU oracle consume what it returns, so it
imports neither of them.

Recipe (the same for every workload):
  * numpy PCG64 streams keyed by ``SeedSequence(seed, spawn_key=(tensor, row))``:
    one independent stream per tensor and per batch row, so rows can be drawn
    in parallel threads and any row can be regenerated on its own;
    tensor ids: Q 0, K 1, V 2, appended K 3, appended V 4, output gradient dO 6;
  * ragged lengths come first, from ``Generator(PCG64(seed))`` itself;
  * values are ``standard_normal(dtype=float32)``, i.e. N(0, 1);
  * bf16 tensors are those float32 draws rounded to bf16, round-to-nearest-even;
    both sides see exactly those bf16 values (the oracle widens them to float64
    exactly);
  * ragged lengths are integers uniform on [1, 32768], both ends inclusive;
  * cache rows a sequence must never read (rows >= its length after the append)
    are filled with a quiet NaN, so an over-read or a 0 * NaN leak shows up in
    the output.

bf16 tensors are returned as ``uint16`` bit patterns, float32 tensors as
``float32``.  ``bf16_bits_to_f32`` widens bit patterns exactly.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional

import numpy as np

SEED_BASE = 1949
BF16_QNAN = np.uint16(0x7FC0)


TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "k_new": 3, "v_new": 4, "lengths": 5, "d_out": 6}


def rng_for(seed: int, tensor: int = 5, row: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, row))))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r = np.where(nan, BF16_QNAN, r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, tensor: str, shape, dtype: str, rows=None) -> np.ndarray:
    """N(0,1) tensor; leading index b is drawn from stream (seed, tensor, b).

    dtype "f32" -> float32 array; "bf16" -> uint16 bf16 bit patterns.
    ``rows`` restricts the draw to those leading indices (others stay zero).
    """
    shape = tuple(int(s) for s in shape)
    out = np.zeros(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype}")
    if len(shape) == 0 or shape[0] == 0:
        return out
    tid = TENSOR_IDS[tensor]

    def fill(i):
        x = rng_for(seed, tid, i).standard_normal(shape[1:], dtype=np.float32)
        out[i] = x if dtype == "f32" else f32_to_bf16_bits(x)

    idx = range(shape[0]) if rows is None else rows
    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, idx))
    return out


def normal_row(seed: int, tensor: str, row: int, shape_tail, dtype: str) -> np.ndarray:
    """Leading-index slice ``row`` of ``normal(seed, tensor, (B,) + shape_tail, dtype)``, alone."""
    x = rng_for(seed, TENSOR_IDS[tensor], row).standard_normal(tuple(shape_tail), dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def ragged_lengths(seed: int, B: int, lo: int = 1, hi: int = 32768) -> np.ndarray:
    """B history lengths uniform on [lo, hi], both ends inclusive, drawn first and
    from a plain ``Generator(PCG64(seed))`` (the tensors keep their keyed streams).
    For seed 1953, B = 32 the histories sum to 543,025 - 32 rows (543,025 with the
    appended token)."""
    return np.random.Generator(np.random.PCG64(seed)).integers(lo, hi, size=B, endpoint=True).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, dtype, seed and path."""

    name: str
    path: str            # "prefill" or "decode" or "append_decode"
    B: int
    h_q: int
    h_kv: int
    d_h: int
    T: int               # prefill length, or cache capacity T_cap for decode
    dtype: str           # "f32" or "bf16"
    seed: int
    causal: bool = True
    ragged: bool = False
    hist_hi: int = 0     # ragged: lengths uniform on [1, hist_hi]


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_prefill_f32", "prefill", 1, 4, 2, 2, 3, "f32", SEED_BASE + 0),
        Workload("prefill_causal_bf16_T4096", "prefill", 1, 32, 8, 128, 4096, "bf16", SEED_BASE + 1),
        Workload("decode_bf16_B64_T8192", "decode", 64, 32, 8, 128, 8192, "bf16", SEED_BASE + 2),
        Workload("decode_mha_B8_T32000", "decode", 8, 32, 32, 128, 32000, "bf16", SEED_BASE + 3),
        Workload("decode_gqa_B8_T32000", "decode", 8, 32, 8, 128, 32000, "bf16", SEED_BASE + 3),
        Workload("decode_mqa_B8_T32000", "decode", 8, 32, 1, 128, 32000, "bf16", SEED_BASE + 3),
        # capacity: first multiple of 64 that holds the longest history plus the appended token
        Workload("ragged_append_decode_B32", "append_decode", 32, 64, 8, 128, round_up(32768 + 1, 64),
                 "bf16", SEED_BASE + 4, ragged=True, hist_hi=32768),
    ]
}


def make_prefill(B, h_q, h_kv, d_h, T, dtype, seed, kv_lens: Optional[np.ndarray] = None):
    """Q (B,h_q,T,d_h), K, V (B,h_kv,T,d_h).  Returns a dict of host arrays."""
    q = normal(seed, "q", (B, h_q, T, d_h), dtype)
    k = normal(seed, "k", (B, h_kv, T, d_h), dtype)
    v = normal(seed, "v", (B, h_kv, T, d_h), dtype)
    d = {"q": q, "k": k, "v": v}
    if kv_lens is not None:
        d["kv_lens"] = np.asarray(kv_lens, dtype=np.int32)
    return d


def make_decode(B, h_q, h_kv, d_h, T_cap, dtype, seed, seq_lens=None, poison=False):
    """Decode inputs: q (B,h_q,1,d_h); caches (B,h_kv,T_cap,d_h); seq_lens (B,).

    seq_lens defaults to T_cap for every sequence (full cache, query at T_cap-1).
    With ``poison``, cache rows >= seq_lens[b] are set to NaN.
    """
    q = normal(seed, "q", (B, h_q, 1, d_h), dtype)
    k = normal(seed, "k", (B, h_kv, T_cap, d_h), dtype)
    v = normal(seed, "v", (B, h_kv, T_cap, d_h), dtype)
    lens = np.full(B, T_cap, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
    if poison:
        _poison_rows(k, lens, dtype)
        _poison_rows(v, lens, dtype)
    return {"q": q, "k_cache": k, "v_cache": v, "seq_lens": lens, "q_pos": (lens - 1).astype(np.int32)}


def make_append_decode(B, h_q, h_kv, d_h, T_cap, dtype, seed, hist_hi, lens=None):
    """Ragged decode step with one appended token per sequence.

    hist[b] ~ U{1..hist_hi} (drawn first) is the history length before the append;
    the append writes row hist[b]; afterwards seq_len = hist+1 and the query sits
    at absolute position hist[b].  Rows >= hist[b] are NaN before the append (row
    hist[b] is then overwritten by the append), rows > hist[b] stay NaN.
    """
    hist = ragged_lengths(seed, B, 1, hist_hi) if lens is None else np.asarray(lens, np.int32)
    if int(hist.max()) + 1 > T_cap:
        raise ValueError("cache capacity too small for the drawn lengths")
    q = normal(seed, "q", (B, h_q, 1, d_h), dtype)
    k = normal(seed, "k", (B, h_kv, T_cap, d_h), dtype)
    v = normal(seed, "v", (B, h_kv, T_cap, d_h), dtype)
    k_new = normal(seed, "k_new", (B, h_kv, 1, d_h), dtype)
    v_new = normal(seed, "v_new", (B, h_kv, 1, d_h), dtype)
    _poison_rows(k, hist, dtype)
    _poison_rows(v, hist, dtype)
    return {
        "q": q, "k_cache": k, "v_cache": v, "k_new": k_new, "v_new": v_new,
        "hist": hist, "write_pos": hist.astype(np.int32),
        "seq_lens": (hist + 1).astype(np.int32), "q_pos": hist.astype(np.int32),
    }


def _poison_rows(cache: np.ndarray, lens: np.ndarray, dtype: str) -> None:
    fill = BF16_QNAN if dtype == "bf16" else np.float32(np.nan)
    for b in range(cache.shape[0]):
        cache[b, :, int(lens[b]):, :] = fill


def make_workload(w: Workload, **overrides):
    """Inputs of a named workload (optionally with sizes overridden, same recipe)."""
    w = dataclasses.replace(w, **overrides) if overrides else w
    if w.path == "prefill":
        return make_prefill(w.B, w.h_q, w.h_kv, w.d_h, w.T, w.dtype, w.seed)
    if w.path == "decode":
        return make_decode(w.B, w.h_q, w.h_kv, w.d_h, w.T, w.dtype, w.seed)
    if w.path == "append_decode":
        return make_append_decode(w.B, w.h_q, w.h_kv, w.d_h, w.T, w.dtype, w.seed, w.hist_hi)
    raise ValueError(w.path)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of generator output (bf16 bits widened; float32 unchanged)."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
