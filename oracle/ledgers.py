"""Byte, FLOP and intensity formulas for the attention path.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

  kv_cache_bytes  [EffSeq] 缓存字节: C_KV = 2 L B T h_kv d_h s (the 2 counts K and V);
                  [AttnVar] 3.2: KVBytes = 2 B L N H_KV d_h s;
                  [Ch09] 09.1: 2 B T L H d s for MHA (H = query heads = KV heads).
  ragged_kv_bytes [AttnVar] 3.2: with unequal request lengths, sum the per-request lengths.
  decode_flops    [MhaMqaGqa] section 8: every query head does one QK and one PV
                  product per visible key, 2 d_h FLOPs each, so 4 h_q d_h per key
                  (the page's printed total is 134,217,728 at h_q=32, d_h=128, T=8192;
                  its formula was lost in extraction and this is the reading that
                  reproduces that total).
  prefill_flops   the same 4 h_q d_h per visible (query, key) pair; a causal row i
                  sees i+1 keys, so the count is 4 B h_q d_h T (T+1) / 2
                  ([EffSeq] 资源变化: arithmetic O(B h_q T^2 d_h) over visible pairs).
  kv_read_intensity  [MhaMqaGqa] section 8 table: FLOPs per KV byte when each cached
                  byte is read from HBM once: 4 h_q d_h / (2 h_kv d_h s).
"""

from __future__ import annotations


def kv_cache_bytes(L: int, B: int, T: int, h_kv: int, d_h: int, s: int) -> int:
    return 2 * L * B * T * h_kv * d_h * s


def ragged_kv_bytes(lengths, L: int, h_kv: int, d_h: int, s: int) -> int:
    return sum(2 * L * int(t) * h_kv * d_h * s for t in lengths)


def kv_bytes_per_token_layer(h_kv: int, d_h: int, s: int) -> int:
    return kv_cache_bytes(1, 1, 1, h_kv, d_h, s)


def decode_flops(h_q: int, d_h: int, lengths) -> int:
    """QK + PV FLOPs of one decode step: 4 h_q d_h per visible key, summed over sequences."""
    return sum(4 * h_q * d_h * int(t) for t in lengths)


def prefill_flops(B: int, h_q: int, d_h: int, T: int, causal: bool = True) -> int:
    pairs = T * (T + 1) // 2 if causal else T * T
    return 4 * B * h_q * d_h * pairs


def kv_read_intensity(h_q: int, h_kv: int, d_h: int, s: int) -> float:
    return (4 * h_q * d_h) / (2 * h_kv * d_h * s)


def projection_params(d: int, h_q: int, h_kv: int, d_h: int) -> int:
    """Bias-free parameter count of the Q, K, V and output projections
    ([EffSeq] 头与投影: W_Q is d x h_q d_h, W_K and W_V are d x h_kv d_h, W_O is h_q d_h x d)."""
    return d * h_q * d_h + 2 * d * h_kv * d_h + h_q * d_h * d
