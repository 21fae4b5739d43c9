"""Helpers for the GPU parity tests: host <-> device marshalling and the parity bar."""

import numpy as np

from grouped_query_attention_prefill_amd import inputs

# parity bar for bf16 inputs with fp32 accumulation, and for the fp32 path
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def to_dev(x: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def ints_dev(x):
    import torch

    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


def to_host64(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return inputs.to_f32(x, dtype).astype(np.float64)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (the rounding of a bf16 output)."""
    a = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(a))
    return 0.5 * np.exp2(e - 7)


def check_parity(got: np.ndarray, want: np.ndarray, *, mode: str, what: str = ""):
    """mode: 'f32' (max-abs 1e-5), 'bf16' (2e-2 / 2e-3), 'bf16out' (bf16 bar + output rounding)."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    if mode == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max-abs {err.max():.3g} > {F32_MAX_ABS}"
        return err.max(), err.mean()
    excess = err - (bf16_half_ulp(want) if mode == "bf16out" else 0.0)
    assert excess.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3g} (excess {excess.max():.3g})"
    assert err.mean() <= BF16_MEAN_ABS + (bf16_half_ulp(want).mean() if mode == "bf16out" else 0.0), \
        f"{what}: mean-abs {err.mean():.3g}"
    return err.max(), err.mean()


def host_workers() -> int:
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def parallel_map(fn, items):
    """fn over items in host threads (numpy releases the GIL in the oracle's array work)."""
    import concurrent.futures

    with concurrent.futures.ThreadPoolExecutor(host_workers()) as ex:
        return list(ex.map(fn, items))
