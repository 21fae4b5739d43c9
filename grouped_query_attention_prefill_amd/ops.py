"""Thin ctypes binding of libgqa.so with the C entry points' names.

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI (``include/gqa.h``).  PyTorch provides device memory
(``torch.empty``) and the current stream; nothing here computes attention.
The library must be built (``python -m grouped_query_attention_prefill_amd.build``);
loading fails loudly otherwise -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgqa.so")

GQA_OK = 0
GQA_ERR_INVALID_ARGUMENT = 1
GQA_ERR_UNSUPPORTED = 2
GQA_ERR_WORKSPACE_TOO_SMALL = 3
GQA_ERR_HIP = 4
GQA_ERR_SCRATCH_LIMIT = 5
GQA_DECODE_SCRATCH_BYTES = 16 << 20
GQA_F32 = 0
GQA_BF16 = 1
GQA_MASK_NONE = 0
GQA_MASK_CAUSAL = 1

# exported symbol -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = {
    "gqa_prefill": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _I, _I, _P]),
    "gqa_prefill_chunk": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _F, _I, _I, _P]),
    "gqa_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I]),
    "gqa_decode": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]),
    "gqa_kv_append": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "gqa_append_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]),
    "gqa_prefill_rope": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _F, _I, _I, _P]),
    "gqa_prefill_chunk_rope": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _F, _F, _I, _I, _P]),
    "gqa_kv_append_paged_rope": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_append_decode_paged_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                          _F, _F, _I, _I, _P, _S, _P]),
    "gqa_append_decode_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I,
                                    _P, _S, _P]),
    "gqa_append_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                     _I, _I, _P, _S, _P]),
    "gqa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]),
    "gqa_kv_append_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "gqa_rope": (_I, [_P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_rope_qk": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_kv_append_rope": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "gqa_prefill_lse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _I, _I, _P]),
    "gqa_prefill_backward_workspace_bytes": (_S, [_I, _I, _I]),
    "gqa_prefill_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _I, _I,
                                  _P, _S, _P]),
    "gqa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "gqa_status_string": (ctypes.c_char_p, [_I]),
}

_lib = None


class GQAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(gqa_status_string(status))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgqa.so and declare its prototypes.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m grouped_query_attention_prefill_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def gqa_status_string(status: int) -> str:
    return load_library().gqa_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != GQA_OK:
        raise GQAError(status)


# ------------------------------------------------------------------ torch marshalling helpers
def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return GQA_F32
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dtype(code: int):
    torch = _torch()
    return torch.float32 if code == GQA_F32 else torch.bfloat16


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t, name, dims=None):
    _require(t.is_cuda, f"{name} must be a device tensor")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    if dims is not None:
        _require(t.dim() == dims, f"{name} must be {dims}-D")


def _int_vec(t, name, B, device):
    if t is None:
        return None
    torch = _torch()
    _dev_tensor(t, name, 1)
    _require(t.dtype == torch.int32 and t.numel() == B, f"{name} must be int32 of shape ({B},)")
    _require(t.device == device, f"{name} must be on {device}")
    return t


def _launch(device, tensors, fn, *args) -> None:
    """Call a C entry point with ``device`` current and its current stream as the
    trailing stream argument; every tensor argument must live on ``device``."""
    torch = _torch()
    for name, t in tensors:
        if t is not None:
            _require(t.device == device, f"{name} must be on {device}")
    with torch.cuda.device(device):
        _check(fn(*args, _stream_handle(device)))


def _out_code(in_code: int, out_dtype) -> int:
    """Output dtype code; only float32 and bfloat16 outputs exist (a caller-supplied
    ``out`` of any other dtype would receive the wrong element size)."""
    if out_dtype is None:
        return GQA_F32
    torch = _torch()
    if out_dtype == torch.float32:
        return GQA_F32
    if out_dtype == torch.bfloat16:
        return GQA_BF16
    raise TypeError(f"output dtype must be torch.float32 or torch.bfloat16, got {out_dtype}")


# ------------------------------------------------------------------ entry points
def _prefill_args(q, k, v, kv_lens, out, out_dtype):
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, n, 4)
    B, h_q, T, d_h = q.shape
    _require(k.shape == v.shape and k.shape[0] == B and k.shape[2] == T and k.shape[3] == d_h,
             "k, v must be (B, h_kv, T, d_h) matching q")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, T, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, T, d_h), "out must be (B, h_q, T, d_h)")
    kv_lens = _int_vec(kv_lens, "kv_lens", B, q.device)
    return B, h_q, k.shape[1], T, d_h, code, oc, out, kv_lens


def gqa_prefill(q, k, v, *, causal: bool = True, scale: Optional[float] = None, kv_lens=None,
                out=None, out_dtype=None):
    """O = grouped-query attention of q (B,h_q,T,d_h) over k, v (B,h_kv,T,d_h).

    Returns ``out`` (allocated with ``torch.empty`` when None); fp32 output by default.
    """
    B, h_q, h_kv, T, d_h, code, oc, out, kv_lens = _prefill_args(q, k, v, kv_lens, out, out_dtype)
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    _launch(q.device, (("k", k), ("v", v), ("out", out)), load_library().gqa_prefill,
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, h_q, h_kv, T, d_h,
            GQA_MASK_CAUSAL if causal else GQA_MASK_NONE, _ptr(kv_lens), sc, code, oc)
    return out


def gqa_prefill_rope(q, k, v, *, causal: bool = True, scale: Optional[float] = None, kv_lens=None,
                     base: float = 10000.0, out=None, out_dtype=None):
    """gqa_prefill with query row i rotated at position i inside the kernel (k must
    already hold rotated keys); equals gqa_prefill(gqa_rope(q), k, v) bit for bit."""
    B, h_q, h_kv, T, d_h, code, oc, out, kv_lens = _prefill_args(q, k, v, kv_lens, out, out_dtype)
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    _launch(q.device, (("k", k), ("v", v), ("out", out)), load_library().gqa_prefill_rope,
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, h_q, h_kv, T, d_h,
            GQA_MASK_CAUSAL if causal else GQA_MASK_NONE, _ptr(kv_lens), sc, float(base), code, oc)
    return out


def gqa_prefill_chunk(q, k_cache, v_cache, *, kv_lens=None, q_pos0=None, causal: bool = True,
                      scale: Optional[float] = None, out=None, out_dtype=None):
    """S_q queries per sequence at absolute positions q_pos0[b] + i against a cache."""
    return _prefill_chunk(q, k_cache, v_cache, kv_lens, q_pos0, causal, scale, out, out_dtype, None)


def gqa_prefill_chunk_rope(q, k_cache, v_cache, *, kv_lens=None, q_pos0=None, causal: bool = True,
                           scale: Optional[float] = None, base: float = 10000.0, out=None, out_dtype=None):
    """gqa_prefill_chunk with each query row rotated at its absolute position inside the kernel."""
    return _prefill_chunk(q, k_cache, v_cache, kv_lens, q_pos0, causal, scale, out, out_dtype, float(base))


def _prefill_chunk(q, k_cache, v_cache, kv_lens, q_pos0, causal, scale, out, out_dtype, rope_base):
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, n, 4)
    B, h_q, S_q, d_h = q.shape
    _require(k_cache.shape == v_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d_h,
             "caches must be (B, h_kv, T_cap, d_h)")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q and caches must share a dtype")
    h_kv, T_cap = k_cache.shape[1], k_cache.shape[2]
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, S_q, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, S_q, d_h), "out must be (B, h_q, S_q, d_h)")
    kv_lens = _int_vec(kv_lens, "kv_lens", B, q.device)
    q_pos0 = _int_vec(q_pos0, "q_pos0", B, q.device)
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    lib = load_library()
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), B, h_q, h_kv, S_q, T_cap, d_h,
            GQA_MASK_CAUSAL if causal else GQA_MASK_NONE, _ptr(kv_lens), _ptr(q_pos0), sc)
    tensors = (("k_cache", k_cache), ("v_cache", v_cache), ("out", out))
    if rope_base is None:
        _launch(q.device, tensors, lib.gqa_prefill_chunk, *head, code, oc)
    else:
        _launch(q.device, tensors, lib.gqa_prefill_chunk_rope, *head, rope_base, code, oc)
    return out


def gqa_decode_workspace_bytes(B: int, h_q: int, h_kv: int, T_cap: int, d_h: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(load_library().gqa_decode_workspace_bytes(B, h_q, h_kv, T_cap, d_h, code))


def gqa_decode(q, k_cache, v_cache, seq_lens, *, q_pos=None, scale: Optional[float] = None,
               max_seq_len: Optional[int] = None, out=None, out_dtype=None, workspace=None):
    """One query per sequence, q (B,h_q,1,d_h), against caches (B,h_kv,T_cap,d_h)."""
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, n, 4)
    B, h_q, S_q, d_h = q.shape
    _require(S_q == 1, "decode takes one query per sequence (S_q = 1)")
    _require(k_cache.shape == v_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d_h,
             "caches must be (B, h_kv, T_cap, d_h)")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q and caches must share a dtype")
    h_kv, T_cap = k_cache.shape[1], k_cache.shape[2]
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, 1, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, 1, d_h), "out must be (B, h_q, 1, d_h)")
    seq_lens = _int_vec(seq_lens, "seq_lens", B, q.device)
    _require(seq_lens is not None, "seq_lens is required")
    q_pos = _int_vec(q_pos, "q_pos", B, q.device)
    lib = load_library()
    ws_bytes = int(lib.gqa_decode_workspace_bytes(B, h_q, h_kv, T_cap, d_h, code))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    msl = 0 if max_seq_len is None else int(max_seq_len)
    _launch(q.device, (("k_cache", k_cache), ("v_cache", v_cache), ("out", out), ("workspace", workspace)),
            lib.gqa_decode, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(q_pos), _ptr(out),
            B, h_q, h_kv, T_cap, d_h, msl, sc, code, oc, _ptr(workspace), ws_have)
    return out


def gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, *, q_pos=None, scale: Optional[float] = None,
                       max_seq_len: Optional[int] = None, out=None, out_dtype=None):
    """gqa_decode whose partial states live in the library's static device scratch
    (GQA_DECODE_SCRATCH_BYTES per GPU): the C call allocates nothing.  Pass ``out``
    to keep this wrapper from allocating the output.  Calls that overlap on one GPU
    share that scratch and race."""
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, n, 4)
    B, h_q, S_q, d_h = q.shape
    _require(S_q == 1, "decode takes one query per sequence (S_q = 1)")
    _require(k_cache.shape == v_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d_h,
             "caches must be (B, h_kv, T_cap, d_h)")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q and caches must share a dtype")
    h_kv, T_cap = k_cache.shape[1], k_cache.shape[2]
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, 1, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, 1, d_h), "out must be (B, h_q, 1, d_h)")
    seq_lens = _int_vec(seq_lens, "seq_lens", B, q.device)
    _require(seq_lens is not None, "seq_lens is required")
    q_pos = _int_vec(q_pos, "q_pos", B, q.device)
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    msl = 0 if max_seq_len is None else int(max_seq_len)
    _launch(q.device, (("k_cache", k_cache), ("v_cache", v_cache), ("out", out)), load_library().gqa_decode_noalloc,
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(q_pos), _ptr(out),
            B, h_q, h_kv, T_cap, d_h, msl, sc, code, oc)
    return out


def gqa_kv_append(k_cache, v_cache, k_new, v_new, write_pos):
    """Write k_new, v_new (B,h_kv,1,d_h) into row write_pos[b] of the caches (in place)."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, n, 4)
    B, h_kv, T_cap, d_h = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "caches must match")
    _require(tuple(k_new.shape) == (B, h_kv, 1, d_h) and k_new.shape == v_new.shape,
             "k_new, v_new must be (B, h_kv, 1, d_h)")
    _require(k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype, "dtypes must match")
    write_pos = _int_vec(write_pos, "write_pos", B, k_cache.device)
    _require(write_pos is not None, "write_pos is required")
    lib = load_library()
    _launch(k_cache.device, (("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)), lib.gqa_kv_append,
            _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(write_pos),
            B, h_kv, T_cap, d_h, _dtype_code(k_cache))
    return k_cache, v_cache


def _new_rows(k_new, v_new, B, h_kv, d_h, dtype, device):
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, n, 4)
        _require(t.device == device, f"{n} must be on {device}")
    _require(tuple(k_new.shape) == (B, h_kv, 1, d_h) and k_new.shape == v_new.shape,
             "k_new, v_new must be (B, h_kv, 1, d_h)")
    _require(k_new.dtype == v_new.dtype == dtype, "k_new, v_new must share the caches' dtype")


def gqa_append_decode(q, k_cache, v_cache, k_new, v_new, write_pos, seq_lens, *, q_pos=None,
                      scale: Optional[float] = None, max_seq_len: Optional[int] = None, out=None, out_dtype=None,
                      workspace=None):
    """gqa_kv_append(k_cache, v_cache, k_new, v_new, write_pos) then gqa_decode(...), in one call."""
    return _append_decode(q, k_cache, v_cache, k_new, v_new, write_pos, seq_lens, q_pos, scale, max_seq_len, out,
                          out_dtype, workspace, None)


def gqa_append_decode_rope(q, k_cache, v_cache, k_new, v_new, write_pos, seq_lens, *, q_pos=None,
                           scale: Optional[float] = None, max_seq_len: Optional[int] = None, base: float = 10000.0,
                           out=None, out_dtype=None, workspace=None):
    """gqa_kv_append_rope (k_new rotated at write_pos) then gqa_decode with each query
    rotated at its position (q_pos, else seq_lens - 1), in one call."""
    return _append_decode(q, k_cache, v_cache, k_new, v_new, write_pos, seq_lens, q_pos, scale, max_seq_len, out,
                          out_dtype, workspace, float(base))


def _append_decode(q, k_cache, v_cache, k_new, v_new, write_pos, seq_lens, q_pos, scale, max_seq_len, out,
                   out_dtype, workspace, rope_base):
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, n, 4)
    B, h_q, S_q, d_h = q.shape
    _require(S_q == 1, "decode takes one query per sequence (S_q = 1)")
    _require(k_cache.shape == v_cache.shape and k_cache.shape[0] == B and k_cache.shape[3] == d_h,
             "caches must be (B, h_kv, T_cap, d_h)")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q and caches must share a dtype")
    h_kv, T_cap = k_cache.shape[1], k_cache.shape[2]
    _new_rows(k_new, v_new, B, h_kv, d_h, q.dtype, q.device)
    write_pos = _int_vec(write_pos, "write_pos", B, q.device)
    _require(write_pos is not None, "write_pos is required")
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, 1, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, 1, d_h), "out must be (B, h_q, 1, d_h)")
    seq_lens = _int_vec(seq_lens, "seq_lens", B, q.device)
    _require(seq_lens is not None, "seq_lens is required")
    q_pos = _int_vec(q_pos, "q_pos", B, q.device)
    lib = load_library()
    ws_bytes = int(lib.gqa_decode_workspace_bytes(B, h_q, h_kv, T_cap, d_h, code))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    msl = 0 if max_seq_len is None else int(max_seq_len)
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(write_pos), _ptr(seq_lens),
            _ptr(q_pos), _ptr(out), B, h_q, h_kv, T_cap, d_h, msl, sc)
    tail = (code, oc, _ptr(workspace), ws_have)
    tensors = (("k_cache", k_cache), ("v_cache", v_cache), ("out", out), ("workspace", workspace))
    if rope_base is None:
        _launch(q.device, tensors, lib.gqa_append_decode, *head, *tail)
    else:
        _launch(q.device, tensors, lib.gqa_append_decode_rope, *head, rope_base, *tail)
    return out


def gqa_append_decode_paged(q, k_pages, v_pages, k_new, v_new, block_table, write_pos, seq_lens, *, q_pos=None,
                            scale: Optional[float] = None, max_seq_len: Optional[int] = None, out=None,
                            out_dtype=None, workspace=None):
    """gqa_kv_append_paged then gqa_decode_paged on the same page pools, in one call."""
    return _append_decode_paged(q, k_pages, v_pages, k_new, v_new, block_table, write_pos, seq_lens, q_pos, scale,
                                max_seq_len, out, out_dtype, workspace, None)


def gqa_append_decode_paged_rope(q, k_pages, v_pages, k_new, v_new, block_table, write_pos, seq_lens, *,
                                 q_pos=None, scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                                 base: float = 10000.0, out=None, out_dtype=None, workspace=None):
    """gqa_kv_append_paged_rope then gqa_decode_paged with each query rotated at its position, in one call."""
    return _append_decode_paged(q, k_pages, v_pages, k_new, v_new, block_table, write_pos, seq_lens, q_pos, scale,
                                max_seq_len, out, out_dtype, workspace, float(base))


def _append_decode_paged(q, k_pages, v_pages, k_new, v_new, block_table, write_pos, seq_lens, q_pos, scale,
                         max_seq_len, out, out_dtype, workspace, rope_base):
    torch = _torch()
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _dev_tensor(t, n, 4)
    B, h_q, S_q, d_h = q.shape
    _require(S_q == 1, "decode takes one query per sequence (S_q = 1)")
    _require(k_pages.shape == v_pages.shape and k_pages.shape[3] == d_h, "pages must be (n_pages, h_kv, page_size, d_h)")
    _require(q.dtype == k_pages.dtype == v_pages.dtype, "q and pages must share a dtype")
    n_pages, h_kv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _new_rows(k_new, v_new, B, h_kv, d_h, q.dtype, q.device)
    _dev_tensor(block_table, "block_table", 2)
    _require(block_table.dtype == torch.int32 and block_table.shape[0] == B, "block_table must be int32 (B, max_pages)")
    max_pages = block_table.shape[1]
    write_pos = _int_vec(write_pos, "write_pos", B, q.device)
    _require(write_pos is not None, "write_pos is required")
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, 1, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, 1, d_h), "out must be (B, h_q, 1, d_h)")
    seq_lens = _int_vec(seq_lens, "seq_lens", B, q.device)
    _require(seq_lens is not None, "seq_lens is required")
    q_pos = _int_vec(q_pos, "q_pos", B, q.device)
    lib = load_library()
    ws_bytes = int(lib.gqa_decode_workspace_bytes(B, h_q, h_kv, page_size * max_pages, d_h, code))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    msl = 0 if max_seq_len is None else int(max_seq_len)
    head = (_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(write_pos),
            _ptr(seq_lens), _ptr(q_pos), _ptr(out), B, h_q, h_kv, page_size, n_pages, max_pages, d_h, msl, sc)
    tail = (code, oc, _ptr(workspace), ws_have)
    tensors = (("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table), ("out", out),
               ("workspace", workspace))
    if rope_base is None:
        _launch(q.device, tensors, lib.gqa_append_decode_paged, *head, *tail)
    else:
        _launch(q.device, tensors, lib.gqa_append_decode_paged_rope, *head, rope_base, *tail)
    return out


def gqa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, *, q_pos=None, scale: Optional[float] = None,
                     max_seq_len: Optional[int] = None, out=None, out_dtype=None, workspace=None):
    """Decode against a paged cache: pages (n_pages, h_kv, page_size, d_h), block_table (B, max_pages) int32."""
    torch = _torch()
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _dev_tensor(t, n, 4)
    B, h_q, S_q, d_h = q.shape
    _require(S_q == 1, "decode takes one query per sequence (S_q = 1)")
    _require(k_pages.shape == v_pages.shape and k_pages.shape[3] == d_h, "pages must be (n_pages, h_kv, page_size, d_h)")
    _require(q.dtype == k_pages.dtype == v_pages.dtype, "q and pages must share a dtype")
    n_pages, h_kv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _dev_tensor(block_table, "block_table", 2)
    _require(block_table.dtype == torch.int32 and block_table.shape[0] == B, "block_table must be int32 (B, max_pages)")
    max_pages = block_table.shape[1]
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, 1, d_h), dtype=_torch_dtype(oc), device=q.device)
    _dev_tensor(out, "out", 4)
    _require(tuple(out.shape) == (B, h_q, 1, d_h), "out must be (B, h_q, 1, d_h)")
    seq_lens = _int_vec(seq_lens, "seq_lens", B, q.device)
    _require(seq_lens is not None, "seq_lens is required")
    q_pos = _int_vec(q_pos, "q_pos", B, q.device)
    lib = load_library()
    ws_bytes = int(lib.gqa_decode_workspace_bytes(B, h_q, h_kv, page_size * max_pages, d_h, code))
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    msl = 0 if max_seq_len is None else int(max_seq_len)
    _launch(q.device, (("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table), ("out", out),
                       ("workspace", workspace)),
            lib.gqa_decode_paged, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens),
            _ptr(q_pos), _ptr(out), B, h_q, h_kv, page_size, n_pages, max_pages, d_h, msl, sc, code, oc,
            _ptr(workspace), ws_have)
    return out


def gqa_kv_append_paged(k_pages, v_pages, k_new, v_new, block_table, write_pos):
    """Write k_new, v_new (B,h_kv,1,d_h) at token position write_pos[b] of each sequence's pages (in place)."""
    torch = _torch()
    for n, t in (("k_pages", k_pages), ("v_pages", v_pages), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, n, 4)
    n_pages, h_kv, page_size, d_h = k_pages.shape
    B = k_new.shape[0]
    _require(v_pages.shape == k_pages.shape, "page pools must match")
    _require(tuple(k_new.shape) == (B, h_kv, 1, d_h) and k_new.shape == v_new.shape, "k_new, v_new must be (B, h_kv, 1, d_h)")
    _require(k_pages.dtype == v_pages.dtype == k_new.dtype == v_new.dtype, "dtypes must match")
    _dev_tensor(block_table, "block_table", 2)
    _require(block_table.dtype == torch.int32 and block_table.shape[0] == B, "block_table must be int32 (B, max_pages)")
    write_pos = _int_vec(write_pos, "write_pos", B, k_pages.device)
    _require(write_pos is not None, "write_pos is required")
    lib = load_library()
    _launch(k_pages.device, (("v_pages", v_pages), ("k_new", k_new), ("v_new", v_new), ("block_table", block_table)),
            lib.gqa_kv_append_paged, _ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new), _ptr(block_table),
            _ptr(write_pos), B, h_kv, page_size, n_pages, block_table.shape[1], d_h, _dtype_code(k_pages))
    return k_pages, v_pages


ROPE_BASE = 10000.0


def gqa_rope(x, *, pos0=None, base: float = ROPE_BASE, out=None):
    """Rotary encoding of x (B, H, S, d_h): row s of sequence b at position pos0[b] + s.

    Returns ``out`` (a new tensor when None; pass ``out=x`` to rotate in place).
    """
    torch = _torch()
    _dev_tensor(x, "x", 4)
    B, H, S, d_h = x.shape
    if out is None:
        out = torch.empty_like(x)
    _dev_tensor(out, "out", 4)
    _require(out.shape == x.shape and out.dtype == x.dtype, "out must match x")
    pos0 = _int_vec(pos0, "pos0", B, x.device)
    _launch(x.device, (("out", out),), load_library().gqa_rope,
            _ptr(x), _ptr(out), _ptr(pos0), B, H, S, d_h, float(base), _dtype_code(x))
    return out


def gqa_rope_qk(q, k, *, pos0=None, base: float = ROPE_BASE, q_out=None, k_out=None):
    """gqa_rope of q (B, h_q, S, d_h) and k (B, h_kv, S, d_h) at the same positions, one launch.

    Returns (q_out, k_out) (new tensors when None; pass q_out=q, k_out=k to rotate in place).
    """
    torch = _torch()
    _dev_tensor(q, "q", 4)
    _dev_tensor(k, "k", 4)
    B, h_q, S, d_h = q.shape
    _require(k.dim() == 4 and k.shape[0] == B and k.shape[2:] == q.shape[2:] and k.dtype == q.dtype,
             "k must be (B, h_kv, S, d_h) of q's dtype")
    h_kv = k.shape[1]
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _dev_tensor(q_out, "q_out", 4)
    _dev_tensor(k_out, "k_out", 4)
    _require(q_out.shape == q.shape and q_out.dtype == q.dtype, "q_out must match q")
    _require(k_out.shape == k.shape and k_out.dtype == k.dtype, "k_out must match k")
    pos0 = _int_vec(pos0, "pos0", B, q.device)
    _launch(q.device, (("q_out", q_out), ("k", k), ("k_out", k_out)), load_library().gqa_rope_qk,
            _ptr(q), _ptr(q_out), _ptr(k), _ptr(k_out), _ptr(pos0), B, h_q, h_kv, S, d_h, float(base),
            _dtype_code(q))
    return q_out, k_out


def gqa_kv_append_paged_rope(k_pages, v_pages, k_new, v_new, block_table, write_pos, *, base: float = ROPE_BASE):
    """gqa_kv_append_paged with k_new rotated at position write_pos[b] (in place on the pools)."""
    torch = _torch()
    for n, t in (("k_pages", k_pages), ("v_pages", v_pages), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, n, 4)
    n_pages, h_kv, page_size, d_h = k_pages.shape
    B = k_new.shape[0]
    _require(v_pages.shape == k_pages.shape, "page pools must match")
    _require(tuple(k_new.shape) == (B, h_kv, 1, d_h) and k_new.shape == v_new.shape, "k_new, v_new must be (B, h_kv, 1, d_h)")
    _require(k_pages.dtype == v_pages.dtype == k_new.dtype == v_new.dtype, "dtypes must match")
    _dev_tensor(block_table, "block_table", 2)
    _require(block_table.dtype == torch.int32 and block_table.shape[0] == B, "block_table must be int32 (B, max_pages)")
    write_pos = _int_vec(write_pos, "write_pos", B, k_pages.device)
    _require(write_pos is not None, "write_pos is required")
    _launch(k_pages.device, (("v_pages", v_pages), ("k_new", k_new), ("v_new", v_new), ("block_table", block_table)),
            load_library().gqa_kv_append_paged_rope, _ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new),
            _ptr(block_table), _ptr(write_pos), B, h_kv, page_size, n_pages, block_table.shape[1], d_h, float(base),
            _dtype_code(k_pages))
    return k_pages, v_pages


def gqa_kv_append_rope(k_cache, v_cache, k_new, v_new, write_pos, *, base: float = ROPE_BASE):
    """kv_append with k_new rotated at position write_pos[b] (in place on the caches)."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, n, 4)
    B, h_kv, T_cap, d_h = k_cache.shape
    _require(v_cache.shape == k_cache.shape, "caches must match")
    _require(tuple(k_new.shape) == (B, h_kv, 1, d_h) and k_new.shape == v_new.shape,
             "k_new, v_new must be (B, h_kv, 1, d_h)")
    _require(k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype, "dtypes must match")
    write_pos = _int_vec(write_pos, "write_pos", B, k_cache.device)
    _require(write_pos is not None, "write_pos is required")
    _launch(k_cache.device, (("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)),
            load_library().gqa_kv_append_rope, _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
            _ptr(write_pos), B, h_kv, T_cap, d_h, float(base), _dtype_code(k_cache))
    return k_cache, v_cache


def gqa_prefill_lse(q, k, v, *, causal: bool = True, scale: Optional[float] = None, kv_lens=None,
                    out=None, out_dtype=None, lse=None):
    """gqa_prefill that also returns the row log-sum-exp (B, h_q, T) fp32 a backward pass needs."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, n, 4)
    B, h_q, T, d_h = q.shape
    _require(k.shape == v.shape and k.shape[0] == B and k.shape[2] == T and k.shape[3] == d_h,
             "k, v must be (B, h_kv, T, d_h) matching q")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    h_kv = k.shape[1]
    code = _dtype_code(q)
    oc = _out_code(code, out_dtype if out is None else out.dtype)
    if out is None:
        out = torch.empty((B, h_q, T, d_h), dtype=_torch_dtype(oc), device=q.device)
    if lse is None:
        lse = torch.empty((B, h_q, T), dtype=torch.float32, device=q.device)
    _dev_tensor(out, "out", 4)
    _dev_tensor(lse, "lse", 3)
    _require(lse.dtype == torch.float32 and tuple(lse.shape) == (B, h_q, T), "lse must be fp32 (B, h_q, T)")
    kv_lens = _int_vec(kv_lens, "kv_lens", B, q.device)
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    _launch(q.device, (("k", k), ("v", v), ("out", out), ("lse", lse)), load_library().gqa_prefill_lse,
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, h_q, h_kv, T, d_h,
            GQA_MASK_CAUSAL if causal else GQA_MASK_NONE, _ptr(kv_lens), sc, code, oc)
    return out, lse


def gqa_prefill_backward_workspace_bytes(B: int, h_q: int, T: int) -> int:
    return int(load_library().gqa_prefill_backward_workspace_bytes(B, h_q, T))


def gqa_prefill_backward(q, k, v, o, d_o, lse, *, causal: bool = True, scale: Optional[float] = None,
                         kv_lens=None, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV (fp32) of bf16 prefill attention from O, dO and the forward's row log-sum-exp."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("d_o", d_o)):
        _dev_tensor(t, n, 4)
    B, h_q, T, d_h = q.shape
    h_kv = k.shape[1]
    _require(k.shape == v.shape and tuple(k.shape) == (B, h_kv, T, d_h), "k, v must be (B, h_kv, T, d_h)")
    _require(o.shape == q.shape and d_o.shape == q.shape, "o and d_o must match q")
    _require(q.dtype == k.dtype == v.dtype == d_o.dtype, "q, k, v, d_o must share a dtype")
    _dev_tensor(lse, "lse", 3)
    _require(lse.dtype == torch.float32 and tuple(lse.shape) == (B, h_q, T), "lse must be fp32 (B, h_q, T)")
    if dq is None:
        dq = torch.empty((B, h_q, T, d_h), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty((B, h_kv, T, d_h), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((B, h_kv, T, d_h), dtype=torch.float32, device=q.device)
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _dev_tensor(t, n, 4)
        _require(t.dtype == torch.float32, f"{n} must be fp32")
    kv_lens = _int_vec(kv_lens, "kv_lens", B, q.device)
    lib = load_library()
    ws_bytes = int(lib.gqa_prefill_backward_workspace_bytes(B, h_q, T))
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_have = workspace.numel() * workspace.element_size()
    sc = 1.0 / math.sqrt(d_h) if scale is None else float(scale)
    _launch(q.device, (("k", k), ("v", v), ("o", o), ("d_o", d_o), ("lse", lse), ("dq", dq), ("dk", dk),
                       ("dv", dv), ("workspace", workspace)),
            lib.gqa_prefill_backward, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk),
            _ptr(dv), B, h_q, h_kv, T, d_h, GQA_MASK_CAUSAL if causal else GQA_MASK_NONE,
            _ptr(kv_lens), sc, _dtype_code(q), _dtype_code(o), _ptr(workspace), ws_have)
    return dq, dk, dv
