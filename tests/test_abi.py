"""The C-ABI library loads and exports every entry point include/gqa.h declares.

CPU only: calls made here return from host-side validation before any HIP call,
so no GPU is touched.
"""

import ctypes
import os
import re

import pytest

from grouped_query_attention_prefill_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

needs_lib = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH), reason="libgqa.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gqa_prefill", "gqa_prefill_chunk", "gqa_decode", "gqa_decode_workspace_bytes",
              "gqa_kv_append", "gqa_status_string", "gqa_decode_paged", "gqa_kv_append_paged",
              "gqa_rope", "gqa_rope_qk", "gqa_kv_append_rope", "gqa_prefill_lse", "gqa_prefill_backward",
              "gqa_prefill_backward_workspace_bytes", "gqa_append_decode", "gqa_append_decode_paged",
              "gqa_prefill_rope", "gqa_append_decode_rope", "gqa_prefill_chunk_rope", "gqa_kv_append_paged_rope",
              "gqa_append_decode_paged_rope", "gqa_decode_noalloc"):
        assert n in names
    assert set(names) == set(ops.SIGNATURES), "binding prototypes must match the header"


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ops.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


@needs_lib
def test_status_strings():
    for s in range(6):
        assert ops.gqa_status_string(s).startswith("GQA_")
    assert "unknown" in ops.gqa_status_string(99)


FAKE = 0x1000  # never dereferenced: validation fails before any launch


@needs_lib
@pytest.mark.parametrize("args,expect", [
    # (B, h_q, h_kv, T, d_h, mask, scale, in, out)
    ((1, 6, 4, 8, 64, 1, 0.125, 1, 0), ops.GQA_ERR_INVALID_ARGUMENT),    # 6 % 4 != 0
    ((0, 4, 2, 8, 64, 1, 0.125, 1, 0), ops.GQA_ERR_INVALID_ARGUMENT),    # B < 1
    ((1, 4, 2, 8, 64, 7, 0.125, 1, 0), ops.GQA_ERR_INVALID_ARGUMENT),    # unknown mask
    ((1, 4, 2, 8, 64, 1, float("nan"), 1, 0), ops.GQA_ERR_INVALID_ARGUMENT),
    ((1, 4, 2, 8, 64, 1, -1.0, 1, 0), ops.GQA_ERR_INVALID_ARGUMENT),
    ((1, 4, 2, 8, 96, 1, 0.1, 1, 0), ops.GQA_ERR_UNSUPPORTED),           # bf16 d_h 96
    ((1, 4, 2, 8, 300, 1, 0.1, 0, 0), ops.GQA_ERR_UNSUPPORTED),          # fp32 d_h > 256
    ((1, 4, 2, 8, 64, 1, 0.1, 0, 1), ops.GQA_ERR_UNSUPPORTED),           # fp32 in, bf16 out
    ((1, 4, 2, 8, 64, 1, 0.1, 5, 0), ops.GQA_ERR_UNSUPPORTED),           # unknown dtype
    ((1, 4, 2, 1 << 23, 128, 1, 0.1, 1, 0), ops.GQA_ERR_UNSUPPORTED),    # one bf16 K head > 2^31 - 1 bytes
    ((1, 4, 2, 1 << 24, 64, 1, 0.1, 1, 0), ops.GQA_ERR_UNSUPPORTED),
])
def test_prefill_validation(args, expect):
    lib = ops.load_library()
    B, h_q, h_kv, T, d_h, mask, scale, i, o = args
    assert lib.gqa_prefill(FAKE, FAKE, FAKE, FAKE, B, h_q, h_kv, T, d_h, mask, None, scale, i, o, None) == expect


@needs_lib
def test_prefill_rejects_null_and_misaligned():
    lib = ops.load_library()
    assert lib.gqa_prefill(None, FAKE, FAKE, FAKE, 1, 4, 2, 8, 64, 1, None, 0.1, 1, 0, None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_prefill(FAKE + 2, FAKE, FAKE, FAKE, 1, 4, 2, 8, 64, 1, None, 0.1, 1, 0, None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_prefill(FAKE, FAKE, FAKE, FAKE + 4, 1, 4, 2, 8, 64, 1, None, 0.1, 1, 0, None) == ops.GQA_ERR_INVALID_ARGUMENT
    # a bf16 output needs 16-byte alignment too (it is written as 16-byte vectors)
    assert lib.gqa_prefill(FAKE, FAKE, FAKE, FAKE + 8, 1, 4, 2, 8, 64, 1, None, 0.1, 1, 1, None) == ops.GQA_ERR_INVALID_ARGUMENT


@needs_lib
def test_decode_validation_and_workspace():
    lib = ops.load_library()
    ws = lib.gqa_decode_workspace_bytes(64, 32, 8, 8192, 128, ops.GQA_BF16)
    assert ws > 0 and ws % 4 == 0
    assert lib.gqa_decode_workspace_bytes(64, 30, 8, 8192, 128, ops.GQA_BF16) == 0     # invalid sizes
    assert lib.gqa_decode_workspace_bytes(64, 32, 8, 8192, 128, ops.GQA_F32) == 0      # fp32 path needs none
    args = (FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 32, 8, 8192, 128, 0, 0.088, ops.GQA_BF16, ops.GQA_F32)
    # workspace too small
    assert lib.gqa_decode(*args, FAKE, ws - 1, None) == ops.GQA_ERR_WORKSPACE_TOO_SMALL
    # max_seq_len above capacity
    bad = list(args); bad[11] = 8193
    assert lib.gqa_decode(*bad, FAKE, ws, None) == ops.GQA_ERR_INVALID_ARGUMENT
    # missing seq_lens
    bad = list(args); bad[3] = None
    assert lib.gqa_decode(*bad, FAKE, ws, None) == ops.GQA_ERR_INVALID_ARGUMENT


@needs_lib
def test_kv_append_validation():
    lib = ops.load_library()
    assert lib.gqa_kv_append(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 8, 64, 1, None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 64, 9, None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_kv_append(FAKE + 2, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 64, 1, None) == ops.GQA_ERR_INVALID_ARGUMENT


@needs_lib
def test_paged_validation():
    lib = ops.load_library()
    # (q, kp, vp, bt, sl, qp, o, B, h_q, h_kv, page, n_pages, max_pages, d_h, msl, scale, in, out, ws, wsb, stream)
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 8, 2, 64, 10, 500, 128, 0, 0.088, ops.GQA_BF16, ops.GQA_F32,
            FAKE, 1 << 30, None]
    def call(**kw):
        a = list(base)
        names = ["q", "kp", "vp", "bt", "sl", "qp", "o", "B", "h_q", "h_kv", "page", "n_pages", "max_pages", "d_h",
                 "msl", "scale", "in", "out", "ws", "wsb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.gqa_decode_paged(*a)
    assert call(page=48) == ops.GQA_ERR_UNSUPPORTED          # page size not a multiple of 64
    assert call(**{"in": ops.GQA_F32}) == ops.GQA_ERR_UNSUPPORTED
    assert call(bt=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(msl=500 * 64 + 1) == ops.GQA_ERR_INVALID_ARGUMENT  # above max_pages x page_size
    assert call(h_q=7) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(wsb=0) == ops.GQA_ERR_WORKSPACE_TOO_SMALL   # 32000 keys per sequence need splits
    assert lib.gqa_kv_append_paged(FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 2, 64, 10, 4, 128, 1, None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_kv_append_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 10, 4, 3, 1, None) == ops.GQA_ERR_UNSUPPORTED


@needs_lib
def test_rope_validation():
    lib = ops.load_library()
    ok = (FAKE, FAKE, None, 2, 8, 16, 128, 10000.0, ops.GQA_BF16, None)
    def call(**kw):
        names = ["x", "y", "pos0", "B", "H", "S", "d", "base", "dtype", "stream"]
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.gqa_rope(*a)
    assert call(d=127) == ops.GQA_ERR_UNSUPPORTED                 # odd width
    assert call(d=258) == ops.GQA_ERR_UNSUPPORTED                 # wider than 256
    assert call(base=1.0) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(base=float("inf")) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(S=0) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(x=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(y=FAKE + 1) == ops.GQA_ERR_INVALID_ARGUMENT       # misaligned bf16
    assert call(dtype=7) == ops.GQA_ERR_UNSUPPORTED
    assert call(x=FAKE + 2, dtype=ops.GQA_F32) == ops.GQA_ERR_INVALID_ARGUMENT
    ok2 = (FAKE, FAKE, FAKE, FAKE, None, 2, 8, 2, 16, 128, 10000.0, ops.GQA_BF16, None)
    def call2(**kw):
        names = ["q", "q_out", "k", "k_out", "pos0", "B", "h_q", "h_kv", "S", "d", "base", "dtype", "stream"]
        a = list(ok2)
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.gqa_rope_qk(*a)
    assert call2(d=127) == ops.GQA_ERR_UNSUPPORTED
    assert call2(base=0.5) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call2(h_kv=0) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call2(k=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call2(k_out=FAKE + 1) == ops.GQA_ERR_INVALID_ARGUMENT   # misaligned bf16
    assert call2(pos0=FAKE + 2) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call2(dtype=7) == ops.GQA_ERR_UNSUPPORTED
    assert lib.gqa_kv_append_rope(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 8, 64, 10000.0, 1, None) == \
        ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_kv_append_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 63, 10000.0, 1, None) == \
        ops.GQA_ERR_UNSUPPORTED
    assert lib.gqa_kv_append_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 64, -1.0, 1, None) == \
        ops.GQA_ERR_INVALID_ARGUMENT


@needs_lib
def test_backward_validation():
    lib = ops.load_library()
    assert lib.gqa_prefill_backward_workspace_bytes(2, 8, 100) == 2 * 8 * 100 * 4
    assert lib.gqa_prefill_backward_workspace_bytes(0, 8, 100) == 0
    ok = [FAKE] * 9 + [1, 8, 2, 64, 128, 1, None, 0.088, ops.GQA_BF16, ops.GQA_F32, FAKE, 1 << 20, None]
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "B", "h_q", "h_kv", "T", "d", "mask", "lens",
             "scale", "in", "o_dt", "ws", "wsb", "stream"]
    def call(**kw):
        a = list(ok)
        for key, val in kw.items():
            a[names.index(key)] = val
        return lib.gqa_prefill_backward(*a)
    assert call(**{"in": ops.GQA_F32}) == ops.GQA_ERR_UNSUPPORTED
    assert call(d=96) == ops.GQA_ERR_UNSUPPORTED
    assert call(h_q=7) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(mask=3) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(lse=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(dq=FAKE + 4) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(wsb=8 * 64 * 4 - 1) == ops.GQA_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_prefill_lse(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 8, 64, 1, None, 0.1, 1, 0, None) == \
        ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_prefill_lse(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, 4, 2, 8, 64, 1, None, 0.1, 1, 0, None) == \
        ops.GQA_ERR_INVALID_ARGUMENT


@needs_lib
def test_bf16_rows_limit_on_chunk_and_backward():
    """The bf16 prefill kernels address one (sequence, head) with 32-bit offsets: chunked
    prefill and the backward reject a head span of more than 2^31 - 1 bytes up front."""
    lib = ops.load_library()
    big = 1 << 23   # 2^23 rows x 128 x 2 bytes = 2^31
    assert lib.gqa_prefill_chunk(FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 16, big, 128, 1, None, None, 0.1,
                                 ops.GQA_BF16, ops.GQA_F32, None) == ops.GQA_ERR_UNSUPPORTED
    ws = lib.gqa_prefill_backward_workspace_bytes(1, 4, big)
    assert lib.gqa_prefill_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, big, 128, 1, None,
                                    0.1, ops.GQA_BF16, ops.GQA_F32, FAKE, ws, None) == ops.GQA_ERR_UNSUPPORTED


def test_binding_requires_one_device_for_every_tensor():
    """The binding checks that every tensor argument lives on the device it makes
    current for the call, before anything reaches the library."""
    torch = pytest.importorskip("torch")
    called = []
    with pytest.raises(ValueError, match="k must be on cuda:0"):
        ops._launch(torch.device("cuda:0"), (("k", torch.empty(1)),), lambda *a: called.append(a) or 0)
    assert not called


@needs_lib
def test_append_decode_validation():
    """The fused append + decode calls check the arguments of both calls before
    anything is launched (every case here fails a host check)."""
    lib = ops.load_library()
    ws = lib.gqa_decode_workspace_bytes(64, 32, 8, 8192, 128, ops.GQA_BF16)
    names = ["q", "kc", "vc", "kn", "vn", "wp", "sl", "qp", "o", "B", "h_q", "h_kv", "T", "d_h", "msl", "scale",
             "in", "out", "ws", "wsb", "stream"]
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 32, 8, 8192, 128, 0, 0.088, ops.GQA_BF16,
            ops.GQA_F32, FAKE, ws, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.gqa_append_decode(*a)

    assert call(kn=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(vn=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(wp=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(kn=FAKE + 8) == ops.GQA_ERR_INVALID_ARGUMENT        # new rows need 16-byte alignment
    assert call(wp=FAKE + 2) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(sl=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(msl=8193) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(h_q=30) == ops.GQA_ERR_INVALID_ARGUMENT
    assert call(wsb=ws - 1) == ops.GQA_ERR_WORKSPACE_TOO_SMALL
    assert call(B=2, h_q=256, wsb=0) == ops.GQA_ERR_WORKSPACE_TOO_SMALL   # r = 32: the two-launch path checks it too
    assert call(**{"in": ops.GQA_F32, "d_h": 40, "kn": None}) == ops.GQA_ERR_INVALID_ARGUMENT

    pnames = ["q", "kp", "vp", "kn", "vn", "bt", "wp", "sl", "qp", "o", "B", "h_q", "h_kv", "page", "n_pages",
              "max_pages", "d_h", "msl", "scale", "in", "out", "ws", "wsb", "stream"]
    pbase = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 8, 2, 64, 10, 500, 128, 0, 0.088,
             ops.GQA_BF16, ops.GQA_F32, FAKE, 1 << 30, None]

    def pcall(**kw):
        a = list(pbase)
        for k, v in kw.items():
            a[pnames.index(k)] = v
        return lib.gqa_append_decode_paged(*a)

    assert pcall(kn=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert pcall(wp=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert pcall(bt=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert pcall(page=48) == ops.GQA_ERR_UNSUPPORTED
    assert pcall(wsb=0) == ops.GQA_ERR_WORKSPACE_TOO_SMALL


@needs_lib
def test_rope_fused_validation():
    """Prefill and decode with rotary encoding in the kernels: bad bases, the fp32
    path and the usual argument errors are caught before any launch."""
    lib = ops.load_library()
    # (q, k, v, o, B, h_q, h_kv, T, d_h, mask, kv_lens, scale, base, in, out, stream)
    ok = [FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 128, ops.GQA_MASK_CAUSAL, None, 0.088, 10000.0, ops.GQA_BF16,
          ops.GQA_F32, None]
    def pre(**kw):
        a = list(ok)
        names = ["q", "k", "v", "o", "B", "h_q", "h_kv", "T", "d_h", "mask", "kv", "scale", "base", "in", "out", "s"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return lib.gqa_prefill_rope(*a)
    assert pre(base=1.0) == ops.GQA_ERR_INVALID_ARGUMENT
    assert pre(base=float("nan")) == ops.GQA_ERR_INVALID_ARGUMENT
    assert pre(**{"in": ops.GQA_F32}) == ops.GQA_ERR_UNSUPPORTED
    assert pre(d_h=96) == ops.GQA_ERR_UNSUPPORTED
    assert pre(h_q=7) == ops.GQA_ERR_INVALID_ARGUMENT
    assert pre(q=FAKE + 8) == ops.GQA_ERR_INVALID_ARGUMENT
    # chunked: (q, kc, vc, o, B, h_q, h_kv, S_q, T_cap, d_h, mask, kv_lens, q_pos0, scale, base, in, out, stream)
    ch = [FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 16, 64, 128, ops.GQA_MASK_CAUSAL, None, None, 0.088, 10000.0,
          ops.GQA_BF16, ops.GQA_F32, None]
    assert lib.gqa_prefill_chunk_rope(*(ch[:14] + [0.0] + ch[15:])) == ops.GQA_ERR_INVALID_ARGUMENT
    assert lib.gqa_prefill_chunk_rope(*(ch[:15] + [ops.GQA_F32] + ch[16:])) == ops.GQA_ERR_UNSUPPORTED
    assert lib.gqa_prefill_chunk_rope(*(ch[:12] + [FAKE + 2] + ch[13:])) == ops.GQA_ERR_INVALID_ARGUMENT
    ws = lib.gqa_decode_workspace_bytes(64, 32, 8, 8192, 128, ops.GQA_BF16)
    dec = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 32, 8, 8192, 128, 0, 0.088, 10000.0,
           ops.GQA_BF16, ops.GQA_F32, FAKE, ws, None]
    def dcall(**kw):
        a = list(dec)
        names = ["q", "kc", "vc", "kn", "vn", "wp", "sl", "qp", "o", "B", "h_q", "h_kv", "T", "d_h", "msl", "scale",
                 "base", "in", "out", "ws", "wsb", "s"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return lib.gqa_append_decode_rope(*a)
    assert dcall(base=0.5) == ops.GQA_ERR_INVALID_ARGUMENT
    assert dcall(**{"in": ops.GQA_F32, "d_h": 40}) == ops.GQA_ERR_UNSUPPORTED
    assert dcall(kn=None) == ops.GQA_ERR_INVALID_ARGUMENT
    assert dcall(wsb=ws - 1) == ops.GQA_ERR_WORKSPACE_TOO_SMALL


@needs_lib
def test_paged_rope_validation():
    lib = ops.load_library()
    # (kp, vp, kn, vn, bt, wp, B, h_kv, page, n_pages, max_pages, d_h, base, dtype, stream)
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 64, 10, 4, 128, 10000.0, ops.GQA_BF16, None]
    def app(i, v):
        a = list(ok); a[i] = v
        return lib.gqa_kv_append_paged_rope(*a)
    assert app(4, None) == ops.GQA_ERR_INVALID_ARGUMENT        # no block table
    assert app(12, 1.0) == ops.GQA_ERR_INVALID_ARGUMENT        # base
    assert app(11, 3) == ops.GQA_ERR_UNSUPPORTED               # odd d_h
    assert app(6, 0) == ops.GQA_ERR_INVALID_ARGUMENT           # B
    # (q, kp, vp, kn, vn, bt, wp, sl, qp, o, B, h_q, h_kv, page, n_pages, max_pages, d_h, msl, scale, base, in, out,
    #  ws, wsb, stream)
    dec = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 2, 8, 2, 64, 10, 500, 128, 0, 0.088, 10000.0,
           ops.GQA_BF16, ops.GQA_F32, FAKE, 1 << 30, None]
    def dcall(i, v):
        a = list(dec); a[i] = v
        return lib.gqa_append_decode_paged_rope(*a)
    assert dcall(19, 0.0) == ops.GQA_ERR_INVALID_ARGUMENT
    assert dcall(13, 48) == ops.GQA_ERR_UNSUPPORTED
    assert dcall(23, 0) == ops.GQA_ERR_WORKSPACE_TOO_SMALL
    assert dcall(3, None) == ops.GQA_ERR_INVALID_ARGUMENT


def test_binding_rejects_other_output_dtypes_before_any_call(monkeypatch):
    """Only float32 and bfloat16 outputs exist: a caller-supplied ``out`` (or an
    ``out_dtype``) of any other dtype raises TypeError before the library is called
    (an int8 ``out`` would otherwise receive 2-byte values into 1-byte elements)."""
    torch = pytest.importorskip("torch")
    calls = []

    class _Stub:
        def __getattr__(self, name):
            def fn(*a):
                calls.append(name)
                return 0
            return fn

    # host tensors stand in for device tensors: the checks under test come first
    monkeypatch.setattr(ops, "_dev_tensor", lambda *a, **k: None)
    monkeypatch.setattr(ops, "load_library", lambda *a, **k: _Stub())
    bf = torch.bfloat16
    q4, kv4 = torch.zeros(1, 4, 8, 64, dtype=bf), torch.zeros(1, 2, 8, 64, dtype=bf)
    qd = torch.zeros(1, 4, 1, 64, dtype=bf)
    for bad in (torch.float16, torch.int8, torch.uint8, torch.bool, torch.float64):
        with pytest.raises(TypeError):
            ops.gqa_prefill(q4, kv4, kv4, out=torch.zeros(1, 4, 8, 64, dtype=bad))
        with pytest.raises(TypeError):
            ops.gqa_prefill(q4, kv4, kv4, out_dtype=bad)
        with pytest.raises(TypeError):
            ops.gqa_prefill_chunk(q4, kv4, kv4, out=torch.zeros(1, 4, 8, 64, dtype=bad))
        with pytest.raises(TypeError):
            ops.gqa_decode(qd, kv4, kv4, torch.full((1,), 8, dtype=torch.int32),
                           out=torch.zeros(1, 4, 1, 64, dtype=bad))
    assert calls == []
    assert ops._out_code(ops.GQA_BF16, torch.float32) == ops.GQA_F32
    assert ops._out_code(ops.GQA_BF16, torch.bfloat16) == ops.GQA_BF16


@needs_lib
def test_decode_noalloc_validation_and_scratch_limit():
    """The allocation-free decode checks its arguments as gqa_decode does, then
    rejects shapes whose split plan needs more than the static scratch -- all before
    the scratch's address is looked up or anything is launched (no GPU here)."""
    lib = ops.load_library()
    cap = ops.GQA_DECODE_SCRATCH_BYTES
    # (q, k, v, seq_lens, q_pos, o, B, h_q, h_kv, T_cap, d_h, msl, scale, in, out, stream)
    # one sequence of 2^23 keys over 16 query heads: 2048 splits of 16 x 130 floats
    big = (FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 16, 1, 1 << 23, 128, 0, 0.088, ops.GQA_BF16, ops.GQA_F32, None)
    assert lib.gqa_decode_workspace_bytes(1, 16, 1, 1 << 23, 128, ops.GQA_BF16) > cap
    assert lib.gqa_decode_noalloc(*big) == ops.GQA_ERR_SCRATCH_LIMIT
    assert "16 MiB" in ops.gqa_status_string(ops.GQA_ERR_SCRATCH_LIMIT)
    # argument errors come first, whatever the size
    bad = list(big); bad[3] = None
    assert lib.gqa_decode_noalloc(*bad) == ops.GQA_ERR_INVALID_ARGUMENT
    bad = list(big); bad[11] = (1 << 23) + 1              # max_seq_len above capacity
    assert lib.gqa_decode_noalloc(*bad) == ops.GQA_ERR_INVALID_ARGUMENT
    bad = list(big); bad[8] = 3                           # 16 % 3 != 0
    assert lib.gqa_decode_noalloc(*bad) == ops.GQA_ERR_INVALID_ARGUMENT
    bad = list(big); bad[10] = 96                         # bf16 d_h 96
    assert lib.gqa_decode_noalloc(*bad) == ops.GQA_ERR_UNSUPPORTED
    # every benchmarked decode shape fits the scratch
    for (B, hq, hkv, T) in ((64, 32, 8, 8192), (8, 32, 32, 32000), (8, 32, 8, 32000), (8, 32, 1, 32000),
                            (32, 64, 8, 32832)):
        assert lib.gqa_decode_workspace_bytes(B, hq, hkv, T, 128, ops.GQA_BF16) <= cap
