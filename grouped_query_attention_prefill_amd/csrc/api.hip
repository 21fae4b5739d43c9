// C ABI of the grouped-query attention library: argument validation and
// dispatch to the kernels.  Every host-checkable error is reported before any
// launch; nothing is allocated, and the only state kept between calls is the
// per-device record of kernels allowed more than 64 KiB of LDS.
#include "gqa.h"
#include "internal.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

namespace {

using gqa::AttnArgs;
using gqa::DecodeArgs;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// dtype/d_h combinations with a kernel behind them
int check_types(int in_dtype, int out_dtype, int d_h) {
  if (in_dtype == GQA_F32) {
    if (out_dtype != GQA_F32) return GQA_ERR_UNSUPPORTED;
    if (d_h < 1 || d_h > 256) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
  }
  if (in_dtype == GQA_BF16) {
    if (out_dtype != GQA_F32 && out_dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
    if (d_h != 64 && d_h != 128) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
  }
  return GQA_ERR_UNSUPPORTED;
}

bool known_dtype(int t) { return t == GQA_F32 || t == GQA_BF16; }

// The bf16 prefill and backward kernels address the rows of one (sequence, head)
// through 32-bit buffer offsets: rows * d_h bf16 values must fit in 2^31 - 1 bytes.
bool bf16_rows_fit(int in_dtype, int rows, int d_h) {
  return in_dtype != GQA_BF16 || (long long)rows * d_h * 2 <= 0x7fffffffLL;
}

// On the bf16 path every tensor, the output included, needs a 16-byte aligned base
// (the prefill writes O as 16-byte vectors whatever its element type); the fp32 path
// needs 4 bytes.
int check_ptrs(int in_dtype, const void* q, const void* k, const void* v, const void* o) {
  if (!q || !k || !v || !o) return GQA_ERR_INVALID_ARGUMENT;
  const uintptr_t al = in_dtype == GQA_BF16 ? 16 : 4;
  if (!aligned(q, al) || !aligned(k, al) || !aligned(v, al) || !aligned(o, al)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

int run_attention(const AttnArgs& a, int in_dtype, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.B == 0) return GQA_OK;
  hipError_t e = in_dtype == GQA_F32 ? gqa::launch_attn_f32(a, s) : gqa::launch_attn_bf16(a, s);
  return hip_status(e);
}

}  // namespace

// ---- gqa_decode_noalloc: the decode workspace in a static device array.
// In host code `scratch` names a host-side stand-in, not device memory: its device
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[GQA_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on the first call
// made on each device.
hipError_t current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

extern "C" {

static int prefill_chunk_impl(const void* q, const void* k_cache, const void* v_cache, void* o,
                              int B, int h_q, int h_kv, int S_q, int T_cap, int d_h,
                              int mask, const int32_t* kv_lens, const int32_t* q_pos0,
                              float scale, int in_dtype, int out_dtype, void* stream, float rope_base) {
  if (B < 1 || h_q < 1 || h_kv < 1 || S_q < 1 || T_cap < 1 || d_h < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (h_q % h_kv != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (mask != GQA_MASK_NONE && mask != GQA_MASK_CAUSAL) return GQA_ERR_INVALID_ARGUMENT;
  if (!scale_ok(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(in_dtype) || !known_dtype(out_dtype)) return GQA_ERR_UNSUPPORTED;
  int st = check_types(in_dtype, out_dtype, d_h);
  if (st != GQA_OK) return st;
  if (!bf16_rows_fit(in_dtype, T_cap, d_h)) return GQA_ERR_UNSUPPORTED;
  st = check_ptrs(in_dtype, q, k_cache, v_cache, o);
  if (st != GQA_OK) return st;
  if ((kv_lens && !aligned(kv_lens, 4)) || (q_pos0 && !aligned(q_pos0, 4))) return GQA_ERR_INVALID_ARGUMENT;
  AttnArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o;
  a.kv_lens = kv_lens; a.q_pos0 = q_pos0;
  a.B = B; a.h_q = h_q; a.h_kv = h_kv; a.S_q = S_q; a.T_cap = T_cap; a.D = d_h;
  a.causal = mask == GQA_MASK_CAUSAL ? 1 : 0;
  // default positions: the newest S_q positions of each history, except when the
  // chunk spans the whole capacity, which is a prefill (row i at position i)
  a.q_pos_from_end = S_q == T_cap ? 0 : 1;
  a.scale = scale;
  a.out_bf16 = out_dtype == GQA_BF16 ? 1 : 0;
  a.rope_base = rope_base;
  return run_attention(a, in_dtype, stream);
}

int gqa_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o,
                      int B, int h_q, int h_kv, int S_q, int T_cap, int d_h,
                      int mask, const int32_t* kv_lens, const int32_t* q_pos0,
                      float scale, int in_dtype, int out_dtype, void* stream) {
  return prefill_chunk_impl(q, k_cache, v_cache, o, B, h_q, h_kv, S_q, T_cap, d_h, mask, kv_lens, q_pos0, scale,
                            in_dtype, out_dtype, stream, 0.f);
}

int gqa_prefill_chunk_rope(const void* q, const void* k_cache, const void* v_cache, void* o,
                           int B, int h_q, int h_kv, int S_q, int T_cap, int d_h,
                           int mask, const int32_t* kv_lens, const int32_t* q_pos0,
                           float scale, float rope_base, int in_dtype, int out_dtype, void* stream) {
  if (!std::isfinite(rope_base) || rope_base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  if (known_dtype(in_dtype) && in_dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  return prefill_chunk_impl(q, k_cache, v_cache, o, B, h_q, h_kv, S_q, T_cap, d_h, mask, kv_lens, q_pos0, scale,
                            in_dtype, out_dtype, stream, rope_base);
}

static int prefill_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int h_q, int h_kv, int T, int d_h, int mask, const int32_t* kv_lens, float scale,
                        int in_dtype, int out_dtype, void* stream, float rope_base = 0.f) {
  if (B < 1 || h_q < 1 || h_kv < 1 || T < 1 || d_h < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (h_q % h_kv != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (mask != GQA_MASK_NONE && mask != GQA_MASK_CAUSAL) return GQA_ERR_INVALID_ARGUMENT;
  if (!scale_ok(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(in_dtype) || !known_dtype(out_dtype)) return GQA_ERR_UNSUPPORTED;
  int st = check_types(in_dtype, out_dtype, d_h);
  if (st != GQA_OK) return st;
  if (!bf16_rows_fit(in_dtype, T, d_h)) return GQA_ERR_UNSUPPORTED;
  st = check_ptrs(in_dtype, q, k, v, o);
  if (st != GQA_OK) return st;
  if (kv_lens && !aligned(kv_lens, 4)) return GQA_ERR_INVALID_ARGUMENT;
  if (lse && !aligned(lse, 4)) return GQA_ERR_INVALID_ARGUMENT;
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.kv_lens = kv_lens; a.q_pos0 = nullptr;
  a.B = B; a.h_q = h_q; a.h_kv = h_kv; a.S_q = T; a.T_cap = T; a.D = d_h;
  a.causal = mask == GQA_MASK_CAUSAL ? 1 : 0;
  a.q_pos_from_end = 0;    // query i sits at position i
  a.scale = scale;
  a.out_bf16 = out_dtype == GQA_BF16 ? 1 : 0;
  a.lse = lse;
  a.rope_base = rope_base;
  return run_attention(a, in_dtype, stream);
}

int gqa_prefill(const void* q, const void* k, const void* v, void* o,
                int B, int h_q, int h_kv, int T, int d_h,
                int mask, const int32_t* kv_lens, float scale,
                int in_dtype, int out_dtype, void* stream) {
  return prefill_impl(q, k, v, o, nullptr, B, h_q, h_kv, T, d_h, mask, kv_lens, scale, in_dtype, out_dtype, stream);
}

int gqa_prefill_rope(const void* q, const void* k, const void* v, void* o,
                     int B, int h_q, int h_kv, int T, int d_h,
                     int mask, const int32_t* kv_lens, float scale, float rope_base,
                     int in_dtype, int out_dtype, void* stream) {
  if (!std::isfinite(rope_base) || rope_base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  if (known_dtype(in_dtype) && in_dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  return prefill_impl(q, k, v, o, nullptr, B, h_q, h_kv, T, d_h, mask, kv_lens, scale, in_dtype, out_dtype, stream,
                      rope_base);
}

int gqa_prefill_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int h_q, int h_kv, int T, int d_h,
                    int mask, const int32_t* kv_lens, float scale,
                    int in_dtype, int out_dtype, void* stream) {
  if (!lse) return GQA_ERR_INVALID_ARGUMENT;
  return prefill_impl(q, k, v, o, lse, B, h_q, h_kv, T, d_h, mask, kv_lens, scale, in_dtype, out_dtype, stream);
}

size_t gqa_prefill_backward_workspace_bytes(int B, int h_q, int T) {
  if (B < 1 || h_q < 1 || T < 1) return 0;
  return gqa::bwd_workspace_bytes(B, h_q, T);
}

int gqa_prefill_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                         const float* lse, float* dq, float* dk, float* dv,
                         int B, int h_q, int h_kv, int T, int d_h, int mask, const int32_t* kv_lens,
                         float scale, int in_dtype, int o_dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || h_q < 1 || h_kv < 1 || T < 1 || d_h < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (h_q % h_kv != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (mask != GQA_MASK_NONE && mask != GQA_MASK_CAUSAL) return GQA_ERR_INVALID_ARGUMENT;
  if (!scale_ok(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(in_dtype) || !known_dtype(o_dtype)) return GQA_ERR_UNSUPPORTED;
  if (in_dtype != GQA_BF16 || (d_h != 64 && d_h != 128)) return GQA_ERR_UNSUPPORTED;
  if (!bf16_rows_fit(in_dtype, T, d_h)) return GQA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) ||
      !aligned(o, o_dtype == GQA_BF16 ? 2 : 4) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || (kv_lens && !aligned(kv_lens, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  const size_t need = gqa::bwd_workspace_bytes(B, h_q, T);
  if (workspace_bytes < need) return GQA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 4)) return GQA_ERR_INVALID_ARGUMENT;
  gqa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.d_o = d_o; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.kv_lens = kv_lens;
  a.B = B; a.h_q = h_q; a.h_kv = h_kv; a.T = T; a.D = d_h;
  a.causal = mask == GQA_MASK_CAUSAL ? 1 : 0;
  a.o_bf16 = o_dtype == GQA_BF16 ? 1 : 0;
  a.scale = scale;
  a.workspace = workspace;
  return hip_status(gqa::launch_backward_bf16(a, static_cast<hipStream_t>(stream)));
}

size_t gqa_decode_workspace_bytes(int B, int h_q, int h_kv, int T_cap, int d_h, int in_dtype) {
  if (B < 1 || h_q < 1 || h_kv < 1 || T_cap < 1 || d_h < 1 || h_q % h_kv != 0) return 0;
  if (in_dtype != GQA_BF16) return 0;
  if (d_h != 64 && d_h != 128) return 0;
  return gqa::plan_decode_bf16(B, h_q, h_kv, T_cap, d_h, T_cap).workspace_bytes;
}

// The new token's rows for the fused append + decode calls.
struct AppendIn {
  const void* k_new;
  const void* v_new;
  const int32_t* write_pos;
};

// kv_append's pointer rules: 16-byte rows need 16-byte aligned bases.
static bool append_ptrs_ok(const AppendIn& ap, const void* k_cache, const void* v_cache, int d_h, int eb) {
  if (!ap.k_new || !ap.v_new || !ap.write_pos || !aligned(ap.write_pos, 4)) return false;
  const uintptr_t al = (d_h * eb) % 16 == 0 ? 16 : (uintptr_t)eb;
  return aligned(ap.k_new, al) && aligned(ap.v_new, al) && aligned(k_cache, al) && aligned(v_cache, al);
}

// Decode over a contiguous cache, after an optional append (ap non-null).  Every
// check runs before the first launch.  The bf16 path with r <= 16 writes the new
// row inside the decode kernel; the other paths launch kv_append first.
static int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int32_t* q_pos, void* o,
                       int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                       float scale, int in_dtype, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream, const AppendIn* ap,
                       float rope_base = 0.f, bool check_only = false) {
  if (B < 1 || h_q < 1 || h_kv < 1 || T_cap < 1 || d_h < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (h_q % h_kv != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (max_seq_len > T_cap) return GQA_ERR_INVALID_ARGUMENT;
  if (!scale_ok(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(in_dtype) || !known_dtype(out_dtype)) return GQA_ERR_UNSUPPORTED;
  int st = check_types(in_dtype, out_dtype, d_h);
  if (st != GQA_OK) return st;
  st = check_ptrs(in_dtype, q, k_cache, v_cache, o);
  if (st != GQA_OK) return st;
  if (!seq_lens || !aligned(seq_lens, 4) || (q_pos && !aligned(q_pos, 4))) return GQA_ERR_INVALID_ARGUMENT;
  const int eb = in_dtype == GQA_BF16 ? 2 : 4;
  if (ap && !append_ptrs_ok(*ap, k_cache, v_cache, d_h, eb)) return GQA_ERR_INVALID_ARGUMENT;
  if (rope_base != 0.f && in_dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  const int len = max_seq_len > 0 ? max_seq_len : T_cap;
  DecodeArgs a;
  a.rope_base = rope_base;
  a.q = q; a.k = k_cache; a.v = v_cache; a.seq_lens = seq_lens; a.q_pos = q_pos; a.o = o;
  a.B = B; a.h_q = h_q; a.h_kv = h_kv; a.T_cap = T_cap; a.D = d_h; a.max_len = len;
  a.scale = scale;
  a.out_bf16 = out_dtype == GQA_BF16 ? 1 : 0;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  gqa::DecodePlan pl{};
  if (check_only) return GQA_OK;   // argument checks only (the workspace is the caller's next step)
  if (in_dtype == GQA_BF16) {
    pl = gqa::plan_decode_bf16(B, h_q, h_kv, T_cap, d_h, len);
    if (pl.n_split > 1) {
      if (workspace_bytes < pl.workspace_bytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
      if (!workspace || !aligned(workspace, 16)) return GQA_ERR_INVALID_ARGUMENT;
    }
  }
  const bool fused = ap && in_dtype == GQA_BF16 && h_q / h_kv <= 16;
  if (ap && !fused) {
    const hipError_t e =
        rope_base != 0.f
            ? gqa::launch_kv_append_rope(const_cast<void*>(k_cache), const_cast<void*>(v_cache), ap->k_new,
                                         ap->v_new, ap->write_pos, B, h_kv, T_cap, d_h, rope_base, eb, s)
            : gqa::launch_kv_append(const_cast<void*>(k_cache), const_cast<void*>(v_cache), ap->k_new, ap->v_new,
                                    ap->write_pos, B, h_kv, T_cap, d_h, eb, s);
    if (e != hipSuccess) return GQA_ERR_HIP;
  }
  if (fused) { a.k_new = ap->k_new; a.v_new = ap->v_new; a.write_pos = ap->write_pos; }
  if (in_dtype == GQA_F32) return hip_status(gqa::launch_decode_f32(a, s));
  return hip_status(gqa::launch_decode_bf16(a, pl, s));
}

// Decode over a paged cache, after an optional append (ap non-null).
static int decode_paged_impl(const void* q, const void* k_pages, const void* v_pages,
                             const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                             int B, int h_q, int h_kv, int page_size, int n_pages, int max_pages_per_seq, int d_h,
                             int max_seq_len, float scale, int in_dtype, int out_dtype,
                             void* workspace, size_t workspace_bytes, void* stream, const AppendIn* ap,
                             float rope_base = 0.f) {
  if (B < 1 || h_q < 1 || h_kv < 1 || page_size < 1 || n_pages < 1 || max_pages_per_seq < 1 || d_h < 1)
    return GQA_ERR_INVALID_ARGUMENT;
  if (h_q % h_kv != 0) return GQA_ERR_INVALID_ARGUMENT;
  const long long cap = (long long)page_size * max_pages_per_seq;
  if (cap > 0x7fffffffLL) return GQA_ERR_INVALID_ARGUMENT;
  const int T_cap = (int)cap;
  if (max_seq_len > T_cap) return GQA_ERR_INVALID_ARGUMENT;
  if (!scale_ok(scale)) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(in_dtype) || !known_dtype(out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (in_dtype != GQA_BF16 || page_size % 64 != 0) return GQA_ERR_UNSUPPORTED;
  int st = check_types(in_dtype, out_dtype, d_h);
  if (st != GQA_OK) return st;
  st = check_ptrs(in_dtype, q, k_pages, v_pages, o);
  if (st != GQA_OK) return st;
  if (!block_table || !seq_lens || !aligned(block_table, 4) || !aligned(seq_lens, 4) || (q_pos && !aligned(q_pos, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  if (ap && !append_ptrs_ok(*ap, k_pages, v_pages, d_h, 2)) return GQA_ERR_INVALID_ARGUMENT;
  const int len = max_seq_len > 0 ? max_seq_len : T_cap;
  DecodeArgs a;
  a.rope_base = rope_base;
  a.q = q; a.k = k_pages; a.v = v_pages; a.seq_lens = seq_lens; a.q_pos = q_pos; a.o = o;
  a.B = B; a.h_q = h_q; a.h_kv = h_kv; a.T_cap = T_cap; a.D = d_h; a.max_len = len;
  a.scale = scale;
  a.out_bf16 = out_dtype == GQA_BF16 ? 1 : 0;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.block_table = block_table; a.page_size = page_size; a.max_pages = max_pages_per_seq; a.n_pages = n_pages;
  const gqa::DecodePlan pl = gqa::plan_decode_bf16(B, h_q, h_kv, T_cap, d_h, len);
  if (pl.n_split > 1) {
    if (workspace_bytes < pl.workspace_bytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned(workspace, 16)) return GQA_ERR_INVALID_ARGUMENT;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = ap && h_q / h_kv <= 16;
  if (ap && !fused) {
    const hipError_t e =
        rope_base != 0.f
            ? gqa::launch_kv_append_paged_rope(const_cast<void*>(k_pages), const_cast<void*>(v_pages), ap->k_new,
                                               ap->v_new, block_table, ap->write_pos, B, h_kv, page_size, n_pages,
                                               max_pages_per_seq, d_h, rope_base, 2, s)
            : gqa::launch_kv_append_paged(const_cast<void*>(k_pages), const_cast<void*>(v_pages), ap->k_new,
                                          ap->v_new, block_table, ap->write_pos, B, h_kv, page_size, n_pages,
                                          max_pages_per_seq, d_h, 2, s);
    if (e != hipSuccess) return GQA_ERR_HIP;
  }
  if (fused) { a.k_new = ap->k_new; a.v_new = ap->v_new; a.write_pos = ap->write_pos; }
  return hip_status(gqa::launch_decode_bf16(a, pl, s));
}

int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* seq_lens, const int32_t* q_pos, void* o,
               int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
               float scale, int in_dtype, int out_dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, q_pos, o, B, h_q, h_kv, T_cap, d_h, max_seq_len, scale,
                     in_dtype, out_dtype, workspace, workspace_bytes, stream, nullptr);
}

int gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int32_t* q_pos, void* o,
                       int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                       float scale, int in_dtype, int out_dtype, void* stream) {
  // every argument is checked first, then the scratch the split plan needs, all
  // before the scratch's address is looked up and before any launch
  const int pre = decode_impl(q, k_cache, v_cache, seq_lens, q_pos, o, B, h_q, h_kv, T_cap, d_h, max_seq_len,
                              scale, in_dtype, out_dtype, nullptr, 0, nullptr, nullptr, 0.f, /*check_only=*/true);
  if (pre != GQA_OK) return pre;
  if (in_dtype == GQA_BF16) {
    const gqa::DecodePlan pl = gqa::plan_decode_bf16(B, h_q, h_kv, T_cap, d_h, max_seq_len > 0 ? max_seq_len : T_cap);
    if (pl.n_split > 1 && pl.workspace_bytes > GQA_DECODE_SCRATCH_BYTES) return GQA_ERR_SCRATCH_LIMIT;
  }
  void* ws = nullptr;
  if (current_scratch(&ws) != hipSuccess) return GQA_ERR_HIP;
  return decode_impl(q, k_cache, v_cache, seq_lens, q_pos, o, B, h_q, h_kv, T_cap, d_h, max_seq_len, scale,
                     in_dtype, out_dtype, ws, GQA_DECODE_SCRATCH_BYTES, stream, nullptr);
}

int gqa_append_decode(const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* write_pos, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                      int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                      float scale, int in_dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const AppendIn ap{k_new, v_new, write_pos};
  return decode_impl(q, k_cache, v_cache, seq_lens, q_pos, o, B, h_q, h_kv, T_cap, d_h, max_seq_len, scale,
                     in_dtype, out_dtype, workspace, workspace_bytes, stream, &ap);
}

int gqa_append_decode_rope(const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* write_pos, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                           int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                           float scale, float rope_base, int in_dtype, int out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!std::isfinite(rope_base) || rope_base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  const AppendIn ap{k_new, v_new, write_pos};
  return decode_impl(q, k_cache, v_cache, seq_lens, q_pos, o, B, h_q, h_kv, T_cap, d_h, max_seq_len, scale,
                     in_dtype, out_dtype, workspace, workspace_bytes, stream, &ap, rope_base);
}

int gqa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                     int B, int h_q, int h_kv, int page_size, int n_pages, int max_pages_per_seq, int d_h,
                     int max_seq_len, float scale, int in_dtype, int out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_paged_impl(q, k_pages, v_pages, block_table, seq_lens, q_pos, o, B, h_q, h_kv, page_size, n_pages,
                           max_pages_per_seq, d_h, max_seq_len, scale, in_dtype, out_dtype, workspace,
                           workspace_bytes, stream, nullptr);
}

int gqa_append_decode_paged(const void* q, void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                            const int32_t* block_table, const int32_t* write_pos, const int32_t* seq_lens,
                            const int32_t* q_pos, void* o, int B, int h_q, int h_kv, int page_size, int n_pages,
                            int max_pages_per_seq, int d_h, int max_seq_len, float scale, int in_dtype,
                            int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const AppendIn ap{k_new, v_new, write_pos};
  return decode_paged_impl(q, k_pages, v_pages, block_table, seq_lens, q_pos, o, B, h_q, h_kv, page_size, n_pages,
                           max_pages_per_seq, d_h, max_seq_len, scale, in_dtype, out_dtype, workspace,
                           workspace_bytes, stream, &ap);
}

int gqa_append_decode_paged_rope(const void* q, void* k_pages, void* v_pages, const void* k_new,
                                 const void* v_new, const int32_t* block_table, const int32_t* write_pos,
                                 const int32_t* seq_lens, const int32_t* q_pos, void* o, int B, int h_q, int h_kv,
                                 int page_size, int n_pages, int max_pages_per_seq, int d_h, int max_seq_len,
                                 float scale, float rope_base, int in_dtype, int out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!std::isfinite(rope_base) || rope_base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  const AppendIn ap{k_new, v_new, write_pos};
  return decode_paged_impl(q, k_pages, v_pages, block_table, seq_lens, q_pos, o, B, h_q, h_kv, page_size, n_pages,
                           max_pages_per_seq, d_h, max_seq_len, scale, in_dtype, out_dtype, workspace,
                           workspace_bytes, stream, &ap, rope_base);
}

int gqa_kv_append_paged_rope(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                             const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                             int page_size, int n_pages, int max_pages_per_seq, int d_h, float base, int dtype,
                             void* stream) {
  if (B < 1 || h_kv < 1 || page_size < 1 || n_pages < 1 || max_pages_per_seq < 1) return GQA_ERR_INVALID_ARGUMENT;
  if ((long long)page_size * max_pages_per_seq > 0x7fffffffLL) return GQA_ERR_INVALID_ARGUMENT;
  if (d_h < 2 || d_h % 2 != 0 || d_h / 2 > gqa::kRopeMaxHalf) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(base) || base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
  const int eb = dtype == GQA_BF16 ? 2 : 4;
  if (!k_pages || !v_pages || !k_new || !v_new || !block_table || !write_pos) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_pages, eb) || !aligned(v_pages, eb) || !aligned(k_new, eb) || !aligned(v_new, eb) ||
      !aligned(block_table, 4) || !aligned(write_pos, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  return hip_status(gqa::launch_kv_append_paged_rope(k_pages, v_pages, k_new, v_new, block_table, write_pos, B, h_kv,
                                                     page_size, n_pages, max_pages_per_seq, d_h, base, eb,
                                                     static_cast<hipStream_t>(stream)));
}

int gqa_kv_append_paged(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                        const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                        int page_size, int n_pages, int max_pages_per_seq, int d_h, int dtype, void* stream) {
  if (B < 1 || h_kv < 1 || page_size < 1 || n_pages < 1 || max_pages_per_seq < 1 || d_h < 1)
    return GQA_ERR_INVALID_ARGUMENT;
  if ((long long)page_size * max_pages_per_seq > 0x7fffffffLL) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype)) return GQA_ERR_INVALID_ARGUMENT;
  const int eb = dtype == GQA_BF16 ? 2 : 4;
  if ((d_h * eb) % 16 != 0) return GQA_ERR_UNSUPPORTED;
  if (!k_pages || !v_pages || !k_new || !v_new || !block_table || !write_pos) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(block_table, 4) || !aligned(write_pos, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  return hip_status(gqa::launch_kv_append_paged(k_pages, v_pages, k_new, v_new, block_table, write_pos, B, h_kv,
                                                page_size, n_pages, max_pages_per_seq, d_h, eb,
                                                static_cast<hipStream_t>(stream)));
}

int gqa_rope(const void* x, void* y, const int32_t* pos0, int B, int H, int S, int d_h, float base,
             int dtype, void* stream) {
  if (B < 1 || H < 1 || S < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (d_h < 2 || d_h % 2 != 0 || d_h / 2 > gqa::kRopeMaxHalf) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(base) || base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
  const int eb = dtype == GQA_BF16 ? 2 : 4;
  if (!x || !y || !aligned(x, eb) || !aligned(y, eb) || (pos0 && !aligned(pos0, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  return hip_status(gqa::launch_rope(x, y, pos0, B, H, S, d_h, base, eb, static_cast<hipStream_t>(stream)));
}

int gqa_rope_qk(const void* q, void* q_out, const void* k, void* k_out, const int32_t* pos0, int B,
                int h_q, int h_kv, int S, int d_h, float base, int dtype, void* stream) {
  if (B < 1 || h_q < 1 || h_kv < 1 || S < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (d_h < 2 || d_h % 2 != 0 || d_h / 2 > gqa::kRopeMaxHalf) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(base) || base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
  const int eb = dtype == GQA_BF16 ? 2 : 4;
  if (!q || !q_out || !k || !k_out || !aligned(q, eb) || !aligned(q_out, eb) || !aligned(k, eb) ||
      !aligned(k_out, eb) || (pos0 && !aligned(pos0, 4)))
    return GQA_ERR_INVALID_ARGUMENT;
  return hip_status(gqa::launch_rope_pair(q, q_out, h_q, k, k_out, h_kv, pos0, B, S, d_h, base, eb,
                                          static_cast<hipStream_t>(stream)));
}

int gqa_kv_append_rope(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* write_pos, int B, int h_kv, int T_cap, int d_h, float base,
                       int dtype, void* stream) {
  if (B < 1 || h_kv < 1 || T_cap < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (d_h < 2 || d_h % 2 != 0 || d_h / 2 > gqa::kRopeMaxHalf) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(base) || base <= 1.f) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
  const int eb = dtype == GQA_BF16 ? 2 : 4;
  if (!k_cache || !v_cache || !k_new || !v_new || !write_pos) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_cache, eb) || !aligned(v_cache, eb) || !aligned(k_new, eb) || !aligned(v_new, eb) ||
      !aligned(write_pos, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  return hip_status(gqa::launch_kv_append_rope(k_cache, v_cache, k_new, v_new, write_pos, B, h_kv, T_cap, d_h,
                                               base, eb, static_cast<hipStream_t>(stream)));
}

int gqa_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  const int32_t* write_pos, int B, int h_kv, int T_cap, int d_h,
                  int dtype, void* stream) {
  if (B < 1 || h_kv < 1 || T_cap < 1 || d_h < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (!known_dtype(dtype)) return GQA_ERR_INVALID_ARGUMENT;
  if (!k_cache || !v_cache || !k_new || !v_new || !write_pos) return GQA_ERR_INVALID_ARGUMENT;
  const int eb = dtype == GQA_BF16 ? 2 : 4;
  const uintptr_t al = (d_h * eb) % 16 == 0 ? 16 : (uintptr_t)eb;
  if (!aligned(k_cache, al) || !aligned(v_cache, al) || !aligned(k_new, al) || !aligned(v_new, al) ||
      !aligned(write_pos, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  return hip_status(gqa::launch_kv_append(k_cache, v_cache, k_new, v_new, write_pos, B, h_kv, T_cap,
                                          d_h, eb, static_cast<hipStream_t>(stream)));
}

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "GQA_OK: success";
    case GQA_ERR_INVALID_ARGUMENT: return "GQA_ERR_INVALID_ARGUMENT: invalid size, pointer, mask or scale";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: unsupported dtype / head-width combination";
    case GQA_ERR_WORKSPACE_TOO_SMALL: return "GQA_ERR_WORKSPACE_TOO_SMALL: decode workspace below gqa_decode_workspace_bytes()";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: HIP launch failure";
    case GQA_ERR_SCRATCH_LIMIT:
      return "GQA_ERR_SCRATCH_LIMIT: these sizes need more decode scratch than the library's static "
             "buffer (GQA_DECODE_SCRATCH_BYTES, 16 MiB); use gqa_decode with a workspace";
    default: return "unknown gqa status";
  }
}

}  // extern "C"
