// Internal launch interface between the C ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>

namespace gqa {

// Kernels with more than 64 KiB of dynamic LDS have to be allowed it
// (hipFuncSetAttribute) on each device they run on.  `done` records the devices
// already allowed, one bit per device ordinal below 64 (other ordinals are set on
// every call); two threads racing on a first call both set the attribute, which
// is harmless.
inline hipError_t allow_dynamic_lds(const void* fn, int bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Attention over a cache for S_q query rows per sequence at absolute positions
// q_pos0[b] + i.  Prefill is the case q_pos0 = 0, S_q = T_cap.
struct AttnArgs {
  const void* q;          // (B, h_q, S_q, D)
  const void* k;          // (B, h_kv, T_cap, D)
  const void* v;          // (B, h_kv, T_cap, D)
  void* o;                // (B, h_q, S_q, D)
  const int32_t* kv_lens; // (B,) or null -> T_cap
  const int32_t* q_pos0;  // (B,) or null -> (kv_len - S_q) when from_end, else 0
  int B, h_q, h_kv, S_q, T_cap, D;
  int causal;
  int q_pos_from_end;     // 1: default position of row 0 is kv_len - S_q
  float scale;
  int out_bf16;           // output dtype of the bf16 path
  float* lse = nullptr;   // (B, h_q, S_q) natural-log row log-sum-exp of the scaled scores, or null
  float rope_base = 0.f;  // > 0: Q rotated at each row's position as it is loaded (bf16 path)
};

// Decode: one query per sequence at q_pos[b] (null -> seq_lens[b] - 1), keys
// j < min(seq_lens[b], q_pos[b] + 1, max_len).
struct DecodeArgs {
  const void* q;          // (B, h_q, 1, D)
  const void* k;          // (B, h_kv, T_cap, D)
  const void* v;
  const int32_t* seq_lens;
  const int32_t* q_pos;
  void* o;                // (B, h_q, 1, D)
  int B, h_q, h_kv, T_cap, D, max_len;
  float scale;
  int out_bf16;
  void* workspace;
  size_t workspace_bytes;
  // paged cache (block_table non-null): k, v point at page pools (n_pages, h_kv,
  // page_size, D); T_cap = max_pages * page_size
  const int32_t* block_table = nullptr;
  int page_size = 0, max_pages = 0, n_pages = 0;
  // fused append (write_pos non-null; 16x16 kernel only, r <= 16): k_new, v_new
  // (B, h_kv, 1, D) written to position write_pos[b] and used by this decode
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* write_pos = nullptr;
  // > 0: rotary encoding inside the kernels, Q at its query position and (fused
  // append) the new key at write_pos[b]
  float rope_base = 0.f;
};

struct DecodePlan {
  int head_chunks;   // ceil(r / 32)
  int chunk;         // keys per split (multiple of the key tile)
  int n_split;       // splits launched
  int n_split_cap;   // splits the workspace is sized for
  size_t workspace_bytes;
};

// Split plan for the bf16 decode path.  `len` is the grid-sizing bound.
DecodePlan plan_decode_bf16(int B, int h_q, int h_kv, int T_cap, int D, int len);

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
hipError_t launch_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* write_pos, int B, int h_kv, int T_cap, int D,
                            int elem_bytes, hipStream_t s);
// Gradients of bf16 prefill attention (dQ, dK, dV in fp32) from the forward's output
// O and row log-sum-exp; the workspace holds delta = rowsum(dO * O), one float per row.
struct BwdArgs {
  const void* q;          // (B, h_q, T, D) bf16
  const void* k;          // (B, h_kv, T, D) bf16
  const void* v;
  const void* o;          // (B, h_q, T, D) fp32 or bf16 (o_bf16)
  const void* d_o;        // (B, h_q, T, D) bf16
  const float* lse;       // (B, h_q, T)
  float* dq;              // (B, h_q, T, D)
  float* dk;              // (B, h_kv, T, D)
  float* dv;
  const int32_t* kv_lens; // (B,) or null -> T
  int B, h_q, h_kv, T, D, causal, o_bf16;
  float scale;
  void* workspace;        // bwd_workspace_bytes(B, h_q, T)
};
size_t bwd_workspace_bytes(int B, int h_q, int T);
hipError_t launch_backward_bf16(const BwdArgs& a, hipStream_t s);

// rotary encoding: head widths up to 2 * kRopeMaxHalf
constexpr int kRopeMaxHalf = 128;
// Two tensors (x: H heads, x2: H2 heads) rotated at the same positions in one launch.
hipError_t launch_rope_pair(const void* x, void* y, int H, const void* x2, void* y2, int H2,
                            const int32_t* pos0, int B, int S, int D, float base, int elem_bytes, hipStream_t s);
hipError_t launch_rope(const void* x, void* y, const int32_t* pos0, int B, int H, int S, int D,
                       float base, int elem_bytes, hipStream_t s);
hipError_t launch_kv_append_rope(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                 const int32_t* write_pos, int B, int h_kv, int T_cap, int D, float base,
                                 int elem_bytes, hipStream_t s);
hipError_t launch_kv_append_paged_rope(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                                       const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                                       int page_size, int n_pages, int max_pages, int D, float base, int elem_bytes,
                                       hipStream_t s);
hipError_t launch_kv_append_paged(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                                  const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                                  int page_size, int n_pages, int max_pages, int D, int elem_bytes,
                                  hipStream_t s);

}  // namespace gqa
