// fp32 grouped-query attention for any head width 1..256 (reference-precision path).
//
// Serves prefill, chunked prefill and decode with one kernel.  A workgroup
// owns one (sequence b, K/V head g) and 32 "rows"; rows are the r query heads
// of the group packed with query positions, position-major
// (row = i * r + head_in_group), so one K/V tile in LDS serves every head of
// the group ([MhaMqaGqa] section 7: one K/V tile is loaded once for all query
// rows of its group; a prefill block packs positions x heads, each row keeping
// its own causal position).  The key loop runs the online softmax of
// [EffSeq] 在线 softmax with per-row state (m, l, u): m is the running maximum
// of scaled scores, l the normalizer, u the unnormalized output; a new tile
// rescales (l, u) by e^{m - m'} and adds its own terms.  Masked keys are
// removed by selection ([MhaMqaGqa] section 1: -inf at invisible positions).
// All arithmetic is fp32 with the accurate expf; the order of additions
// differs from a materialized softmax only by rounding ([EffSeq] 资源变化).
#include "internal.h"

#include <cmath>

namespace gqa {
namespace {

constexpr int kRows = 32;    // query rows per workgroup
constexpr int kKeys = 32;    // keys per tile
constexpr int kThreads = 256;
constexpr int kMaxD = 256;
constexpr int kUPerThread = kMaxD / 8;

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;             // (B, h_q, S_q) or null
  const int32_t* kv_lens;
  const int32_t* q_pos0;
  int h_q, h_kv, r, S_q, T_cap, D;
  int causal, from_end, max_len;
  float scale;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__global__ void __launch_bounds__(kThreads)
attn_f32_kernel(F32Params p) {
  extern __shared__ float smem[];
  const int D = p.D;
  const int ld = D + 1;                    // padded row stride (bank spread)
  float* Qs = smem;                        // [kRows][ld]
  float* Ks = Qs + kRows * ld;             // [kKeys][ld]
  float* Vs = Ks + kKeys * ld;             // [kKeys][ld]
  float* Ps = Vs + kKeys * ld;             // [kRows][kKeys + 1]

  const int tid = threadIdx.x;
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int row0 = blockIdx.x * kRows;
  const int n_rows = p.r * p.S_q;

  const int len_b = clampi(p.kv_lens ? p.kv_lens[b] : p.T_cap, 0, p.T_cap);
  const int pos0 = p.q_pos0 ? p.q_pos0[b] : (p.from_end ? len_b - p.S_q : 0);
  const int kv_len = min(len_b, p.max_len);

  // this thread's row in the score / output mapping
  const int ri = tid / 8;
  const int rlane = tid % 8;
  const int rho = row0 + ri;
  const bool row_valid = rho < n_rows;
  const int qi = row_valid ? rho / p.r : 0;
  const int hh = row_valid ? rho % p.r : 0;
  const int head = g * p.r + hh;
  const int pos = pos0 + qi;

  // the block's key extent: up to the largest position of its valid rows
  int kv_end = kv_len;
  if (p.causal) {
    const int last = min(row0 + kRows, n_rows) - 1;
    const int max_pos = pos0 + last / p.r;
    kv_end = min(kv_len, max(max_pos + 1, 0));
  }

  // stage the block's queries
  for (int e = tid; e < kRows * D; e += kThreads) {
    const int i = e / D, d = e % D;
    const int rr = row0 + i;
    float x = 0.f;
    if (rr < n_rows) {
      const int h2 = g * p.r + rr % p.r;
      const int q2 = rr / p.r;
      x = p.q[((size_t)(b * p.h_q + h2) * p.S_q + q2) * D + d];
    }
    Qs[i * ld + d] = x;
  }

  float m = -INFINITY, l = 0.f;
  float u[kUPerThread];
#pragma unroll
  for (int e = 0; e < kUPerThread; ++e) u[e] = 0.f;

  const size_t kv_base = (size_t)(b * p.h_kv + g) * p.T_cap * D;
  for (int j0 = 0; j0 < kv_end; j0 += kKeys) {
    __syncthreads();   // previous tile fully consumed (and Qs staged on the first pass)
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int j = e / D, d = e % D;
      const int key = j0 + j;
      float kx = 0.f, vx = 0.f;
      if (key < kv_end) {
        kx = p.k[kv_base + (size_t)key * D + d];
        vx = p.v[kv_base + (size_t)key * D + d];
      }
      Ks[j * ld + d] = kx;
      Vs[j * ld + d] = vx;
    }
    __syncthreads();

    // scores of row ri against keys rlane + 8c
    float s[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = rlane + 8 * c;
      const int key = j0 + j;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(Qs[ri * ld + d], Ks[j * ld + d], acc);
      const bool vis = row_valid && key < kv_len && (!p.causal || key <= pos);
      s[c] = vis ? acc * p.scale : -INFINITY;
      tmax = fmaxf(tmax, s[c]);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 8));
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // no -inf - (-inf)
    const float alpha = expf(m - m_use);                      // 0 while nothing was visible
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float pr = (s[c] == -INFINITY) ? 0.f : expf(s[c] - m_use);
      psum += pr;
      Ps[ri * (kKeys + 1) + rlane + 8 * c] = pr;
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) psum += __shfl_xor(psum, off, 8);
    l = alpha * l + psum;
    m = m_new;
    __syncthreads();

    // u[ri][d] = alpha u + sum_j P[ri][j] V[j][d] for d = rlane + 8e
#pragma unroll
    for (int e = 0; e < kUPerThread; ++e) {
      const int d = rlane + 8 * e;
      if (d < D) {
        float acc = alpha * u[e];
        for (int j = 0; j < kKeys; ++j) acc = fmaf(Ps[ri * (kKeys + 1) + j], Vs[j * ld + d], acc);
        u[e] = acc;
      }
    }
  }

  if (row_valid) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    float* orow = p.o + ((size_t)(b * p.h_q + head) * p.S_q + qi) * D;
#pragma unroll
    for (int e = 0; e < kUPerThread; ++e) {
      const int d = rlane + 8 * e;
      if (d < D) orow[d] = u[e] * inv;
    }
    // m is the running maximum of the scaled scores, l the sum of exp(s - m)
    if (p.lse && rlane == 0) p.lse[(size_t)(b * p.h_q + head) * p.S_q + qi] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

size_t f32_smem_bytes(int D) {
  const int ld = D + 1;
  return sizeof(float) * ((size_t)kRows * ld + 2 * (size_t)kKeys * ld + (size_t)kRows * (kKeys + 1));
}

hipError_t launch(const F32Params& prm, int B, hipStream_t s) {
  const int n_rows = prm.r * prm.S_q;
  dim3 grid((n_rows + kRows - 1) / kRows, prm.h_kv, B);
  const size_t smem = f32_smem_bytes(prm.D);
  if (smem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_f32_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(kThreads), smem, s, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  F32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.kv_lens = a.kv_lens;
  p.q_pos0 = a.q_pos0;
  p.h_q = a.h_q; p.h_kv = a.h_kv; p.r = a.h_q / a.h_kv;
  p.S_q = a.S_q; p.T_cap = a.T_cap; p.D = a.D;
  p.causal = a.causal; p.from_end = a.q_pos_from_end; p.max_len = a.T_cap;
  p.scale = a.scale;
  return launch(p, a.B, s);
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
  F32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = nullptr;
  p.kv_lens = a.seq_lens;
  p.q_pos0 = a.q_pos;
  p.h_q = a.h_q; p.h_kv = a.h_kv; p.r = a.h_q / a.h_kv;
  p.S_q = 1; p.T_cap = a.T_cap; p.D = a.D;
  p.causal = 1; p.from_end = 1; p.max_len = a.max_len;
  p.scale = a.scale;
  return launch(p, a.B, s);
}

}  // namespace gqa
