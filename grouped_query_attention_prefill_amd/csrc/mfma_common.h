// Device helpers shared by the bf16 matrix-core kernels (gfx950 / CDNA4).
//
// Matrix-core tile used throughout: v_mfma_f32_32x32x16_bf16, wave64.
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + t], t = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + t][l % 32]
//   C (32 x 32): lane l, element e holds C[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32]
// The attention kernels compute S^T = K Q^T and O^T = V^T P^T, so that a lane's
// column is one query row: every per-row softmax quantity (running max m,
// normalizer l, rescale factor) then lives in the lane that owns the row, and
// only lanes l and l ^ 32 share a row.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value of x in lane l ^ 32 combined with this lane's: max / sum over the two
// lanes that share a query row.  permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; called with x twice, the two
// results hold {own, partner} in some order on every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pack 8 floats into bf16 (round to nearest even, the hardware conversion).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Workgroup barrier that waits only for this wave's LDS traffic, not for its
// outstanding global loads, so prefetched tiles stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Interleave two bf16 lanes of 8 dwords: lo -> the low halves, hi -> the high halves.
// x[t] holds (d, d+1) of key t; the result rows hold 8 keys of one d.
__device__ __forceinline__ void split_pairs(const uint32_t x[8], uint4& lo, uint4& hi) {
  lo.x = (x[0] & 0xffffu) | (x[1] << 16);
  lo.y = (x[2] & 0xffffu) | (x[3] << 16);
  lo.z = (x[4] & 0xffffu) | (x[5] << 16);
  lo.w = (x[6] & 0xffffu) | (x[7] << 16);
  hi.x = (x[0] >> 16) | (x[1] & 0xffff0000u);
  hi.y = (x[2] >> 16) | (x[3] & 0xffff0000u);
  hi.z = (x[4] >> 16) | (x[5] & 0xffff0000u);
  hi.w = (x[6] >> 16) | (x[7] & 0xffff0000u);
}

// Key held by slot t (0..7) of lane half h within 16-key chunk kc of a tile:
// slots 0..7 of half h are keys {4h..4h+3, 8+4h..8+4h+3}.  This is the key order
// in which the S^T accumulator rows come out of the matrix core, so P feeds the
// next product straight from registers; V^T is stored in LDS in the same order.
__device__ __forceinline__ int chunk_key(int kc, int h, int t) {
  return kc * 16 + 8 * (t >> 2) + 4 * h + (t & 3);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace gqa
