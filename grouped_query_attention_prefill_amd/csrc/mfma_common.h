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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer resource over [base, base + bytes): loads at or past `bytes` return 0
// (checked per dword), which zero-fills partial tiles without branches.  base and
// bytes must be the same on every lane of the wave; readfirstlane tells the
// compiler so, which keeps the descriptor in scalar registers (a descriptor it
// believes divergent costs a loop over lanes around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* const ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// A operand of O^T += V^T P^T for 16 keys (chunk kc of the LDS tile) and 32 values
// of d starting at d0, read from row-major V in LDS with two transposing reads.
// ds_read_b64_tr_b16 works in groups of 16 lanes: source lane s = 4j + q supplies
// 4 consecutive 16-bit values, and output lane i receives, as its value j, element
// i % 4 of source lane 4j + i / 4.  Pointing source lane (j, q) of group G at row
// (16 kc + 8u + 4(G / 2) + j), columns d0 + 16(G % 2) + 4q .. +3 hands output lane
// l the values V[16 kc + 8u + 4(l / 32) + j][d0 + l % 32], j = 0..3: exactly the
// keys chunk_key() assigns to slots 4u .. 4u + 3 of lane half l / 32.
__device__ __forceinline__ bf16x8 load_vt_operand(const unsigned char* vrow0, int vs_bytes, int kc, int d0,
                                                  int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int j = s >> 2, q = s & 3;
  const unsigned char* base = vrow0 + (16 * kc + 4 * (G >> 1) + j) * vs_bytes + (d0 + 16 * (G & 1) + 4 * q) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * vs_bytes));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Key held by slot t (0..7) of lane half h within 16-key chunk kc of a tile:
// slots 0..7 of half h are keys {4h..4h+3, 8+4h..8+4h+3}.  This is the key order
// in which the S^T accumulator rows come out of the matrix core, so P feeds the
// next product straight from registers; load_vt_operand() reads V in that order.
__device__ __forceinline__ int chunk_key(int kc, int h, int t) {
  return kc * 16 + 8 * (t >> 2) + 4 * h + (t & 3);
}

// Running maximum is only moved when a tile's maximum exceeds it by more than
// this many powers of two; until then exp2 arguments stay <= kLazyRescale, the
// probabilities stay <= 2^kLazyRescale, and the rescale of O and l is skipped.
// The final o = u / l is unchanged: numerator and denominator carry the same
// factor ([EffSeq] 在线 softmax: any common base m gives the same ratio).
constexpr float kLazyRescale = 8.0f;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace gqa
