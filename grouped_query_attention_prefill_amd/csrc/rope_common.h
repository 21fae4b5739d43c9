// Rotary position encoding arithmetic shared by the rotation kernels and the
// attention kernels that rotate Q (and the appended key) as they load them, so the
// fused and the separate paths produce the same bits.
//
// The pages print no rotation formula; the form used is the common one, pair
// (x[i], x[i + d/2]) turned by the angle p * theta_i, theta_i = base^(-2 i / d):
//     y[i]       = x[i] cos - x[i + d/2] sin,   y[i + d/2] = x[i + d/2] cos + x[i] sin.
// theta_i / (2 pi) comes from the host as a 64-bit fixed-point fraction of a turn
// F_i; the device forms p * F_i modulo 2^64 with integer products, which drops the
// whole turns exactly (angles reach 3e4 radians at the lengths served) and leaves
// the fraction, whose top 32 bits, read as a signed fraction in [-1/2, 1/2), feed
// the hardware sine and cosine (which take turns) in single precision.
#pragma once

#include <cmath>

#include "internal.h"
#include "mfma_common.h"

namespace gqa {

struct RopeFreq {
  uint64_t turn_frac[kRopeMaxHalf];   // round(2^64 theta_i / (2 pi)), i < d / 2
};

inline RopeFreq make_rope_freq(int d, float base) {
  RopeFreq f;
  const int half = d / 2;
  const long double two_pi = 6.283185307179586476925286766559L;
  for (int i = 0; i < kRopeMaxHalf; ++i) {
    if (i >= half) { f.turn_frac[i] = 0; continue; }
    const long double turns = std::pow((long double)base, -2.0L * i / d) / two_pi;   // < 1 turn
    f.turn_frac[i] = (uint64_t)std::llround(std::ldexp(turns, 63)) << 1;
  }
  return f;
}

// cos and sin of p * theta for theta = 2 pi F / 2^64: p * F modulo 2^64 is the
// fraction of a turn; its top 32 bits, signed, are that fraction in [-1/2, 1/2).
__device__ __forceinline__ void rope_cos_sin(int p, uint64_t F, float& c, float& s) {
  const uint64_t t = (uint64_t)(int64_t)p * F;
  const float f = (float)(int32_t)(uint32_t)(t >> 32) * 0x1p-32f;
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// One pair turned, with the rounding of each step fixed (one product, one fused
// multiply-add) so every caller gets the same bits.
__device__ __forceinline__ void rope_rotate(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = __builtin_fmaf(x0, c, -(x1 * s));
  y1 = __builtin_fmaf(x1, c, x0 * s);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  const __bf16 b = (__bf16)v;                  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

// Turn fractions F_i of the head widths the attention kernels serve (d_h <= 128), as
// kernel arguments: a lane reads the entries its elements need with scalar loads
// and a select, never by a lane-varying index into the argument block.
constexpr int kRopeKernelHalf = 64;
struct RopeTheta {
  uint64_t t[kRopeKernelHalf];       // the first entries of RopeFreq::turn_frac
};

inline RopeTheta make_rope_theta(int d, float base) {
  const RopeFreq f = make_rope_freq(d, base);
  RopeTheta r;
  for (int i = 0; i < kRopeKernelHalf; ++i) r.t[i] = f.turn_frac[i];
  return r;
}

// Rotate the bf16 pairs (lo[e], hi[e]), e < 8, of one row at position p: lo[e] is
// element i_e of the first half, hi[e] its partner i_e + d/2, th[e] = F_{i_e}.
__device__ __forceinline__ void rope_rotate8(bf16x8& lo, bf16x8& hi, int p, const uint64_t (&th)[8]) {
  typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
  u16x8 l = __builtin_bit_cast(u16x8, lo), u = __builtin_bit_cast(u16x8, hi);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float c, s, y0, y1;
    rope_cos_sin(p, th[e], c, s);
    rope_rotate(bf16_bits_to_f32(l[e]), bf16_bits_to_f32(u[e]), c, s, y0, y1);
    l[e] = f32_to_bf16_bits(y0);
    u[e] = f32_to_bf16_bits(y1);
  }
  lo = __builtin_bit_cast(bf16x8, l);
  hi = __builtin_bit_cast(bf16x8, u);
}

}  // namespace gqa
