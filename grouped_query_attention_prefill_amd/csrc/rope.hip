// Rotary position encoding of query and key rows, and the key-rotating append.
//
// Every query head and every stored key head is rotated by its position before
// the scores are formed ([EffSeq] 分组查询注意力: under rotary encoding all query
// heads and each key head actually kept are rotated; [MhaMqaGqa] note under the
// parameter table: attention uses the position-processed Q and K).  A group's key
// head is therefore rotated once, when it is written, not once per query head that
// reads it; and the rotation is applied to the new key on its way into the cache,
// never to rows already stored, which other readers may share ([Ch09] 09.4).
//
// The rotation (pair (x[i], x[i + d/2]) turned by p * base^(-2 i / d), angles
// reduced to a fraction of a turn in fixed point, hardware sine and cosine) is in
// rope_common.h, shared with the attention kernels that rotate Q as they load it.
// Elements are read and written in the tensor's own precision; the arithmetic is fp32.
#include "internal.h"
#include "rope_common.h"

namespace gqa {
namespace {

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }

template <typename T, int VEC>
struct Vec;
template <>
struct Vec<float, 4> { typedef float4 type; };
template <>
struct Vec<uint16_t, 8> { typedef uint4 type; };
template <typename T>
struct Vec<T, 1> { typedef T type; };

// One thread per (row, VEC consecutive pairs).  Rows are (b, h, s) of a (B, H, S, d)
// tensor; row s of sequence b sits at position pos0[b] + s.  With VEC > 1 both halves
// of the pairs move as 16-byte vectors (the launcher uses rope_heads_kernel below for
// those).  One launch may rotate two tensors of the same rows' positions (Q and K):
// chunk indices past the first tensor's fall to the second.
struct RopeSeg {
  const void* x;
  void* y;
  int H;
  long long n_chunks;
};

template <typename T, int VEC>
__global__ void __launch_bounds__(256)
rope_kernel(RopeSeg a, RopeSeg a2, const int32_t* pos0, int S, int half, RopeFreq f) {
  typedef typename Vec<T, VEC>::type V;
  long long cidx = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool second = cidx >= a.n_chunks;
  if (second) {
    cidx -= a.n_chunks;
    if (cidx >= a2.n_chunks) return;
  }
  const T* x = static_cast<const T*>(second ? a2.x : a.x);
  T* y = static_cast<T*>(second ? a2.y : a.y);
  const int H = second ? a2.H : a.H;
  const int chunks = half / VEC;
  const long long row = cidx / chunks;
  const int i0 = (int)(cidx - row * chunks) * VEC;
  const int s = (int)(row % S);
  const int b = (int)(row / ((long long)S * H));
  const int p = (pos0 ? pos0[b] : 0) + s;
  const T* xr = x + row * 2 * half + i0;
  T* yr = y + row * 2 * half + i0;
  V lo = *reinterpret_cast<const V*>(xr);
  V hi = *reinterpret_cast<const V*>(xr + half);
  T* l = reinterpret_cast<T*>(&lo);
  T* u = reinterpret_cast<T*>(&hi);
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    float c, sn, y0, y1;
    rope_cos_sin(p, f.turn_frac[i0 + v], c, sn);
    rope_rotate(ld(l + v), ld(u + v), c, sn, y0, y1);
    st(l + v, y0);
    st(u + v, y1);
  }
  *reinterpret_cast<V*>(yr) = lo;
  *reinterpret_cast<V*>(yr + half) = hi;
}

// The vectorized form: one thread per (sequence, group of kHeadGroup heads, position,
// VEC consecutive pairs).  The angles depend only on the position and the pair, so a
// thread computes its VEC sines and cosines once and turns the same pairs of every
// head of its group; it requests all of the group's rows before it turns any, so
// 2 kHeadGroup 16-byte loads are in flight per thread.  Consecutive threads take
// consecutive pairs, then positions, so each head's rows are read and written as
// contiguous runs.  The arithmetic per element is the one above, bit for bit.
constexpr int kHeadGroup = 8;

template <typename T, int VEC>
__global__ void __launch_bounds__(256)
rope_heads_kernel(RopeSeg a, RopeSeg a2, long long n1, long long n2, const int32_t* pos0, int S, int half,
                  RopeFreq f) {
  typedef typename Vec<T, VEC>::type V;
  long long cidx = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool second = cidx >= n1;
  if (second) {
    cidx -= n1;
    if (cidx >= n2) return;
  }
  const T* x = static_cast<const T*>(second ? a2.x : a.x);
  T* y = static_cast<T*>(second ? a2.y : a.y);
  const int H = second ? a2.H : a.H;
  const int n_groups = (H + kHeadGroup - 1) / kHeadGroup;
  const int chunks = half / VEC;
  const int i0 = (int)(cidx % chunks) * VEC;
  long long rest = cidx / chunks;
  const int s = (int)(rest % S);
  rest /= S;
  const int grp = (int)(rest % n_groups);
  const int b = (int)(rest / n_groups);
  const int p = (pos0 ? pos0[b] : 0) + s;
  const int h0 = grp * kHeadGroup;
  const int nh = min(kHeadGroup, H - h0);
  const long long row_stride = (long long)S * 2 * half;        // elements between heads
  const long long base = ((long long)(b * H + h0) * S + s) * 2 * half + i0;
  V lo[kHeadGroup], hi[kHeadGroup];
#pragma unroll
  for (int j = 0; j < kHeadGroup; ++j)
    if (j < nh) {
      lo[j] = *reinterpret_cast<const V*>(x + base + j * row_stride);
      hi[j] = *reinterpret_cast<const V*>(x + base + j * row_stride + half);
    }
  float c[VEC], sn[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) rope_cos_sin(p, f.turn_frac[i0 + v], c[v], sn[v]);
#pragma unroll
  for (int j = 0; j < kHeadGroup; ++j)
    if (j < nh) {
      T* l = reinterpret_cast<T*>(&lo[j]);
      T* u = reinterpret_cast<T*>(&hi[j]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float y0, y1;
        rope_rotate(ld(l + v), ld(u + v), c[v], sn[v], y0, y1);
        st(l + v, y0);
        st(u + v, y1);
      }
      *reinterpret_cast<V*>(y + base + j * row_stride) = lo[j];
      *reinterpret_cast<V*>(y + base + j * row_stride + half) = hi[j];
    }
}

// Append with the key rotated at its own position: one workgroup per (K/V head,
// sequence); threads < d/2 rotate key pairs, all threads copy the value row.  With
// a block table (paged pools (n_pages, h_kv, page_size, d)) the row is found through
// the sequence's page, and a page outside the pool skips the sequence.
template <typename T>
__global__ void __launch_bounds__(128)
kv_append_rope_kernel(T* kc, T* vc, const T* kn, const T* vn, const int32_t* write_pos, int h_kv,
                      int T_cap, int half, RopeFreq f, const int32_t* block_table, int page_size,
                      int n_pages, int max_pages) {
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int wp = write_pos[b];
  if (wp < 0 || wp >= T_cap) return;
  const int d = 2 * half;
  size_t row = ((size_t)(b * h_kv + g) * T_cap + wp) * d;
  if (block_table) {
    const int pg = block_table[(size_t)b * max_pages + wp / page_size];
    if (pg < 0 || pg >= n_pages) return;
    row = (((size_t)pg * h_kv + g) * page_size + wp % page_size) * d;
  }
  const T* ks = kn + (size_t)(b * h_kv + g) * d;
  const T* vs = vn + (size_t)(b * h_kv + g) * d;
  T* kd = kc + row;
  T* vd = vc + row;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float c, sn, y0, y1;
    rope_cos_sin(wp, f.turn_frac[i], c, sn);
    rope_rotate(ld(ks + i), ld(ks + i + half), c, sn, y0, y1);
    st(kd + i, y0);
    st(kd + i + half, y1);
  }
  for (int i = threadIdx.x; i < d; i += blockDim.x) vd[i] = vs[i];
}

}  // namespace

hipError_t launch_rope_pair(const void* x, void* y, int H, const void* x2, void* y2, int H2,
                            const int32_t* pos0, int B, int S, int D, float base, int elem_bytes, hipStream_t s) {
  const int half = D / 2;
  const RopeFreq f = make_rope_freq(D, base);
  auto al = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  const bool al16 = al(x) && al(y) && (H2 == 0 || (al(x2) && al(y2)));
  const int vec = !al16 ? 1 : (elem_bytes == 4 ? (half % 4 == 0 ? 4 : 1) : (half % 8 == 0 ? 8 : 1));
  const RopeSeg a{x, y, H, (long long)B * H * S * (half / vec)};
  const RopeSeg a2{x2, y2, H2, (long long)B * H2 * S * (half / vec)};
  if (vec > 1) {
    // head groups: each thread turns the same pairs of up to kHeadGroup heads
    const long long n1 = (long long)B * ((H + kHeadGroup - 1) / kHeadGroup) * S * (half / vec);
    const long long n2 = (long long)B * ((H2 + kHeadGroup - 1) / kHeadGroup) * S * (half / vec);
    const long long blocks = (n1 + n2 + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(256);
    if (elem_bytes == 4)
      hipLaunchKernelGGL((rope_heads_kernel<float, 4>), grid, block, 0, s, a, a2, n1, n2, pos0, S, half, f);
    else
      hipLaunchKernelGGL((rope_heads_kernel<uint16_t, 8>), grid, block, 0, s, a, a2, n1, n2, pos0, S, half, f);
    return hipGetLastError();
  }
  // element by element (unaligned tensors, or half widths the vectors do not divide)
  const long long blocks = (a.n_chunks + a2.n_chunks + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (elem_bytes == 4) hipLaunchKernelGGL((rope_kernel<float, 1>), grid, block, 0, s, a, a2, pos0, S, half, f);
  else hipLaunchKernelGGL((rope_kernel<uint16_t, 1>), grid, block, 0, s, a, a2, pos0, S, half, f);
  return hipGetLastError();
}

hipError_t launch_rope(const void* x, void* y, const int32_t* pos0, int B, int H, int S, int D,
                       float base, int elem_bytes, hipStream_t s) {
  return launch_rope_pair(x, y, H, nullptr, nullptr, 0, pos0, B, S, D, base, elem_bytes, s);
}

namespace {
hipError_t append_rope(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* write_pos, int B, int h_kv, int T_cap, int D, float base, int elem_bytes,
                       const int32_t* block_table, int page_size, int n_pages, int max_pages, hipStream_t s) {
  const RopeFreq f = make_rope_freq(D, base);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(kv_append_rope_kernel<float>, dim3(h_kv, B), dim3(128), 0, s,
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), static_cast<const float*>(k_new),
                       static_cast<const float*>(v_new), write_pos, h_kv, T_cap, D / 2, f, block_table, page_size,
                       n_pages, max_pages);
  else
    hipLaunchKernelGGL(kv_append_rope_kernel<uint16_t>, dim3(h_kv, B), dim3(128), 0, s,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), write_pos, h_kv,
                       T_cap, D / 2, f, block_table, page_size, n_pages, max_pages);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_kv_append_rope(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                 const int32_t* write_pos, int B, int h_kv, int T_cap, int D, float base,
                                 int elem_bytes, hipStream_t s) {
  return append_rope(k_cache, v_cache, k_new, v_new, write_pos, B, h_kv, T_cap, D, base, elem_bytes, nullptr, 0, 0,
                     0, s);
}

hipError_t launch_kv_append_paged_rope(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                                       const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                                       int page_size, int n_pages, int max_pages, int D, float base, int elem_bytes,
                                       hipStream_t s) {
  return append_rope(k_pages, v_pages, k_new, v_new, write_pos, B, h_kv, page_size * max_pages, D, base, elem_bytes,
                     block_table, page_size, n_pages, max_pages, s);
}

}  // namespace gqa
