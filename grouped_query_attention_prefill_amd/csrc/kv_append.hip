// Append one new token's key and value rows to a KV cache (B, h_kv, T_cap, d_h).
//
// A decode step first projects the new token's own K and V and appends them to
// the cache, then attends over every visible row ([AttnVar] 3.1; [MhaMqaGqa]
// section 4).  Row write_pos[b] of every cache head of sequence b receives
// k_new[b, :, 0, :] and v_new[b, :, 0, :]; a write_pos outside [0, T_cap)
// skips the sequence.  One workgroup per (K/V head, sequence), 16-byte
// copies when the row allows them.  The paged variant finds the row through the
// sequence's block table (rows of 16-byte multiples only).
#include "internal.h"

namespace gqa {
namespace {

__global__ void __launch_bounds__(64)
kv_append_kernel(unsigned char* kc, unsigned char* vc, const unsigned char* kn, const unsigned char* vn,
                 const int32_t* write_pos, int h_kv, int T_cap, int row_bytes) {
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int wp = write_pos[b];
  if (wp < 0 || wp >= T_cap) return;
  const size_t src = (size_t)(b * h_kv + g) * row_bytes;
  const size_t dst = ((size_t)(b * h_kv + g) * T_cap + wp) * row_bytes;
  if (row_bytes % 16 == 0) {
    for (int i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) {
      reinterpret_cast<uint4*>(kc + dst)[i] = reinterpret_cast<const uint4*>(kn + src)[i];
      reinterpret_cast<uint4*>(vc + dst)[i] = reinterpret_cast<const uint4*>(vn + src)[i];
    }
  } else {
    for (int i = threadIdx.x; i < row_bytes / 2; i += blockDim.x) {
      reinterpret_cast<uint16_t*>(kc + dst)[i] = reinterpret_cast<const uint16_t*>(kn + src)[i];
      reinterpret_cast<uint16_t*>(vc + dst)[i] = reinterpret_cast<const uint16_t*>(vn + src)[i];
    }
  }
}

// Paged cache: token position write_pos[b] lives in page
// block_table[b * max_pages + write_pos[b] / page_size], row write_pos[b] % page_size.
__global__ void __launch_bounds__(64)
kv_append_paged_kernel(unsigned char* kc, unsigned char* vc, const unsigned char* kn, const unsigned char* vn,
                       const int32_t* block_table, const int32_t* write_pos, int h_kv, int page_size,
                       int n_pages, int max_pages, int row_bytes) {
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int wp = write_pos[b];
  if (wp < 0 || wp >= max_pages * page_size) return;
  const int pg = block_table[(size_t)b * max_pages + wp / page_size];
  if (pg < 0 || pg >= n_pages) return;
  const size_t src = (size_t)(b * h_kv + g) * row_bytes;
  const size_t dst = (((size_t)pg * h_kv + g) * page_size + wp % page_size) * row_bytes;
  for (int i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) {
    reinterpret_cast<uint4*>(kc + dst)[i] = reinterpret_cast<const uint4*>(kn + src)[i];
    reinterpret_cast<uint4*>(vc + dst)[i] = reinterpret_cast<const uint4*>(vn + src)[i];
  }
}

}  // namespace

hipError_t launch_kv_append_paged(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                                  const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                                  int page_size, int n_pages, int max_pages, int D, int elem_bytes,
                                  hipStream_t s) {
  hipLaunchKernelGGL(kv_append_paged_kernel, dim3(h_kv, B), dim3(64), 0, s,
                     static_cast<unsigned char*>(k_pages), static_cast<unsigned char*>(v_pages),
                     static_cast<const unsigned char*>(k_new), static_cast<const unsigned char*>(v_new),
                     block_table, write_pos, h_kv, page_size, n_pages, max_pages, D * elem_bytes);
  return hipGetLastError();
}

hipError_t launch_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* write_pos, int B, int h_kv, int T_cap, int D,
                            int elem_bytes, hipStream_t s) {
  const int row_bytes = D * elem_bytes;
  hipLaunchKernelGGL(kv_append_kernel, dim3(h_kv, B), dim3(64), 0, s,
                     static_cast<unsigned char*>(k_cache), static_cast<unsigned char*>(v_cache),
                     static_cast<const unsigned char*>(k_new), static_cast<const unsigned char*>(v_new),
                     write_pos, h_kv, T_cap, row_bytes);
  return hipGetLastError();
}

}  // namespace gqa
