// Streaming-read reference kernel for the benchmark (libgqa_readfloor.so; not part of
// the attention library).  It reads a buffer once, 16 bytes per load, four loads in
// flight per thread, with a grid of two 256-thread workgroups per compute unit,
// which was the fastest of the grid sizes tried (512 to 8192 workgroups).  The time
// it takes for a decode row's algorithmic byte count, measured the same way as that
// row (inputs evicted from the Infinity Cache, HIP events around one call), is the
// floor the row's own time is compared with.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

__global__ void __launch_bounds__(256) read_floor_kernel(const uint4* __restrict__ x, size_t n16, unsigned* out) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = x[i], b = x[i + stride], c = x[i + 2 * stride], d = x[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = x[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // one word per workgroup, so the loads cannot be dropped
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Workgroups launched by gqa_read_floor on the current device (the size `out` needs, in words).
int gqa_read_floor_grid(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return 2 * cus;
}

// Read bytes (a multiple of 16) of device buffer x once on `stream`; out: device buffer of
// gqa_read_floor_grid() unsigned words.  Returns 0, or 1 on a bad argument or launch error.
int gqa_read_floor(const void* x, size_t bytes, unsigned* out, void* stream) {
  if (!x || !out || bytes % 16 != 0) return 1;   // checked before any HIP call
  const int grid = gqa_read_floor_grid();
  if (grid < 1) return 1;
  hipLaunchKernelGGL(read_floor_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(x), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
