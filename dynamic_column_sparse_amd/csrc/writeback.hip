// Cache writeback: scatter packed new activations into the block-column-major
// activation cache (gfx950).  Hidden unit j of block b is 128 contiguous bf16
// (256 bytes) in both layouts, so each group of 16 threads moves one whole
// segment with 16-byte loads and stores.
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

__global__ __launch_bounds__(256) void cache_writeback(const uint16_t* __restrict__ packed,
                                                       const int32_t* __restrict__ idx,
                                                       uint16_t* __restrict__ a_cache, int h, int k) {
  const int64_t b = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t p = t >> 4;
  const int c = (int)(t & 15) * 8;
  if (p >= k) return;
  const int j = clamp_index(idx[b * k + p], h);
  *(uint4*)(a_cache + (b * h + j) * kRowBlock + c) = *(const uint4*)(packed + (b * k + p) * kRowBlock + c);
}

}  // namespace

hipError_t launch_writeback(const uint16_t* packed, const int32_t* idx, uint16_t* a_cache, int64_t n, int h, int k,
                            hipStream_t s) {
  const int64_t nb = row_blocks(n);
  dim3 grid((unsigned)(((int64_t)k * 16 + 255) / 256), (unsigned)nb);
  timing_before(K_WRITEBACK, s);
  hipLaunchKernelGGL(cache_writeback, grid, dim3(256), 0, s, packed, idx, a_cache, h, k);
  hipError_t e = hipGetLastError();
  timing_after(K_WRITEBACK, s);
  return e;
}

}  // namespace chipmunk
