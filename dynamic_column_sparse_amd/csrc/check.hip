// Check of caller-built index sets against the library's contract: every value
// in [0, cols), each row strictly ascending (hence unique).  The compute
// kernels clamp out-of-range values instead of faulting, which hides such a
// mistake; this reports it.
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

// result = {0, rows}: no bad row yet; rows stands for "none".
__global__ void check_init(int64_t* result, int64_t rows) {
  if (threadIdx.x == 0) {
    result[0] = 0;
    result[1] = rows;
  }
}

// One wave per row: lane j looks at elements j, j + 64, ... and at each one's
// predecessor; the wave's verdict is a ballot, recorded by lane 0 with two
// device-scope atomics (count, smallest bad row).
__global__ __launch_bounds__(256) void check_rows(const int32_t* __restrict__ idx, int64_t rows, int k, int64_t cols,
                                                  int64_t* __restrict__ result) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;   // wave-uniform
  const int32_t* row = idx + r * k;
  bool bad = false;
  for (int j = lane; j < k; j += 64) {
    const int32_t v = row[j];
    bad |= v < 0 || (int64_t)v >= cols;
    if (j > 0) bad |= row[j - 1] >= v;
  }
  if (__ballot(bad) != 0 && lane == 0) {
    atomicAdd(reinterpret_cast<unsigned long long*>(result), 1ull);
    atomicMin(reinterpret_cast<long long*>(result + 1), (long long)r);
  }
}

}  // namespace

hipError_t launch_check_index_sets(const int32_t* idx, int64_t rows, int k, int64_t cols, int64_t* result,
                                   hipStream_t s) {
  hipLaunchKernelGGL(check_init, dim3(1), dim3(64), 0, s, result, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows == 0 || k == 0) return e;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL(check_rows, grid, dim3(256), 0, s, idx, rows, k, cols, result);
  return hipGetLastError();
}

}  // namespace chipmunk
