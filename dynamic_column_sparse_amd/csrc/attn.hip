// Launchers of the attention kernels (kernel code: attn_kernels.h).
#include "attn_kernels.h"

namespace chipmunk {

hipError_t launch_attn_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* m, float* num, float* den,
                             float* o, float* score, int64_t n, int heads, float scale, hipStream_t s) {
  const int64_t nb = row_blocks(n);
  const dim3 grid((unsigned)(nb * heads));
  timing_before(K_ATTN_STATS, s);
  hipLaunchKernelGGL(attn_stats, grid, dim3(256), 0, s, q, k, m, den, n, heads, scale);
  hipError_t e = hipGetLastError();
  timing_after(K_ATTN_STATS, s);
  if (e != hipSuccess) return e;
  timing_before(K_ATTN_DENSE, s);
  hipLaunchKernelGGL(attn_dense, grid, dim3(256), 0, s, q, k, v, m, den, num, o, score, n, heads, scale);
  e = hipGetLastError();
  timing_after(K_ATTN_DENSE, s);
  return e;
}

hipError_t launch_attn_sparse(bool refresh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, const float* m, float* num, float* den, float* o, int64_t n,
                              int heads, int kk, float scale, hipStream_t s) {
  const int64_t nb = row_blocks(n);
  const dim3 grid((unsigned)(nb * heads));
  const int kid = refresh ? K_ATTN_REFRESH : K_ATTN_SPARSE;
  timing_before(kid, s);
  if (refresh)
    hipLaunchKernelGGL((attn_sparse<true>), grid, dim3(256), 0, s, q, k, v, idx, m, num, den, o, n, heads, kk, scale);
  else
    hipLaunchKernelGGL((attn_sparse<false>), grid, dim3(256), 0, s, q, k, v, idx, m, num, den, o, n, heads, kk, scale);
  hipError_t e = hipGetLastError();
  timing_after(kid, s);
  return e;
}

hipError_t launch_attn_reident(const uint16_t* q_prev, const uint16_t* k_prev, const uint16_t* v_prev,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                               const float* m, float* num, float* den, float* score, float* o, int64_t n, int heads,
                               int kk, float scale, hipStream_t s) {
  const int64_t nb = row_blocks(n);
  const dim3 grid((unsigned)(nb * heads));
  timing_before(K_ATTN_REIDENT, s);
  hipLaunchKernelGGL(attn_reident, grid, dim3(256), 0, s, q_prev, k_prev, v_prev, q, k, v, idx, m, num, den, score, o,
                     n, heads, kk, scale);
  hipError_t e = hipGetLastError();
  timing_after(K_ATTN_REIDENT, s);
  return e;
}

}  // namespace chipmunk
