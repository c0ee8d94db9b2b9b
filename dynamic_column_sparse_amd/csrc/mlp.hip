// Launchers of the MLP kernels (kernel code: mlp_kernels.h).
#include "mlp_kernels.h"

namespace chipmunk {

#ifndef MLP_WIDE_WASTE_PCT
#define MLP_WIDE_WASTE_PCT 25
#endif
// Largest share of computed-but-unused columns (percent) accepted for 256-wide
// phase-1 tiles.
constexpr int kWideWastePct = MLP_WIDE_WASTE_PCT;

hipError_t launch_mlp_gemm1(bool dense, const uint16_t* x, const uint16_t* w1t, const float* b1,
                            const int32_t* idx, uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed,
                            float* score, int64_t n, int d, int h, int k, hipStream_t s, const Fp8Rows* f8,
                            bool fp8_d) {
  const int nb = (int)row_blocks(n);
  const int cols = dense ? h : k;
  const int kp = padded_k(k);
  // 256-wide tiles when they waste little of the last tile, else 128-wide.
  const int t256 = (cols + 255) / 256, t128 = (cols + 127) / 128;
  const bool wide = t128 > 1 && (int64_t)t256 * 256 * 100 <= (int64_t)cols * (100 + kWideWastePct);
  const int kid = dense ? K_MLP_GEMM1_DENSE : K_MLP_GEMM1_SPARSE;
  const void* xa = f8 ? (const void*)f8->x : (const void*)x;
  const void* wa = f8 ? (const void*)f8->w : (const void*)w1t;
  const uint8_t* xs = f8 ? f8->x_scale : nullptr;
  const uint8_t* ws = f8 ? f8->w_scale : nullptr;
  const dim3 grid((unsigned)xcd_grid((wide ? t256 : t128) * nb));
#define G1_LAUNCH(BN_, DENSE_, F8_, FD_)                                                                    \
  hipLaunchKernelGGL((mlp_gemm1<BN_, DENSE_, F8_, FD_>), grid, dim3(256), 0, s, xa, wa, xs, ws, b1, idx, a_cache, \
                     dbuf, a_packed, score, n, d, h, k, kp)
  // (the dense step writes no D, so it has no fp8-D form)
#define G1_LAUNCH_F8(BN_, DENSE_)                 \
  {                                               \
    if (!DENSE_ && fp8_d) {                       \
      if (f8)                                     \
        G1_LAUNCH(BN_, false, true, true);        \
      else                                        \
        G1_LAUNCH(BN_, false, false, true);       \
    } else if (f8) {                              \
      G1_LAUNCH(BN_, DENSE_, true, false);        \
    } else {                                      \
      G1_LAUNCH(BN_, DENSE_, false, false);       \
    }                                             \
  }
  timing_before(kid, s);
  if (wide) {
    if (dense)
      G1_LAUNCH_F8(256, true)
    else
      G1_LAUNCH_F8(256, false)
  } else {
    if (dense)
      G1_LAUNCH_F8(128, true)
    else
      G1_LAUNCH_F8(128, false)
  }
#undef G1_LAUNCH_F8
#undef G1_LAUNCH
  hipError_t e = hipGetLastError();
  timing_after(kid, s);
  return e;
}

hipError_t launch_mlp_gemm2(bool dense, const uint16_t* src, const uint16_t* w2, const int32_t* idx,
                            const float* b2, float* y, int64_t n, int d, int h, int k, int kp, hipStream_t s,
                            const Fp8Cols* f8w) {
  const int nb = (int)row_blocks(n);
  const int kid = dense ? K_MLP_GEMM2_DENSE : K_MLP_GEMM2_SPARSE;
  const int bn = d % 256 == 0 ? 256 : 128;
  const dim3 grid((unsigned)xcd_grid(d / bn * nb));
  timing_before(kid, s);
  if (dense) {
    if (bn == 256)
      hipLaunchKernelGGL((mlp_gemm2<256, true>), grid, dim3(256), 0, s, src, w2, idx, b2, y, n, d, h, k, kp);
    else
      hipLaunchKernelGGL((mlp_gemm2<128, true>), grid, dim3(256), 0, s, src, w2, idx, b2, y, n, d, h, k, kp);
  } else if (f8w) {
    const unsigned char* d8 = (const unsigned char*)src;
    if (bn == 256)
      hipLaunchKernelGGL((mlp_gemm2_rows_f8<256>), grid, dim3(256), 0, s, d8, f8w->w, f8w->w_scale, idx, y, n, d, h,
                         k, kp);
    else
      hipLaunchKernelGGL((mlp_gemm2_rows_f8<128>), grid, dim3(256), 0, s, d8, f8w->w, f8w->w_scale, idx, y, n, d, h,
                         k, kp);
  } else {
    if (bn == 256)
      hipLaunchKernelGGL((mlp_gemm2_rows<256>), grid, dim3(256), 0, s, src, w2, idx, y, n, d, h, k, kp);
    else
      hipLaunchKernelGGL((mlp_gemm2_rows<128>), grid, dim3(256), 0, s, src, w2, idx, y, n, d, h, k, kp);
  }
  hipError_t e = hipGetLastError();
  timing_after(kid, s);
  return e;
}

}  // namespace chipmunk
