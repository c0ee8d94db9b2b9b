// Row-wise fp8 quantization for the fp8 variant of the MLP's first product
// (gfx950).  Each row of a bf16 matrix becomes OCP e4m3 codes with one
// power-of-two scale 2^e per row: e is the smallest integer (at least -126)
// with max|row| * 2^-e <= 448, e = 0 for an all-zero row, and each element is
// rounded to nearest even after the exact scaling by 2^-e (v_cvt_pk_fp8_f32;
// scaled values never exceed 448, so no code is NaN).  The scale is stored as
// its E8M0 byte 127 + e, the form the scaled matrix-core instructions take.
//
// One wave per row, four rows per workgroup: the row maximum is a wave
// reduction (no LDS, no barrier).  Rows of up to kCachedUnits * 64 * 8 values
// stay in registers between the maximum and the conversion (one read of the
// row; all of a lane's 16-byte loads are in flight together); longer rows are
// read twice.  Conversion goes 8 elements at a time (8-byte stores).
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

constexpr int kCachedUnits = 8;   // 16-byte units per lane kept in registers (rows up to 4096)

template <bool CACHED>
__global__ __launch_bounds__(256) void quantize_fp8_rows(const uint16_t* __restrict__ src, int64_t rows, int cols,
                                                         uint8_t* __restrict__ dst, uint8_t* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* s = src + row * cols;
  uint8_t* o = dst + row * cols;
  const int units = cols >> 3;
  // |x| as bf16 bits (sign cleared) orders like the values (finite inputs).
  uint32_t mx = 0;
  uint4 keep[CACHED ? kCachedUnits : 1];
  if (CACHED) {
#pragma unroll
    for (int i = 0; i < kCachedUnits; ++i) {
      const int u = lane + 64 * i;
      keep[i] = u < units ? *(const uint4*)(s + u * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kCachedUnits; ++i) mx = max(mx, abs_max_bf16x8(keep[i]));
  } else {
    for (int u = lane; u < units; u += 64) mx = max(mx, abs_max_bf16x8(*(const uint4*)(s + u * 8)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  const int e = fp8_exponent(mx);
  if (lane == 0) scale[row] = (uint8_t)(127 + e);
  if (CACHED) {
#pragma unroll
    for (int i = 0; i < kCachedUnits; ++i) {
      const int u = lane + 64 * i;
      if (u < units) *(uint2*)(o + u * 8) = bf16x8_to_fp8(keep[i], e);
    }
  } else {
    for (int u = lane; u < units; u += 64) *(uint2*)(o + u * 8) = bf16x8_to_fp8(*(const uint4*)(s + u * 8), e);
  }
}

// Column-wise variant (the output features of W2 for the fp8 second product):
// every column gets its own power-of-two scale, the same rule as a row above.
// One workgroup per strip of 128 columns: thread (row group rg = t/16, column
// group cg = t%16) takes 8 columns (16-byte loads) of rows rg, rg+16, ...; the
// 16 partial maxima of a column meet in LDS, then each thread converts its
// rows again with its columns' scales.  Used once per layer at set-up.
__global__ __launch_bounds__(256) void quantize_fp8_cols(const uint16_t* __restrict__ src, int64_t rows, int cols,
                                                         uint8_t* __restrict__ dst, uint8_t* __restrict__ scale) {
  __shared__ uint32_t smax[16][128 + 1];
  __shared__ int sexp[128];
  const int t = threadIdx.x, cg = t & 15, rg = t >> 4;
  const int c0 = blockIdx.x * 128 + cg * 8;
  const bool live = c0 < cols;   // cols % 8 == 0: a column group is wholly in or out
  uint32_t mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0;
  if (live) {
    for (int64_t r = rg; r < rows; r += 16) {
      const uint4 v = *(const uint4*)(src + r * cols + c0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx[2 * i] = max(mx[2 * i], w[i] & 0x7fffu);
        mx[2 * i + 1] = max(mx[2 * i + 1], (w[i] >> 16) & 0x7fffu);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) smax[rg][cg * 8 + e] = mx[e];
  __syncthreads();
  if (t < 128) {
    uint32_t m = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) m = max(m, smax[g][t]);
    const int e = fp8_exponent(m);
    sexp[t] = e;
    if (blockIdx.x * 128 + t < cols) scale[blockIdx.x * 128 + t] = (uint8_t)(127 + e);
  }
  __syncthreads();
  if (!live) return;
  float mul[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mul[e] = __uint_as_float((uint32_t)(127 - sexp[cg * 8 + e]) << 23);
  for (int64_t r = rg; r < rows; r += 16) {
    const uint4 v = *(const uint4*)(src + r * cols + c0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf2f(w[i] & 0xffffu) * mul[2 * i];
      x[2 * i + 1] = bf2f(w[i] >> 16) * mul[2 * i + 1];
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
    *(uint2*)(dst + r * cols + c0) = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

}  // namespace

hipError_t launch_quantize_fp8_cols(const uint16_t* src, int64_t rows, int cols, uint8_t* dst, uint8_t* scale,
                                    hipStream_t s) {
  const dim3 grid((unsigned)((cols + 127) / 128));
  timing_before(K_QUANTIZE_FP8, s);
  hipLaunchKernelGGL(quantize_fp8_cols, grid, dim3(256), 0, s, src, rows, cols, dst, scale);
  hipError_t e = hipGetLastError();
  timing_after(K_QUANTIZE_FP8, s);
  return e;
}

hipError_t launch_quantize_fp8(const uint16_t* src, int64_t rows, int cols, uint8_t* dst, uint8_t* scale,
                               hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  timing_before(K_QUANTIZE_FP8, s);
  if (cols <= kCachedUnits * 64 * 8)
    hipLaunchKernelGGL(quantize_fp8_rows<true>, grid, dim3(256), 0, s, src, rows, cols, dst, scale);
  else
    hipLaunchKernelGGL(quantize_fp8_rows<false>, grid, dim3(256), 0, s, src, rows, cols, dst, scale);
  hipError_t e = hipGetLastError();
  timing_after(K_QUANTIZE_FP8, s);
  return e;
}

}  // namespace chipmunk
