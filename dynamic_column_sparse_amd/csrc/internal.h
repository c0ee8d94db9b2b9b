// Internal launch interface between the C ABI (validation, timing) and the
// kernel translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace chipmunk {

constexpr int kRowBlock = 128;
constexpr int kHeadDim = 128;

// Kernel ids for the optional per-kernel timer (order = chipmunk_kernel_name ids).
enum KernelId {
  K_MLP_GEMM1_SPARSE = 0,
  K_MLP_GEMM1_DENSE,
  K_MLP_GEMM2_SPARSE,
  K_MLP_GEMM2_DENSE,
  K_TOPK,
  K_WRITEBACK,
  K_ATTN_STATS,
  K_ATTN_DENSE,
  K_ATTN_SPARSE,
  K_ATTN_REFRESH,
  K_SPARSE_STEP_FUSED,
  K_ATTN_REIDENT,
  K_QUANTIZE_FP8,
  K_SPARSE_STEP_REIDENT_FUSED,
  K_COUNT
};
const char* kernel_name(int kid);

// Size of the library-owned scratch array of the allocation-free entry point
// (CHIPMUNK_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of that array on the current device (looked up once per
// device, then cached).  Allocates nothing.
hipError_t noalloc_scratch(void** out);

// Timer hooks (no-ops unless chipmunk_timing_enable(1)).
void timing_before(int kid, hipStream_t s);
void timing_after(int kid, hipStream_t s);

__host__ __device__ inline int64_t row_blocks(int64_t n) { return (n + kRowBlock - 1) / kRowBlock; }
// Rows per block of the D tiles: k rounded up to the 64-wide reduction chunk
// (the rows past k are zero, so phase 2 streams whole chunks).
__host__ __device__ inline int padded_k(int k) { return (k + 63) / 64 * 64; }

// fp8 operands of the MLP's first product: e4m3 codes of x [n][d] and W1^T
// [h][d] with one E8M0 scale byte per row.
struct Fp8Rows {
  const uint8_t* x;
  const uint8_t* x_scale;
  const uint8_t* w;
  const uint8_t* w_scale;
};
// fp8 W2 of the fp8 second product: e4m3 codes [h][d] with one E8M0 scale
// byte per column (output feature).
struct Fp8Cols {
  const uint8_t* w;
  const uint8_t* w_scale;
};
// MLP phase 1: gathered x W1[:,S] + GELU, then either the sparse epilogue
// (D tiles, cache writeback; with a score array, also S's column L1 of D) or
// the dense one (score, full cache write).  f8 non-NULL: the product runs on
// the fp8 operands instead of x and w1t; fp8_d (sparse): D leaves as fp8
// codes with (row, 32-unit) scales for the fp8 second product.
hipError_t launch_mlp_gemm1(bool dense, const uint16_t* x, const uint16_t* w1t, const float* b1,
                            const int32_t* idx, uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed,
                            float* score, int64_t n, int d, int h, int k, hipStream_t s,
                            const Fp8Rows* f8 = nullptr, bool fp8_d = false);
// Row-wise fp8 quantization of a bf16 [rows][cols] matrix (cols % 8 == 0).
hipError_t launch_quantize_fp8(const uint16_t* src, int64_t rows, int cols, uint8_t* dst, uint8_t* scale,
                               hipStream_t s);
// Column-wise: scale[c] for each column (cols % 8 == 0).
hipError_t launch_quantize_fp8_cols(const uint16_t* src, int64_t rows, int cols, uint8_t* dst, uint8_t* scale,
                                    hipStream_t s);
// MLP phase 2: y (+)= src[b] W2[S] where src is [nb][kc][128] (D tiles, or the cache).
// f8w (sparse only): src holds phase 1's fp8 D and the product runs on f8w.
hipError_t launch_mlp_gemm2(bool dense, const uint16_t* src, const uint16_t* w2, const int32_t* idx,
                            const float* b2, float* y, int64_t n, int d, int h, int k, int kc,
                            hipStream_t s, const Fp8Cols* f8w = nullptr);
hipError_t launch_writeback(const uint16_t* packed, const int32_t* idx, uint16_t* a_cache, int64_t n, int h,
                            int k, hipStream_t s);
hipError_t launch_topk(const float* score, int64_t rows, int64_t cols, int k, int32_t* idx, hipStream_t s);
// Index-set check: result[0] = rows breaking the contract, result[1] = the
// smallest such row (rows if none).
hipError_t launch_check_index_sets(const int32_t* idx, int64_t rows, int k, int64_t cols, int64_t* result,
                                   hipStream_t s);
hipError_t launch_attn_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* m, float* num,
                             float* den, float* o, float* score, int64_t n, int heads, float scale,
                             hipStream_t s);
hipError_t launch_attn_sparse(bool refresh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, const float* m, float* num, float* den, float* o, int64_t n,
                              int heads, int kk, float scale, hipStream_t s);
// Sparse attention step with per-step re-identification (num, den hold totals).
hipError_t launch_attn_reident(const uint16_t* q_prev, const uint16_t* k_prev, const uint16_t* v_prev,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                               const float* m, float* num, float* den, float* score, float* o, int64_t n, int heads,
                               int kk, float scale, hipStream_t s);
// Sparse MLP phase 1, then one kernel with the MLP phase-2 tiles first and the
// sparse attention units after them (k = 0: attention units only).
hipError_t launch_sparse_step(const uint16_t* x, const uint16_t* w1t, const float* b1, const int32_t* midx,
                              uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed, float* mscore,
                              const uint16_t* w2, float* y,
                              int64_t n, int d, int h, int k, const uint16_t* q, const uint16_t* kx,
                              const uint16_t* v, const int32_t* aidx, const float* m, const float* num,
                              const float* den, float* o, int64_t na, int heads, int kk, float scale,
                              hipStream_t s, const Fp8Rows* f8 = nullptr, const Fp8Cols* f8w = nullptr);

// The same with the re-identifying attention step in the shared grid.
hipError_t launch_sparse_step_reident(const uint16_t* x, const uint16_t* w1t, const float* b1, const int32_t* midx,
                                      uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed, float* mscore,
                                      const uint16_t* w2, float* y, int64_t n, int d, int h, int k,
                                      const uint16_t* q_prev, const uint16_t* k_prev, const uint16_t* v_prev,
                                      const uint16_t* q, const uint16_t* kx, const uint16_t* v, const int32_t* aidx,
                                      const float* m, float* num, float* den, float* ascore, float* o, int64_t na,
                                      int heads, int kk, float scale, hipStream_t s, const Fp8Rows* f8,
                                      const Fp8Cols* f8w);

}  // namespace chipmunk
