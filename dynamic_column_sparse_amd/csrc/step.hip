// The sparse step of one transformer block as two launches: the MLP's sparse
// phase 1, then ONE kernel whose first workgroups run the MLP's phase-2 tiles
// and whose remaining workgroups run the attention delta.
//
// The attention delta and the MLP delta of a step read different inputs and
// write different outputs, so nothing orders them.  Run one after the other,
// the phase-2 tiles (one wave of long units) leave part of the chip idle at
// their tail and the attention units (1.6 waves of short ones) leave a ragged
// tail of their own.  Sharing one grid lets the short attention units fill the
// workgroup slots beside the long phase-2 units (longest work first), and the
// two kernels' tails overlap.
//
// Both bodies are the single-kernel ones (same tiles, same order of sums), so
// the fused step gives bit-identical results to the two separate calls.
#include "attn_kernels.h"
#include "mlp_kernels.h"

namespace chipmunk {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// blockIdx.x < g2: phase-2 unit blockIdx.x of xcd_grid(ntn * nb) units.
// Otherwise: attention unit blockIdx.x - g2.  g2 is a multiple of 8, so both
// bodies keep their own unit -> XCD mapping (unit id mod 8).
template <int BN>
__global__ __launch_bounds__(256, 2) void sparse_step_fused(
    int g2, const uint16_t* __restrict__ dsrc, const uint16_t* __restrict__ w2, const int32_t* __restrict__ midx,
    float* __restrict__ y, int64_t n, int d, int h, int k, int kp, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kx, const uint16_t* __restrict__ v, const int32_t* __restrict__ aidx,
    const float* __restrict__ m, const float* __restrict__ num, const float* __restrict__ den,
    float* __restrict__ o, int64_t na, int heads, int kk, float scale) {
  __shared__ __align__(16) unsigned char smem[cmax(Gemm2RowsLds<BN>::kRing, AttnSparseLds::kRing)];
  __shared__ __align__(16) int sIdx[8][32];
  __shared__ float sDen[kRowBlock];
  __shared__ float sDenRest[kRowBlock];
  static_assert(Gemm2RowsLds<BN>::kIds == 8 * 32 && AttnSparseLds::kIds == 8 * 32, "id ring size");
  const int bid = blockIdx.x;
  if (bid < g2)
    gemm2_rows_body<BN>(bid, smem, sIdx, dsrc, w2, midx, y, n, d, h, k, kp);
  else
    // The sparse (non-refresh) body only reads num and den.
    attn_sparse_body<false>(bid - g2, smem, sIdx, sDen, sDenRest, q, kx, v, aidx, m, const_cast<float*>(num),
                            const_cast<float*>(den), o, na, heads, kk, scale);
}

}  // namespace

hipError_t launch_sparse_step(const uint16_t* x, const uint16_t* w1t, const float* b1, const int32_t* midx,
                              uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed, float* mscore,
                              const uint16_t* w2, float* y, int64_t n, int d, int h, int k, const uint16_t* q,
                              const uint16_t* kx, const uint16_t* v, const int32_t* aidx, const float* m,
                              const float* num, const float* den, float* o, int64_t na, int heads, int kk,
                              float scale, hipStream_t s, const Fp8Rows* f8) {
  const int kp = padded_k(k);
  int g2 = 0;
  const int bn = d % 256 == 0 ? 256 : 128;
  if (k > 0) {
    hipError_t e = launch_mlp_gemm1(false, x, w1t, b1, midx, a_cache, dbuf, a_packed, mscore, n, d, h, k, s, f8);
    if (e != hipSuccess) return e;
    g2 = xcd_grid(d / bn * (int)row_blocks(n));
  }
  const int ga = (int)(row_blocks(na) * heads);
  const dim3 grid((unsigned)(g2 + ga));
  timing_before(K_SPARSE_STEP_FUSED, s);
  if (bn == 256)
    hipLaunchKernelGGL((sparse_step_fused<256>), grid, dim3(256), 0, s, g2, dbuf, w2, midx, y, n, d, h, k, kp, q, kx,
                       v, aidx, m, num, den, o, na, heads, kk, scale);
  else
    hipLaunchKernelGGL((sparse_step_fused<128>), grid, dim3(256), 0, s, g2, dbuf, w2, midx, y, n, d, h, k, kp, q, kx,
                       v, aidx, m, num, den, o, na, heads, kk, scale);
  hipError_t e = hipGetLastError();
  timing_after(K_SPARSE_STEP_FUSED, s);
  return e;
}

}  // namespace chipmunk
