// The sparse step of one transformer block as two launches: the MLP's sparse
// phase 1, then ONE kernel whose workgroups run the MLP's phase-2 tiles and the
// attention delta (the fixed-set step, or the step that re-identifies its keys
// every step).
//
// The attention delta and the MLP delta of a step read different inputs and
// write different outputs, so nothing orders them.  Run one after the other,
// each leaves a ragged tail (at FLUX the phase-2 tiles are one wave of long
// units, the attention units 1.6 waves of short ones).  Sharing one grid
// overlaps the tails, and the longer kind of unit goes first so that the
// shorter kind fills the grid's end: the phase-2 tiles at FLUX, the attention
// units (8316 keys each) at HunyuanVideo.
//
// Both bodies are the single-kernel ones (same tiles, same order of sums), so
// the fused step gives bit-identical results to the two separate calls.
#include "attn_kernels.h"
#include "mlp_kernels.h"

namespace chipmunk {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// With ga_first == 0: blockIdx.x < g2 is phase-2 unit blockIdx.x of
// xcd_grid(ntn * nb) units, and the rest are attention units.  With
// ga_first > 0 (the attention units are the longer ones): the first ga_first
// workgroups (the heads * nb attention units, rounded up to a multiple of 8)
// are attention units and the rest phase-2 units, so the short phase-2 tiles
// fill the grid's tail.  g2 and ga_first are multiples of 8, so both bodies
// keep their own unit -> XCD mapping (unit id mod 8).  F8W: the phase-2 tiles
// run the fp8 second product (fp8 D from phase 1, fp8 W2 rows).
template <int BN, bool F8W>
__global__ __launch_bounds__(256, 2) void sparse_step_fused(
    int g2, int ga_first, const uint16_t* __restrict__ dsrc, const uint16_t* __restrict__ w2, const uint8_t* __restrict__ w2f8,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ midx, float* __restrict__ y, int64_t n, int d, int h,
    int k, int kp, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kx, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ aidx, const float* __restrict__ m, const float* __restrict__ num,
    const float* __restrict__ den, float* __restrict__ o, int64_t na, int heads, int kk, float scale) {
  constexpr int kG2Ring = F8W ? Gemm2RowsF8Lds<BN>::kRing : Gemm2RowsLds<BN>::kRing;
  constexpr int kG2Ids = F8W ? Gemm2RowsF8Lds<BN>::kIds : Gemm2RowsLds<BN>::kIds;
  __shared__ __align__(16) unsigned char smem[cmax(kG2Ring, AttnSparseLds::kRing)];
  __shared__ __align__(16) int sIdx[cmax(kG2Ids, AttnSparseLds::kIds)];
  __shared__ float sDen[kRowBlock];
  __shared__ float sDenRest[kRowBlock];
  static_assert(AttnSparseLds::kIds == 8 * 32, "id ring size");
  const int bid = blockIdx.x;
  const bool phase2 = ga_first > 0 ? bid >= ga_first : bid < g2;
  if (phase2) {
    const int lin = ga_first > 0 ? bid - ga_first : bid;
    if constexpr (F8W)
      gemm2_rows_body_f8<BN>(lin, smem, reinterpret_cast<int(*)[64]>(sIdx), (const unsigned char*)dsrc, w2f8, w2s,
                             midx, y, n, d, h, k, kp);
    else
      gemm2_rows_body<BN>(lin, smem, reinterpret_cast<int(*)[32]>(sIdx), dsrc, w2, midx, y, n, d, h, k, kp);
  } else {
    const int lin = ga_first > 0 ? bid : bid - g2;
    if (lin >= (int)row_blocks(na) * heads) return;   // padding up to a multiple of 8
    // The sparse (non-refresh) body only reads num and den.
    attn_sparse_body<false>(lin, smem, reinterpret_cast<int(*)[32]>(sIdx), sDen, sDenRest, q, kx, v, aidx, m,
                            const_cast<float*>(num), const_cast<float*>(den), o, na, heads, kk, scale);
  }
}

// LDS of a phase-2 tile (ring and id ring), for the overlay below.
template <int BN, bool F8W>
struct Gemm2TileLds {
  unsigned char ring[F8W ? Gemm2RowsF8Lds<BN>::kRing : Gemm2RowsLds<BN>::kRing];
  int ids[F8W ? Gemm2RowsF8Lds<BN>::kIds : Gemm2RowsLds<BN>::kIds];
};
template <int BN, bool F8W>
union ReidentStepLds {
  Gemm2TileLds<BN, F8W> g2;
  AttnReidentLds at;
};

// The same shared grid with the re-identifying attention step (num, den hold
// totals; the previous step's q, k, v give the share taken out) in place of
// the fixed-set one, with the same ordering (ga_first).  The two bodies' LDS
// overlay each other.
template <int BN, bool F8W>
__global__ __launch_bounds__(256, 2) void sparse_step_reident_fused(
    int g2, int ga_first, const uint16_t* __restrict__ dsrc, const uint16_t* __restrict__ w2, const uint8_t* __restrict__ w2f8,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ midx, float* __restrict__ y, int64_t n, int d, int h,
    int k, int kp, const uint16_t* __restrict__ q_prev, const uint16_t* __restrict__ k_prev,
    const uint16_t* __restrict__ v_prev, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kx,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ aidx, const float* __restrict__ m,
    float* __restrict__ num, float* __restrict__ den, float* __restrict__ ascore, float* __restrict__ o, int64_t na,
    int heads, int kk, float scale) {
  __shared__ __align__(16) ReidentStepLds<BN, F8W> lds;
  const int bid = blockIdx.x;
  const bool phase2 = ga_first > 0 ? bid >= ga_first : bid < g2;
  if (phase2) {
    const int lin = ga_first > 0 ? bid - ga_first : bid;
    if constexpr (F8W)
      gemm2_rows_body_f8<BN>(lin, lds.g2.ring, reinterpret_cast<int(*)[64]>(lds.g2.ids),
                             (const unsigned char*)dsrc, w2f8, w2s, midx, y, n, d, h, k, kp);
    else
      gemm2_rows_body<BN>(lin, lds.g2.ring, reinterpret_cast<int(*)[32]>(lds.g2.ids), dsrc, w2, midx, y, n, d, h, k,
                          kp);
  } else {
    const int lin = ga_first > 0 ? bid : bid - g2;
    if (lin >= (int)row_blocks(na) * heads) return;   // padding up to a multiple of 8
    attn_reident_body(lin, lds.at, q_prev, k_prev, v_prev, q, kx, v, aidx, m, num, den, ascore, o, na, heads, kk,
                      scale);
  }
}

}  // namespace

hipError_t launch_sparse_step_reident(const uint16_t* x, const uint16_t* w1t, const float* b1, const int32_t* midx,
                                      uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed, float* mscore,
                                      const uint16_t* w2, float* y, int64_t n, int d, int h, int k,
                                      const uint16_t* q_prev, const uint16_t* k_prev, const uint16_t* v_prev,
                                      const uint16_t* q, const uint16_t* kx, const uint16_t* v, const int32_t* aidx,
                                      const float* m, float* num, float* den, float* ascore, float* o, int64_t na,
                                      int heads, int kk, float scale, hipStream_t s, const Fp8Rows* f8,
                                      const Fp8Cols* f8w) {
  const int kp = padded_k(k);
  int g2 = 0;
  const int bn = d % 256 == 0 ? 256 : 128;
  if (k > 0) {
    hipError_t e =
        launch_mlp_gemm1(false, x, w1t, b1, midx, a_cache, dbuf, a_packed, mscore, n, d, h, k, s, f8, f8w != nullptr);
    if (e != hipSuccess) return e;
    g2 = xcd_grid(d / bn * (int)row_blocks(n));
  }
  const int ga = (int)(row_blocks(na) * heads);
  // Longest units first (see launch_sparse_step); a re-identifying unit
  // streams its key chunks twice, once per step's inputs.
  const int64_t attn_bytes = 2 * (int64_t)((kk + 31) / 32) * 16384;
  const int64_t g2_bytes = f8w ? (int64_t)(kp / 64) * (kRowBlock * 64 + 64 * bn)
                               : (int64_t)(kp / 32) * (kRowBlock * 64 + 32 * bn * 2);
  const int ga_first = (g2 > 0 && ga > 0 && attn_bytes > g2_bytes) ? xcd_grid(ga) : 0;
  const dim3 grid((unsigned)(ga_first > 0 ? ga_first + g2 : g2 + ga));
  timing_before(K_SPARSE_STEP_REIDENT_FUSED, s);
  const uint8_t* w2f8 = f8w ? f8w->w : nullptr;
  const uint8_t* w2s = f8w ? f8w->w_scale : nullptr;
#define REID_LAUNCH(BN_, F8W_)                                                                                       \
  hipLaunchKernelGGL((sparse_step_reident_fused<BN_, F8W_>), grid, dim3(256), 0, s, g2, ga_first, dbuf, w2, w2f8,   \
                     w2s, midx, y, n, d, h, k, kp, q_prev, k_prev, v_prev, q, kx, v, aidx, m, num, den, ascore, o,   \
                     na, heads, kk, scale)
  if (bn == 256) {
    if (f8w)
      REID_LAUNCH(256, true);
    else
      REID_LAUNCH(256, false);
  } else {
    if (f8w)
      REID_LAUNCH(128, true);
    else
      REID_LAUNCH(128, false);
  }
#undef REID_LAUNCH
  hipError_t e = hipGetLastError();
  timing_after(K_SPARSE_STEP_REIDENT_FUSED, s);
  return e;
}

hipError_t launch_sparse_step(const uint16_t* x, const uint16_t* w1t, const float* b1, const int32_t* midx,
                              uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed, float* mscore,
                              const uint16_t* w2, float* y, int64_t n, int d, int h, int k, const uint16_t* q,
                              const uint16_t* kx, const uint16_t* v, const int32_t* aidx, const float* m,
                              const float* num, const float* den, float* o, int64_t na, int heads, int kk,
                              float scale, hipStream_t s, const Fp8Rows* f8, const Fp8Cols* f8w) {
  const int kp = padded_k(k);
  int g2 = 0;
  const int bn = d % 256 == 0 ? 256 : 128;
  if (k > 0) {
    hipError_t e =
        launch_mlp_gemm1(false, x, w1t, b1, midx, a_cache, dbuf, a_packed, mscore, n, d, h, k, s, f8, f8w != nullptr);
    if (e != hipSuccess) return e;
    g2 = xcd_grid(d / bn * (int)row_blocks(n));
  }
  const int ga = (int)(row_blocks(na) * heads);
  // Longest units first: the attention units lead when each streams more
  // operand bytes through LDS than a phase-2 tile (ceil(kk/32) chunks of
  // 16 KB against the tile's K-chunks of D and W2 rows).
  const int64_t attn_bytes = (int64_t)((kk + 31) / 32) * 16384;
  const int64_t g2_bytes = f8w ? (int64_t)(kp / 64) * (kRowBlock * 64 + 64 * bn)
                               : (int64_t)(kp / 32) * (kRowBlock * 64 + 32 * bn * 2);
  const int ga_first = (g2 > 0 && ga > 0 && attn_bytes > g2_bytes) ? xcd_grid(ga) : 0;
  const dim3 grid((unsigned)(ga_first > 0 ? ga_first + g2 : g2 + ga));
  timing_before(K_SPARSE_STEP_FUSED, s);
  const uint8_t* w2f8 = f8w ? f8w->w : nullptr;
  const uint8_t* w2s = f8w ? f8w->w_scale : nullptr;
#define FUSED_LAUNCH(BN_, F8W_)                                                                                      \
  hipLaunchKernelGGL((sparse_step_fused<BN_, F8W_>), grid, dim3(256), 0, s, g2, ga_first, dbuf, w2, w2f8, w2s, midx, \
                     y, n, d, h, k, kp, q, kx, v, aidx, m, num, den, o, na, heads, kk, scale)
  if (bn == 256) {
    if (f8w)
      FUSED_LAUNCH(256, true);
    else
      FUSED_LAUNCH(256, false);
  } else {
    if (f8w)
      FUSED_LAUNCH(128, true);
    else
      FUSED_LAUNCH(128, false);
  }
#undef FUSED_LAUNCH
  hipError_t e = hipGetLastError();
  timing_after(K_SPARSE_STEP_FUSED, s);
  return e;
}

}  // namespace chipmunk
