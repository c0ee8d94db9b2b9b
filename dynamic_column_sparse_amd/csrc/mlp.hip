// MLP kernels of the column-sparse delta (gfx950).
//
// Phase 1 (mlp_gemm1): one workgroup per (128-row block b, tile of BN gathered
// hidden units).  The tile's hidden units are rows of W1^T ([h][d], one
// contiguous 2*d-byte row each), so gathering them is a set of coalesced row
// reads; the x rows of block b are contiguous too.  Both operands stream through
// double-buffered LDS tiles in K-chunks of 64 and feed the bf16 matrix cores
// (32x32x16, fp32 accumulate).  Epilogue per element: + b1, GELU (tanh form),
// round to bf16, then
//   sparse: D = a_new - a_cache (exact in fp32, rounded to bf16 as the next
//           product's operand) -> D tiles; a_new -> cache (fused writeback) or
//           a packed buffer;
//   dense:  score[b][j] = sum over real rows |a_new - a_cache|; a_new -> cache.
// Phase 2 (mlp_gemm2): one workgroup per (block b, BN output columns); the
// reduction runs over the block's k gathered hidden units: D tile rows
// ([nb][k][128]) times the gathered W2 rows ([h][d], contiguous per unit).  Both
// tiles sit in LDS as they come from memory ([unit][column]) and are read with
// the transposing LDS read, so no shuffle is needed to put the reduction index
// in registers.  y rows are read, added to and written once (no atomics: every
// output element has exactly one writer, so results are deterministic).
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

constexpr int BM = 128;      // rows per block (one row block)
constexpr int BK = 64;       // reduction chunk
constexpr int LDA = BK + 8;  // padded K-contiguous row: 144 B (16-byte reads conflict-free)

template <int BN, bool DENSE>
__global__ __launch_bounds__(256, 1) void mlp_gemm1(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ w1t,
                                                    const float* __restrict__ b1,
                                                    const int32_t* __restrict__ idx,
                                                    uint16_t* __restrict__ a_cache,
                                                    uint16_t* __restrict__ dbuf,
                                                    uint16_t* __restrict__ a_packed,
                                                    float* __restrict__ score, int64_t n, int d, int h, int k) {
  constexpr int WN = BN / 2;                 // columns per wave (2x2 wave grid)
  constexpr int NI = WN / 32;                // 32-wide column subtiles per wave
  constexpr int MI = 2;                      // 32-row subtiles per wave (64 rows)
  constexpr int A_CH = BM * BK / 8 / 256;    // 16-byte chunks per thread, x tile
  constexpr int B_CH = BN * BK / 8 / 256;    // 16-byte chunks per thread, W1^T tile

  __shared__ __align__(16) uint16_t sA[2][BM][LDA];
  __shared__ __align__(16) uint16_t sB[2][BN][LDA];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int b = blockIdx.y;
  const int c0 = blockIdx.x * BN;
  const int64_t r0 = (int64_t)b * BM;
  const int rows = (int)(n - r0 < BM ? n - r0 : BM);
  const int kcols = DENSE ? h : k;

  const uint16_t* a_src[A_CH];
  bool a_ok[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + 256 * i, row = c >> 3, col8 = c & 7;
    a_ok[i] = row < rows;
    a_src[i] = x + (r0 + (a_ok[i] ? row : 0)) * (int64_t)d + col8 * 8;
  }
  const uint16_t* b_src[B_CH];
  bool b_ok[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + 256 * i, row = c >> 3, col8 = c & 7;
    const int p = c0 + row;
    b_ok[i] = p < kcols;
    int j = 0;
    if (b_ok[i]) j = DENSE ? p : clamp_index(idx[(int64_t)b * k + p], h);
    b_src[i] = w1t + (int64_t)j * d + col8 * 8;
  }

  uint4 ra[A_CH], rb[B_CH];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#define G1_LOAD(kt_)                                                                          \
  _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                          \
    if (a_ok[i]) ra[i] = *(const uint4*)(a_src[i] + (kt_) * BK); else ra[i] = z4;             \
  }                                                                                           \
  _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                          \
    if (b_ok[i]) rb[i] = *(const uint4*)(b_src[i] + (kt_) * BK); else rb[i] = z4;             \
  }
#define G1_STORE(buf_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                          \
    const int c = tid + 256 * i;                                                              \
    *(uint4*)&sA[buf_][c >> 3][(c & 7) * 8] = ra[i];                                          \
  }                                                                                           \
  _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                          \
    const int c = tid + 256 * i;                                                              \
    *(uint4*)&sB[buf_][c >> 3][(c & 7) * 8] = rb[i];                                          \
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int KT = d / BK;
  G1_LOAD(0);
  G1_STORE(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) {
      G1_LOAD(kt + 1);
    }
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8_t af[MI], bfr[NI];
      const int ko = s * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = *(const bf16x8_t*)&sA[buf][wm * 64 + mi * 32 + (lane & 31)][ko];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = *(const bf16x8_t*)&sB[buf][wn * WN + ni * 32 + (lane & 31)][ko];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < KT) {
      G1_STORE(buf ^ 1);
    }
    __syncthreads();
  }
#undef G1_LOAD
#undef G1_STORE

  // ---- epilogue ----
  float colsum[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    colsum[ni] = 0.f;
    const int jl = wn * WN + ni * 32 + (lane & 31);
    const int p = c0 + jl;
    const bool valid = p < kcols;
    int j = 0;
    if (valid) j = DENSE ? p : clamp_index(idx[(int64_t)b * k + p], h);
    const float bias = (valid && b1) ? b1[j] : 0.f;
    uint16_t* cache_col = a_cache + ((int64_t)b * h + j) * BM;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m0 = wm * 64 + mi * 32 + g * 8 + (lane >> 5) * 4;
        float av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf2f(f2bf(gelu_tanh(acc[mi][ni][g * 4 + e] + bias)));
          av[e] = (m0 + e < rows) ? a : 0.f;
        }
        if (!valid) continue;
        const uint2 old = *(const uint2*)(cache_col + m0);
        const float o0 = bf2f(old.x & 0xffffu), o1 = bf2f(old.x >> 16);
        const float o2 = bf2f(old.y & 0xffffu), o3 = bf2f(old.y >> 16);
        const uint2 nw = make_uint2(pack2(av[0], av[1]), pack2(av[2], av[3]));
        if (DENSE) {
          colsum[ni] += (m0 + 0 < rows ? fabsf(av[0] - o0) : 0.f) + (m0 + 1 < rows ? fabsf(av[1] - o1) : 0.f) +
                        (m0 + 2 < rows ? fabsf(av[2] - o2) : 0.f) + (m0 + 3 < rows ? fabsf(av[3] - o3) : 0.f);
          *(uint2*)(cache_col + m0) = nw;
        } else {
          const uint2 dd = make_uint2(pack2(av[0] - o0, av[1] - o1), pack2(av[2] - o2, av[3] - o3));
          *(uint2*)(dbuf + ((int64_t)b * k + p) * BM + m0) = dd;
          if (a_packed)
            *(uint2*)(a_packed + ((int64_t)b * k + p) * BM + m0) = nw;
          else
            *(uint2*)(cache_col + m0) = nw;
        }
      }
    }
  }
  if (DENSE) {
    // Column L1 over the block's rows: lanes l and l^32 hold the two 4-row halves
    // of each 8-row group; the wm=1 waves hold rows 64..127.
    float* sred = (float*)&sA[0][0][0];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      colsum[ni] += __shfl_xor(colsum[ni], 32);
      if (wm == 1 && lane < 32) sred[wn * WN + ni * 32 + lane] = colsum[ni];
    }
    __syncthreads();
    if (wm == 0 && lane < 32) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int p = c0 + wn * WN + ni * 32 + lane;
        if (p < kcols) score[(int64_t)b * h + p] = colsum[ni] + sred[wn * WN + ni * 32 + lane];
      }
    }
  }
}

template <int BN, bool DENSE>
__global__ __launch_bounds__(256, 1) void mlp_gemm2(const uint16_t* __restrict__ src,
                                                    const uint16_t* __restrict__ w2,
                                                    const int32_t* __restrict__ idx,
                                                    const float* __restrict__ b2, float* __restrict__ y,
                                                    int64_t n, int d, int h, int k, int kc) {
  constexpr int WN = BN / 2, NI = WN / 32, MI = 2;
  constexpr int LDD = BM + 16;   // 288-byte rows for the transposing reads
  constexpr int LDW = BN + 16;
  constexpr int D_CH = BK * BM / 8 / 256;   // 4
  constexpr int W_CH = BK * BN / 8 / 256;   // BN/32
  constexpr int WROW = BN / 8;              // 16-byte chunks per W2 tile row

  __shared__ __align__(16) uint16_t sD[2][BK][LDD];
  __shared__ __align__(16) uint16_t sW[2][BK][LDW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int b = blockIdx.y;
  const int n0 = blockIdx.x * BN;
  const int64_t r0 = (int64_t)b * BM;
  const int rows = (int)(n - r0 < BM ? n - r0 : BM);
  const int kk = DENSE ? h : k;
  const uint16_t* sblk = src + (int64_t)b * kc * BM;
  const int32_t* sidx = DENSE ? nullptr : idx + (int64_t)b * k;

  uint4 rd[D_CH], rw[W_CH];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#define G2_LOAD(kt_)                                                                          \
  {                                                                                           \
    const int j0 = (kt_) * BK;                                                                \
    _Pragma("unroll") for (int i = 0; i < D_CH; ++i) {                                        \
      const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;                          \
      const int jr = j0 + row;                                                                \
      if (jr < kk) rd[i] = *(const uint4*)(sblk + (int64_t)jr * BM + col); else rd[i] = z4;   \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < W_CH; ++i) {                                        \
      const int c = tid + 256 * i, row = c / WROW, col = (c % WROW) * 8;                      \
      const int jr = j0 + row;                                                                \
      if (jr < kk) {                                                                          \
        const int g = DENSE ? jr : clamp_index(sidx[jr], h);                                  \
        rw[i] = *(const uint4*)(w2 + (int64_t)g * d + n0 + col);                              \
      } else {                                                                                \
        rw[i] = z4;                                                                           \
      }                                                                                       \
    }                                                                                         \
  }
#define G2_STORE(buf_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < D_CH; ++i) {                                          \
    const int c = tid + 256 * i;                                                              \
    *(uint4*)&sD[buf_][c >> 4][(c & 15) * 8] = rd[i];                                         \
  }                                                                                           \
  _Pragma("unroll") for (int i = 0; i < W_CH; ++i) {                                          \
    const int c = tid + 256 * i;                                                              \
    *(uint4*)&sW[buf_][c / WROW][(c % WROW) * 8] = rw[i];                                     \
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int KT = (kk + BK - 1) / BK;
  if (KT > 0) {
    G2_LOAD(0);
    G2_STORE(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) {
      G2_LOAD(kt + 1);
    }
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8_t af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = tr_operand(&sD[buf][0][0], LDD, s * 16, wm * 64 + mi * 32, lane);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = tr_operand(&sW[buf][0][0], LDW, s * 16, wn * WN + ni * 32, lane);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < KT) {
      G2_STORE(buf ^ 1);
    }
    __syncthreads();
  }
#undef G2_LOAD
#undef G2_STORE

#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int col = n0 + wn * WN + ni * 32 + (lane & 31);
    const float bias = (DENSE && b2) ? b2[col] : 0.f;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < rows) {
          float* yp = y + (r0 + m) * (int64_t)d + col;
          if (DENSE)
            *yp = acc[mi][ni][r] + bias;
          else
            *yp += acc[mi][ni][r];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_mlp_gemm1(bool dense, const uint16_t* x, const uint16_t* w1t, const float* b1,
                            const int32_t* idx, uint16_t* a_cache, uint16_t* dbuf, uint16_t* a_packed,
                            float* score, int64_t n, int d, int h, int k, hipStream_t s) {
  const int64_t nb = row_blocks(n);
  const int cols = dense ? h : k;
  // 256-wide tiles when they waste little of the last tile, else 128-wide.
  const int t256 = (cols + 255) / 256, t128 = (cols + 127) / 128;
  const bool wide = t128 > 1 && (int64_t)t256 * 256 * 100 <= (int64_t)cols * 106;
  const int kid = dense ? K_MLP_GEMM1_DENSE : K_MLP_GEMM1_SPARSE;
  timing_before(kid, s);
  if (wide) {
    dim3 grid(t256, (unsigned)nb);
    if (dense)
      hipLaunchKernelGGL((mlp_gemm1<256, true>), grid, dim3(256), 0, s, x, w1t, b1, idx, a_cache, dbuf, a_packed,
                         score, n, d, h, k);
    else
      hipLaunchKernelGGL((mlp_gemm1<256, false>), grid, dim3(256), 0, s, x, w1t, b1, idx, a_cache, dbuf,
                         a_packed, score, n, d, h, k);
  } else {
    dim3 grid(t128, (unsigned)nb);
    if (dense)
      hipLaunchKernelGGL((mlp_gemm1<128, true>), grid, dim3(256), 0, s, x, w1t, b1, idx, a_cache, dbuf, a_packed,
                         score, n, d, h, k);
    else
      hipLaunchKernelGGL((mlp_gemm1<128, false>), grid, dim3(256), 0, s, x, w1t, b1, idx, a_cache, dbuf,
                         a_packed, score, n, d, h, k);
  }
  hipError_t e = hipGetLastError();
  timing_after(kid, s);
  return e;
}

hipError_t launch_mlp_gemm2(bool dense, const uint16_t* src, const uint16_t* w2, const int32_t* idx,
                            const float* b2, float* y, int64_t n, int d, int h, int k, int kc, hipStream_t s) {
  const int64_t nb = row_blocks(n);
  const int kid = dense ? K_MLP_GEMM2_DENSE : K_MLP_GEMM2_SPARSE;
  timing_before(kid, s);
  if (d % 256 == 0) {
    dim3 grid(d / 256, (unsigned)nb);
    if (dense)
      hipLaunchKernelGGL((mlp_gemm2<256, true>), grid, dim3(256), 0, s, src, w2, idx, b2, y, n, d, h, k, kc);
    else
      hipLaunchKernelGGL((mlp_gemm2<256, false>), grid, dim3(256), 0, s, src, w2, idx, b2, y, n, d, h, k, kc);
  } else {
    dim3 grid(d / 128, (unsigned)nb);
    if (dense)
      hipLaunchKernelGGL((mlp_gemm2<128, true>), grid, dim3(256), 0, s, src, w2, idx, b2, y, n, d, h, k, kc);
    else
      hipLaunchKernelGGL((mlp_gemm2<128, false>), grid, dim3(256), 0, s, src, w2, idx, b2, y, n, d, h, k, kc);
  }
  hipError_t e = hipGetLastError();
  timing_after(kid, s);
  return e;
}

}  // namespace chipmunk
