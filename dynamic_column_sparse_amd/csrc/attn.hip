// Attention kernels of the column-sparse delta (gfx950), head_dim 128.
//
// Every kernel runs one workgroup (4 waves) per (head, 128-query block); wave w
// owns queries 32w .. 32w+31 of the block and keeps their Q rows in registers
// for the whole key loop.  Keys stream through double-buffered LDS tiles of 64
// (K rows for the scores, V rows for the numerator).  Scores are computed
// transposed, s^T = K_tile Q^T, so each lane holds one query and 16 keys: the
// exponentials then feed P V directly as the left operand, with V read through
// the transposing LDS read in the same reduction order as the accumulator rows.
//
//   attn_stats  (refresh pass 1): online row max m and sum l over all keys.
//   attn_dense  (refresh pass 2): p = exp(s - m), num = p V, den = sum p,
//               o = num / den, and the key-mass score sum_i p_ij / l_i per key,
//               reduced over the block's queries inside the workgroup.
//   attn_sparse (sparse step / REFRESH): the same loop over the gathered keys
//               S only, with the cached m; SPARSE writes
//               o = (num + num_S) / (den + den_S); REFRESH subtracts the S part
//               from num and den.
// Heads are spread over the 8 XCDs so that all query blocks of one head share
// one XCD's L2, where that head's K and V rows are re-read.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

constexpr int KT = 64;          // keys per tile
constexpr int LDK = 128 + 8;    // 272-byte rows: 16-byte reads conflict-free
constexpr int LDV = 128 + 16;   // 288-byte rows for the transposing reads
constexpr int CH = KT * 128 / 8 / 256;  // 16-byte chunks per thread per tile (4)

// Block -> (head, query block): all blocks of a head land on one XCD (workgroups
// are dispatched to the 8 XCDs round-robin by linear id) when heads % 8 == 0.
__device__ __forceinline__ void head_block(int heads, int nb, int& hh, int& b) {
  const int L = blockIdx.x;
  if ((heads & 7) == 0) {
    const int xcd = L & 7, slot = L >> 3;
    hh = xcd + 8 * (slot / nb);
    b = slot % nb;
  } else {
    hh = L / nb;
    b = L % nb;
  }
}

struct QFrag {
  bf16x8_t f[8];
};

__device__ __forceinline__ void load_q(QFrag& q, const uint16_t* qh, int64_t qrow, bool ok, int lane) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (ok)
      q.f[s] = *(const bf16x8_t*)(qh + qrow * 128 + s * 16 + (lane >> 5) * 8);
    else
      q.f[s] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }
}

// s^T for 32 keys (tile rows kb .. kb+31) against the wave's 32 queries.
__device__ __forceinline__ f32x16_t scores_t(const uint16_t* sk, int kb, const QFrag& q, int lane) {
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8_t kf = *(const bf16x8_t*)(sk + (kb + (lane & 31)) * LDK + s * 16 + (lane >> 5) * 8);
    acc = mfma32(kf, q.f[s], acc);
  }
  return acc;
}

// Tile key index of accumulator element r in lane `lane`, relative to the subtile.
__device__ __forceinline__ int acc_key(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

__global__ __launch_bounds__(256, 1) void attn_stats(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     float* __restrict__ m_out, float* __restrict__ l_out, int64_t n,
                                                     int heads, float scale) {
  __shared__ __align__(16) uint16_t sK[2][KT][LDK];
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block(heads, nb, hh, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const uint16_t* qh = q + (int64_t)hh * n * 128;
  const uint16_t* kh = k + (int64_t)hh * n * 128;
  const int qi = wave * 32 + (lane & 31);
  QFrag qf;
  load_q(qf, qh, r0 + qi, qi < rows, lane);

  uint4 rk[CH];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#define ST_LOAD(t_)                                                                           \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                                            \
    const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;                            \
    const int64_t key = (int64_t)(t_) * KT + row;                                             \
    if (key < n) rk[i] = *(const uint4*)(kh + key * 128 + col); else rk[i] = z4;              \
  }
#define ST_STORE(buf_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                                            \
    const int c = tid + 256 * i;                                                              \
    *(uint4*)&sK[buf_][c >> 4][(c & 15) * 8] = rk[i];                                         \
  }

  float mr = -INFINITY, lr = 0.f;
  const int ntiles = (int)((n + KT - 1) / KT);
  ST_LOAD(0);
  ST_STORE(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      ST_LOAD(t + 1);
    }
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      const f32x16_t sacc = scores_t(&sK[buf][0][0], kt2 * 32, qf, lane);
      float sc[16], tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t key = (int64_t)t * KT + kt2 * 32 + acc_key(r, lane);
        sc[r] = key < n ? sacc[r] * scale : -INFINITY;
        tmax = fmaxf(tmax, sc[r]);
      }
      if (tmax > -INFINITY) {
        const float mnew = fmaxf(mr, tmax);
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += __expf(sc[r] - mnew);
        lr = lr * __expf(mr - mnew) + sum;
        mr = mnew;
      }
    }
    if (t + 1 < ntiles) {
      ST_STORE(buf ^ 1);
    }
    __syncthreads();
  }
#undef ST_LOAD
#undef ST_STORE
  const float m2 = __shfl_xor(mr, 32), l2 = __shfl_xor(lr, 32);
  const float M = fmaxf(mr, m2);
  const float L = (mr > -INFINITY ? lr * __expf(mr - M) : 0.f) + (m2 > -INFINITY ? l2 * __expf(m2 - M) : 0.f);
  if (lane < 32 && qi < rows) {
    m_out[(int64_t)hh * n + r0 + qi] = M;
    l_out[(int64_t)hh * n + r0 + qi] = L;
  }
}

__global__ __launch_bounds__(256, 1) void attn_dense(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, const float* __restrict__ m,
                                                     float* __restrict__ den, float* __restrict__ num,
                                                     float* __restrict__ o, float* __restrict__ score, int64_t n,
                                                     int heads, float scale) {
  __shared__ __align__(16) uint16_t sK[2][KT][LDK];
  __shared__ __align__(16) uint16_t sV[2][KT][LDV];
  __shared__ float sScore[4][KT];
  __shared__ float sDen[kRowBlock];
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block(heads, nb, hh, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const int64_t hoff = (int64_t)hh * n;
  const uint16_t* qh = q + hoff * 128;
  const uint16_t* kh = k + hoff * 128;
  const uint16_t* vh = v + hoff * 128;
  const int qi = wave * 32 + (lane & 31);
  const bool qok = qi < rows;
  QFrag qf;
  load_q(qf, qh, r0 + qi, qok, lane);
  const float mrow = qok ? m[hoff + r0 + qi] : 0.f;
  // den holds pass 1's row sums on entry; they normalise the key-mass scores.
  const float invl = qok ? 1.f / den[hoff + r0 + qi] : 0.f;

  uint4 rk[CH], rv[CH];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#define DN_LOAD(t_)                                                                           \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                                            \
    const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;                            \
    const int64_t key = (int64_t)(t_) * KT + row;                                             \
    if (key < n) {                                                                            \
      rk[i] = *(const uint4*)(kh + key * 128 + col);                                          \
      rv[i] = *(const uint4*)(vh + key * 128 + col);                                          \
    } else {                                                                                  \
      rk[i] = z4;                                                                             \
      rv[i] = z4;                                                                             \
    }                                                                                         \
  }
#define KV_STORE(buf_)                                                                        \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                                            \
    const int c = tid + 256 * i;                                                              \
    *(uint4*)&sK[buf_][c >> 4][(c & 15) * 8] = rk[i];                                         \
    *(uint4*)&sV[buf_][c >> 4][(c & 15) * 8] = rv[i];                                         \
  }

  f32x16_t acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ni][r] = 0.f;
  float dpart = 0.f;
  const int ntiles = (int)((n + KT - 1) / KT);
  DN_LOAD(0);
  KV_STORE(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      DN_LOAD(t + 1);
    }
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      const f32x16_t sacc = scores_t(&sK[buf][0][0], kt2 * 32, qf, lane);
      float p[16], w[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t key = (int64_t)t * KT + kt2 * 32 + acc_key(r, lane);
        p[r] = key < n ? __expf(sacc[r] * scale - mrow) : 0.f;
        dpart += p[r];
        w[r] = p[r] * invl;
      }
      const float tot = halfwave_transpose_sum16(w, lane);
      if ((lane & 1) == 0) sScore[wave][kt2 * 32 + acc_key((lane >> 1) & 15, lane)] = tot;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8_t pa;
        uint4 pk = make_uint4(pack2(p[hf * 8 + 0], p[hf * 8 + 1]), pack2(p[hf * 8 + 2], p[hf * 8 + 3]),
                              pack2(p[hf * 8 + 4], p[hf * 8 + 5]), pack2(p[hf * 8 + 6], p[hf * 8 + 7]));
        pa = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const bf16x8_t vb = tr_operand(&sV[buf][0][0], LDV, kt2 * 32 + hf * 16, ni * 32, lane);
          acc[ni] = mfma32(pa, vb, acc[ni]);
        }
      }
    }
    __syncthreads();
    if (tid < KT) {
      const int64_t key = (int64_t)t * KT + tid;
      if (key < n)
        score[((int64_t)hh * nb + b) * n + key] = sScore[0][tid] + sScore[1][tid] + sScore[2][tid] + sScore[3][tid];
    }
    if (t + 1 < ntiles) {
      KV_STORE(buf ^ 1);
    }
    __syncthreads();
  }
#undef DN_LOAD
  dpart += __shfl_xor(dpart, 32);
  if (lane < 32) sDen[qi] = dpart;
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int c = ni * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = wave * 32 + acc_key(r, lane);
      if (qr < rows) {
        const int64_t g = (hoff + r0 + qr) * 128 + c;
        num[g] = acc[ni][r];
        o[g] = acc[ni][r] / sDen[qr];
      }
    }
  }
  if (lane < 32 && qok) den[hoff + r0 + qi] = sDen[qi];
}

template <bool REFRESH>
__global__ __launch_bounds__(256, 1) void attn_sparse(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
                                                      const float* __restrict__ m, float* __restrict__ num,
                                                      float* __restrict__ den, float* __restrict__ o, int64_t n,
                                                      int heads, int kk, float scale) {
  __shared__ __align__(16) uint16_t sK[2][KT][LDK];
  __shared__ __align__(16) uint16_t sV[2][KT][LDV];
  __shared__ float sDen[kRowBlock];
  __shared__ int sIdx[3][KT];   // gathered key ids of the next three tiles
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block(heads, nb, hh, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const int64_t hoff = (int64_t)hh * n;
  const uint16_t* qh = q + hoff * 128;
  const uint16_t* kh = k + hoff * 128;
  const uint16_t* vh = v + hoff * 128;
  const int32_t* S = idx + ((int64_t)hh * nb + b) * kk;
  const int qi = wave * 32 + (lane & 31);
  const bool qok = qi < rows;
  QFrag qf;
  load_q(qf, qh, r0 + qi, qok, lane);
  const float mrow = qok ? m[hoff + r0 + qi] : 0.f;
  const int nn = (int)(n < 0x7fffffff ? n : 0x7fffffff);

  uint4 rk[CH], rv[CH];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#define SP_LOAD(t_)                                                                           \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                                            \
    const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;                            \
    const int j = (t_) * KT + row;                                                            \
    if (j < kk) {                                                                             \
      const int64_t key = sIdx[(t_) % 3][row];                                                \
      rk[i] = *(const uint4*)(kh + key * 128 + col);                                          \
      rv[i] = *(const uint4*)(vh + key * 128 + col);                                          \
    } else {                                                                                  \
      rk[i] = z4;                                                                             \
      rv[i] = z4;                                                                             \
    }                                                                                         \
  }

  f32x16_t acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ni][r] = 0.f;
  float dpart = 0.f;
  const int ntiles = (kk + KT - 1) / KT;
  // Index ring: slot t%3 holds the key ids of tile t, loaded two tiles ahead so
  // no K/V row load waits on its index load.
  auto key_of = [&](int t, int r) -> int {
    const int j = t * KT + r;
    return j < kk ? clamp_index(S[j], nn) : 0;
  };
  if (tid < KT) {
    sIdx[0][tid] = key_of(0, tid);
    sIdx[1][tid] = key_of(1, tid);
    sIdx[2][tid] = key_of(2, tid);
  }
  __syncthreads();
  if (ntiles > 0) {
    SP_LOAD(0);
    KV_STORE(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    int pre = 0;
    if (t + 1 < ntiles) {
      SP_LOAD(t + 1);
    }
    if (tid < KT) pre = key_of(t + 3, tid);
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      const f32x16_t sacc = scores_t(&sK[buf][0][0], kt2 * 32, qf, lane);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = t * KT + kt2 * 32 + acc_key(r, lane);
        p[r] = j < kk ? __expf(sacc[r] * scale - mrow) : 0.f;
        dpart += p[r];
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint4 pk = make_uint4(pack2(p[hf * 8 + 0], p[hf * 8 + 1]), pack2(p[hf * 8 + 2], p[hf * 8 + 3]),
                              pack2(p[hf * 8 + 4], p[hf * 8 + 5]), pack2(p[hf * 8 + 6], p[hf * 8 + 7]));
        const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const bf16x8_t vb = tr_operand(&sV[buf][0][0], LDV, kt2 * 32 + hf * 16, ni * 32, lane);
          acc[ni] = mfma32(pa, vb, acc[ni]);
        }
      }
    }
    if (t + 1 < ntiles) {
      KV_STORE(buf ^ 1);
    }
    if (tid < KT) sIdx[t % 3][tid] = pre;
    __syncthreads();
  }
#undef SP_LOAD
  dpart += __shfl_xor(dpart, 32);
  if (lane < 32) sDen[qi] = dpart;
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int c = ni * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = wave * 32 + acc_key(r, lane);
      if (qr < rows) {
        const int64_t row = hoff + r0 + qr;
        const int64_t g = row * 128 + c;
        if (REFRESH)
          num[g] = num[g] - acc[ni][r];
        else
          o[g] = (num[g] + acc[ni][r]) / (den[row] + sDen[qr]);
      }
    }
  }
  if (REFRESH && lane < 32 && qok) den[hoff + r0 + qi] = den[hoff + r0 + qi] - sDen[qi];
}

#undef KV_STORE

}  // namespace

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

}  // namespace chipmunk
