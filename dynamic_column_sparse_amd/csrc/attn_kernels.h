#pragma once
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

#include <type_traits>

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
__device__ __forceinline__ void head_block(int heads, int nb, int& hh, int& b, int L) {
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
  head_block(heads, nb, hh, b, blockIdx.x);
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
  head_block(heads, nb, hh, b, blockIdx.x);
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

// Sparse step / REFRESH over the gathered keys S of one (head, query block).
// Gathered K and V rows (256 bytes each) move by direct global->LDS loads in
// 32-key chunks through a 4-stage ring (64 KB, two workgroups per CU); their
// key ids arrive in an 8-chunk LDS ring far enough ahead that no row load
// waits on its id.  K rows store 16-byte chunk c at c ^ (row % 16) (plain
// 16-byte operand reads, no bank conflicts); V rows store 32-byte column pairs
// at pair ^ swzp(row) for the transposing reads.  The score products of chunk
// t+1 are issued before the exponentials and value products of chunk t, so the
// matrix cores always have independent work.  The rest numerator (in the
// coalesced 16-byte layout of the epilogue) is loaded behind the last stage.
// Every load issued between direct-load stages is unconditional, once per
// wave, so the per-wave load counts that the waits rely on are exact.
// LDS of one attn_sparse workgroup.
struct AttnSparseLds {
  static constexpr int kRing = 4 * 2 * 32 * 256;   // 4 stages of 32 K rows + 32 V rows
  static constexpr int kIds = 8 * 32;
};

// Body of the sparse step / REFRESH for workgroup `lin` of its grid; `smem`
// (ring, 16-byte aligned), `sIdx` (8 x 32 ids), `sDen` and `sDenRest` (128
// floats each) are LDS provided by the caller.
template <bool REFRESH>
__device__ __forceinline__ void attn_sparse_body(int lin, unsigned char* smem, int (*sIdx)[32], float* sDen,
                                                 float* sDenRest, const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                 const int32_t* __restrict__ idx, const float* __restrict__ m,
                                                 float* __restrict__ num, float* __restrict__ den,
                                                 float* __restrict__ o, int64_t n, int heads, int kk, float scale) {
  constexpr int SK = 32;                 // keys per chunk
  constexpr int NSS = 4;                 // ring stages
  constexpr int TILE = SK * 256;         // 8 KB per tensor per stage
  constexpr int STAGE = 2 * TILE;
  constexpr int INS = TILE / 1024 / 4;   // direct loads per wave per tensor per stage (2)
  constexpr int L = 2 * INS;
  constexpr int DID = 2 * NSS - 1;       // id lookahead: chunk t+NSS's ids are older than stage t
  constexpr int RID = 8;                 // id ring slots
  constexpr int PIECES = kRowBlock * 128 / 4 / 256;   // 16-byte rest/output pieces per thread (16)
  constexpr int PRE = PIECES / 2;        // of which loaded early (register budget)
  static_assert(RID >= DID - NSS + 1 && (RID & (RID - 1)) == 0, "id ring");
  static_assert(NSS * STAGE == AttnSparseLds::kRing && RID * SK == AttnSparseLds::kIds, "LDS layout");
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block(heads, nb, hh, b, lin);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_lds = lds_addr(smem);
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const int64_t hoff = (int64_t)hh * n;
  const uint16_t* qh = q + hoff * 128;
  const uint16_t* kh = k + hoff * 128;
  const uint16_t* vh = v + hoff * 128;
  const int32_t* S = idx + ((int64_t)hh * nb + b) * kk;
  const int nn = (int)(n < 0x7fffffff ? n : 0x7fffffff);
  const int qi = wave * 32 + (lane & 31);
  const bool qok = qi < rows;
  const int qc = qok ? qi : rows - 1;    // clamped row: loads stay unconditional

  // Direct-load geometry: instruction i of a wave covers rows (wave*INS+i)*4 ..
  // +3 of the tile; lane -> row lane/16, physical 16-byte chunk lane%16.
  const int pc = lane & 15;
  int krow[INS], koff[INS], voff[INS];
#pragma unroll
  for (int i = 0; i < INS; ++i) {
    const int r = (wave * INS + i) * 4 + (lane >> 4);
    krow[i] = r;
    koff[i] = (pc ^ (r & 15)) * 8;
    voff[i] = ((((pc >> 1) ^ swzp(r)) << 1) | (pc & 1)) * 8;
  }
  auto load_ids = [&](int t, int (&ids)[INS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < INS; ++i) ids[i] = clamp_index(sIdx[t & (RID - 1)][krow[i]], nn);
  };
  // Chunk t's 32 key ids -> ring slot t % RID (lanes 0..31 of wave 0; positions
  // past kk read id 0, whose scores are masked to p = 0).
  auto id_dma = [&](int t) __attribute__((always_inline)) {
    if (wave == 0 && lane < SK) {
      const int j = t * SK + lane;
      dma4_at(S + (j < kk ? j : 0), lds_addr(&sIdx[t & (RID - 1)][0]));
    }
  };
#define AS_ISSUE(buf_, ids_)                                                                 \
  {                                                                                          \
    const uint32_t st_ = smem_lds + (buf_) * STAGE;                                          \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                          \
        dma16_at(kh + (int64_t)ids_[i] * 128 + koff[i], st_ + (wave * INS + i) * 1024);      \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                          \
        dma16_at(vh + (int64_t)ids_[i] * 128 + voff[i], st_ + TILE + (wave * INS + i) * 1024); \
  }
  float4 rest[PIECES];
  auto load_rest = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < PRE; ++it) {
      const int e = it * 256 + tid, qr = e >> 5, c4 = e & 31;
      const int qrc = qr < rows ? qr : rows - 1;
      rest[it] = *(const float4*)(num + (hoff + r0 + qrc) * 128 + c4 * 4);
    }
  };
  QFrag qf;
  float mrow = 0.f, dr_pre = 1.f;
  auto load_qmd = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf.f[s2] = *(const bf16x8_t*)(qh + (r0 + qc) * 128 + s2 * 16 + (lane >> 5) * 8);
    mrow = m[hoff + r0 + qc];
    const int dq = (tid & (kRowBlock - 1)) < rows ? (tid & (kRowBlock - 1)) : rows - 1;
    dr_pre = den[hoff + r0 + dq];
  };

  f32x16_t acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ni][r] = 0.f;
  float dpart = 0.f;
  const int KT = (kk + SK - 1) / SK;

  if (KT > 0) {
    if (wave == 0 && lane < SK) {
#pragma unroll
      for (int t = 0; t < DID; ++t)
        if (t < KT) dma4_at(S + (t * SK + lane < kk ? t * SK + lane : 0), lds_addr(&sIdx[t][0]));
    }
    wait_vmcnt<0>();
    __syncthreads();
    // Q, the row max and the rest denominator go out before the first stages.
    // Their first use (the scores of chunk 0) then waits for them once, before
    // the key loop; issued after the stages, they would make the compiler's own
    // waits inside the loop (which do not count the direct loads) drain the
    // whole prefetch ring on every iteration.
    load_qmd();
    int ids_a[INS], ids_b[INS];
#pragma unroll
    for (int t = 0; t < NSS - 1; ++t) {
      if (t < KT) {
        load_ids(t, ids_a);
        AS_ISSUE(t, ids_a);
      }
    }
    if (NSS - 1 < KT) load_ids(NSS - 1, ids_a);
    // The rest numerator follows the last stage: in the prologue when every
    // stage is issued there, else at iteration t_r = KT - NSS.
    const int t_r = KT - NSS;
    if (t_r < 0) load_rest();

    const int ksw = lane & 15;   // K row (lane % 32) % 16
    // s^T = K_chunk Q^T for the chunk in stage slot `slot`: lane holds query
    // lane%32 and 16 keys (accumulator rows).
    auto scores = [&](int slot) __attribute__((always_inline)) {
      const unsigned char* st = smem + slot * STAGE;
      f32x16_t sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const bf16x8_t kf = *(const bf16x8_t*)(st + (lane & 31) * 256 + (((2 * s2 + (lane >> 5)) ^ ksw) << 4));
        sc = mfma32(kf, qf.f[s2], sc);
      }
      return sc;
    };
    // Stage 0 (issued in the prologue) must be complete; newer than it: the
    // other prologue stages and the rest numerator if it went out in the
    // prologue.
    {
      const int ahead = (KT - 1) < (NSS - 2) ? (KT - 1) : (NSS - 2);
      wait_vmcnt_upto<(NSS - 2) * L + PRE>(ahead * L + (t_r < 0 ? PRE : 0));
      barrier();
    }
    const float sl2 = scale * 1.4426950408889634f, ml2 = mrow * 1.4426950408889634f;
    f32x16_t sacc = scores(0);
    // Software pipeline: iteration t issues the score products of chunk t+1,
    // then the exponentials and the value products of chunk t, so the matrix
    // cores have independent work while the exponentials run.  Iterations with
    // t + DID < KT are the steady state: every stage, id and score issue
    // happens, the chunk is full, the rest numerator is not yet issued, and the
    // loads newer than stage t+1 are one stage (L) plus, on wave 0 after the
    // first iteration, one id load.  They run without run-time conditions.
    auto body = [&](int t, auto STEADY) __attribute__((always_inline)) {
      constexpr bool steady = decltype(STEADY)::value;
      f32x16_t snext;
      if (steady || t + 1 < KT) {
        if (steady) {
          if (wave == 0 && t >= 1)
            wait_vmcnt<L + 1>();
          else
            wait_vmcnt<L>();
        } else {
          // Stage t+1 must be complete.  Newer than it: the stages after it
          // already issued (L each), the rest numerator if already issued, and
          // on wave 0 the id loads of iterations t-NSS+3 .. t-1 (stage t+1
          // went out at iteration t-NSS+2).  Chunk t+NSS's ids (issued at
          // iteration t+NSS-DID) are older, so they are complete too.
          const int issued_to = (t + NSS - 2) < (KT - 1) ? (t + NSS - 2) : (KT - 1);
          const int ahead = issued_to - (t + 1);
          int newer = ahead * L + (t > t_r ? PRE : 0);
          if (wave == 0) {
            const int j0 = t - NSS + 3 > 0 ? t - NSS + 3 : 0;
            const int j1 = (t - 1) < (KT - DID - 1) ? (t - 1) : (KT - DID - 1);
            newer += j1 >= j0 ? j1 - j0 + 1 : 0;
          }
          wait_vmcnt_upto<(NSS - 2) * L + PRE + NSS>(newer);
        }
        barrier();
        // Slot of stage t+NSS-1 is stage t-1's: its keys were read at
        // iteration t-2 and its values at t-1, before this barrier.
        if (steady || t + DID < KT) id_dma(t + DID);
        if (steady || t + NSS - 1 < KT) AS_ISSUE((t + NSS - 1) % NSS, ids_a);
        if (!steady && t == t_r) load_rest();
        if (steady || t + NSS < KT) load_ids(t + NSS, ids_b);
        snext = scores((t + 1) % NSS);
      }
      const unsigned char* st = smem + (t % NSS) * STAGE;
      // p = exp(s*scale - m) = 2^(s*scale*log2e - m*log2e): one FMA and one
      // exp2 per element.  Only the last chunk can hold positions past kk.
      // Query rows past the block end hold finite values (their loads are
      // clamped) and are never stored, so they need no mask.
      float p[16];
      if (steady || t * SK + SK <= kk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -ml2));
          dpart += p[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = t * SK + acc_key(r, lane);
          p[r] = j < kk ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -ml2)) : 0.f;
          dpart += p[r];
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint4 pk = make_uint4(pack2(p[hf * 8 + 0], p[hf * 8 + 1]), pack2(p[hf * 8 + 2], p[hf * 8 + 3]),
                                    pack2(p[hf * 8 + 4], p[hf * 8 + 5]), pack2(p[hf * 8 + 6], p[hf * 8 + 7]));
        const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const bf16x8_t vb = tr_operand_swz(st + TILE, 256, hf * 16, ni * 32, lane);
          acc[ni] = mfma32(pa, vb, acc[ni]);
        }
      }
      if (steady || t + 1 < KT) {
        sacc = snext;
#pragma unroll
        for (int i = 0; i < INS; ++i) ids_a[i] = ids_b[i];
      }
    };
    int t = 0;
    for (; t + DID < KT; ++t) body(t, std::true_type{});
    for (; t < KT; ++t) body(t, std::false_type{});
  } else {
    load_qmd();
    load_rest();
  }
#undef AS_ISSUE
  dpart += __shfl_xor(dpart, 32);
  // Epilogue through the idle ring: the numerator part goes to LDS as fp32
  // [128 rows][128 columns] (16-byte chunk c of row r at c ^ ((r / 4) % 2) * 8,
  // so the two row groups of one store hit different banks), then every
  // thread combines and stores whole 16-byte pieces.
  __syncthreads();
  float* sacc_t = (float*)smem;
  if (lane < 32) sDen[qi] = dpart;
  if (tid < kRowBlock) sDenRest[tid] = dr_pre;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = wave * 32 + acc_key(r, lane);
      const int cc = ni * 32 + (lane & 31);
      sacc_t[qr * 128 + (((cc >> 2) ^ (((qr >> 2) & 1) << 3)) << 2) + (cc & 3)] = acc[ni][r];
    }
#pragma unroll
  for (int it = PRE; it < PIECES; ++it) {
    const int e = it * 256 + tid, qr = e >> 5, c4 = e & 31;
    const int qrc = qr < rows ? qr : rows - 1;
    rest[it] = *(const float4*)(num + (hoff + r0 + qrc) * 128 + c4 * 4);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
    const int e = it * 256 + tid, qr = e >> 5, c4 = e & 31;
    if (qr >= rows) continue;
    const float4 a = *(const float4*)(sacc_t + qr * 128 + ((c4 ^ (((qr >> 2) & 1) << 3)) << 2));
    const int64_t g = (hoff + r0 + qr) * 128 + c4 * 4;
    if (REFRESH) {
      *(float4*)(num + g) = make_float4(rest[it].x - a.x, rest[it].y - a.y, rest[it].z - a.z, rest[it].w - a.w);
    } else {
      const float dt = sDenRest[qr] + sDen[qr];
      *(float4*)(o + g) = make_float4((rest[it].x + a.x) / dt, (rest[it].y + a.y) / dt, (rest[it].z + a.z) / dt,
                                      (rest[it].w + a.w) / dt);
    }
  }
  if (REFRESH && tid < rows) den[hoff + r0 + tid] = sDenRest[tid] - sDen[tid];
}

template <bool REFRESH>
__global__ __launch_bounds__(256, 2) void attn_sparse(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
                                                      const float* __restrict__ m, float* __restrict__ num,
                                                      float* __restrict__ den, float* __restrict__ o, int64_t n,
                                                      int heads, int kk, float scale) {
  __shared__ __align__(16) unsigned char smem[AttnSparseLds::kRing];
  __shared__ __align__(16) int sIdx[8][32];
  __shared__ float sDen[kRowBlock];
  __shared__ float sDenRest[kRowBlock];
  attn_sparse_body<REFRESH>(blockIdx.x, smem, sIdx, sDen, sDenRest, q, k, v, idx, m, num, den, o, n, heads, kk, scale);
}

#undef KV_STORE

}  // namespace
}  // namespace chipmunk
