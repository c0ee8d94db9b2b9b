#pragma once
// Attention kernels of the column-sparse delta (gfx950), head_dim 128.
//
// Every kernel runs one workgroup (4 waves) per (head, 128-query block); wave w
// owns queries 32w .. 32w+31 of the block and keeps their Q rows in registers
// for the whole key loop.  Keys stream in 32-row chunks through a ring of LDS
// stages filled by direct global->LDS loads.  Scores are computed transposed,
// s^T = K_chunk Q^T, so each lane holds one query and 16 keys: the
// exponentials then feed P V directly as the left operand, with V read through
// the transposing LDS read in the same reduction order as the accumulator rows.
// Exponentials are exp(scale s - m) = 2^(s * scale*log2e - m*log2e): one FMA
// and one exp2 per element.
//
//   attn_stats  (refresh pass 1): row max m and row sum l over all keys
//               (l is the refresh's den = sum_j p_ij).
//   attn_dense  (refresh pass 2): p = exp(s - m), num = p V, o = num / l, and
//               the key-mass score sum_i p_ij / l_i per key, reduced over the
//               block's queries on the matrix cores.
//   attn_sparse (sparse step / REFRESH): the same loop over the gathered keys
//               S only, with the cached m; SPARSE writes
//               o = (num + num_S) / (den + den_S); REFRESH subtracts the S part
//               from num and den.
// The dense passes spread heads over the 8 XCDs so that all query blocks of
// one head share one XCD's L2, where that head's K and V rows are re-read;
// the sparse passes run head-major, so all XCDs gather from the same head's
// rows, which the last-level cache then holds.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

// Workgroup -> (head, query block) for the dense passes: all blocks of a head
// land on one XCD (workgroups are dispatched to the 8 XCDs round-robin by
// linear id) when heads % 8 == 0, so the head's K and V rows, which every
// query block streams in full and in the same order, are re-read from that
// XCD's L2.
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

// Workgroup -> (head, query block) for the sparse passes: head-major in
// launch order, so the resident workgroups of all 8 XCDs work on the same head
// (or two) at a time.  Each query block gathers its own scattered subset of
// the head's keys; what the XCDs share then is the last-level cache, which
// holds one head's K and V (2 x 256 bytes x n: 61 MB at n = 118 800) but not
// eight.  Measured at the HunyuanVideo shape: 12.4 ms against 13.6 ms per
// sparse step with the dense passes' XCD-per-head order.
__device__ __forceinline__ void head_block_sparse(int nb, int& hh, int& b, int L) {
  hh = L / nb;
  b = L % nb;
}

struct QFrag {
  bf16x8_t f[8];
};

// Tile key index of accumulator element r in lane `lane`, relative to the subtile.
__device__ __forceinline__ int acc_key(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// Geometry shared by the dense passes: 32-key chunks, K rows store 16-byte
// chunk c at c ^ (row % 16) (plain 16-byte operand reads, no bank conflicts),
// V rows store 32-byte column pairs at pair ^ swzp(row) for the transposing
// reads.  Direct-load instruction i of a wave covers rows (wave*2+i)*4 .. +3
// of a chunk; lane -> row lane/16, physical 16-byte chunk lane%16.
constexpr int kSK = 32;                       // keys per chunk
constexpr int kTile = kSK * 256;              // 8 KB per tensor per chunk
constexpr int kIns = kTile / 1024 / 4;        // direct loads per wave per tensor per chunk (2)

struct ChunkGeom {
  int krow[kIns], koff[kIns], voff[kIns];
  __device__ __forceinline__ explicit ChunkGeom(int wave, int lane) {
    const int pc = lane & 15;
#pragma unroll
    for (int i = 0; i < kIns; ++i) {
      const int r = (wave * kIns + i) * 4 + (lane >> 4);
      krow[i] = r;
      koff[i] = (pc ^ (r & 15)) * 8;
      voff[i] = ((((pc >> 1) ^ swzp(r)) << 1) | (pc & 1)) * 8;
    }
  }
};

// s^T = K_chunk Q^T for the chunk stored at `st`: lane holds query lane%32 and
// the 16 keys acc_key(r, lane).
__device__ __forceinline__ f32x16_t chunk_scores(const unsigned char* st, const QFrag& qf, int lane) {
  const int ksw = lane & 15;   // K row (lane % 32) % 16
  f32x16_t sc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) {
    const bf16x8_t kf = *(const bf16x8_t*)(st + (lane & 31) * 256 + (((2 * s2 + (lane >> 5)) ^ ksw) << 4));
    sc = mfma32(kf, qf.f[s2], sc);
  }
  return sc;
}

// Q fragments of query row `row` (a valid row: callers clamp), optionally with
// every sign bit flipped (= the fragments of -Q).
__device__ __forceinline__ void load_q_row(QFrag& qf, const uint16_t* qh, int64_t row, uint32_t flip, int lane) {
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) {
    uint4 u = *(const uint4*)(qh + row * 128 + s2 * 16 + (lane >> 5) * 8);
    u.x ^= flip;
    u.y ^= flip;
    u.z ^= flip;
    u.w ^= flip;
    qf.f[s2] = __builtin_bit_cast(bf16x8_t, u);
  }
}

// Refresh pass 1 for one (head, query block): m_i = max_j scale*s_ij and
// l_i = sum_j exp(scale*s_ij - m_i) over all n keys.  Keys stream through a
// 4-stage ring of 32-key chunks (32 KB; four workgroups per CU, so a
// 24-head, 34-block layer runs in one round).  Full chunks load from a scalar
// base and fixed lane offsets; the chunks past the last full one clamp their
// rows to row n-1 (every load stays unconditional, so the per-wave load counts
// behind the waits are exact) and mask them.  For a negative scale the kernel
// runs on -Q with |scale|, so the running maximum is always a maximum of raw
// scores: m = max_j(s'_ij) * |scale| exactly.
constexpr int kStatsStages = 4;

__global__ __launch_bounds__(256, 4) void attn_stats(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     float* __restrict__ m_out, float* __restrict__ l_out, int64_t n,
                                                     int heads, float scale) {
  constexpr int NS = kStatsStages, L = kIns;
  __shared__ __align__(16) unsigned char smem[NS * kTile];
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block(heads, nb, hh, b, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_lds = lds_addr(smem);
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const int64_t hoff = (int64_t)hh * n;
  const uint16_t* kh = k + hoff * 128;
  const int nn = (int)n;
  const int qi = wave * 32 + (lane & 31);
  const int qc = qi < rows ? qi : rows - 1;
  const float as = fabsf(scale), sl2 = as * 1.4426950408889634f;
  const ChunkGeom geo(wave, lane);
  const int KT = (nn + kSK - 1) / kSK, KF = nn / kSK;   // chunks, full chunks
  uint32_t kofs[kIns];
#pragma unroll
  for (int i = 0; i < kIns; ++i) kofs[i] = geo.krow[i] * 256 + geo.koff[i] * 2;

  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + (t % NS) * kTile;
#pragma unroll
    for (int i = 0; i < kIns; ++i) {
      const int key = t * kSK + geo.krow[i];
      dma16_at(kh + (int64_t)(key < nn ? key : nn - 1) * 128 + geo.koff[i], st + (wave * kIns + i) * 1024);
    }
  };
  auto issue_full = [&](int t, int slot) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + slot * kTile;
    const unsigned char* base = (const unsigned char*)kh + (int64_t)t * kTile;
#pragma unroll
    for (int i = 0; i < kIns; ++i) dma16_sa(base, kofs[i], st + (wave * kIns + i) * 1024);
  };

  // Q goes out before the stages: its first use (chunk 0's scores, before the
  // loop) then waits for it once.
  QFrag qf;
  load_q_row(qf, q + hoff * 128, r0 + qc, scale < 0.f ? 0x80008000u : 0u, lane);
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < KT) issue(t);
  {
    const int ahead = (KT - 1) < (NS - 2) ? (KT - 1) : (NS - 2);
    wait_vmcnt_upto<(NS - 2) * L>(ahead * L);
    barrier();
  }
  f32x16_t sa = chunk_scores(smem, qf, lane), sb;
  // mr: the lane's running maximum of raw scores (exact).  lr: the sum of
  // 2^(s*sl2 - ms2) over the lane's keys so far, where the base ms2 moves only
  // when the scaled running maximum passes it by more than kLazy, so every
  // exponent stays <= kLazy (terms <= 2^kLazy, far inside fp32) and rescaling
  // lr (one more exp2) is rare instead of once per chunk.
  constexpr float kLazy = 8.f;
  float mr = -INFINITY, lr = 0.f, ms2 = -INFINITY;
  // Iteration t issues chunk t+1's score products into `nxt`, then folds chunk
  // t (in `cur`) into the running (m, l).  Steady iterations issue a full
  // chunk (t + NS - 1 < KF); their own chunk is full too.  SLOT >= 0 is t % NS
  // known at compile time (the unrolled steady loop), so the stage addresses
  // become immediate offsets of the LDS reads.
  auto body = [&](int t, f32x16_t& cur, f32x16_t& nxt, auto STEADY, auto SLOT) __attribute__((always_inline)) {
    constexpr bool steady = decltype(STEADY)::value;
    constexpr int slot = decltype(SLOT)::value;
    const int s1 = slot >= 0 ? (slot + 1) % NS : (t + 1) % NS;
    const int sl = slot >= 0 ? (slot + NS - 1) % NS : (t + NS - 1) % NS;
    if (steady || t + 1 < KT) {
      // Stage t+1 must be complete; newer than it are the stages issued up to
      // min(t + NS - 2, KT - 1).
      if (steady) {
        wait_vmcnt<(NS - 3) * L>();
      } else {
        const int last = (t + NS - 2) < (KT - 1) ? (t + NS - 2) : (KT - 1);
        wait_vmcnt_upto<(NS - 3) * L>((last - t - 1) * L);
      }
      barrier();
      // Stage t+NS-1 reuses the slot of chunk t-1, read at iteration t-2.
      if (steady)
        issue_full(t + NS - 1, sl);
      else if (t + NS - 1 < KT)
        issue(t + NS - 1);
      nxt = chunk_scores(smem + s1 * kTile, qf, lane);
    }
    const bool full = steady || t * kSK + kSK <= nn;
    float mloc;
    if (steady) {
      mloc = cur[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, cur[r]);
    } else {
      mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = full || t * kSK + acc_key(r, lane) < nn;
        mloc = ok ? fmaxf(mloc, cur[r]) : mloc;
      }
    }
    // A lane whose keys so far are all masked (only when n < 32) keeps
    // mr = ms2 = -inf and lr = 0: its comparison below is false.
    mr = fmaxf(mr, mloc);
    const float mr2 = mr * sl2;
    if (__ballot(mr2 > ms2 + kLazy)) {
      const bool up = mr2 > ms2 + kLazy;
      lr *= up ? __builtin_amdgcn_exp2f(ms2 - mr2) : 1.f;   // 2^-inf = 0 on a lane's first keys
      ms2 = up ? mr2 : ms2;
    }
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = full || t * kSK + acc_key(r, lane) < nn;
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[r], sl2, -ms2));
      sum += ok ? e : 0.f;
    }
    lr += sum;
  };
  static_assert(NS == 4, "the steady loop is unrolled by the ring size");
  using Dyn = std::integral_constant<int, -1>;
  int t = 0;
  for (; t + 3 + NS < KF; t += 4) {
    body(t, sa, sb, std::true_type{}, std::integral_constant<int, 0>{});
    body(t + 1, sb, sa, std::true_type{}, std::integral_constant<int, 1>{});
    body(t + 2, sa, sb, std::true_type{}, std::integral_constant<int, 2>{});
    body(t + 3, sb, sa, std::true_type{}, std::integral_constant<int, 3>{});
  }
  for (; t + NS < KF; t += 2) {
    body(t, sa, sb, std::true_type{}, Dyn{});
    body(t + 1, sb, sa, std::true_type{}, Dyn{});
  }
  while (t < KT) {
    body(t, sa, sb, std::false_type{}, Dyn{});
    if (++t >= KT) break;
    body(t, sb, sa, std::false_type{}, Dyn{});
    ++t;
  }

  // Lanes l and l^32 hold the same query (different keys).  Each lane's sum
  // is taken from its base ms2 to the row maximum M.
  const float m2 = __shfl_xor(mr, 32), l2 = __shfl_xor(lr, 32), s2 = __shfl_xor(ms2, 32);
  const float M = fmaxf(mr, m2), M2 = M * sl2;
  const float la = mr > -INFINITY ? lr * __builtin_amdgcn_exp2f(ms2 - M2) : 0.f;
  const float lb = m2 > -INFINITY ? l2 * __builtin_amdgcn_exp2f(s2 - M2) : 0.f;
  if (lane < 32 && qi < rows) {
    m_out[hoff + r0 + qi] = M * as;
    l_out[hoff + r0 + qi] = la + lb;
  }
}

// The p tile of one wave for the score products: [32 queries][32 keys] fp16,
// rows of 64 bytes, with 8-byte unit u of row r stored at unit
// u ^ g(r / 4), g(x) = x ^ ((x & 2) << 1).  The 32 rows written at one
// unit cover all 64 banks once, and the two 16-lane groups of each half of a
// transposing read (query rows 8 apart) land on opposite halves of the row.
__device__ __forceinline__ int p_unit(int u, int r) {
  const int x = (r >> 2) & 7;
  return u ^ x ^ ((x & 2) << 1);
}

// Reads the p tile as the right operand of a 16x16x32 product with the QUERIES
// as the reduction index: lane l gets key 16*half + l%16 and queries
// 8*(l/16) .. +7 in order.
__device__ __forceinline__ f16x8_t p_operand(const unsigned char* tile, int half, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int u = half * 4 + (i & 3);   // 8-byte unit of keys 4u .. 4u+3
  const int kr = G * 8 + (i >> 2);    // query row; the second read is 4 rows on
  i16x4_t lo = lds_read_tr16((const uint16_t*)(tile + kr * 64 + (p_unit(u, kr) << 3)));
  i16x4_t hi = lds_read_tr16((const uint16_t*)(tile + (kr + 4) * 64 + (p_unit(u, kr + 4) << 3)));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8_t, v);
}

// Refresh pass 2 for one (head, query block), given pass 1's m and l: with
// p_ij = exp(scale*s_ij - m_i), num = p V (fp32 accumulate of bf16 p and V),
// o = num / l, and the key-mass score score[h][b][j] = sum over the block's
// queries of p_ij / l_i.  den keeps pass 1's l, which is sum_j p_ij.  K and V
// move through a 4-stage ring of 32-key chunks (64 KB, two workgroups per CU);
// the score products of chunk t+1 are issued before the exponentials and value
// products of chunk t.  The score is a matrix product too: each wave writes
// its p tile to LDS in fp16, reads it back transposed (queries as the
// reduction index) and multiplies it by the row of its queries' 2^15/l in fp16
// (1 <= l <= n keeps those normal up to n = 2^29; the 2^-15 is applied after
// the fp32 sum, exactly), one 16x16x32 product per 16 keys, each over all 32
// of the wave's queries (a 32x32x16 product would compute 32 equal rows).  fp16 rather than bf16 operands: the sums then carry
// about 2^-12 relative error per term, small enough for the index sets even
// when a block has few valid queries.  The four waves' partial sums meet in LDS and are stored for four chunks (128 keys) at a time
// by wave 3.  Those stores are not counted in the waits (which then wait for a
// little more than needed, never less).
constexpr int kDenseStages = 4;
constexpr int kScoreGroup = 4;   // chunks per score store

__global__ __launch_bounds__(256, 2) void attn_dense(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, const float* __restrict__ m,
                                                     float* __restrict__ den, float* __restrict__ num,
                                                     float* __restrict__ o, float* __restrict__ score, int64_t n,
                                                     int heads, float scale) {
  constexpr int NS = kDenseStages, G = kScoreGroup;
  constexpr int STAGE = 2 * kTile;
  constexpr int L = 2 * kIns;
  constexpr int PIECES = kRowBlock * 128 / 4 / 256;   // 16-byte output pieces per thread (16)
  __shared__ __align__(16) unsigned char smem[NS * STAGE];
  __shared__ __align__(16) unsigned char sP[4][32 * 64];
  __shared__ float sSc[2][G][4][kSK];
  __shared__ float sInv[kRowBlock];
  __shared__ float sL[kRowBlock];
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block(heads, nb, hh, b, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_lds = lds_addr(smem);
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const int64_t hoff = (int64_t)hh * n;
  const uint16_t* kh = k + hoff * 128;
  const uint16_t* vh = v + hoff * 128;
  float* srow = score + ((int64_t)hh * nb + b) * n;
  const int nn = (int)n;
  const int qi = wave * 32 + (lane & 31);
  const bool qok = qi < rows;
  const int qc = qok ? qi : rows - 1;
  const ChunkGeom geo(wave, lane);
  const int KT = (nn + kSK - 1) / kSK, KF = nn / kSK;
  uint32_t kofs[kIns], vofs[kIns];
#pragma unroll
  for (int i = 0; i < kIns; ++i) {
    kofs[i] = geo.krow[i] * 256 + geo.koff[i] * 2;
    vofs[i] = geo.krow[i] * 256 + geo.voff[i] * 2;
  }

  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + (t % NS) * STAGE;
    int key[kIns];
#pragma unroll
    for (int i = 0; i < kIns; ++i) {
      const int j = t * kSK + geo.krow[i];
      key[i] = j < nn ? j : nn - 1;
    }
#pragma unroll
    for (int i = 0; i < kIns; ++i)
      dma16_at(kh + (int64_t)key[i] * 128 + geo.koff[i], st + (wave * kIns + i) * 1024);
#pragma unroll
    for (int i = 0; i < kIns; ++i)
      dma16_at(vh + (int64_t)key[i] * 128 + geo.voff[i], st + kTile + (wave * kIns + i) * 1024);
  };
  auto issue_full = [&](int t, int slot) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + slot * STAGE;
    const unsigned char* kb = (const unsigned char*)kh + (int64_t)t * kTile;
    const unsigned char* vb = (const unsigned char*)vh + (int64_t)t * kTile;
#pragma unroll
    for (int i = 0; i < kIns; ++i) dma16_sa(kb, kofs[i], st + (wave * kIns + i) * 1024);
#pragma unroll
    for (int i = 0; i < kIns; ++i) dma16_sa(vb, vofs[i], st + kTile + (wave * kIns + i) * 1024);
  };
  // Wave 3 stores the block's scores of chunks g*G .. g*G+G-1 (two keys per lane).
  auto store_scores = [&](int g) __attribute__((always_inline)) {
    if (wave == 3) {
      const int c = lane >> 4, kc = (lane & 15) * 2;
      const int j = (g * G + c) * kSK + kc;
      const float (*ps)[kSK] = sSc[g & 1][c];
      const float s0 = ps[0][kc] + ps[1][kc] + ps[2][kc] + ps[3][kc];
      const float s1 = ps[0][kc + 1] + ps[1][kc + 1] + ps[2][kc + 1] + ps[3][kc + 1];
      if (j < nn) srow[j] = s0;
      if (j + 1 < nn) srow[j + 1] = s1;
    }
  };

  QFrag qf;
  load_q_row(qf, q + hoff * 128, r0 + qc, 0u, lane);
  const float mrow = m[hoff + r0 + qc];
  const float lrow = den[hoff + r0 + qc];   // pass 1's l
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < KT) issue(t);
  // Rows past the block end weigh nothing in the scores.
  if (lane < 32) {
    sInv[qi] = qok ? 1.f / lrow : 0.f;
    sL[qi] = lrow;
  }
  {
    const int ahead = (KT - 1) < (NS - 2) ? (KT - 1) : (NS - 2);
    wait_vmcnt_upto<(NS - 2) * L>(ahead * L);
    barrier();
  }
  // Left operand of the score products: every row holds 2^15/l of the wave's
  // 32 queries, in the order p_operand delivers them.
  f16x8_t wq;
  {
    const float* w = sInv + wave * 32 + (lane >> 4) * 8;
    constexpr float S = 32768.f;
    const uint4 pk = make_uint4(pack2h(w[0] * S, w[1] * S), pack2h(w[2] * S, w[3] * S),
                                pack2h(w[4] * S, w[5] * S), pack2h(w[6] * S, w[7] * S));
    wq = __builtin_bit_cast(f16x8_t, pk);
  }
  const float sl2 = scale * 1.4426950408889634f, ml2 = mrow * 1.4426950408889634f;
  f32x16_t acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ni][r] = 0.f;
  unsigned char* pw = sP[wave];
  const int pq = lane & 31, ph = lane >> 5;
  f32x16_t sa = chunk_scores(smem, qf, lane), sb;

  // SLOT >= 0 is t % NS known at compile time (the unrolled steady loop), so
  // the stage addresses become immediate offsets of the LDS reads.
  auto body = [&](int t, f32x16_t& cur, f32x16_t& nxt, auto STEADY, auto SLOT) __attribute__((always_inline)) {
    constexpr bool steady = decltype(STEADY)::value;
    constexpr int slot = decltype(SLOT)::value;
    const int s0 = slot >= 0 ? slot : t % NS;
    const int s1 = slot >= 0 ? (slot + 1) % NS : (t + 1) % NS;
    const int sl = slot >= 0 ? (slot + NS - 1) % NS : (t + NS - 1) % NS;
    if (steady || t + 1 < KT) {
      if (steady) {
        wait_vmcnt<(NS - 3) * L>();
      } else {
        const int last = (t + NS - 2) < (KT - 1) ? (t + NS - 2) : (KT - 1);
        wait_vmcnt_upto<(NS - 3) * L>((last - t - 1) * L);
      }
      barrier();
      // Every wave's partial scores of chunks t-G .. t-1 are in LDS.
      if (t % G == 0 && t >= G) store_scores(t / G - 1);
      // Stage t+NS-1 reuses the slot of chunk t-1: its keys were read at
      // iteration t-2 and its values at t-1, before this barrier.
      if (steady)
        issue_full(t + NS - 1, sl);
      else if (t + NS - 1 < KT)
        issue(t + NS - 1);
      nxt = chunk_scores(smem + s1 * STAGE, qf, lane);
    }
    const unsigned char* st = smem + s0 * STAGE;
    const bool full = steady || t * kSK + kSK <= nn;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[r], sl2, -ml2));
      p[r] = (full || t * kSK + acc_key(r, lane) < nn) ? e : 0.f;
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint4 pk = make_uint4(pack2(p[hf * 8 + 0], p[hf * 8 + 1]), pack2(p[hf * 8 + 2], p[hf * 8 + 3]),
                                  pack2(p[hf * 8 + 4], p[hf * 8 + 5]), pack2(p[hf * 8 + 6], p[hf * 8 + 7]));
      // This lane's keys 8*(2hf) + 4*ph .. +3 and 8*(2hf+1) + 4*ph .. +3 of query
      // pq, in fp16 for the score products.
      *(uint2*)(pw + pq * 64 + (p_unit(4 * hf + ph, pq) << 3)) =
          make_uint2(pack2h(p[hf * 8 + 0], p[hf * 8 + 1]), pack2h(p[hf * 8 + 2], p[hf * 8 + 3]));
      *(uint2*)(pw + pq * 64 + (p_unit(4 * hf + 2 + ph, pq) << 3)) =
          make_uint2(pack2h(p[hf * 8 + 4], p[hf * 8 + 5]), pack2h(p[hf * 8 + 6], p[hf * 8 + 7]));
      const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const bf16x8_t vb = tr_operand_swz(st + kTile, 256, hf * 16, ni * 32, lane);
        acc[ni] = mfma32(pa, vb, acc[ni]);
      }
    }
    // Keys 0..15 and 16..31 of the chunk, each summed over the wave's 32
    // queries by one 16x16x32 product (every output row is the same).
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t sc0 = mfma16h(wq, p_operand(pw, 0, lane), z);
    const f32x4_t sc1 = mfma16h(wq, p_operand(pw, 1, lane), z);
    if (lane < 16) {
      sSc[(t / G) & 1][t % G][wave][lane] = sc0[0] * (1.f / 32768.f);
      sSc[(t / G) & 1][t % G][wave][16 + lane] = sc1[0] * (1.f / 32768.f);
    }
  };
  static_assert(NS == 4 && G == 4, "the steady loop is unrolled by the ring size");
  using Dyn = std::integral_constant<int, -1>;
  int t = 0;
  for (; t + 3 + NS < KF; t += 4) {
    body(t, sa, sb, std::true_type{}, std::integral_constant<int, 0>{});
    body(t + 1, sb, sa, std::true_type{}, std::integral_constant<int, 1>{});
    body(t + 2, sa, sb, std::true_type{}, std::integral_constant<int, 2>{});
    body(t + 3, sb, sa, std::true_type{}, std::integral_constant<int, 3>{});
  }
  for (; t + NS < KF; t += 2) {
    body(t, sa, sb, std::true_type{}, Dyn{});
    body(t + 1, sb, sa, std::true_type{}, Dyn{});
  }
  while (t < KT) {
    body(t, sa, sb, std::false_type{}, Dyn{});
    if (++t >= KT) break;
    body(t, sb, sa, std::false_type{}, Dyn{});
    ++t;
  }

  // Epilogue through the idle ring: the numerator goes to LDS as fp32 [128
  // rows][128 columns] (16-byte chunk c of row r at c ^ ((r / 4) % 2) * 8), then
  // every thread stores whole 16-byte pieces of num and o.
  __syncthreads();
  // Score groups not yet stored: the last one, and the one before it when the
  // loop's final iteration (which has no barrier) was due to store it.
  {
    const int glast = (KT - 1) / G;
    if ((KT - 1) % G == 0 && glast >= 1) store_scores(glast - 1);
    store_scores(glast);
  }
  float* sacc_t = (float*)smem;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = wave * 32 + acc_key(r, lane);
      const int cc = ni * 32 + (lane & 31);
      sacc_t[qr * 128 + (((cc >> 2) ^ (((qr >> 2) & 1) << 3)) << 2) + (cc & 3)] = acc[ni][r];
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
    const int e = it * 256 + tid, qr = e >> 5, c4 = e & 31;
    if (qr >= rows) continue;
    const float4 a = *(const float4*)(sacc_t + qr * 128 + ((c4 ^ (((qr >> 2) & 1) << 3)) << 2));
    const int64_t g = (hoff + r0 + qr) * 128 + c4 * 4;
    // o = num / den with den = l, divided as the sparse step divides.
    const float dl = sL[qr];
    *(float4*)(num + g) = a;
    *(float4*)(o + g) = make_float4(a.x / dl, a.y / dl, a.z / dl, a.w / dl);
  }
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
  head_block_sparse(nb, hh, b, lin);
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
  // Gathered rows load from the head's K / V base (wave-uniform, in SGPRs) plus
  // a 32-bit byte offset id * 256 + the lane's chunk (n < 2^24 keeps it exact).
#define AS_ISSUE(buf_, ids_)                                                                 \
  {                                                                                          \
    const uint32_t st_ = smem_lds + (buf_) * STAGE;                                          \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                          \
        dma16_sa(kh, (uint32_t)ids_[i] * 256u + (uint32_t)koff[i] * 2u, st_ + (wave * INS + i) * 1024); \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                          \
        dma16_sa(vh, (uint32_t)ids_[i] * 256u + (uint32_t)voff[i] * 2u, st_ + TILE + (wave * INS + i) * 1024); \
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
    // SLOT >= 0 is t % NSS known at compile time (the unrolled steady loop),
    // so the stage addresses become immediate offsets of the LDS reads.
    auto body = [&](int t, auto STEADY, auto SLOT) __attribute__((always_inline)) {
      constexpr bool steady = decltype(STEADY)::value;
      constexpr int slot = decltype(SLOT)::value;
      const int s0 = slot >= 0 ? slot : t % NSS;
      const int s1 = slot >= 0 ? (slot + 1) % NSS : (t + 1) % NSS;
      const int sl = slot >= 0 ? (slot + NSS - 1) % NSS : (t + NSS - 1) % NSS;
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
        if (steady || t + NSS - 1 < KT) AS_ISSUE(sl, ids_a);
        if (!steady && t == t_r) load_rest();
        if (steady || t + NSS < KT) load_ids(t + NSS, ids_b);
        snext = scores(s1);
      }
      const unsigned char* st = smem + s0 * STAGE;
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
    static_assert(NSS == 4, "the steady loop is unrolled by the ring size");
    using Dyn = std::integral_constant<int, -1>;
    int t = 0;
    for (; t + 3 + DID < KT; t += 4) {
      body(t, std::true_type{}, std::integral_constant<int, 0>{});
      body(t + 1, std::true_type{}, std::integral_constant<int, 1>{});
      body(t + 2, std::true_type{}, std::integral_constant<int, 2>{});
      body(t + 3, std::true_type{}, std::integral_constant<int, 3>{});
    }
    for (; t + DID < KT; ++t) body(t, std::true_type{}, Dyn{});
    for (; t < KT; ++t) body(t, std::false_type{}, Dyn{});
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

// Sparse step with per-step re-identification, for one (head, query block).
// The cache holds totals over all keys (as the dense step leaves them), and S
// may differ from the previous step's.  For the gathered keys S, the share
// computed from the previous step's q, k, v is taken out of num and den and
// this step's share is put in; then o = num / den, and each key of S gets the
// score sum over the block's queries of p_ij / den_i, with den as it stood
// when the step began.  The keys of S pass through the ring twice, as one
// sequence of 2 * ceil(kk / 32) chunks: first the previous step's rows (their
// p enter the sums with a minus sign), then this step's.  Both passes
// accumulate into the same numerator and denominator registers, and the ring,
// id ring and load accounting are those of the sparse step over the doubled
// sequence (every chunk loads its own copy of its 32 ids; the id ring has 16
// slots so that a chunk's ids outlive its score store).  One Q fragment set
// is live at a time: the current step's Q rows replace the previous step's
// right after the scores of the last old chunk are issued (a compiler-visible
// load there drains the ring once per workgroup).  The scores of new chunk c
// are a matrix product of this step's p tile (fp16, written to LDS and read
// back transposed) with 2^14 / den (fp16); the four waves' partial sums meet
// in LDS and wave 3 stores them one chunk later, after a barrier (those
// stores are not counted in the waits, which then wait a little longer than
// needed, never less).
constexpr int kReidIdSlots = 16;

__device__ __forceinline__ void load_q_frag(QFrag& qf, const uint16_t* row, int lane) {
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) qf.f[s2] = *(const bf16x8_t*)(row + s2 * 16 + (lane >> 5) * 8);
}

// LDS of one attn_reident workgroup (a struct, so that a shared-grid kernel can
// overlay it with another body's LDS).
struct AttnReidentLds {
  unsigned char ring[4 * 2 * kTile];      // 4 stages of 32 K rows + 32 V rows
  int ids[kReidIdSlots][kSK];
  unsigned char p[4][32 * 64];            // each wave's fp16 p tile
  float sc[2][4][kSK];                    // partial scores of two chunks
  float inv[kRowBlock], den[kRowBlock], den_old[kRowBlock];
};

// Body of the re-identifying step for workgroup `lin` of its grid.
__device__ __forceinline__ void attn_reident_body(
    int lin, AttnReidentLds& lds, const uint16_t* __restrict__ q_prev, const uint16_t* __restrict__ k_prev,
    const uint16_t* __restrict__ v_prev, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, const float* __restrict__ m,
    float* __restrict__ num, float* __restrict__ den, float* __restrict__ score, float* __restrict__ o, int64_t n,
    int heads, int kk, float scale) {
  constexpr int SK = kSK;
  constexpr int NSS = 4;
  constexpr int STAGE = 2 * kTile;
  constexpr int INS = kIns;
  constexpr int L = 2 * INS;
  constexpr int DID = 2 * NSS - 1;
  constexpr int RID = kReidIdSlots;
  constexpr int PIECES = kRowBlock * 128 / 4 / 256;
  constexpr float kW = 16384.f;   // score weights 2^14 / den: normal fp16 for den in [2^-2, 2^28]
  static_assert((RID & (RID - 1)) == 0 && RID >= DID + 2, "id ring: a new chunk's slot lives until its score store");
  static_assert(sizeof(lds.ring) == NSS * STAGE, "LDS layout");
  unsigned char* smem = lds.ring;
  int (*sIdx)[SK] = lds.ids;
  unsigned char (*sP)[32 * 64] = lds.p;
  float (*sSc)[4][SK] = lds.sc;
  float* sInv = lds.inv;
  float* sDen = lds.den;
  float* sDenOld = lds.den_old;
  const int nb = (int)row_blocks(n);
  int hh, b;
  head_block_sparse(nb, hh, b, lin);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_lds = lds_addr(smem);
  const int64_t r0 = (int64_t)b * kRowBlock;
  const int rows = (int)(n - r0 < kRowBlock ? n - r0 : kRowBlock);
  const int64_t hoff = (int64_t)hh * n;
  const uint16_t* khp = k_prev + hoff * 128;
  const uint16_t* vhp = v_prev + hoff * 128;
  const uint16_t* khn = k + hoff * 128;
  const uint16_t* vhn = v + hoff * 128;
  const int32_t* S = idx + ((int64_t)hh * nb + b) * kk;
  float* srow = score + ((int64_t)hh * nb + b) * n;
  const int nn = (int)n;
  const int qi = wave * 32 + (lane & 31);
  const bool qok = qi < rows;
  const int qc = qok ? qi : rows - 1;   // clamped row: loads stay unconditional
  const ChunkGeom geo(wave, lane);
  const int KR = (kk + SK - 1) / SK;     // chunks of S
  const int KT = 2 * KR;                 // chunks of the sequence: KR old, then KR new

  auto load_ids = [&](int t, int (&ids)[INS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < INS; ++i) ids[i] = clamp_index(sIdx[t & (RID - 1)][geo.krow[i]], nn);
  };
  // Sequence chunk t's 32 key ids (chunk t mod KR of S) -> ring slot t % RID;
  // positions past kk read id 0, whose p are masked to 0.
  auto id_dma = [&](int t) __attribute__((always_inline)) {
    if (wave == 0 && lane < SK) {
      const int j = (t < KR ? t : t - KR) * SK + lane;
      dma4_at(S + (j < kk ? j : 0), lds_addr(&sIdx[t & (RID - 1)][0]));
    }
  };
  // Rows of sequence chunk t from the wave-uniform K / V bases of its step plus
  // 32-bit byte offsets id * 256 + the lane's chunk (n < 2^24 keeps them exact).
#define AR_ISSUE(t_, ids_, new_)                                                                       \
  {                                                                                                    \
    const uint32_t st_ = smem_lds + ((t_) % NSS) * STAGE;                                              \
    const uint16_t* kb_ = (new_) ? khn : khp;                                                          \
    const uint16_t* vb_ = (new_) ? vhn : vhp;                                                          \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                                    \
        dma16_sa(kb_, (uint32_t)ids_[i] * 256u + (uint32_t)geo.koff[i] * 2u, st_ + (wave * INS + i) * 1024); \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                                    \
        dma16_sa(vb_, (uint32_t)ids_[i] * 256u + (uint32_t)geo.voff[i] * 2u,                           \
                 st_ + kTile + (wave * INS + i) * 1024);                                               \
  }
  // Wave 3 stores the scores of new chunk c (lanes 0..31: one key each); its
  // ids are in the slot of sequence chunk KR + c.
  auto store_scores = [&](int c) __attribute__((always_inline)) {
    if (wave == 3 && lane < SK) {
      const int j = c * SK + lane;
      if (j < kk) {
        const float (*ps)[SK] = sSc[c & 1];
        srow[clamp_index(sIdx[(KR + c) & (RID - 1)][lane], nn)] = ps[0][lane] + ps[1][lane] + ps[2][lane] + ps[3][lane];
      }
    }
  };

  QFrag qf;
  const float mrow = m[hoff + r0 + qc];
  const float drow = den[hoff + r0 + qc];
  f32x16_t acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ni][r] = 0.f;
  float dpart = 0.f;

  if (KT > 0) {
    if (wave == 0 && lane < SK) {
#pragma unroll
      for (int t = 0; t < DID; ++t)
        if (t < KT) {
          const int j = (t < KR ? t : t - KR) * SK + lane;
          dma4_at(S + (j < kk ? j : 0), lds_addr(&sIdx[t][0]));
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    // The previous step's Q rows go out before the first stages (their first
    // use, before the loop, then waits for them once).
    load_q_frag(qf, q_prev + (hoff + r0 + qc) * 128, lane);
    int ids_a[INS], ids_b[INS];
#pragma unroll
    for (int t = 0; t < NSS - 1; ++t) {
      if (t < KT) {
        load_ids(t, ids_a);
        AR_ISSUE(t, ids_a, t >= KR);
      }
    }
    if (NSS - 1 < KT) load_ids(NSS - 1, ids_a);
    {
      const int ahead = (KT - 1) < (NSS - 2) ? (KT - 1) : (NSS - 2);
      wait_vmcnt_upto<(NSS - 2) * L>(ahead * L);
      barrier();
    }
    // Score weights of this wave's queries (rows past the block end weigh 0),
    // in the order p_operand delivers the queries; written and read back by
    // the same wave.
    if (lane < 32) sInv[qi] = qok ? 1.f / drow : 0.f;
    f16x8_t wq;
    {
      const float* w = sInv + wave * 32 + (lane >> 4) * 8;
      const uint4 pk = make_uint4(pack2h(w[0] * kW, w[1] * kW), pack2h(w[2] * kW, w[3] * kW),
                                  pack2h(w[4] * kW, w[5] * kW), pack2h(w[6] * kW, w[7] * kW));
      wq = __builtin_bit_cast(f16x8_t, pk);
    }
    const float sl2 = scale * 1.4426950408889634f, ml2 = mrow * 1.4426950408889634f;
    f32x16_t sacc = chunk_scores(smem, qf, lane);
    // With a single old chunk, this step's Q rows are due for chunk 1 already.
    if (KR == 1) load_q_frag(qf, q + (hoff + r0 + qc) * 128, lane);
    unsigned char* pw = sP[wave];
    const int pq = lane & 31, ph = lane >> 5;

    // Iteration t: scores of chunk t+1, then the exponentials and value
    // products of chunk t.  NEW: chunk t is one of this step's.  STEADY: every
    // stage, id and score issue happens, chunk t is full, and chunks t+1 and
    // t+NSS-1 belong to the same step as chunk t.
    auto body = [&](int t, auto NEW, auto STEADY) __attribute__((always_inline)) {
      constexpr bool steady = decltype(STEADY)::value;
      constexpr bool cur_new = decltype(NEW)::value;
      const int c = cur_new ? t - KR : t;   // chunk of S
      f32x16_t snext;
      if (steady || t + 1 < KT) {
        if (steady) {
          if (wave == 0 && t >= 1)
            wait_vmcnt<L + 1>();
          else
            wait_vmcnt<L>();
        } else {
          // Stage t+1 must be complete.  Newer than it: the stages after it
          // already issued, and on wave 0 the id loads of iterations
          // t-NSS+3 .. t-1.
          const int issued_to = (t + NSS - 2) < (KT - 1) ? (t + NSS - 2) : (KT - 1);
          int newer = (issued_to - (t + 1)) * L;
          if (wave == 0) {
            const int j0 = t - NSS + 3 > 0 ? t - NSS + 3 : 0;
            const int j1 = (t - 1) < (KT - DID - 1) ? (t - 1) : (KT - DID - 1);
            newer += j1 >= j0 ? j1 - j0 + 1 : 0;
          }
          wait_vmcnt_upto<(NSS - 2) * L + NSS>(newer);
        }
        barrier();
        // Every wave's partial scores of new chunk c-1 are in LDS.
        if (cur_new && c >= 1) store_scores(c - 1);
        if (steady || t + DID < KT) id_dma(t + DID);
        if (steady) {
          AR_ISSUE(t + NSS - 1, ids_a, cur_new);
        } else if (t + NSS - 1 < KT) {
          AR_ISSUE(t + NSS - 1, ids_a, t + NSS - 1 >= KR);
        }
        if (steady || t + NSS < KT) load_ids(t + NSS, ids_b);
        snext = chunk_scores(smem + ((t + 1) % NSS) * STAGE, qf, lane);
        // After the scores of the last old chunk: this step's Q rows.
        if (!cur_new && !steady && t + 2 == KR) load_q_frag(qf, q + (hoff + r0 + qc) * 128, lane);
      }
      const unsigned char* st = smem + (t % NSS) * STAGE;
      float p[16];
      if (steady || c * SK + SK <= kk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -ml2));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = c * SK + acc_key(r, lane);
          p[r] = j < kk ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sl2, -ml2)) : 0.f;
        }
      }
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) psum += p[r];
      dpart += cur_new ? psum : -psum;
      constexpr float sg = cur_new ? 1.f : -1.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint4 pk = make_uint4(pack2(sg * p[hf * 8 + 0], sg * p[hf * 8 + 1]),
                                    pack2(sg * p[hf * 8 + 2], sg * p[hf * 8 + 3]),
                                    pack2(sg * p[hf * 8 + 4], sg * p[hf * 8 + 5]),
                                    pack2(sg * p[hf * 8 + 6], sg * p[hf * 8 + 7]));
        if (cur_new) {
          // This lane's keys 8*(2hf) + 4*ph .. +3 and 8*(2hf+1) + 4*ph .. +3 of
          // query pq, in fp16 for the score products.
          *(uint2*)(pw + pq * 64 + (p_unit(4 * hf + ph, pq) << 3)) =
              make_uint2(pack2h(p[hf * 8 + 0], p[hf * 8 + 1]), pack2h(p[hf * 8 + 2], p[hf * 8 + 3]));
          *(uint2*)(pw + pq * 64 + (p_unit(4 * hf + 2 + ph, pq) << 3)) =
              make_uint2(pack2h(p[hf * 8 + 4], p[hf * 8 + 5]), pack2h(p[hf * 8 + 6], p[hf * 8 + 7]));
        }
        const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const bf16x8_t vb = tr_operand_swz(st + kTile, 256, hf * 16, ni * 32, lane);
          acc[ni] = mfma32(pa, vb, acc[ni]);
        }
      }
      if (cur_new) {
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t sc0 = mfma16h(wq, p_operand(pw, 0, lane), z);
        const f32x4_t sc1 = mfma16h(wq, p_operand(pw, 1, lane), z);
        if (lane < 16) {
          sSc[c & 1][wave][lane] = sc0[0] * (1.f / kW);
          sSc[c & 1][wave][16 + lane] = sc1[0] * (1.f / kW);
        }
      }
      if (steady || t + 1 < KT) {
        sacc = snext;
#pragma unroll
        for (int i = 0; i < INS; ++i) ids_a[i] = ids_b[i];
      }
    };
    int t = 0;
    // Old chunks: steady while chunks t .. t+NSS-1 are all old (then chunk t is
    // not the last old one, so it is full, and t + DID < KT).
    for (; t + NSS - 1 < KR; ++t) body(t, std::false_type{}, std::true_type{});
    for (; t < KR; ++t) body(t, std::false_type{}, std::false_type{});
    for (; t + DID < KT; ++t) body(t, std::true_type{}, std::true_type{});
    for (; t < KT; ++t) body(t, std::true_type{}, std::false_type{});
  }
#undef AR_ISSUE
  dpart += __shfl_xor(dpart, 32);
  // Epilogue through the idle ring, as in the sparse step: the numerator change
  // goes to LDS as fp32 [128 rows][128 columns], then every thread updates
  // whole 16-byte pieces of num and stores o.
  __syncthreads();
  // Score stores not yet done: the last new chunk's, and the one before it,
  // due at the final iteration (which has no barrier).
  if (KR >= 2) store_scores(KR - 2);
  if (KR >= 1) store_scores(KR - 1);
  float* sacc_t = (float*)smem;
  if (lane < 32) {
    sDen[qi] = dpart;
    sDenOld[qi] = drow;
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = wave * 32 + acc_key(r, lane);
      const int cc = ni * 32 + (lane & 31);
      sacc_t[qr * 128 + (((cc >> 2) ^ (((qr >> 2) & 1) << 3)) << 2) + (cc & 3)] = acc[ni][r];
    }
  float4 rest[PIECES];
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
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
    const float4 nw = make_float4(rest[it].x + a.x, rest[it].y + a.y, rest[it].z + a.z, rest[it].w + a.w);
    const float dt = sDenOld[qr] + sDen[qr];
    *(float4*)(num + g) = nw;
    *(float4*)(o + g) = make_float4(nw.x / dt, nw.y / dt, nw.z / dt, nw.w / dt);
  }
  if (tid < rows) den[hoff + r0 + tid] = sDenOld[tid] + sDen[tid];
}

__global__ __launch_bounds__(256, 2) void attn_reident(
    const uint16_t* __restrict__ q_prev, const uint16_t* __restrict__ k_prev, const uint16_t* __restrict__ v_prev,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ m, float* __restrict__ num, float* __restrict__ den,
    float* __restrict__ score, float* __restrict__ o, int64_t n, int heads, int kk, float scale) {
  __shared__ __align__(16) AttnReidentLds lds;
  attn_reident_body(blockIdx.x, lds, q_prev, k_prev, v_prev, q, k, v, idx, m, num, den, score, o, n, heads, kk,
                    scale);
}

}  // namespace
}  // namespace chipmunk
