#pragma once
// MLP kernels of the column-sparse delta (gfx950).
//
// Phase 1 (mlp_gemm1): one workgroup per (128-row block b, tile of BN gathered
// hidden units).  The tile's hidden units are rows of W1^T ([h][d], one
// contiguous 2*d-byte row each), so gathering them is a set of coalesced row
// reads; the x rows of block b are contiguous too.  Both operands stream
// through a 3-stage LDS ring in K-chunks of 64, filled by direct global->LDS
// loads two chunks ahead, and feed the bf16 matrix cores (32x32x16, fp32
// accumulate).  Epilogue per element: + b1, GELU (tanh form), round to bf16, then
//   sparse: D = a_new - a_cache (exact in fp32, rounded to bf16 as the next
//           product's operand); a_new -> cache (fused writeback) or a packed
//           buffer;
//   dense:  D = a_new; score[b][j] = sum over real rows |a_new - a_cache|;
//           a_new -> cache.
// Phase 2 (mlp_gemm2): one workgroup per (block b, BN output columns); the
// reduction runs over the block's hidden units: the activation cache
// ([nb][h][128]) of the dense step times the W2 rows ([h][d], contiguous per
// unit).  (The sparse step's gathered product is gemm2_rows_body below.)  Both tiles are copied into
// LDS as they lie in memory ([unit][column]) by direct global->LDS loads and
// read back with the transposing LDS read, so no register staging is needed.
// y rows are read, added to and written once (no atomics: every output element
// has exactly one writer, so results are deterministic).
//
// Work order: units are numbered tile-major (all row blocks of one column tile
// consecutively) and each XCD runs one contiguous range of them.  Row blocks
// that run together then gather weight rows from the same range of hidden units
// (index sets are ascending), which that XCD's L2 serves after the first fetch.
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

constexpr int BM = 128;   // rows per block (one row block)
constexpr int BK = 64;    // reduction chunk
constexpr int NS = 3;     // LDS ring stages: one consumed, two in flight
#ifndef MLP_GROUP_TILES
#define MLP_GROUP_TILES 2
#endif
constexpr int kGroupTiles = MLP_GROUP_TILES;   // column tiles of one row block run back to back


// F8: x and W1^T are e4m3 codes (one byte per element) with one E8M0 scale
// byte per row (xs for the token rows, ws1 for the hidden units); each 64-byte
// row piece of a chunk is then 64 reduction steps instead of 32, and one
// scaled fp8 product (32x32x64) replaces the two bf16 ones.  Lane l's operand
// bytes are the same two 16-byte LDS pieces (K bytes 16g.. and 32+16g.., g =
// l/32) that feed the two bf16 substeps.  The row scales are fixed for a
// tile, so each lane keeps its row's and its column's scale byte in a
// register for the whole loop; the products come out scaled.
//
// FD (sparse only): D leaves as e4m3 codes for the fp8 second product instead
// of bf16: dbuf holds [nb][kp/64][128][64] codes, followed by one E8M0 scale byte per
// (row, 32 consecutive units), stored per 64-unit chunk as [nb][kp/64][128][2]
// so that the second product streams a chunk's scales with its codes.  D is
// first rounded to bf16, as the bf16 path stores it.
template <int BN, bool DENSE, bool F8, bool FD>
__global__ __launch_bounds__(256, 2) void mlp_gemm1(const void* __restrict__ xv,
                                                    const void* __restrict__ wv,
                                                    const uint8_t* __restrict__ xs,
                                                    const uint8_t* __restrict__ ws1,
                                                    const float* __restrict__ b1,
                                                    const int32_t* __restrict__ idx,
                                                    uint16_t* __restrict__ a_cache,
                                                    uint16_t* __restrict__ dbuf,
                                                    uint16_t* __restrict__ a_packed,
                                                    float* __restrict__ score, int64_t n, int d, int h, int k,
                                                    int kp) {
  constexpr int WN = BN / 2;          // columns per wave (2x2 wave grid)
  constexpr int NI = WN / 32;         // 32-wide column subtiles per wave
  constexpr int MI = 2;               // 32-row subtiles per wave (64 rows)
  constexpr int BK = 32, NS = 3;      // 32-deep (bf16) K-chunks, 3-stage ring: 72 KB, two workgroups per CU
  constexpr int ROWB = 64;            // LDS row: 64 bytes = 4 chunks of 16 bytes (32 bf16 or 64 fp8)
  constexpr int CPR = ROWB / 16, RPI = 1024 / ROWB;   // chunks per row, rows per direct load
  constexpr int A_INS = BM / RPI / 4; // direct loads per wave per stage, x tile
  constexpr int B_INS = BN / RPI / 4; // same, W1^T tile
  constexpr int L = A_INS + B_INS;    // DMA instructions per thread per stage
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + BN) * ROWB;

  __shared__ __align__(16) unsigned char smem[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in SGPRs
  const uint32_t smem_lds = lds_addr(smem);
  const int wm = wave >> 1, wn = wave & 1;
  const int kcols = DENSE ? h : k;
  const int nb = (int)row_blocks(n), ntiles = (kcols + BN - 1) / BN;
  const int u = xcd_unit(blockIdx.x, ntiles * nb);
  if (u >= ntiles * nb) return;
  int b, tile;
  grouped_tile(u, nb, ntiles, kGroupTiles, b, tile);
  const int c0 = tile * BN;
  const int64_t r0 = (int64_t)b * BM;
  const int rows = (int)(n - r0 < BM ? n - r0 : BM);

  // Source of the 16-byte chunk this lane fills in each DMA instruction: row
  // (instruction's first row + lane/8), physical chunk lane%8, logical chunk
  // (lane%8) ^ swz8(row).  Rows past the data are clamped to a valid row: their
  // products only reach output rows/columns the epilogue never stores.
  const int64_t RB = F8 ? (int64_t)d : 2 * (int64_t)d;   // bytes per x / W1^T row
  const unsigned char* x = (const unsigned char*)xv;
  const unsigned char* w1t = (const unsigned char*)wv;
  const int lrow = lane / CPR, pch = lane % CPR;
  const unsigned char* asrc[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int r = (wave * A_INS + i) * RPI + lrow;
    const int rg = r < rows ? r : rows - 1;
    asrc[i] = x + (r0 + rg) * RB + ((pch ^ swz4(r)) << 4);
  }
  const unsigned char* bsrc[B_INS];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int r = (wave * B_INS + i) * RPI + lrow;
    const int p = c0 + r;
    int j = 0;
    if (p < kcols) j = DENSE ? p : clamp_index(idx[(int64_t)b * k + p], h);
    bsrc[i] = w1t + (int64_t)j * RB + ((pch ^ swz4(r)) << 4);
  }

#define G1_ISSUE(kt_, buf_)                                                                 \
  {                                                                                         \
    const uint32_t st_ = smem_lds + (buf_) * STAGE;                                         \
    _Pragma("unroll") for (int i = 0; i < A_INS; ++i)                                       \
        dma16_at(asrc[i] + (kt_) * ROWB, st_ + (wave * A_INS + i) * 1024);                  \
    _Pragma("unroll") for (int i = 0; i < B_INS; ++i)                                       \
        dma16_at(bsrc[i] + (kt_) * ROWB, st_ + A_BYTES + (wave * B_INS + i) * 1024);        \
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // Epilogue column ids and biases, fetched before the main loop so their
  // latency hides under it.
  int jcol[NI];
  bool valid[NI];
  float bias[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int p = c0 + wn * WN + ni * 32 + (lane & 31);
    valid[ni] = p < kcols;
    jcol[ni] = valid[ni] ? (DENSE ? p : clamp_index(idx[(int64_t)b * k + p], h)) : 0;
    bias[ni] = (valid[ni] && b1) ? b1[jcol[ni]] : 0.f;
  }

  // fp8: the scale bytes of this lane's rows (one per 32-row subtile) and
  // columns (one per 32-column subtile), the same for both 32-deep halves of a
  // product (lanes l and l+32 carry the same row / column).
  int sa[MI], sb[NI];
  if (F8) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int r = wm * 64 + mi * 32 + (lane & 31);
      sa[mi] = xs[r0 + (r < rows ? r : rows - 1)];
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) sb[ni] = ws1[jcol[ni]];
  }

  // Operand reads: lane l reads row (base + l%32), logical chunk 2s + l/32.  Every
  // row base is a multiple of 32, so the swizzle depends on the lane only.
  const int sw = swz4(lane & 31);
  const int KT = (int)(RB / ROWB);
  G1_ISSUE(0, 0);
  if (KT > 1) G1_ISSUE(1, 1);
  // One K-chunk; `slot` is kt % NS (a constant in the unrolled loop below, so
  // the stage base becomes an immediate offset of the LDS reads).
  auto chunk = [&](int kt, int slot) __attribute__((always_inline)) {
    if (kt + 1 < KT)
      wait_vmcnt<L>();
    else
      wait_vmcnt<0>();
    barrier();
    if (kt + 2 < KT) G1_ISSUE(kt + 2, (slot + 2) % NS);
    const unsigned char* st = smem + slot * STAGE;
    // Operand fragments of K-substep s+1 are read while substep s multiplies.
    bf16x8_t af[2][MI], bfr[2][NI];
#define G1_FRAG(s_, q_)                                                                              \
    {                                                                                                \
      const int coff = (((2 * (s_) + (lane >> 5)) ^ sw) << 4);                                       \
      _Pragma("unroll") for (int mi = 0; mi < MI; ++mi)                                              \
        af[q_][mi] = *(const bf16x8_t*)(st + (wm * 64 + mi * 32 + (lane & 31)) * ROWB + coff);       \
      _Pragma("unroll") for (int ni = 0; ni < NI; ++ni)                                              \
        bfr[q_][ni] = *(const bf16x8_t*)(st + A_BYTES + (wn * WN + ni * 32 + (lane & 31)) * ROWB + coff); \
    }
    G1_FRAG(0, 0);
    if constexpr (F8) {
      // Both 16-byte halves form one 64-deep fp8 operand.
      G1_FRAG(1, 1);
      typedef int i32x4_t __attribute__((ext_vector_type(4)));
      typedef int i32x8_t __attribute__((ext_vector_type(8)));
      auto cat = [](bf16x8_t lo, bf16x8_t hi) __attribute__((always_inline)) {
        const i32x4_t a = __builtin_bit_cast(i32x4_t, lo), c = __builtin_bit_cast(i32x4_t, hi);
        const i32x8_t r = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
        return r;
      };
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const i32x8_t a8 = cat(af[0][mi], af[1][mi]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, cat(bfr[0][ni], bfr[1][ni]), acc[mi][ni],
                                                                        0, 0, 0, sa[mi], 0, sb[ni]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        if (s + 1 < BK / 16) G1_FRAG(s + 1, (s + 1) & 1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(af[s & 1][mi], bfr[s & 1][ni], acc[mi][ni]);
      }
    }
#undef G1_FRAG
  };
  static_assert(NS == 3, "the K loop is unrolled by the ring size");
  int kt = 0;
  if constexpr (!F8) {   // the fp8 body, unrolled, would spill
    for (; kt + 2 < KT; kt += 3) {
      chunk(kt, 0);
      chunk(kt + 1, 1);
      chunk(kt + 2, 2);
    }
  }
  for (; kt < KT; ++kt) chunk(kt, kt % NS);
#undef G1_ISSUE

  // ---- epilogue ----
  // a_new = bf16(GELU(acc + b1)) is staged in the (now idle) LDS ring as
  // [tile column][128 rows], so that the cache columns (256 contiguous bytes
  // each) are then read and written as whole 16-byte chunks by 16 consecutive
  // lanes.  Chunk c (rows 8c..8c+7) of tile column t is stored at chunk
  // c ^ (t % 16); the column's hidden-unit id follows the tile.
  constexpr int CI = BN / 16;                // tile columns per thread in the coalesced phase
  static_assert(BN * 256 + BN * 4 <= NS * STAGE, "staging tile exceeds the LDS ring");
  unsigned char* stile = smem;
  int* scol = (int*)(smem + BN * 256);
  barrier();                                 // every wave is done reading the ring
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int t = wn * WN + ni * 32 + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m0 = wm * 64 + mi * 32 + g * 8 + (lane >> 5) * 4;
        // Evaluated for every element, then selected: a branch per element
        // would cost more than the arithmetic.
        float av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gv = gelu_tanh(acc[mi][ni][g * 4 + e] + bias[ni]);
          av[e] = (valid[ni] && m0 + e < rows) ? gv : 0.f;
        }
        *(uint2*)(stile + t * 256 + (((m0 >> 3) ^ (t & 15)) << 4) + (m0 & 7) * 2) =
            make_uint2(pack2(av[0], av[1]), pack2(av[2], av[3]));
      }
    if (wm == 0 && lane < 32) scol[t] = jcol[ni];
  }
  __syncthreads();

  const int ch = tid & 15, tc = tid >> 4;
  uint4 oldv[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int t = tc + 16 * i;
    if (c0 + t < kcols)
      oldv[i] = *(const uint4*)(a_cache + ((int64_t)b * h + scol[t]) * BM + ch * 8);
    else
      oldv[i] = make_uint4(0, 0, 0, 0);
  }
  // Column L1 of D over the block's real rows: the dense step's score; on a
  // sparse step, the rescore of the recomputed units when a score array is given.
  const bool rescore = !DENSE && score != nullptr;
  float colsum[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int t = tc + 16 * i, p = c0 + t;
    const uint4 an = *(const uint4*)(stile + t * 256 + ((ch ^ tc) << 4));
    uint32_t dw[4];
    colsum[i] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a2 = word_of(an, w), o2 = word_of(oldv[i], w);
      float dv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool live = ch * 8 + w * 2 + e < rows;
        dv[e] = live ? bf2f((a2 >> (16 * e)) & 0xffffu) - bf2f((o2 >> (16 * e)) & 0xffffu) : 0.f;
        if (DENSE || rescore) colsum[i] += fabsf(dv[e]);
      }
      dw[w] = pack2(dv[0], dv[1]);
    }
    if (p < kcols) {
      if (DENSE || !a_packed)
        *(uint4*)(a_cache + ((int64_t)b * h + scol[t]) * BM + ch * 8) = an;
      else
        *(uint4*)(a_packed + ((int64_t)b * k + p) * BM + ch * 8) = an;
    }
    // D replaces a_new in the staging tile: this thread is the only reader and
    // writer of this 16-byte slot.
    if (!DENSE) *(uint4*)(stile + t * 256 + ((ch ^ tc) << 4)) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
  }
  if (DENSE || rescore) {
    // The 16 lanes of a column hold 8 rows each.
#pragma unroll
    for (int i = 0; i < CI; ++i) {
      float v = colsum[i];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      const int t = tc + 16 * i, p = c0 + t;
      if (ch == 0 && p < kcols) score[(int64_t)b * h + (DENSE ? p : scol[t])] = v;
    }
  }
  if (!DENSE) {
    // D leaves K-contiguous in chunks of one phase-2 K-step ([block][kp/32]
    // [128 rows][32] bf16; fp8 codes [block][kp/64][128 rows][64]) so phase 2
    // reads it as a plain K-contiguous operand, each chunk's tile as 8 KB in
    // one piece.  A 16-lane group transposes 8 units x 16 rows out of
    // the [unit][row] tile with two transposing reads (units u..u+3, u+4..u+7):
    // lane j points at unit row u + j/4, tokens 4(j%4)..+3 of its 16-row block,
    // and receives the 4 units of token j.  Units k..kp of the tile are zero
    // (their a_new and cached values are zero), so phase 2 can stream whole
    // 32-unit chunks.
    __syncthreads();
    const int grp = lane >> 4, j = lane & 15;
#pragma unroll 4
    for (int it = 0; it < BN / 16; ++it) {
      const int task = it * 16 + wave * 4 + grp;
      const int u8 = task % (BN / 8), mb = task / (BN / 8);
      const int p = c0 + u8 * 8;
      const int mp = mb * 16 + 4 * (j & 3);
      const int t0 = u8 * 8 + (j >> 2), t1 = t0 + 4;
      const i16x4_t lo = lds_read_tr16((const uint16_t*)(stile + t0 * 256 + (((mp >> 3) ^ (t0 & 15)) << 4) + (mp & 7) * 2));
      const i16x4_t hi = lds_read_tr16((const uint16_t*)(stile + t1 * 256 + (((mp >> 3) ^ (t1 & 15)) << 4) + (mp & 7) * 2));
      const int m = mb * 16 + j;
      const uint4 v = make_uint4((uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16), (uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                                 (uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16), (uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
      if constexpr (FD) {
        // The wave's four 16-lane groups hold units u8 = 4w'..4w'+3 (32
        // consecutive units, one scale block) of the same 16 rows: lanes j,
        // j+16, j+32, j+48 share row m, and two exchanges give the block's
        // maximum.  A block is wholly below kp or wholly past it (kp % 64 == 0).
        uint32_t mx = abs_max_bf16x8(v);
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
        const int e = fp8_exponent(mx);
        if (p < kp) {
          unsigned char* d8 = (unsigned char*)dbuf;
          *(uint2*)(d8 + (int64_t)b * BM * kp + (p >> 6) * (BM * 64) + m * 64 + (p & 63)) = bf16x8_to_fp8(v, e);
          if (grp == 0) {
            unsigned char* dsc = d8 + (int64_t)nb * BM * kp;
            dsc[(((int64_t)b * (kp / 64) + p / 64) * BM + m) * 2 + ((p >> 5) & 1)] = (unsigned char)(127 + e);
          }
        }
      } else {
        // [block][kp/32][128 rows][32 units]: a wave's four groups write one
        // row's 64 bytes each for 16 rows, 1 KB contiguous.
        if (p < kp) *(uint4*)(dbuf + (int64_t)b * BM * kp + (p >> 5) * (BM * 32) + m * 32 + (p & 31)) = v;
      }
    }
  }
}

// 32-deep chunks: a 72 KB ring, so two workgroups share a CU (with 64-deep
// chunks and one workgroup per CU the refresh took 7-9% longer).
template <int BN, bool DENSE>
__global__ __launch_bounds__(256, 2) void mlp_gemm2(const uint16_t* __restrict__ src,
                                                    const uint16_t* __restrict__ w2,
                                                    const int32_t* __restrict__ idx,
                                                    const float* __restrict__ b2, float* __restrict__ y,
                                                    int64_t n, int d, int h, int k, int kp) {
  constexpr int BK = 32;
  constexpr int WN = BN / 2, NI = WN / 32, MI = 2;
  constexpr int D_ROWB = BM * 2;             // 256-byte D tile rows
  constexpr int W_ROWB = BN * 2;             // W2 tile rows
  constexpr int D_BYTES = BK * D_ROWB;       // 8 KB
  constexpr int STAGE = D_BYTES + BK * W_ROWB;
  constexpr int D_INS = D_BYTES / 1024 / 4;  // DMA instructions per wave per stage
  constexpr int W_INS = BK * W_ROWB / 1024 / 4;
  constexpr int D_RPI = 1024 / D_ROWB;       // rows per DMA instruction
  constexpr int W_RPI = 1024 / W_ROWB;

  __shared__ __align__(16) unsigned char smem[NS * STAGE];
  // W2 row ids, ring of 8 chunks (chunk c in slot c % 8), filled by 4-byte
  // direct loads six chunks ahead (sparse step only).
  __shared__ __align__(16) int sIdx[8][BK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in SGPRs
  const uint32_t smem_lds = lds_addr(smem);
  const int wm = wave >> 1, wn = wave & 1;
  const int nb = (int)row_blocks(n), ntn = d / BN;
  const int u = xcd_unit(blockIdx.x, ntn * nb);
  if (u >= ntn * nb) return;
  const int b = u % nb;
  const int n0 = (u / nb) * BN;
  const int64_t r0 = (int64_t)b * BM;
  const int rows = (int)(n - r0 < BM ? n - r0 : BM);
  const int kk = DENSE ? h : k;             // real reduction length (rows kk .. kp of D are zero)
  const uint16_t* sblk = src + (int64_t)b * kp * BM;
  const int32_t* sidx = DENSE ? nullptr : idx + (int64_t)b * k;

  // Per-lane DMA geometry.  D: row (instruction's first row + lane/16), 32-byte
  // pair ((lane%16)/2 ^ swzp(row)), half lane%2.  W2: row (instruction's first
  // row + lane/(BN/8)), pair ((lane%(BN/8))/2 ^ swzp(row)), half lane%2.
  const int d_lr = lane / (D_ROWB / 16), d_pc = lane % (D_ROWB / 16);
  const int w_lr = lane / (W_ROWB / 16), w_pc = lane % (W_ROWB / 16);
  int d_off[D_INS], w_row[W_INS], w_off[W_INS];
#pragma unroll
  for (int i = 0; i < D_INS; ++i) {
    const int r = (wave * D_INS + i) * D_RPI + d_lr;
    d_off[i] = r * BM + ((((d_pc >> 1) ^ swzp(r)) << 1) | (d_pc & 1)) * 8;
  }
#pragma unroll
  for (int i = 0; i < W_INS; ++i) {
    const int r = (wave * W_INS + i) * W_RPI + w_lr;
    w_row[i] = r;
    w_off[i] = ((((w_pc >> 1) ^ swzp(r)) << 1) | (w_pc & 1)) * 8;
  }
  // Ids of chunk t for this lane's W2 rows (identity for the dense step).
  auto load_ids = [&](int t, int (&ids)[W_INS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < W_INS; ++i) {
      const int j = t * BK + w_row[i];
      ids[i] = DENSE ? (j < kk ? j : 0) : clamp_index(sIdx[t & 7][w_row[i]], h);
    }
  };
  // 4-byte direct load of chunk t's 64 ids into ring slot t % 8 (wave 0; lanes
  // past k read id 0 of the block, whose D rows are zero).
  auto id_dma = [&](int t) __attribute__((always_inline)) {
    if (!DENSE && wave == 0) {
      const int j = t * BK + lane;
      dma4_at(sidx + (j < kk ? j : 0), lds_addr(&sIdx[t & 7][0]));
    }
  };

#define G2_ISSUE(kt_, buf_, ids_)                                                           \
  {                                                                                         \
    const uint32_t st_ = smem_lds + (buf_) * STAGE;                                         \
    const uint16_t* dsrc_ = sblk + (int64_t)(kt_) * BK * BM;                                \
    _Pragma("unroll") for (int i = 0; i < D_INS; ++i)                                       \
        dma16_at(dsrc_ + d_off[i], st_ + (wave * D_INS + i) * 1024);                        \
    _Pragma("unroll") for (int i = 0; i < W_INS; ++i)                                       \
        dma16_at(w2 + (int64_t)ids_[i] * d + n0 + w_off[i], st_ + D_BYTES + (wave * W_INS + i) * 1024); \
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // Pipeline.  Iteration kt: (a) wait for chunk kt's loads and barrier; (b) wave 0
  // requests the ids of chunk kt+6; (c) chunk kt+2 is requested with ids read in
  // the previous iteration; (d) the ids of chunk kt+3 are read from the ring;
  // (e) chunk kt is multiplied.  Every global load in the loop is a direct-to-LDS
  // load, so no register result is waited on inside it.  Wave 0 has one more
  // load in flight per iteration (the id chunk, issued before the stage loads
  // so that waiting for a stage also covers the ids issued with it).
  const int KT = kp / BK;
  constexpr int L = D_INS + W_INS;
#pragma unroll
  for (int t = 0; t < 6; ++t) id_dma(t);
  wait_vmcnt<0>();
  __syncthreads();
  int ids_a[W_INS], ids_b[W_INS];
  load_ids(0, ids_a);
  if (KT > 0) G2_ISSUE(0, 0, ids_a);
  load_ids(1, ids_b);
  if (KT > 1) G2_ISSUE(1, 1, ids_b);
  load_ids(2, ids_a);
  // One K-chunk; `slot` is kt % NS (a constant in the unrolled loop below, so
  // the stage base becomes an immediate offset of the LDS reads).
  auto chunk = [&](int kt, int slot) __attribute__((always_inline)) {
    // Outstanding loads of this wave, newest first: stage kt+1 (L) and, on wave
    // 0 of the sparse step, the id load of chunk kt+5 if the previous
    // iteration issued one.  Everything older (stage kt) must be complete.
    if (kt + 1 < KT) {
      if (!DENSE && wave == 0 && kt >= 1 && kt + 5 < KT)
        wait_vmcnt<L + 1>();
      else
        wait_vmcnt<L>();
    } else {
      wait_vmcnt<0>();
    }
    barrier();
    if (kt + 6 < KT) id_dma(kt + 6);
    if (kt + 2 < KT) G2_ISSUE(kt + 2, (slot + 2) % NS, ids_a);
    load_ids(kt + 3, ids_b);
    const unsigned char* st = smem + slot * STAGE;
    bf16x8_t af[2][MI], bfr[2][NI];
#define G2_FRAG(s_, q_)                                                                              \
    {                                                                                                \
      _Pragma("unroll") for (int mi = 0; mi < MI; ++mi)                                              \
        af[q_][mi] = tr_operand_swz(st, D_ROWB, (s_) * 16, wm * 64 + mi * 32, lane);                 \
      _Pragma("unroll") for (int ni = 0; ni < NI; ++ni)                                              \
        bfr[q_][ni] = tr_operand_swz(st + D_BYTES, W_ROWB, (s_) * 16, wn * WN + ni * 32, lane);       \
    }
    G2_FRAG(0, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) G2_FRAG(s + 1, (s + 1) & 1);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(af[s & 1][mi], bfr[s & 1][ni], acc[mi][ni]);
    }
#undef G2_FRAG
#pragma unroll
    for (int i = 0; i < W_INS; ++i) ids_a[i] = ids_b[i];
  };
  static_assert(NS == 3, "the K loop is unrolled by the ring size");
  int kt = 0;
  for (; kt + 2 < KT; kt += 3) {
    chunk(kt, 0);
    chunk(kt + 1, 1);
    chunk(kt + 2, 2);
  }
  for (; kt < KT; ++kt) chunk(kt, kt % NS);
#undef G2_ISSUE

  // Epilogue in two phases (every old y value or bias loaded, then every sum
  // stored): row offsets depend on d, so the compiler cannot reorder a store
  // past a later load itself, and one-at-a-time read-modify-writes would each
  // wait a full memory round trip.
  float yold[NI][MI][16];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int col = n0 + wn * WN + ni * 32 + (lane & 31);
    const float bias = (DENSE && b2) ? b2[col] : 0.f;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (DENSE)
          yold[ni][mi][r] = bias;
        else
          yold[ni][mi][r] = m < rows ? y[(r0 + m) * (int64_t)d + col] : 0.f;
      }
  }
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int col = n0 + wn * WN + ni * 32 + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < rows) y[(r0 + m) * (int64_t)d + col] = yold[ni][mi][r] + acc[mi][ni][r];
      }
  }
}

// Sparse phase 2 over the D tiles ([block][kp/32][128 rows][32], written by
// the sparse phase 1: chunk t of a block is 8 KB in one piece).  Four waves side by side (1x4): each wave owns all 128 rows
// and BN/4 output columns, so per 16-deep K-substep it reads four D fragments
// with plain 16-byte LDS reads and only BN/128 W2 fragments with the (slower)
// transposing read.  32-deep K-chunks in a 3-stage ring (72 KB) leave room for
// two workgroups per CU, which overlap each other's epilogue and barriers.
// LDS of one mlp_gemm2_rows workgroup: the operand ring and the W2 id ring.
template <int BN>
struct Gemm2RowsLds {
  static constexpr int kRing = 3 * (BM * 64 + 32 * BN * 2);
  static constexpr int kIds = 8 * 32;
};

// Body of the sparse phase 2 for workgroup `lin` of its grid; `smem` (ring,
// 16-byte aligned) and `sIdx` (8 x 32 ids) are LDS provided by the caller.
template <int BN>
__device__ __forceinline__ void gemm2_rows_body(int lin, unsigned char* smem, int (*sIdx)[32],
                                                const uint16_t* __restrict__ dsrc, const uint16_t* __restrict__ w2,
                                                const int32_t* __restrict__ idx, float* __restrict__ y, int64_t n,
                                                int d, int h, int k, int kp) {
  constexpr int BK = 32, NS = 3;
  constexpr int WN = BN / 4, NI = WN / 32, MI = BM / 32;
  constexpr int D_ROWB = BK * 2;             // 64-byte D rows (4 chunks)
  constexpr int W_ROWB = BN * 2;             // W2 tile rows
  constexpr int D_BYTES = BM * D_ROWB;       // 8 KB
  constexpr int STAGE = D_BYTES + BK * W_ROWB;
  constexpr int D_RPI = 1024 / D_ROWB;       // rows per direct load
  constexpr int W_RPI = 1024 / W_ROWB;
  constexpr int D_INS = BM / D_RPI / 4;      // direct loads per wave per stage
  constexpr int W_INS = BK / W_RPI / 4;
  constexpr int L = D_INS + W_INS;

  static_assert(NS * STAGE == Gemm2RowsLds<BN>::kRing && BK == 32, "LDS layout");
  // W2 row ids: ring of 8 chunks (chunk c in slot c % 8), filled by 4-byte
  // direct loads six chunks ahead.

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_lds = lds_addr(smem);
  const int nb = (int)row_blocks(n), ntn = d / BN;
  const int u = xcd_unit(lin, ntn * nb);
  if (u >= ntn * nb) return;
  int b, tile;
  grouped_tile(u, nb, ntn, kGroupTiles, b, tile);
  const int n0 = tile * BN;
  const int64_t r0 = (int64_t)b * BM;
  const int rows = (int)(n - r0 < BM ? n - r0 : BM);
  const uint16_t* dblk = dsrc + (int64_t)b * BM * kp;
  const int32_t* sidx = idx + (int64_t)b * k;

  // D: row (instruction's first row + lane/4), physical chunk lane%4, logical
  // chunk (lane%4) ^ swz4(row).  W2: row (instruction's first row +
  // lane/(BN/8)), 32-byte pair ((lane%(BN/8))/2 ^ swzp(row)), half lane%2.
  const int d_lr = lane >> 2, d_pc = lane & 3;
  const int w_lr = lane / (W_ROWB / 16), w_pc = lane % (W_ROWB / 16);
  const uint16_t* dsrc_l[D_INS];
#pragma unroll
  for (int i = 0; i < D_INS; ++i) {
    const int r = (wave * D_INS + i) * D_RPI + d_lr;
    dsrc_l[i] = dblk + r * BK + ((d_pc ^ swz4(r)) << 3);
  }
  int w_row[W_INS], w_off[W_INS];
#pragma unroll
  for (int i = 0; i < W_INS; ++i) {
    const int r = (wave * W_INS + i) * W_RPI + w_lr;
    w_row[i] = r;
    w_off[i] = ((((w_pc >> 1) ^ swzp(r)) << 1) | (w_pc & 1)) * 8;
  }
  // Ids of chunk t for this lane's W2 rows.
  auto load_ids = [&](int t, int (&ids)[W_INS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < W_INS; ++i) ids[i] = clamp_index(sIdx[t & 7][w_row[i]], h);
  };
  // 4-byte direct load of chunk t's 32 ids into ring slot t % 8 (lanes 0..31 of
  // wave 0; positions past k read id 0 of the block, whose D columns are zero).
  auto id_dma = [&](int t) __attribute__((always_inline)) {
    if (wave == 0 && lane < BK) {
      const int j = t * BK + lane;
      dma4_at(sidx + (j < k ? j : 0), lds_addr(&sIdx[t & 7][0]));
    }
  };

#define G2R_ISSUE(kt_, buf_, ids_)                                                          \
  {                                                                                         \
    const uint32_t st_ = smem_lds + (buf_) * STAGE;                                         \
    _Pragma("unroll") for (int i = 0; i < D_INS; ++i)                                       \
        dma16_at(dsrc_l[i] + (int64_t)(kt_) * BK * BM, st_ + (wave * D_INS + i) * 1024);    \
    _Pragma("unroll") for (int i = 0; i < W_INS; ++i)                                       \
        dma16_at(w2 + (int64_t)ids_[i] * d + n0 + w_off[i], st_ + D_BYTES + (wave * W_INS + i) * 1024); \
  }

  f32x16_t acc[MI][NI];
  const int KT = kp / BK;
  // Prologue: ids of chunks 0..5, then stages 0 and 1, then the tile's old y
  // into the accumulators (so the sums start from y and the epilogue only
  // stores; the y loads' latency overlaps the first stages).
  if (wave == 0 && lane < BK) {
#pragma unroll
    for (int t = 0; t < 6; ++t)
      if (t < KT) dma4_at(sidx + (t * BK + lane < k ? t * BK + lane : 0), lds_addr(&sIdx[t][0]));
  }
  wait_vmcnt<0>();
  __syncthreads();
  int ids_a[W_INS], ids_b[W_INS];
  load_ids(0, ids_a);
  G2R_ISSUE(0, 0, ids_a);
  if (KT > 1) {
    load_ids(1, ids_a);
    G2R_ISSUE(1, 1, ids_a);
  }
  if (KT > 2) load_ids(2, ids_a);
  // Row bases are wave-uniform; a lane adds one 32-bit offset (its 4-row half
  // and column).  Rows past the block end start at 0 and are never stored.
  const int lane_off = (lane >> 5) * 4 * d + wave * WN + (lane & 31);
  const int mhalf = (lane >> 5) * 4;
  const bool full = rows == BM;   // wave-uniform: only a ragged last block clamps
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = mi * 32 + (r >> 2) * 8 + (r & 3);
        if (full) {
          acc[mi][ni][r] = y[(r0 + R) * (int64_t)d + n0 + ni * 32 + lane_off];
        } else {
          const int rr = R + mhalf < rows ? R + mhalf : rows - 1;
          acc[mi][ni][r] = y[(r0 + rr) * (int64_t)d + n0 + ni * 32 + wave * WN + (lane & 31)];
        }
      }

  const int sw = swz4(lane & 31);
  // One K-chunk; `slot` is kt % NS (a constant in the unrolled loop below, so
  // the stage base becomes an immediate offset of the LDS reads).
  auto chunk = [&](int kt, int slot) __attribute__((always_inline)) {
    // Outstanding loads of this wave, newest first: stage kt+1 (L) and, on wave
    // 0, the id load of chunk kt+5 if the previous iteration issued one.
    // Everything older (stage kt, and y) must be complete.
    if (kt + 1 < KT) {
      if (wave == 0 && kt >= 1 && kt + 5 < KT)
        wait_vmcnt<L + 1>();
      else
        wait_vmcnt<L>();
    } else {
      wait_vmcnt<0>();
    }
    barrier();
    if (kt + 6 < KT) id_dma(kt + 6);
    if (kt + 2 < KT) G2R_ISSUE(kt + 2, (slot + 2) % NS, ids_a);
    if (kt + 3 < KT) load_ids(kt + 3, ids_b);
    const unsigned char* st = smem + slot * STAGE;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int coff = (((2 * s + (lane >> 5)) ^ sw) << 4);
      bf16x8_t af[MI], bfr[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = tr_operand_swz_nat(st + D_BYTES, W_ROWB, s * 16, wave * WN + ni * 32, lane);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = *(const bf16x8_t*)(st + (mi * 32 + (lane & 31)) * D_ROWB + coff);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(af[mi], bfr[ni], acc[mi][ni]);
    }
#pragma unroll
    for (int i = 0; i < W_INS; ++i) ids_a[i] = ids_b[i];
  };
  static_assert(NS == 3, "the K loop is unrolled by the ring size");
  int kt = 0;
  for (; kt + 2 < KT; kt += 3) {
    chunk(kt, 0);
    chunk(kt + 1, 1);
    chunk(kt + 2, 2);
  }
  for (; kt < KT; ++kt) chunk(kt, kt % NS);
#undef G2R_ISSUE

  // y = acc (which started from the old y).
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = mi * 32 + (r >> 2) * 8 + (r & 3);
        float* yrow = y + (r0 + R) * (int64_t)d + n0 + ni * 32;
        if (full || R + mhalf < rows) yrow[lane_off] = acc[mi][ni][r];
      }
}

// Sparse phase 2 on fp8 operands (the fp8 second product): D as e4m3 codes
// with a scale byte per (row, 32 units) (written by phase 1, see FD above) and
// the gathered W2 rows as e4m3 codes with one scale per output column.  The
// ring and its accounting are those of gemm2_rows_body with 64-unit chunks:
// a stage holds D's 128 rows x 64 bytes, 64 gathered W2 rows x BN bytes and
// the chunk's 256 D scale bytes (one 4-byte direct load of 16 lanes per
// wave, so every wave issues the same number of loads per stage).  W2 rows
// store 16-byte chunk c at c ^ (row % 8); each fp8 B operand is four 8-bit
// transposing reads (ds_read_b64_tr_b8: within 16 lanes, lane i receives byte
// i % 8 of the vectors that lanes 2e + i/8 read, e = 0..7), lane pair 2e, 2e+1
// pointing at row k0 + e, columns c .. c+7 and c+8 .. c+15, so that lane i
// gets column c + i of rows k0 .. k0+7.  Four runs of 8 rows (K bytes 16g..,
// 16g+8.., 32+16g.., 40+16g.. for g = lane/32) make the operand layout of
// v_mfma_scale_f32_32x32x64_f8f6f4.  The D scales are read per product from
// the stage (a byte per lane: row lane%32, block lane/32); the W2 column
// scales stay in registers.
template <int BN>
struct Gemm2RowsF8Lds {
  static constexpr int kStage = BM * 64 + 64 * BN + 256;
  static constexpr int kRing = 3 * kStage;
  static constexpr int kIds = 8 * 64;
};

__device__ __forceinline__ uint2 lds_read_tr8(const unsigned char* p) {
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i_t lds_v2i;
  const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p));
  return make_uint2((uint32_t)r[0], (uint32_t)r[1]);
}

template <int BN>
__device__ __forceinline__ void gemm2_rows_body_f8(int lin, unsigned char* smem, int (*sIdx)[64],
                                                   const unsigned char* __restrict__ dsrc,
                                                   const unsigned char* __restrict__ w2,
                                                   const uint8_t* __restrict__ w2s, const int32_t* __restrict__ idx,
                                                   float* __restrict__ y, int64_t n, int d, int h, int k, int kp) {
  constexpr int BK = 64, NS = 3;
  constexpr int WN = BN / 4, NI = WN / 32, MI = BM / 32;
  constexpr int D_ROWB = 64;                 // 64 units of a D row
  constexpr int W_ROWB = BN;                 // a W2 row of the tile
  constexpr int D_BYTES = BM * D_ROWB;       // 8 KB
  constexpr int W_BYTES = BK * W_ROWB;
  constexpr int STAGE = D_BYTES + W_BYTES + 256;
  constexpr int D_RPI = 1024 / D_ROWB;
  constexpr int W_RPI = 1024 / W_ROWB;
  constexpr int D_INS = BM / D_RPI / 4;
  constexpr int W_INS = BK / W_RPI / 4;
  constexpr int L = D_INS + W_INS + 1;       // + the scale bytes
  constexpr int WCH = BN / 16;               // 16-byte chunks per W2 tile row
  static_assert(NS * STAGE == Gemm2RowsF8Lds<BN>::kRing, "LDS layout");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_lds = lds_addr(smem);
  const int nb = (int)row_blocks(n), ntn = d / BN;
  const int u = xcd_unit(lin, ntn * nb);
  if (u >= ntn * nb) return;
  int b, tile;
  grouped_tile(u, nb, ntn, kGroupTiles, b, tile);
  const int n0 = tile * BN;
  const int64_t r0 = (int64_t)b * BM;
  const int rows = (int)(n - r0 < BM ? n - r0 : BM);
  const int KT = kp / BK;
  const unsigned char* dblk = dsrc + (int64_t)b * BM * kp;
  const unsigned char* sblk = dsrc + (int64_t)nb * BM * kp + (int64_t)b * KT * 256;   // chunk scales
  const int32_t* sidx = idx + (int64_t)b * k;

  // D: row (instruction's first row + lane/4), physical chunk lane%4, logical
  // chunk (lane%4) ^ swz4(row).  W2: row (instruction's first row + lane/WCH),
  // physical chunk lane%WCH, logical chunk (lane%WCH) ^ (row % 8).
  const int d_lr = lane >> 2, d_pc = lane & 3;
  const int w_lr = lane / WCH, w_pc = lane % WCH;
  const unsigned char* dsrc_l[D_INS];
#pragma unroll
  for (int i = 0; i < D_INS; ++i) {
    const int r = (wave * D_INS + i) * D_RPI + d_lr;
    dsrc_l[i] = dblk + r * BK + ((d_pc ^ swz4(r)) << 4);
  }
  int w_row[W_INS], w_off[W_INS];
#pragma unroll
  for (int i = 0; i < W_INS; ++i) {
    const int r = (wave * W_INS + i) * W_RPI + w_lr;
    w_row[i] = r;
    w_off[i] = n0 + ((w_pc ^ (r & 7)) << 4);
  }
  auto load_ids = [&](int t, int (&ids)[W_INS]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < W_INS; ++i) ids[i] = clamp_index(sIdx[t & 7][w_row[i]], h);
  };
  auto id_dma = [&](int t) __attribute__((always_inline)) {
    if (wave == 0) {
      const int j = t * BK + lane;
      dma4_at(sidx + (j < k ? j : 0), lds_addr(&sIdx[t & 7][0]));
    }
  };
#define G2F_ISSUE(kt_, buf_, ids_)                                                                  \
  {                                                                                                 \
    const uint32_t st_ = smem_lds + (buf_) * STAGE;                                                 \
    _Pragma("unroll") for (int i = 0; i < D_INS; ++i)                                               \
        dma16_at(dsrc_l[i] + (int64_t)(kt_) * BK * BM, st_ + (wave * D_INS + i) * 1024);            \
    _Pragma("unroll") for (int i = 0; i < W_INS; ++i)                                               \
        dma16_at(w2 + (int64_t)ids_[i] * d + w_off[i], st_ + D_BYTES + (wave * W_INS + i) * 1024);  \
    if (lane < 16) dma4_at(sblk + (kt_) * 256 + wave * 64 + lane * 4, st_ + D_BYTES + W_BYTES + wave * 64); \
  }

  f32x16_t acc[MI][NI];
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 6; ++t)
      if (t < KT) dma4_at(sidx + (t * BK + lane < k ? t * BK + lane : 0), lds_addr(&sIdx[t][0]));
  }
  wait_vmcnt<0>();
  __syncthreads();
  int ids_a[W_INS], ids_b[W_INS];
  load_ids(0, ids_a);
  G2F_ISSUE(0, 0, ids_a);
  if (KT > 1) {
    load_ids(1, ids_a);
    G2F_ISSUE(1, 1, ids_a);
  }
  if (KT > 2) load_ids(2, ids_a);
  // W2 column scales of this lane's output columns, then the tile's old y.
  int sb[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) sb[ni] = w2s[n0 + wave * WN + ni * 32 + (lane & 31)];
  const int lane_off = (lane >> 5) * 4 * d + wave * WN + (lane & 31);
  const int mhalf = (lane >> 5) * 4;
  const bool full = rows == BM;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = mi * 32 + (r >> 2) * 8 + (r & 3);
        if (full) {
          acc[mi][ni][r] = y[(r0 + R) * (int64_t)d + n0 + ni * 32 + lane_off];
        } else {
          const int rr = R + mhalf < rows ? R + mhalf : rows - 1;
          acc[mi][ni][r] = y[(r0 + rr) * (int64_t)d + n0 + ni * 32 + wave * WN + (lane & 31)];
        }
      }

  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const int sw = swz4(lane & 31);
  const int g = lane >> 5;
  // transposing-read geometry: lane pair (2e, 2e+1) of a 16-lane group reads
  // row e of a run, bytes (lane%2)*8 of the group's 16-column chunk
  const int tj = lane & 15, trow = tj >> 1, thalf = (tj & 1) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) {
      if (wave == 0 && kt >= 1 && kt + 5 < KT)
        wait_vmcnt<L + 1>();
      else
        wait_vmcnt<L>();
    } else {
      wait_vmcnt<0>();
    }
    barrier();
    if (kt + 6 < KT) id_dma(kt + 6);
    if (kt + 2 < KT) G2F_ISSUE(kt + 2, (kt + 2) % NS, ids_a);
    if (kt + 3 < KT) load_ids(kt + 3, ids_b);
    const unsigned char* st = smem + (kt % NS) * STAGE;
    const unsigned char* sw2 = st + D_BYTES;
    const unsigned char* ssc = st + D_BYTES + W_BYTES;
    i32x8_t bop[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int cchunk = (wave * WN + ni * 32 + (lane & 16)) >> 4;   // the group's 16-column chunk
      uint2 q[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int krow = (rr >> 1) * 32 + (rr & 1) * 8 + g * 16 + trow;
        q[rr] = lds_read_tr8(sw2 + krow * W_ROWB + ((cchunk ^ (krow & 7)) << 4) + thalf);
      }
      const i32x8_t v = {(int)q[0].x, (int)q[0].y, (int)q[1].x, (int)q[1].y,
                         (int)q[2].x, (int)q[2].y, (int)q[3].x, (int)q[3].y};
      bop[ni] = v;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const unsigned char* arow = st + (mi * 32 + (lane & 31)) * D_ROWB;
      const i32x4_t lo = *(const i32x4_t*)(arow + ((g ^ sw) << 4));
      const i32x4_t hi = *(const i32x4_t*)(arow + (((2 + g) ^ sw) << 4));
      const i32x8_t aop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int sa = ssc[(mi * 32 + (lane & 31)) * 2 + g];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[ni], acc[mi][ni], 0, 0, 0, sa, 0, sb[ni]);
    }
#pragma unroll
    for (int i = 0; i < W_INS; ++i) ids_a[i] = ids_b[i];
  }
#undef G2F_ISSUE

#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = mi * 32 + (r >> 2) * 8 + (r & 3);
        float* yrow = y + (r0 + R) * (int64_t)d + n0 + ni * 32;
        if (full || R + mhalf < rows) yrow[lane_off] = acc[mi][ni][r];
      }
}

template <int BN>
__global__ __launch_bounds__(256, 2) void mlp_gemm2_rows_f8(const unsigned char* __restrict__ dsrc,
                                                            const unsigned char* __restrict__ w2,
                                                            const uint8_t* __restrict__ w2s,
                                                            const int32_t* __restrict__ idx, float* __restrict__ y,
                                                            int64_t n, int d, int h, int k, int kp) {
  __shared__ __align__(16) unsigned char smem[Gemm2RowsF8Lds<BN>::kRing];
  __shared__ __align__(16) int sIdx[8][64];
  gemm2_rows_body_f8<BN>(blockIdx.x, smem, sIdx, dsrc, w2, w2s, idx, y, n, d, h, k, kp);
}

template <int BN>
__global__ __launch_bounds__(256, 2) void mlp_gemm2_rows(const uint16_t* __restrict__ dsrc,
                                                         const uint16_t* __restrict__ w2,
                                                         const int32_t* __restrict__ idx, float* __restrict__ y,
                                                         int64_t n, int d, int h, int k, int kp) {
  __shared__ __align__(16) unsigned char smem[Gemm2RowsLds<BN>::kRing];
  __shared__ __align__(16) int sIdx[8][32];
  gemm2_rows_body<BN>(blockIdx.x, smem, sIdx, dsrc, w2, idx, y, n, d, h, k, kp);
}

}  // namespace
}  // namespace chipmunk
