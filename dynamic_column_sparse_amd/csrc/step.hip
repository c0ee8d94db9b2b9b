// The sparse step of one transformer block as two launches: the MLP's sparse
// phase 1, then ONE kernel whose first workgroups run the MLP's phase-2 tiles
// and whose remaining workgroups run the attention delta (the fixed-set step,
// or the step that re-identifies its keys every step).
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
#include "topk_kernels.h"

#include <algorithm>
#include <atomic>

namespace chipmunk {
namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// blockIdx.x < g2: phase-2 unit blockIdx.x of xcd_grid(ntn * nb) units.
// Otherwise: attention unit blockIdx.x - g2.  g2 is a multiple of 8, so both
// bodies keep their own unit -> XCD mapping (unit id mod 8).  F8W: the phase-2
// tiles run the fp8 second product (fp8 D from phase 1, fp8 W2 rows).
template <int BN, bool F8W>
__global__ __launch_bounds__(256, 2) void sparse_step_fused(
    int g2, const uint16_t* __restrict__ dsrc, const uint16_t* __restrict__ w2, const uint8_t* __restrict__ w2f8,
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
  if (bid < g2) {
    if constexpr (F8W)
      gemm2_rows_body_f8<BN>(bid, smem, reinterpret_cast<int(*)[64]>(sIdx), (const unsigned char*)dsrc, w2f8, w2s,
                             midx, y, n, d, h, k, kp);
    else
      gemm2_rows_body<BN>(bid, smem, reinterpret_cast<int(*)[32]>(sIdx), dsrc, w2, midx, y, n, d, h, k, kp, k);
  } else {
    // The sparse (non-refresh) body only reads num and den.
    attn_sparse_body<false>(bid - g2, smem, reinterpret_cast<int(*)[32]>(sIdx), sDen, sDenRest, q, kx, v, aidx, m,
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
// the fixed-set one.  The two bodies' LDS overlay each other.
template <int BN, bool F8W>
__global__ __launch_bounds__(256, 2) void sparse_step_reident_fused(
    int g2, const uint16_t* __restrict__ dsrc, const uint16_t* __restrict__ w2, const uint8_t* __restrict__ w2f8,
    const uint8_t* __restrict__ w2s, const int32_t* __restrict__ midx, float* __restrict__ y, int64_t n, int d, int h,
    int k, int kp, const uint16_t* __restrict__ q_prev, const uint16_t* __restrict__ k_prev,
    const uint16_t* __restrict__ v_prev, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kx,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ aidx, const float* __restrict__ m,
    float* __restrict__ num, float* __restrict__ den, float* __restrict__ ascore, float* __restrict__ o, int64_t na,
    int heads, int kk, float scale) {
  __shared__ __align__(16) ReidentStepLds<BN, F8W> lds;
  const int bid = blockIdx.x;
  if (bid < g2) {
    if constexpr (F8W)
      gemm2_rows_body_f8<BN>(bid, lds.g2.ring, reinterpret_cast<int(*)[64]>(lds.g2.ids),
                             (const unsigned char*)dsrc, w2f8, w2s, midx, y, n, d, h, k, kp);
    else
      gemm2_rows_body<BN>(bid, lds.g2.ring, reinterpret_cast<int(*)[32]>(lds.g2.ids), dsrc, w2, midx, y, n, d, h, k,
                          kp, k);
  } else {
    attn_reident_body(bid - g2, lds.at, q_prev, k_prev, v_prev, q, kx, v, aidx, m, num, den, ascore, o, na, heads,
                      kk, scale);
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
  const dim3 grid((unsigned)(g2 + ga));
  timing_before(K_SPARSE_STEP_REIDENT_FUSED, s);
  const uint8_t* w2f8 = f8w ? f8w->w : nullptr;
  const uint8_t* w2s = f8w ? f8w->w_scale : nullptr;
#define REID_LAUNCH(BN_, F8W_)                                                                                       \
  hipLaunchKernelGGL((sparse_step_reident_fused<BN_, F8W_>), grid, dim3(256), 0, s, g2, dbuf, w2, w2f8, w2s, midx, y, \
                     n, d, h, k, kp, q_prev, k_prev, v_prev, q, kx, v, aidx, m, num, den, ascore, o, na, heads, kk,  \
                     scale)
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
  const dim3 grid((unsigned)(g2 + ga));
  timing_before(K_SPARSE_STEP_FUSED, s);
  const uint8_t* w2f8 = f8w ? f8w->w : nullptr;
  const uint8_t* w2s = f8w ? f8w->w_scale : nullptr;
#define FUSED_LAUNCH(BN_, F8W_)                                                                                      \
  hipLaunchKernelGGL((sparse_step_fused<BN_, F8W_>), grid, dim3(256), 0, s, g2, dbuf, w2, w2f8, w2s, midx, y, n, d, h, \
                     k, kp, q, kx, v, aidx, m, num, den, o, na, heads, kk, scale)
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

namespace {

// ---------------------------------------------------------------------------
// The whole sparse step in one launch: the MLP's identification (top-k of each
// row block's scores), its phase 1 and phase 2, and the fixed-set attention
// delta, one work item per workgroup:
//   identification: the top-k of one row block's MLP scores (256 threads, the
//      register body of the identification kernel), written to the caller's
//      index array and to a padded copy that the MLP items read;
//   attention: one (head, query block) unit of the sparse attention delta;
//   phase 1: one (row block, column tile) of the gathered GEMM1, once that
//      block is identified;
//   phase 2: one (row block, output tile) of the gathered GEMM2, once every
//      phase-1 tile of that block is done.
// Every item runs the same body as the separate kernels, so the results are
// bit-identical to chipmunk_identify_topk followed by chipmunk_sparse_step.
// The attention units need nothing from the MLP, so they cover the time the
// identification takes and fill the slots that phase-2 tiles leave while they
// wait; the three kernel boundaries of the separate launches (each a drain of
// the chip) are gone.
//
// Order.  Workgroups whose id is x (mod 8) run on XCD x.  Each XCD has its own
// sequence of items, claimed in order with one atomic per workgroup: its share
// of the identification rows (b = 8s + x), the first `seg[1]` of its attention
// units, its phase-1 tiles, the rest of its attention units, its phase-2
// tiles.  Each kind keeps the unit -> XCD mapping of its own kernel (item s of
// XCD x is the unit a separate launch gives workgroup 8s + x), so the weight
// rows and activation blocks that the GEMM tiles share stay in that XCD's L2.
// The grid is 8 x the sequence length, so every workgroup claims one item
// (units past the end of a kind are empty).
//
// Progress.  Items wait only for items earlier in the dependency order
// (identification < phase 1 < phase 2), and every XCD's sequence lists them in
// that order.  A workgroup waits only for an item that is either running or
// unclaimed; an unclaimed one is preceded in its XCD's sequence only by items
// claimed by running workgroups, whose own waits go to strictly earlier kinds.
// The earliest unfinished item in the dependency order can therefore always
// run, however many workgroups are resident.  Each wait is still bounded
// (kSpinLimit polls): one that gives up sets the status word and goes on, so
// the kernel always ends.
//
// Visibility across XCDs (each has its own L2).  A producer's stores finish
// (vmcnt 0), the workgroup meets at a barrier, and one lane writes the XCD's
// L2 back (an agent-scope release fence) before it bumps the flag with an
// atomic.  The consumer polls the flag with agent-scope loads and then reads
// the data with plain loads: the lines it reads (a block's padded index row,
// its D tiles; both start on 128-byte lines) are read by nobody before their
// flag is set, and kernel start leaves no stale copy in any cache, so those
// reads miss to memory and see the written values.  An acquire fence is left
// out on purpose: it would invalidate the whole L2 of the consumer's XCD, and
// with it the weight rows that the GEMM tiles running there share.
//
// The last workgroup to finish (an exit count) clears the counters and flags,
// so the sync block is zero again for the next call.
constexpr int kSpinLimit = 1 << 20;

struct WholeStepArgs {
  const float* mscore;
  int32_t* midx;
  int32_t* midx_pad;
  const uint16_t* x;
  const uint16_t* w1t;
  const float* b1;
  uint16_t* a_cache;
  uint16_t* dbuf;
  const uint16_t* w2;
  float* y;
  int64_t n;
  int d, h, k, kp, ild, nb, ntiles1, ntn;
  const uint16_t* q;
  const uint16_t* kx;
  const uint16_t* v;
  const int32_t* aidx;
  const float* m;
  const float* num;
  const float* den;
  float* o;
  int64_t na;
  int heads, kk;
  float scale;
  uint32_t* sync;
  // Items per XCD sequence: identification, attention (first part), phase 1,
  // attention (rest), phase 2.
  int seg[5];
};

template <int BN1, int BN2>
union WholeStepLds {
  unsigned char g1[Gemm1Lds<BN1>::kRing];
  Gemm2TileLds<BN2, false> g2;
  struct {
    unsigned char ring[AttnSparseLds::kRing];
    int ids[AttnSparseLds::kIds];
    float den[kRowBlock];
    float den_rest[kRowBlock];
  } at;
  TopkRegLds<256, kWholeTopkKeys> tk;
};

// Waits (one lane) until *flag >= target, for at most kSpinLimit polls.
__device__ __forceinline__ void whole_wait(uint32_t* sync, const uint32_t* flag, uint32_t target) {
  for (int spins = 0; __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target;) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins >= kSpinLimit) {
      atomicOr(&sync[kSyncStatus], 1u);
      break;
    }
  }
}

// Publishes the workgroup's finished stores: every lane's stores complete, the
// workgroup meets, then one lane writes the L2 back and bumps the flag.
__device__ __forceinline__ void whole_signal(uint32_t* flag) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    atomicAdd(flag, 1u);
  }
}

template <int BN1, int BN2>
__global__ __launch_bounds__(256, 2) void sparse_step_whole(const WholeStepArgs a) {
  __shared__ __align__(16) WholeStepLds<BN1, BN2> lds;
  __shared__ int s_item, s_last;
  const int tid = threadIdx.x;
  const int x = blockIdx.x & 7;
  uint32_t* sync = a.sync;
  uint32_t* ident_done = sync + kSyncFlags;
  uint32_t* g1_done = ident_done + a.nb;
  if (tid == 0) s_item = (int)atomicAdd(&sync[kSyncClaim + x], 1u);
  __syncthreads();
  int t = s_item;
  if (t < a.seg[0]) {
    const int b = 8 * t + x;
    if (b < a.nb) {
      topk_reg_body<256, kWholeTopkKeys>(b, lds.tk, a.mscore, a.h, a.k, a.midx, a.midx_pad, a.ild);
      whole_signal(&ident_done[b]);
    }
  } else if ((t -= a.seg[0]) < a.seg[1] || (t >= a.seg[1] + a.seg[2] && t < a.seg[1] + a.seg[2] + a.seg[3])) {
    // Attention unit s of this XCD (s counts both attention parts).
    const int s = t < a.seg[1] ? t : t - a.seg[2];
    const int L = 8 * s + x;
    if (L < a.heads * (int)row_blocks(a.na))
      // The sparse (non-refresh) body only reads num and den.
      attn_sparse_body<false>(L, lds.at.ring, reinterpret_cast<int(*)[32]>(lds.at.ids), lds.at.den,
                              lds.at.den_rest, a.q, a.kx, a.v, a.aidx, a.m, const_cast<float*>(a.num),
                              const_cast<float*>(a.den), a.o, a.na, a.heads, a.kk, a.scale);
  } else if ((t -= a.seg[1]) < a.seg[2]) {
    const int lin = 8 * t + x, units = a.ntiles1 * a.nb;
    const int u = xcd_unit(lin, units);
    if (u < units) {
      int b, tile;
      grouped_tile(u, a.nb, a.ntiles1, kGroupTiles, b, tile);
      if (tid == 0) whole_wait(sync, &ident_done[b], 1u);
      __syncthreads();
      gemm1_body<BN1, false, false, false>(lin, lds.g1, a.x, a.w1t, nullptr, nullptr, a.b1, a.midx_pad, a.a_cache,
                                           a.dbuf, nullptr, nullptr, a.n, a.d, a.h, a.k, a.kp, a.ild);
      whole_signal(&g1_done[b]);
    }
  } else if ((t -= a.seg[2] + a.seg[3]) >= 0 && t < a.seg[4]) {
    const int lin = 8 * t + x, units = a.ntn * a.nb;
    const int u = xcd_unit(lin, units);
    if (u < units) {
      int b, tile;
      grouped_tile(u, a.nb, a.ntn, kGroupTiles, b, tile);
      if (tid == 0) whole_wait(sync, &g1_done[b], (uint32_t)a.ntiles1);
      __syncthreads();
      gemm2_rows_body<BN2>(lin, lds.g2.ring, reinterpret_cast<int(*)[32]>(lds.g2.ids), a.dbuf, a.w2, a.midx_pad,
                           a.y, a.n, a.d, a.h, a.k, a.kp, a.ild);
    }
  }
  // The last workgroup out clears the counters and flags for the next call
  // (every other workgroup has made its last access to them).
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&sync[kSyncExit], 1u) == gridDim.x - 1;
  __syncthreads();
  if (s_last) {
    const int words = kSyncFlags + 2 * a.nb;
    for (int i = tid; i < words; i += 256)
      if (i != kSyncStatus) sync[i] = 0u;
  }
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

}  // namespace

hipError_t launch_sparse_step_whole(const float* mscore, int32_t* midx, int32_t* midx_pad, const uint16_t* x,
                                    const uint16_t* w1t, const float* b1, uint16_t* a_cache, uint16_t* dbuf,
                                    const uint16_t* w2, float* y, int64_t n, int d, int h, int k, const uint16_t* q,
                                    const uint16_t* kx, const uint16_t* v, const int32_t* aidx, const float* m,
                                    const float* num, const float* den, float* o, int64_t na, int heads, int kk,
                                    float scale, uint32_t* sync, hipStream_t s) {
  WholeStepArgs a{};
  a.mscore = mscore;
  a.midx = midx;
  a.midx_pad = midx_pad;
  a.x = x;
  a.w1t = w1t;
  a.b1 = b1;
  a.a_cache = a_cache;
  a.dbuf = dbuf;
  a.w2 = w2;
  a.y = y;
  a.n = n;
  a.d = d;
  a.h = h;
  a.k = k;
  a.kp = padded_k(k);
  a.ild = padded_ids(k);
  a.nb = (int)row_blocks(n);
  const bool wide = mlp_gemm1_wide(k);
  const int bn1 = wide ? 256 : 128, bn2 = d % 256 == 0 ? 256 : 128;
  a.ntiles1 = (k + bn1 - 1) / bn1;
  a.ntn = d / bn2;
  a.q = q;
  a.kx = kx;
  a.v = v;
  a.aidx = aidx;
  a.m = m;
  a.num = num;
  a.den = den;
  a.o = o;
  a.na = na;
  a.heads = heads;
  a.kk = kk;
  a.scale = scale;
  a.sync = sync;
  const int64_t ua = row_blocks(na) * heads;
  const int per_a = (int)((ua + 7) / 8);
  // Attention units before phase 1: enough to fill the chip while the
  // identification runs (two workgroups per CU), the rest after it.
  const int first_a = std::min(per_a, 2 * device_cus() / 8);
  a.seg[0] = k > 0 ? (a.nb + 7) / 8 : 0;
  a.seg[1] = first_a;
  a.seg[2] = k > 0 ? (a.ntiles1 * a.nb + 7) / 8 : 0;
  a.seg[3] = per_a - first_a;
  a.seg[4] = k > 0 ? (a.ntn * a.nb + 7) / 8 : 0;
  const int64_t len = (int64_t)a.seg[0] + a.seg[1] + a.seg[2] + a.seg[3] + a.seg[4];
  const dim3 grid((unsigned)(8 * (len > 0 ? len : 1)));
  timing_before(K_SPARSE_STEP_WHOLE, s);
#define WHOLE_LAUNCH(BN1_, BN2_) hipLaunchKernelGGL((sparse_step_whole<BN1_, BN2_>), grid, dim3(256), 0, s, a)
  if (wide) {
    if (bn2 == 256)
      WHOLE_LAUNCH(256, 256);
    else
      WHOLE_LAUNCH(256, 128);
  } else {
    if (bn2 == 256)
      WHOLE_LAUNCH(128, 256);
    else
      WHOLE_LAUNCH(128, 128);
  }
#undef WHOLE_LAUNCH
  hipError_t e = hipGetLastError();
  timing_after(K_SPARSE_STEP_WHOLE, s);
  return e;
}

}  // namespace chipmunk
