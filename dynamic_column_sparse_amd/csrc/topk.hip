// Sparsity identification: exact top-k per score row (gfx950).
//
// One workgroup (512 threads, 8 waves) per row.  Scores become monotone 32-bit
// keys (NaN -> 0, the lowest; -0 -> +0; sign-magnitude -> offset binary), so the
// choice is integer work and matches any exact reference bit for bit.
//   1. Radix select, 8 bits per pass from the top: an LDS histogram of the
//      candidates that still match the prefix finds the k-th largest key T and
//      how many keys equal to T must still be taken (ties go to the lower index).
//   2. One pass in index order emits key > T plus the first `need` keys == T,
//      using wave ballots for the in-order ranks, so the output is ascending.
// Rows of up to kLdsCap scores are staged in LDS once; longer rows (attention
// at long sequence lengths) are re-read from global memory on each pass.
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsCap = 15360;  // 60 KB of keys

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks lowest
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void topk_rows(const float* __restrict__ score, int64_t cols, int k,
                                                      int32_t* __restrict__ idx) {
  extern __shared__ uint32_t skey[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[kWaves];
  __shared__ uint32_t wtot2[kWaves];
  __shared__ uint32_t sh_prefix, sh_remaining;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* srow = score + row * cols;
  int32_t* orow = idx + row * (int64_t)k;

  if (IN_LDS) {
    for (int64_t i = tid; i < cols; i += kThreads) skey[i] = score_key(srow[i]);
  }
  __syncthreads();
  auto key_at = [&](int64_t i) -> uint32_t { return IN_LDS ? skey[i] : score_key(srow[i]); };

  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < cols; i += kThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Inclusive scan of the counts from the top digit down (threads 0..255).
    uint32_t hv = 0, incl = 0;
    if (tid < 256) {
      hv = hist[255 - tid];
      incl = hv;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      if (lane == 63) wtot[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += wtot[w];
      const uint32_t excl = incl - hv;
      if (excl < remaining && remaining <= incl) {
        sh_prefix = prefix | ((uint32_t)(255 - tid) << shift);
        sh_remaining = remaining - excl;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    mask |= 255u << shift;
  }

  const uint32_t T = prefix, need = remaining;
  uint32_t taken = 0, eq_seen = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int64_t base = 0; base < cols && taken < (uint32_t)k; base += kThreads) {
    const int64_t i = base + tid;
    const bool in = i < cols;
    const uint32_t key = in ? key_at(i) : 0u;
    const bool gt = in && key > T;
    const bool eq = in && key == T;
    const uint64_t em = __ballot(eq);
    if (lane == 0) wtot[wave] = (uint32_t)__popcll(em);
    __syncthreads();
    uint32_t eq_before = eq_seen, eq_chunk = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) eq_before += wtot[w];
      eq_chunk += wtot[w];
    }
    const uint32_t eq_rank = eq_before + (uint32_t)__popcll(em & lt_mask);
    const bool take = gt || (eq && eq_rank < need);
    const uint64_t tm = __ballot(take);
    if (lane == 0) wtot2[wave] = (uint32_t)__popcll(tm);
    __syncthreads();
    uint32_t t_before = taken, t_chunk = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) t_before += wtot2[w];
      t_chunk += wtot2[w];
    }
    const uint32_t pos = t_before + (uint32_t)__popcll(tm & lt_mask);
    if (take && pos < (uint32_t)k) orow[pos] = (int32_t)i;
    taken += t_chunk;
    eq_seen += eq_chunk;
    __syncthreads();
  }
}

// Register-resident variant for rows of up to kRegCols scores: 1024 threads,
// thread t holds keys t + 1024 j (j < kRegKeys).
//   1. Min and max of the row's keys: every key shares their common bit
//      prefix, so the radix passes start at the first bit where they differ
//      (positive scores of similar size share sign and exponent bits; starting
//      at the top would send every key of the first passes to one bin).
//   2. Radix select over the remaining bits, up to 8 per pass, with one
//      256-bin histogram per wave (contention only inside a wave).
//   3. Emit in index order from one ballot pair per (batch j, wave) and a
//      single 16 x 16 prefix table of packed (above, equal) counts.
constexpr int kRegThreads = 1024;
constexpr int kRegWaves = kRegThreads / 64;
constexpr int kRegKeys = 16;
constexpr int kRegCols = kRegThreads * kRegKeys;

// Exclusive prefix sum over tab[0..255] in (batch, wave) order, in place;
// returns the total.  Threads 0..255 take part; ends with a barrier.
__device__ __forceinline__ uint32_t table_scan(uint32_t* tab, uint32_t* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t v = 0, incl = 0;
  if (tid < 256) {
    v = tab[tid];
    incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
  }
  __syncthreads();
  uint32_t total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  if (tid < 256) {
    for (int w = 0; w < wave; ++w) incl += wsum[w];
    tab[tid] = incl - v;
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kRegThreads) void topk_rows_reg(const float* __restrict__ score, int cols, int k,
                                                             int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kRegWaves][256];
  __shared__ uint32_t tab[kRegKeys * kRegWaves];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t red[2][kRegWaves];
  __shared__ uint32_t sh_prefix, sh_remaining;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* srow = score + row * (int64_t)cols;
  int32_t* orow = idx + row * (int64_t)k;

  uint32_t key[kRegKeys];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const int i = tid + kRegThreads * j;
    key[j] = i < cols ? score_key(srow[i]) : 0u;
    if (i < cols) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = red[0][0];
  kmax = red[1][0];
#pragma unroll
  for (int w = 1; w < kRegWaves; ++w) {
    kmin = min(kmin, red[0][w]);
    kmax = max(kmax, red[1][w]);
  }
  // Bits above `hi` are common to every key.
  int hi = (kmin == kmax) ? -1 : 31 - __clz((int)(kmin ^ kmax));
  uint32_t prefix = hi >= 31 ? 0u : (kmin & ~((2u << hi) - 1u));
  if (hi < 0) prefix = kmin;
  uint32_t remaining = (uint32_t)k;
  while (hi >= 0) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t above = hi >= 31 ? 0u : ~((2u << hi) - 1u);   // bits already fixed
    for (int i = tid; i < kRegWaves * 256; i += kRegThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegKeys; ++j) {
      const int i = tid + kRegThreads * j;
      if (i < cols && (key[j] & above) == prefix) atomicAdd(&hist[wave][(key[j] >> lo) & ((2u << (hi - lo)) - 1u)], 1u);
    }
    __syncthreads();
    // Bin counts summed over the waves, scanned from the top bin down.
    const int nbins = 2 << (hi - lo);
    uint32_t hv = 0, incl = 0;
    if (tid < 256) {
      const int bin = nbins - 1 - tid;
      if (bin >= 0) {
#pragma unroll
        for (int w = 0; w < kRegWaves; ++w) hv += hist[w][bin];
      }
      incl = hv;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += wsum[w];
      const uint32_t excl = incl - hv;
      if (tid < nbins && excl < remaining && remaining <= incl) {
        sh_prefix = prefix | ((uint32_t)(nbins - 1 - tid) << lo);
        sh_remaining = remaining - excl;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    hi = lo - 1;
  }

  const uint32_t T = prefix, need = remaining;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  // One scan places every output: index i is taken if its key is above T, or
  // equal to T with fewer than `need` equal keys before it; its position is
  // (keys above T before i) + min(keys equal to T before i, need).  Both counts
  // of each (batch, wave) travel packed in one word (each fits in 16 bits).
  uint64_t gm[kRegKeys], em[kRegKeys];
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const bool valid = tid + kRegThreads * j < cols;
    gm[j] = __ballot(valid && key[j] > T);
    em[j] = __ballot(valid && key[j] == T);
    if (lane == 0) tab[j * kRegWaves + wave] = (uint32_t)__popcll(gm[j]) | ((uint32_t)__popcll(em[j]) << 16);
  }
  __syncthreads();
  table_scan(tab, wsum, tid);
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const uint32_t base = tab[j * kRegWaves + wave];
    const uint32_t gt_before = (base & 0xffffu) + (uint32_t)__popcll(gm[j] & lt_mask);
    const uint32_t eq_before = (base >> 16) + (uint32_t)__popcll(em[j] & lt_mask);
    const bool gt = (gm[j] >> lane) & 1ull, eq = (em[j] >> lane) & 1ull;
    if (gt || (eq && eq_before < need)) {
      const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
      if (pos < (uint32_t)k) orow[pos] = tid + kRegThreads * j;
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* score, int64_t rows, int64_t cols, int k, int32_t* idx, hipStream_t s) {
  timing_before(K_TOPK, s);
  if (cols <= kRegCols)
    hipLaunchKernelGGL(topk_rows_reg, dim3((unsigned)rows), dim3(kRegThreads), 0, s, score, (int)cols, k, idx);
  else if (cols <= kLdsCap)
    hipLaunchKernelGGL((topk_rows<true>), dim3((unsigned)rows), dim3(kThreads), (size_t)cols * 4, s, score, cols, k,
                       idx);
  else
    hipLaunchKernelGGL((topk_rows<false>), dim3((unsigned)rows), dim3(kThreads), 0, s, score, cols, k, idx);
  hipError_t e = hipGetLastError();
  timing_after(K_TOPK, s);
  return e;
}

}  // namespace chipmunk
