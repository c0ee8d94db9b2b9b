// Sparsity identification: exact top-k per score row (gfx950).
//
// Scores become monotone 32-bit keys (NaN -> 0, the lowest; -0 -> +0;
// sign-magnitude -> offset binary), so the choice is integer work and matches
// any exact reference bit for bit.  The k-th largest key T and the number of
// keys equal to T still to take (ties go to the lower index) come from radix
// passes over LDS histograms; a final pass in index order emits key > T and the
// first `need` keys == T, so the output is ascending.  Rows of up to 16384
// scores stay in registers (one workgroup of 1024 threads); longer rows are
// read three times by a 512-thread workgroup (see topk_rows_long).
#include "device_common.h"
#include "internal.h"

namespace chipmunk {
namespace {

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks lowest
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rows longer than the register variant holds (attention rows at long sequence
// lengths), one workgroup of 512 threads per row, three reads of the row:
//   1. an 8192-bin histogram of the keys' top 13 bits finds the bin B that
//      holds the k-th largest key, the count above it and how many of the
//      bin's keys are still needed;
//   2. the keys of bin B (their low 19 bits) are gathered into LDS (wave-
//      aggregated slots), and radix passes of 10 and 9 bits over them give the
//      exact k-th key T and how many keys equal to T are taken (ties to the
//      lower index); a bin larger than the LDS buffer is resolved with the
//      same two passes over the row in global memory instead;
//   3. one pass in index order emits key > T and the first `need` keys == T,
//      each thread taking 16 consecutive scores per iteration (the next 16 are
//      loaded before this iteration's scan), with a block scan of packed
//      (above, equal) counts for the output positions.
// Loads are 16-byte when the row is 16-byte aligned (cols % 4 == 0).  LDS is
// 32 KB of bins and 47 KB of candidates, so two workgroups share a CU.
constexpr int kLongThreads = 512;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kTopBits = 13;
constexpr int kTopBins = 1 << kTopBits;
constexpr int kLowBits = 32 - kTopBits;   // 19: resolved as 10 + 9
constexpr int kCandCap = 12000;   // candidate keys (47 KB)

// Exclusive block scan (in thread order) of one 32-bit value per thread;
// returns the exclusive prefix and sets `total`.  Ends with a barrier (wsum
// may be reused after it).
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kLongWaves; ++w) {
    const uint32_t x = wsum[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  __syncthreads();
  return before + incl - v;
}

template <bool VEC>
__global__ __launch_bounds__(kLongThreads) void topk_rows_long(const float* __restrict__ score, int64_t cols, int k,
                                                               int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kTopBins];
  __shared__ uint32_t cand[kCandCap];
  __shared__ uint32_t wsum[kLongWaves];
  __shared__ uint32_t sh_bin, sh_above, sh_fill;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = blockIdx.x;
  const float* srow = score + row * cols;
  int32_t* orow = idx + row * (int64_t)k;
  const int64_t nvec = VEC ? cols / 4 : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));

  // f(key, valid) for every score of the row (any order), four 16-byte loads
  // per thread in flight before any of them is used; every lane of a wave
  // runs the same calls (invalid ones with valid = false), so f may use
  // wave-wide operations.
  auto for_each = [&](auto&& f) __attribute__((always_inline)) {
    if (VEC) {
      for (int64_t v0 = 0; v0 < nvec; v0 += 4 * kLongThreads) {
        float4 x[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t v = v0 + u * kLongThreads + tid;
          ok[u] = v < nvec;
          x[u] = ok[u] ? *(const float4*)(srow + 4 * v) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          f(score_key(x[u].x), ok[u]);
          f(score_key(x[u].y), ok[u]);
          f(score_key(x[u].z), ok[u]);
          f(score_key(x[u].w), ok[u]);
        }
      }
    }
    for (int64_t i0 = 4 * nvec; i0 < cols; i0 += kLongThreads) {
      const int64_t i = i0 + tid;
      const bool ok = i < cols;
      f(ok ? score_key(srow[i]) : 0u, ok);
    }
  };
  // Bin of the kth largest among `nbins` (8192, 1024 or 512) counts in hist,
  // from the top bin down: sets sh_bin and sh_above (the count in higher bins).
  auto select_bin = [&](int nbins, uint32_t kth) __attribute__((always_inline)) {
    const int per = nbins / kLongThreads;    // 16, 2 or 1 bins per thread, highest first
    uint32_t c[16], tot = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      c[j] = j < per ? hist[nbins - 1 - tid * per - j] : 0u;
      tot += c[j];
    }
    uint32_t all;
    const uint32_t excl = block_scan_excl(tot, wsum, all);
    uint32_t run = excl;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < per && run < kth && kth <= run + c[j]) {
        sh_bin = (uint32_t)(nbins - 1 - tid * per - j);
        sh_above = run;
      }
      run += c[j];
    }
    __syncthreads();
  };

  // ---- 1. top 13 bits
  for (int i = tid; i < kTopBins; i += kLongThreads) hist[i] = 0u;
  if (tid == 0) sh_fill = 0u;
  __syncthreads();
  for_each([&](uint32_t key, bool ok) {
    if (ok) atomicAdd(&hist[key >> kLowBits], 1u);
  });
  __syncthreads();
  select_bin(kTopBins, (uint32_t)k);
  const uint32_t B = sh_bin;
  uint32_t remaining = (uint32_t)k - sh_above;      // still needed from bin B
  const uint32_t candN = hist[B];
  const bool in_lds = candN <= (uint32_t)kCandCap;
  __syncthreads();

  // ---- 2. the keys of bin B
  if (in_lds) {
    // wave-aggregated slots: one LDS atomic per wave and ballot
    auto keep = [&](uint32_t key, bool hit) __attribute__((always_inline)) {
      const uint64_t m = __ballot(hit);
      if (m == 0) return;
      const int first = __builtin_ctzll(m);
      uint32_t base = 0;
      if (lane == first) base = atomicAdd(&sh_fill, (uint32_t)__popcll(m));
      base = __shfl(base, first);
      if (hit) cand[base + __popcll(m & lt_mask)] = key & ((1u << kLowBits) - 1u);
    };
    for_each([&](uint32_t key, bool ok) { keep(key, ok && (key >> kLowBits) == B); });
    __syncthreads();
  }
  // low 19 bits: passes of 10 and 9 bits over bin B's keys (in LDS, or the row)
  uint32_t prefix = B << kLowBits;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 9 : 0;
    const int nbins = pass == 0 ? 1024 : 512;
    const uint32_t mask = pass == 0 ? ~((1u << kLowBits) - 1u) : ~((1u << 9) - 1u);
    for (int i = tid; i < nbins; i += kLongThreads) hist[i] = 0u;
    __syncthreads();
    if (in_lds) {
      for (uint32_t c = tid; c < candN; c += kLongThreads) {
        const uint32_t key = cand[c] | (B << kLowBits);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
    } else {
      for_each([&](uint32_t key, bool ok) {
        if (ok && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
      });
    }
    __syncthreads();
    select_bin(nbins, remaining);
    prefix |= sh_bin << shift;
    remaining -= sh_above;
  }
  const uint32_t T = prefix, need = remaining;

  // ---- 3. emit in index order: thread t takes scores base + 16t .. base + 16t + 15
  constexpr int EPT = 16;
  auto load_run = [&](int64_t i0, uint32_t (&key)[EPT]) __attribute__((always_inline)) {
    if (VEC && i0 + EPT <= cols) {
#pragma unroll
      for (int q = 0; q < EPT / 4; ++q) {
        const float4 x = *(const float4*)(srow + i0 + 4 * q);
        key[4 * q] = score_key(x.x);
        key[4 * q + 1] = score_key(x.y);
        key[4 * q + 2] = score_key(x.z);
        key[4 * q + 3] = score_key(x.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) key[e] = i0 + e < cols ? score_key(srow[i0 + e]) : 0u;
    }
  };
  uint32_t gt_total = 0, eq_total = 0;
  uint32_t cur[EPT], nxt[EPT];
  load_run(EPT * (int64_t)tid, cur);
  for (int64_t base = 0; base < cols; base += EPT * kLongThreads) {
    if (gt_total + (eq_total < need ? eq_total : need) >= (uint32_t)k) break;   // uniform
    const int64_t i0 = base + EPT * tid;
    if (base + EPT * kLongThreads < cols) load_run(i0 + EPT * kLongThreads, nxt);
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool in = i0 + e < cols;
      cg += (in && cur[e] > T) ? 1u : 0u;
      ce += (in && cur[e] == T) ? 1u : 0u;
    }
    uint32_t chunk;
    const uint32_t excl = block_scan_excl(cg | (ce << 16), wsum, chunk);
    uint32_t gt_before = gt_total + (excl & 0xffffu), eq_before = eq_total + (excl >> 16);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool in = i0 + e < cols;
      if (in && cur[e] > T) {
        const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
        if (pos < (uint32_t)k) orow[pos] = (int32_t)(i0 + e);
        ++gt_before;
      } else if (in && cur[e] == T) {
        if (eq_before < need) {
          const uint32_t pos = gt_before + eq_before;
          if (pos < (uint32_t)k) orow[pos] = (int32_t)(i0 + e);
        }
        ++eq_before;
      }
    }
    gt_total += chunk & 0xffffu;
    eq_total += chunk >> 16;
#pragma unroll
    for (int e = 0; e < EPT; ++e) cur[e] = nxt[e];
  }
}

// Register-resident variant for rows of up to kRegCols scores: THREADS
// threads (256, 512 or 1024: the smallest that holds the row, so short rows
// leave no idle lanes and more rows share a CU), each holding kRegKeys keys.
// Scalar layout: thread t holds keys t + THREADS j (j < kRegKeys).  VEC layout
// (rows of a multiple of 4 scores, 16-byte aligned): key j of thread t is
// score 4 (t + THREADS (j / 4)) + j % 4, read as one 16-byte load per group of
// four (a quarter of the load instructions).
//   1. Min and max of the row's keys: every key shares their common bit
//      prefix, so the radix passes start at the first bit where they differ
//      (positive scores of similar size share sign and exponent bits; starting
//      at the top would send every key of the first passes to one bin).
//   2. Radix select over the remaining bits, up to 8 per pass, with one
//      256-bin histogram per wave (contention only inside a wave).
//   3. Emit in index order from ballots per (batch, wave) and a single
//      prefix table of packed (above, equal) counts per (batch, wave); a
//      batch is one key per thread (scalar) or one group of four (VEC), and
//      either way the batches, then the waves, then the lanes run in index
//      order.
constexpr int kRegKeys = 16;
constexpr int kRegCols = 1024 * kRegKeys;

// Exclusive prefix sum over tab[0..N-1] (N = 64, 128 or 256) in (batch, wave)
// order, in place; returns the total.  Threads 0..N-1 take part; ends with a
// barrier.
template <int N>
__device__ __forceinline__ uint32_t table_scan(uint32_t* tab, uint32_t* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t v = 0, incl = 0;
  if (tid < N) {
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
  uint32_t total = 0;
#pragma unroll
  for (int w = 0; w < N / 64; ++w) total += wsum[w];
  if (tid < N) {
    for (int w = 0; w < wave; ++w) incl += wsum[w];
    tab[tid] = incl - v;
  }
  __syncthreads();
  return total;
}

template <int THREADS, bool VEC>
__global__ __launch_bounds__(THREADS) void topk_rows_reg(const float* __restrict__ score, int cols, int k,
                                                        int32_t* __restrict__ idx) {
  constexpr int kWaves = THREADS / 64;
  constexpr int kBatches = VEC ? kRegKeys / 4 : kRegKeys;   // prefix-table rows
  constexpr int kPer = VEC ? 4 : 1;                          // keys per batch and thread
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t tab[kBatches * kWaves];
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t red[2][kWaves];
  __shared__ uint32_t sh_prefix, sh_remaining;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* srow = score + row * (int64_t)cols;
  int32_t* orow = idx + row * (int64_t)k;

  // Key j of this thread is score index i0(j / kPer) + j % kPer, valid when
  // its batch is inside the row (VEC: cols % 4 == 0, so a group is whole).
  auto i0 = [&](int bt) __attribute__((always_inline)) { return kPer * (tid + THREADS * bt); };
  uint32_t key[kRegKeys];
  bool ok[kBatches];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    ok[bt] = i0(bt) < cols;
    if constexpr (VEC) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok[bt]) v = reinterpret_cast<const float4*>(srow)[tid + THREADS * bt];
      key[4 * bt] = score_key(v.x);
      key[4 * bt + 1] = score_key(v.y);
      key[4 * bt + 2] = score_key(v.z);
      key[4 * bt + 3] = score_key(v.w);
    } else {
      key[bt] = ok[bt] ? score_key(srow[i0(bt)]) : 0u;
    }
    if (ok[bt]) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        kmin = min(kmin, key[kPer * bt + e]);
        kmax = max(kmax, key[kPer * bt + e]);
      }
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
  for (int w = 1; w < kWaves; ++w) {
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
    for (int i = tid; i < kWaves * 256; i += THREADS) (&hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegKeys; ++j) {
      if (ok[j / kPer] && (key[j] & above) == prefix)
        atomicAdd(&hist[wave][(key[j] >> lo) & ((2u << (hi - lo)) - 1u)], 1u);
    }
    __syncthreads();
    // Bin counts summed over the waves, scanned from the top bin down.
    const int nbins = 2 << (hi - lo);
    uint32_t hv = 0, incl = 0;
    if (tid < 256) {
      const int bin = nbins - 1 - tid;
      if (bin >= 0) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) hv += hist[w][bin];
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
  // Index i is taken if its key is above T, or equal to T with fewer than
  // `need` equal keys before it; its position is (keys above T before i) +
  // min(keys equal to T before i, need).  Both counts of each (batch, wave)
  // travel packed in one word (each fits in 16 bits).
  uint64_t gm[kRegKeys], em[kRegKeys];
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = kPer * bt + e;
      gm[j] = __ballot(ok[bt] && key[j] > T);
      em[j] = __ballot(ok[bt] && key[j] == T);
      cg += (uint32_t)__popcll(gm[j]);
      ce += (uint32_t)__popcll(em[j]);
    }
    if (lane == 0) tab[bt * kWaves + wave] = cg | (ce << 16);
  }
  __syncthreads();
  table_scan<kBatches * kWaves>(tab, wsum, tid);
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    const uint32_t base = tab[bt * kWaves + wave];
    // Keys of this batch before this thread's: those of the lower lanes (all
    // kPer of each), then this thread's own, one at a time.
    uint32_t g = base & 0xffffu, q = base >> 16;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      g += (uint32_t)__popcll(gm[kPer * bt + e] & lt_mask);
      q += (uint32_t)__popcll(em[kPer * bt + e] & lt_mask);
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = kPer * bt + e;
      const bool gt = (gm[j] >> lane) & 1ull, eq = (em[j] >> lane) & 1ull;
      if (gt) {
        const uint32_t pos = g + (q < need ? q : need);
        if (pos < (uint32_t)k) orow[pos] = i0(bt) + e;
        ++g;
      } else if (eq) {
        if (q < need && g + q < (uint32_t)k) orow[g + q] = i0(bt) + e;
        ++q;
      }
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* score, int64_t rows, int64_t cols, int k, int32_t* idx, hipStream_t s) {
  timing_before(K_TOPK, s);
  // 16-byte loads when every row starts 16-byte aligned.
  const bool vec = cols % 4 == 0 && ((uintptr_t)score & 15) == 0;
#define REG_LAUNCH(T_)                                                                                         \
  {                                                                                                            \
    if (vec)                                                                                                   \
      hipLaunchKernelGGL((topk_rows_reg<T_, true>), dim3((unsigned)rows), dim3(T_), 0, s, score, (int)cols, k, idx); \
    else                                                                                                       \
      hipLaunchKernelGGL((topk_rows_reg<T_, false>), dim3((unsigned)rows), dim3(T_), 0, s, score, (int)cols, k, idx); \
  }
  if (cols <= 256 * kRegKeys)
    REG_LAUNCH(256)
  else if (cols <= 512 * kRegKeys)
    REG_LAUNCH(512)
  else if (cols <= kRegCols)
    REG_LAUNCH(1024)
  else if (vec)
    hipLaunchKernelGGL((topk_rows_long<true>), dim3((unsigned)rows), dim3(kLongThreads), 0, s, score, cols, k, idx);
  else
    hipLaunchKernelGGL((topk_rows_long<false>), dim3((unsigned)rows), dim3(kLongThreads), 0, s, score, cols, k, idx);
#undef REG_LAUNCH
  hipError_t e = hipGetLastError();
  timing_after(K_TOPK, s);
  return e;
}

}  // namespace chipmunk
