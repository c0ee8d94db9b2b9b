// Exact top-k of one score row held in registers (gfx950): the body shared by
// the identification kernel (topk.hip) and the whole-step kernel (step.hip).
//
// Scores become monotone 32-bit keys (NaN -> 0, the lowest; -0 -> +0;
// sign-magnitude -> offset binary), so the choice is integer work and matches
// any exact reference bit for bit.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace chipmunk {

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks lowest
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Keys per thread of the identification kernel's register variant, and the
// longest row it holds (1024 threads).
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

// LDS of one row's selection: one 256-bin histogram per wave, the (batch,
// wave) prefix table and a few shared words.
template <int THREADS, int KEYS>
struct TopkRegLds {
  uint32_t hist[THREADS / 64][256];
  uint32_t tab[KEYS * (THREADS / 64)];
  uint32_t wsum[4];
  uint32_t red[2][THREADS / 64];
  uint32_t prefix, remaining;
};

// Top-k of row `row` of score [rows][cols] (cols <= THREADS * KEYS) by one
// workgroup of THREADS threads; thread t holds keys t + THREADS j (j < KEYS).
// Writes the k chosen column ids in ascending order to idx[row][0..k) and, when
// idx2 is given, to idx2[row * ld2 + 0..k) as well.
//   1. Min and max of the row's keys: every key shares their common bit
//      prefix, so the radix passes start at the first bit where they differ
//      (positive scores of similar size share sign and exponent bits; starting
//      at the top would send every key of the first passes to one bin).
//   2. Radix select over the remaining bits, up to 8 per pass, with one
//      256-bin histogram per wave (contention only inside a wave): the k-th
//      largest key T and how many keys equal to T are still to be taken (ties
//      go to the lower index).
//   3. Emit in index order: index i is taken if its key is above T, or equal
//      to T with fewer than `need` equal keys before it; its position is (keys
//      above T before i) + min(keys equal to T before i, need).  Both counts of
//      each (batch j, wave) travel packed in one word of a prefix table (each
//      fits in 16 bits).  Up to 16 keys per thread the batch ballots stay in
//      scalar registers between the count and the emit; beyond that they are
//      taken again for the emit.
template <int THREADS, int KEYS>
__device__ __forceinline__ void topk_reg_body(int64_t row, TopkRegLds<THREADS, KEYS>& L,
                                              const float* __restrict__ score, int cols, int k,
                                              int32_t* __restrict__ idx, int32_t* __restrict__ idx2, int64_t ld2) {
  constexpr int kWaves = THREADS / 64;
  static_assert(THREADS >= 256 && KEYS * kWaves <= 256 && KEYS * kWaves >= 64, "prefix table size");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = score + row * (int64_t)cols;
  int32_t* orow = idx + row * (int64_t)k;
  int32_t* orow2 = idx2 ? idx2 + row * ld2 : nullptr;

  uint32_t key[KEYS];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < KEYS; ++j) {
    const int i = tid + THREADS * j;
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
    L.red[0][wave] = kmin;
    L.red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = L.red[0][0];
  kmax = L.red[1][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    kmin = min(kmin, L.red[0][w]);
    kmax = max(kmax, L.red[1][w]);
  }
  // Bits above `hi` are common to every key.
  int hi = (kmin == kmax) ? -1 : 31 - __clz((int)(kmin ^ kmax));
  uint32_t prefix = hi >= 31 ? 0u : (kmin & ~((2u << hi) - 1u));
  if (hi < 0) prefix = kmin;
  uint32_t remaining = (uint32_t)k;
  while (hi >= 0) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t above = hi >= 31 ? 0u : ~((2u << hi) - 1u);   // bits already fixed
    for (int i = tid; i < kWaves * 256; i += THREADS) (&L.hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KEYS; ++j) {
      const int i = tid + THREADS * j;
      if (i < cols && (key[j] & above) == prefix)
        atomicAdd(&L.hist[wave][(key[j] >> lo) & ((2u << (hi - lo)) - 1u)], 1u);
    }
    __syncthreads();
    // Bin counts summed over the waves, scanned from the top bin down.
    const int nbins = 2 << (hi - lo);
    uint32_t hv = 0, incl = 0;
    if (tid < 256) {
      const int bin = nbins - 1 - tid;
      if (bin >= 0) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) hv += L.hist[w][bin];
      }
      incl = hv;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      if (lane == 63) L.wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += L.wsum[w];
      const uint32_t excl = incl - hv;
      if (tid < nbins && excl < remaining && remaining <= incl) {
        L.prefix = prefix | ((uint32_t)(nbins - 1 - tid) << lo);
        L.remaining = remaining - excl;
      }
    }
    __syncthreads();
    prefix = L.prefix;
    remaining = L.remaining;
    hi = lo - 1;
  }

  const uint32_t T = prefix, need = remaining;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  auto place = [&](uint64_t gm, uint64_t em, uint32_t base, int i) __attribute__((always_inline)) {
    const uint32_t gt_before = (base & 0xffffu) + (uint32_t)__popcll(gm & lt_mask);
    const uint32_t eq_before = (base >> 16) + (uint32_t)__popcll(em & lt_mask);
    const bool gt = (gm >> lane) & 1ull, eq = (em >> lane) & 1ull;
    if (gt || (eq && eq_before < need)) {
      const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
      if (pos < (uint32_t)k) {
        orow[pos] = i;
        if (orow2) orow2[pos] = i;
      }
    }
  };
  if constexpr (KEYS <= 16) {
    uint64_t gm[KEYS], em[KEYS];
#pragma unroll
    for (int j = 0; j < KEYS; ++j) {
      const bool valid = tid + THREADS * j < cols;
      gm[j] = __ballot(valid && key[j] > T);
      em[j] = __ballot(valid && key[j] == T);
      if (lane == 0) L.tab[j * kWaves + wave] = (uint32_t)__popcll(gm[j]) | ((uint32_t)__popcll(em[j]) << 16);
    }
    __syncthreads();
    table_scan<KEYS * kWaves>(L.tab, L.wsum, tid);
#pragma unroll
    for (int j = 0; j < KEYS; ++j) place(gm[j], em[j], L.tab[j * kWaves + wave], tid + THREADS * j);
  } else {
#pragma unroll
    for (int j = 0; j < KEYS; ++j) {
      const bool valid = tid + THREADS * j < cols;
      const uint64_t gm = __ballot(valid && key[j] > T);
      const uint64_t em = __ballot(valid && key[j] == T);
      if (lane == 0) L.tab[j * kWaves + wave] = (uint32_t)__popcll(gm) | ((uint32_t)__popcll(em) << 16);
    }
    __syncthreads();
    table_scan<KEYS * kWaves>(L.tab, L.wsum, tid);
#pragma unroll
    for (int j = 0; j < KEYS; ++j) {
      const bool valid = tid + THREADS * j < cols;
      place(__ballot(valid && key[j] > T), __ballot(valid && key[j] == T), L.tab[j * kWaves + wave],
            tid + THREADS * j);
    }
  }
}

}  // namespace chipmunk
