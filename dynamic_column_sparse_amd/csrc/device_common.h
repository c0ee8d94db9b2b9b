// Device helpers shared by the gfx950 kernels: bf16/fp16 packing, the matrix-core
// instructions, the transposing LDS read and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace chipmunk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest, ties to even, through gfx950's packed
// conversion (v_cvt_pk_bf16_f32).  Checked against a software round-to-nearest-
// even on all 2^32 fp32 patterns: identical on every non-NaN input (subnormals
// and overflow to infinity included); NaN inputs give NaN.  Branch-free, unlike
// a software version with a NaN test, which the compiler turns into divergent
// branches per element.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f2bf(float x) { return pack2(x, 0.f) & 0xffffu; }
// fp32 pair -> fp16 bits (v_cvt_pk_f16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 operands.  Operand layout (checked on
// gfx950): lane l holds A row l%32 / B column l%32, reduction indices
// (l/32)*8 .. +7; accumulator element r of lane l is row (r/4)*8 + (l/32)*4 + r%4,
// column l%32.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The same product with fp16 operands (same register layout).
__device__ __forceinline__ f32x16_t mfma32h(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// 16x16x32 fp16 product: lane l holds A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; the result D[4*(l/16) + e][l%16] is element e.
__device__ __forceinline__ f32x4_t mfma16h(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i%4 of the 4-element vector read by lane 4e + i/4, for
// e = 0..3.  Used on tiles stored [reduction][column] (rows of W2 or V as they
// come from memory): if lane j of the group points at row kb + j/4, columns
// cb + 4*(j%4) .. +3, lane i gets column cb + i of rows kb .. kb+3.
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// One 32x32x16 operand (8 bf16 per lane) from a [reduction][column] LDS tile with
// row stride `ld` elements, via two transposing reads.  Lane l gets column
// cb + l%32 and the 16 reduction rows k0 .. k0+15 in the order
//   element tt*4 + e  <-  row k0 + tt*8 + (l/32)*4 + e     (tt in 0..1, e in 0..3)
// This is a fixed permutation of the reduction index; a product is correct as
// long as both operands use the same one.  It is also the order in which a
// 32x32 accumulator holds its rows, so a softmax tile kept in registers can be
// fed straight back as the other operand.
__device__ __forceinline__ bf16x8_t tr_operand(const uint16_t* tile, int ld, int k0, int cb, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int col = cb + (G & 1) * 16 + (i & 3) * 4;
  const int kr = k0 + (G >> 1) * 4 + (i >> 2);
  i16x4_t lo = lds_read_tr16(tile + kr * ld + col);
  i16x4_t hi = lds_read_tr16(tile + (kr + 8) * ld + col);
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// ---- direct global -> LDS loads (gfx950 global_load_lds_dwordx4) ----------
// Each lane's 16 bytes land at lds + 16 * lane: one instruction fills 1 KB of
// LDS (wave-uniform destination, passed in M0) from 64 arbitrary 16-byte
// global chunks, with no register staging.  Completion is tracked by vmcnt like
// any vector load.
//
// Issued through inline assembly on purpose: the compiler cannot tell which
// LDS bytes such a load writes, so for the builtin form it drains every
// outstanding vector load (vmcnt(0)) before any later LDS read of the same
// buffer, which would empty the prefetch ring each K-step.  Here the kernels
// order these loads themselves: wait_vmcnt for the stage, then barrier(), and
// only then read it.  The instruction has no register outputs; the compiler's
// own vmcnt waits stay correct because extra loads it does not count can only
// make a vmcnt(N) wait stricter.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(m0)
      : "memory", "m0");
}
// 4-byte variant: 64 lanes x 4 bytes = 256 contiguous LDS bytes (e.g. 64 ids).
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(g), "s"(m0)
      : "memory", "m0");
}

// Forms taking the LDS destination as a 32-bit LDS address that is already
// wave-uniform (computed from the workgroup's LDS base, the loop counter and a
// wave index made uniform with readfirstlane), so each load costs one M0 write.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
}
__device__ __forceinline__ void dma16_at(const void* g, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(lds)
      : "memory", "m0");
}
// Form with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit byte
// offset: advancing the base costs scalar work only.
__device__ __forceinline__ void dma16_sa(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds)
      : "memory", "m0");
}
__device__ __forceinline__ void dma4_at(const void* g, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(g), "s"(lds)
      : "memory", "m0");
}

// Wait until at most N vector-memory instructions of this wave are in flight
// (also waits for this wave's LDS instructions).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
// wait_vmcnt with a count known only at run time (wave-uniform, LO .. HI):
// a binary search down to the immediate form.
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_range(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID)
      wait_vmcnt_range<LO, MID>(n);
    else
      wait_vmcnt_range<MID + 1, HI>(n);
  }
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  wait_vmcnt_range<0, N>(n);
}

// Workgroup barrier without the release/acquire fences of __syncthreads (which
// would wait for every outstanding global load, draining the prefetch ring).
// Callers order their own LDS traffic with wait_vmcnt before it.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

// K-contiguous tiles (rows of 64 bf16 = 8 chunks of 16 bytes): chunk c of row r
// is stored at chunk c ^ swz8(r).  16-byte reads of one chunk by consecutive
// rows then hit distinct banks in groups of 8 and of 16 lanes.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// 64-byte rows (32 bf16 = 4 chunks of 16 bytes): chunk c of row r is stored at
// chunk c ^ swz4(r).  Rows r..r+3 share one 256-byte bank window, so the XOR
// term follows r/4: 16 consecutive rows reading the same logical chunk then
// cover all 64 banks once.
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

// Tiles read with the transposing read ([k][col] rows): 32-byte column pairs
// (q = col / 16) of row r are stored at pair q ^ swzp(r).  The 4 rows x 2 pairs
// that 32 lanes of one transposing read touch then land in distinct banks.
__device__ __forceinline__ int swzp(int r) { return (r & 3) << 1; }

// One 32x32x16 operand from a swizzled [k][col] tile (row_bytes per row), in
// the reduction order of tr_operand.
__device__ __forceinline__ bf16x8_t tr_operand_swz(const unsigned char* tile, int row_bytes, int k0, int cb,
                                                   int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int col = cb + (G & 1) * 16 + (i & 3) * 4;
  const int kr = k0 + (G >> 1) * 4 + (i >> 2);
  const int off = (((col >> 4) ^ swzp(kr)) << 5) + ((col & 15) << 1);
  i16x4_t lo = lds_read_tr16((const uint16_t*)(tile + kr * row_bytes + off));
  i16x4_t hi = lds_read_tr16((const uint16_t*)(tile + (kr + 8) * row_bytes + off));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Same, in the natural reduction order of a K-contiguous operand: lane l gets
// column cb + l%32 and rows k0 + (l/32)*8 .. +7 in order, so it pairs with an
// operand read by plain 16-byte loads from a row-major tile.
__device__ __forceinline__ bf16x8_t tr_operand_swz_nat(const unsigned char* tile, int row_bytes, int k0, int cb,
                                                       int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int col = cb + (G & 1) * 16 + (i & 3) * 4;
  const int kr = k0 + (G >> 1) * 8 + (i >> 2);
  const int off = (((col >> 4) ^ swzp(kr)) << 5) + ((col & 15) << 1);
  i16x4_t lo = lds_read_tr16((const uint16_t*)(tile + kr * row_bytes + off));
  i16x4_t hi = lds_read_tr16((const uint16_t*)(tile + (kr + 4) * row_bytes + off));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// 8x8 transpose of bf16: in[r] holds elements (r, 0..7) of an 8x8 block as 4
// dwords; out[c] receives elements (0..7, c).  32 byte permutes.
__device__ __forceinline__ void transpose8x8_bf16(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t o0 = __builtin_amdgcn_perm(word_of(in[1], c >> 1), word_of(in[0], c >> 1), sel);
    const uint32_t o1 = __builtin_amdgcn_perm(word_of(in[3], c >> 1), word_of(in[2], c >> 1), sel);
    const uint32_t o2 = __builtin_amdgcn_perm(word_of(in[5], c >> 1), word_of(in[4], c >> 1), sel);
    const uint32_t o3 = __builtin_amdgcn_perm(word_of(in[7], c >> 1), word_of(in[6], c >> 1), sel);
    out[c] = make_uint4(o0, o1, o2, o3);
  }
}

// GELU, tanh form: 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)) (the same function: 0.5 (1 + tanh u) is the
// logistic function of 2u), with the hardware reciprocal (about 1 ulp; the
// result is rounded to bf16 next).  exp(-2u) overflowing to +inf gives z * 0.
//
// The exponent -2u, in base 2, is z * (a + b z^2) with a = -2c log2(e) and
// b = -2c * 0.044715 * log2(e) (c = sqrt(2/pi)): one FMA and two products
// before the hardware exp2, and no branches.
__device__ __forceinline__ float gelu_tanh(float z) {
  constexpr float a = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float b = a * 0.044715f;
  const float t = z * __builtin_fmaf(b, z * z, a);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// fp8 (OCP e4m3) power-of-two scale of a set of values whose largest |bf16|
// bit pattern (sign cleared) is mx: the smallest e >= -126 with
// max * 2^-e <= 448 (e = 0 when mx = 0).  With the maximum as fp32
// 2^(E-127) (1 + f/2^23) and 448 = 1.75 * 2^8: e = E - 135, plus one when
// 1 + f/2^23 > 1.75.
__device__ __forceinline__ int fp8_exponent(uint32_t mx) {
  if (mx == 0) return 0;
  const uint32_t ab = mx << 16;
  const int E = (int)(ab >> 23), f = (int)(ab & 0x7fffff);
  return E == 0 ? -126 : max(E - 135 + (f > 0x600000 ? 1 : 0), -126);
}
// Largest |bf16| bit pattern among the 8 values of v (sign bits cleared).
__device__ __forceinline__ uint32_t abs_max_bf16x8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) mx = max(mx, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  return mx;
}
// 8 bf16 values times 2^-e (exact) as e4m3 codes, rounded to nearest even
// (v_cvt_pk_fp8_f32); the caller's scale keeps every product within 448.
__device__ __forceinline__ uint2 bf16x8_to_fp8(const uint4& v, int e) {
  const float mul = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf2f(w[i] & 0xffffu) * mul;
    x[2 * i + 1] = bf2f(w[i] >> 16) * mul;
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__device__ __forceinline__ int clamp_index(int j, int hi) { return j < 0 ? 0 : (j >= hi ? hi - 1 : j); }

// Workgroups are handed to the 8 XCDs round-robin by linear id.  This maps the
// linear id to a unit index so that each XCD runs one contiguous range of units
// (in unit order): units that share data then share that XCD's L2.  Launch
// 8 * ceil(units / 8) workgroups; ids mapped past `units` have no work.
__device__ __forceinline__ int xcd_unit(int linear_id, int units) {
  const int per = (units + 7) >> 3;
  return (linear_id & 7) * per + (linear_id >> 3);
}
__host__ __device__ inline int xcd_grid(int units) { return ((units + 7) >> 3) << 3; }

// Unit -> (row block b, column tile t) with the column tiles in groups of `gt`:
// inside a group, the gt tiles of one row block are consecutive units, then
// those of the next block.  A contiguous range of units (one XCD's share) then
// covers a few tiles of many blocks, so both the blocks' activation rows and the
// tiles' weight rows are reused from that XCD's L2.
__device__ __forceinline__ void grouped_tile(int u, int nb, int ntiles, int gt, int& b, int& t) {
  const int per = nb * gt;
  const int tg = u / per;
  const int r = u - tg * per;
  const int g = (ntiles - tg * gt) < gt ? (ntiles - tg * gt) : gt;
  b = r / g;
  t = tg * gt + r % g;
}

// Sum 16 per-lane values over the 32 lanes of each half-wave with one exchange
// per halving: after the exchanges lane l holds the total of value
// ((l >> 1) & 15) over its half-wave (lanes l and l^1 agree).
__device__ __forceinline__ float halfwave_transpose_sum16(const float (&v)[16], int lane) {
  const bool b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  float w8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float send = b4 ? v[i] : v[i + 8];
    const float keep = b4 ? v[i + 8] : v[i];
    w8[i] = keep + __shfl_xor(send, 16);
  }
  float w4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float send = b3 ? w8[i] : w8[i + 4];
    const float keep = b3 ? w8[i + 4] : w8[i];
    w4[i] = keep + __shfl_xor(send, 8);
  }
  float w2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = b2 ? w4[i] : w4[i + 2];
    const float keep = b2 ? w4[i + 2] : w4[i];
    w2[i] = keep + __shfl_xor(send, 4);
  }
  const float send = b1 ? w2[0] : w2[1];
  const float keep = b1 ? w2[1] : w2[0];
  const float w1 = keep + __shfl_xor(send, 2);
  return w1 + __shfl_xor(w1, 1);
}

}  // namespace chipmunk
