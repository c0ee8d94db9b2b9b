// Device helpers shared by the gfx950 kernels: bf16 packing, the bf16 matrix-core
// instructions, the transposing LDS read and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace chipmunk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f2bf(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 operands.  Operand layout (checked on
// gfx950): lane l holds A row l%32 / B column l%32, reduction indices
// (l/32)*8 .. +7; accumulator element r of lane l is row (r/4)*8 + (l/32)*4 + r%4,
// column l%32.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// GELU, tanh form: 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)) (the same function: 0.5 (1 + tanh u) is the
// logistic function of 2u).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;
  const float u = c * (z + 0.044715f * z * z * z);
  return z / (1.0f + __expf(-2.0f * u));
}

__device__ __forceinline__ int clamp_index(int j, int hi) { return j < 0 ? 0 : (j >= hi ? hi - 1 : j); }

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
