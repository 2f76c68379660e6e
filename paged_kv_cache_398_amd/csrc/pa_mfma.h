// pa_mfma.h -- device helpers shared by the kernels that run their products
// on the matrix cores (v_mfma_f32_16x16x32_bf16): operand types, the 4-lane
// maximum of a 16x16 result column, and the two-term bf16 split of the
// softmax weights.  Internal; included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

// 1.0 in all eight bf16 lanes (the "ones" operand whose product gives row sums)
__device__ __forceinline__ bf16x8_t bf16x8_ones() {
  return as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
}

// Maximum over lanes c, c+16, c+32, c+48 (the four lanes of one column of a
// 16x16 product).  A compare and select: the values are scores or -inf,
// never NaN, so no quieting of NaN inputs (which fmaxf would add after the
// lane swaps) is needed.
__device__ __forceinline__ float max4q(float x) {
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float u = __uint_as_float(r[0]), v = __uint_as_float(r[1]);
    x = u > v ? u : v;
  }
  {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float u = __uint_as_float(r[0]), v = __uint_as_float(r[1]);
    x = u > v ? u : v;
  }
  return x;
}

__device__ __forceinline__ float max8(const float (&x)[2][4]) {
  return fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
               fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
}

// p = hi + lo in bf16: hi is p truncated to bf16 (the upper half of its
// bits, one byte permute per pair), the remainder p - hi is exact in fp32
// and below 2^-7 p, and lo is that remainder rounded to the nearest bf16;
// so hi + lo is within a relative 2^-16 of p.
__device__ __forceinline__ void split_bf16(const float (&p)[8], bf16x8_t &hi, bf16x8_t &lo) {
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __float_as_uint(p[2 * i]), b = __float_as_uint(p[2 * i + 1]);
    h[i] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // upper halves of a (low), b (high)
    lo[2 * i] = (__bf16)(p[2 * i] - __uint_as_float(a & 0xFFFF0000u));
    lo[2 * i + 1] = (__bf16)(p[2 * i + 1] - __uint_as_float(b & 0xFFFF0000u));
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
}

}  // namespace pa
