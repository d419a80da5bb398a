// Dynamic int8 quantisation helpers shared by the dispatch kernels
// ("UMDK/CAM communication acceleration library deep analysis v2", section
// 2.5, QuantProcess).  Included by .hip files compiled with floating-point
// contraction off.
#pragma once

#include "device_util.h"

namespace moe {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Running maximum of |x| over eight 16-bit elements, two at a time: with the
// sign bits cleared, bf16 and fp16 magnitudes order like unsigned integers,
// so a packed 16-bit integer max (v_pk_max_u16) does the comparison.
__device__ __forceinline__ u16x2 max_magnitude(u16x2 m, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu));
  return m;
}

// int8 code of one element in the low byte of the result.  y = f * s is one
// rounded binary32 multiply; adding 1.5 * 2^23 (binade [2^23, 2^24), ulp 1)
// rounds y half-to-even to an integer n exactly, since |y| < 127.5 < 2^22,
// and the sum's bit pattern is 0x4b400000 + n, whose low byte is n as a
// two's-complement int8 -- the same code as rint, int32 conversion and
// narrowing, in two instructions.  (This file is compiled with contraction
// off, so the multiply and the add stay separate.)
__device__ __forceinline__ uint32_t code_bits(float f, float s) {
  const float y = f * s;
  return __float_as_uint(y + 12582912.0f);
}

// Eight elements -> eight int8 codes packed little-endian in two dwords.
template <bool kFp16>
__device__ __forceinline__ uint2 quantise_chunk(const uint4& v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t a = w[2 * d], b = w[2 * d + 1];
    const uint32_t c0 = code_bits(half_to_f32<kFp16>(a & 0xffffu), s);
    const uint32_t c1 = code_bits(half_to_f32<kFp16>(a >> 16), s);
    const uint32_t c2 = code_bits(half_to_f32<kFp16>(b & 0xffffu), s);
    const uint32_t c3 = code_bits(half_to_f32<kFp16>(b >> 16), s);
    out[d] = (c0 & 0xffu) | ((c1 & 0xffu) << 8) | ((c2 & 0xffu) << 16) | (c3 << 24);
  }
  return make_uint2(out[0], out[1]);
}

// Scale and inverse scale of a row whose largest magnitude has the 16-bit
// pattern m (sign cleared): s = 127 / (amax + 1e-12f), inv = 1 / s, both
// correctly rounded binary32 divisions.
template <bool kFp16>
__device__ __forceinline__ void row_scale(uint32_t m, float& s, float& inv) {
  const float amax = half_to_f32<kFp16>(m);
  s = 127.0f / (amax + 1e-12f);
  inv = 1.0f / s;
}

}  // namespace moe
