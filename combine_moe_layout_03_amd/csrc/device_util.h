// Device helpers shared by the HIP kernels of libmoe_ep (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---- 16-bit float patterns <-> binary32 --------------------------------------

// bfloat16 is the high half of a binary32, so widening is a shift (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary16 widening through the hardware conversion (exact, subnormals kept).
__device__ __forceinline__ float f16_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

template <bool kFp16>
__device__ __forceinline__ float half_to_f32(uint32_t b) {
  return kFp16 ? f16_to_f32(b) : bf16_to_f32(b);
}

// binary32 -> bfloat16, round half to even: add 0x7fff plus the lowest kept
// bit, then truncate.  NaNs stay quiet NaNs.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// binary32 -> binary16 through the hardware conversion, which rounds to
// nearest even in the default FP mode and keeps binary16 subnormals.
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---- wave-level helpers ------------------------------------------------------

// Number of set bits of `mask` in lanes below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), d, kWave));
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// A value known to be the same in every lane, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace moe
