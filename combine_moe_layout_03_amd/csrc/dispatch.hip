// Stage 3, dispatch ("UMDK/CAM communication acceleration library deep
// analysis v2", section 2.5, moe_dispatch_normal_zb and QuantProcess).
//
// One wave per token.  The wave reads the token's row once, 16 bytes (eight
// 16-bit elements) per lane per load, coalesced, and keeps it in registers;
// then it writes the row (or its int8 codes and inverse scale) to each of the
// token's k receive rows.  Quantisation:
//   amax = max |x_i|            -- taken on the 16-bit patterns with the sign
//                                  bit cleared (magnitude order = integer
//                                  order), reduced across the wave (DPP)
//   s    = 127.0f / (amax + 1e-12f),  inv = 1.0f / s
//                               -- correctly rounded binary32 divisions
//   q_i  = rint(x_i * s)        -- one binary32 multiply, then round half to
//                                  even to an integer (see code_bits)
// |x_i * s| < 127.5, so the page's int32 -> half -> int8 casts are exact and
// q_i is the integer narrowed.
//
// Each int8 row holds h code bytes, then the float inverse scale at byte
// align32(h); each lane stores eight codes (8 bytes) per chunk.  The token
// row is loaded non-temporally (it is read once); the stores are ordinary
// (non-temporal stores of the scattered receive rows measured 60 % slower).
#include "device_util.h"
#include "launch.h"
#include "quant.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kDispatchThreads = 256;
constexpr int kTokensPerBlock = kDispatchThreads / kWave;  // one wave per token
constexpr int kGroup = 8;  // destinations resolved together

// One wave per token; a lane holds chunks lane + 64 i, i < kVpl, of the row
// (8 elements, 16 bytes each).
template <bool kFp16, bool kQuant, int kVpl>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(RouteArgs a,
                                                                    const uint16_t* __restrict__ x,
                                                                    uint8_t* __restrict__ recv) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(static_cast<int>(threadIdx.x / kWave));
  const int t = uniform(blockIdx.x * kTokensPerBlock + wave);
  if (t >= a.bs) return;
  const int chunks = a.hidden >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * a.hidden);

  uint4 v[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const int c = lane + i * kWave;
    if (c < chunks) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c));
      v[i] = make_uint4(w.x, w.y, w.z, w.w);
    } else {
      v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  if constexpr (!kQuant) {
    for (int j0 = 0; j0 < a.k; j0 += kGroup) {
      int64_t row_off[kGroup];
      bool valid[kGroup];
      resolve_rows<kGroup>(a, t, j0, lane, row_off, valid);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (!valid[j]) continue;
        uint4* dst = reinterpret_cast<uint4*>(recv + row_off[j]);
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
          const int c = lane + i * kWave;
          if (c < chunks) dst[c] = v[i];
        }
      }
    }
  } else {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < kVpl; ++i) m2 = max_magnitude(m2, v[i]);
    const uint32_t m = wave_max_u32(m2.x > m2.y ? m2.x : m2.y);
    float s, inv;
    row_scale<kFp16>(m, s, inv);
    uint2 q[kVpl];
#pragma unroll
    for (int i = 0; i < kVpl; ++i) q[i] = quantise_chunk<kFp16>(v[i], s);
    for (int j0 = 0; j0 < a.k; j0 += kGroup) {
      int64_t row_off[kGroup];
      bool valid[kGroup];
      resolve_rows<kGroup>(a, t, j0, lane, row_off, valid);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (!valid[j]) continue;
        uint8_t* base = recv + row_off[j];
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
          const int c = lane + i * kWave;
          if (c < chunks) reinterpret_cast<uint2*>(base)[c] = q[i];
        }
        if (lane == 0) *reinterpret_cast<float*>(base + a.scale_off) = inv;
      }
    }
  }
}

// One case per entry of select::kDispatchVpl.
template <bool kFp16, bool kQuant>
hipError_t launch_vpl(const RouteArgs& a, const uint16_t* x, uint8_t* recv, hipStream_t stream) {
  const dim3 grid((a.bs + kTokensPerBlock - 1) / kTokensPerBlock);
  const dim3 block(kDispatchThreads);
#define MOE_DISPATCH_CASE(V)                                                                              \
  case V:                                                                                                 \
    hipLaunchKernelGGL((dispatch_kernel<kFp16, kQuant, V>), grid, block, 0, stream, a, x, recv);          \
    return hipGetLastError();
  switch (select::dispatch_vpl(a.hidden)) {
    MOE_DISPATCH_CASE(1)
    MOE_DISPATCH_CASE(2)
    MOE_DISPATCH_CASE(4)
    MOE_DISPATCH_CASE(8)
    MOE_DISPATCH_CASE(16)
    MOE_DISPATCH_CASE(32)
  }
#undef MOE_DISPATCH_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dispatch(const RouteArgs& r, const void* x, Half x_type, bool quant,
                           void* recv_x, hipStream_t stream) {
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  uint8_t* recv = static_cast<uint8_t*>(recv_x);
  if (x_type == Half::kFp16) {
    return quant ? launch_vpl<true, true>(r, xs, recv, stream)
                 : launch_vpl<true, false>(r, xs, recv, stream);
  }
  return quant ? launch_vpl<false, true>(r, xs, recv, stream)
               : launch_vpl<false, false>(r, xs, recv, stream);
}

}  // namespace moe
