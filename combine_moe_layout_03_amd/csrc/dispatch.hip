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
constexpr int kGroup = 8;  // destinations resolved together

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16- and 8-byte stores; kNt marks them non-temporal (streaming).
template <bool kNt>
__device__ __forceinline__ void put(uint4* p, const uint4& v) {
  if constexpr (kNt) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}
template <bool kNt>
__device__ __forceinline__ void put(uint2* p, const uint2& v) {
  if constexpr (kNt) {
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
  } else {
    *p = v;
  }
}

// kWpt waves per token (a workgroup holds kDispatchThreads / 64 / kWpt
// tokens).  Wave part p of a token owns the 64-chunk groups p, p + kWpt,
// p + 2 kWpt, ... of the row; a lane holds chunk lane + 64 * group, i.e.
// kVpl chunks of 8 elements (16 bytes) each.  With kWpt > 1 the parts combine
// their maxima through LDS.  kNt selects non-temporal stores.
template <bool kFp16, bool kQuant, int kVpl, int kWpt, bool kNt>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(RouteArgs a,
                                                                    const uint16_t* __restrict__ x,
                                                                    uint8_t* __restrict__ recv) {
  constexpr int kTok = kDispatchThreads / kWave / kWpt;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(static_cast<int>(threadIdx.x / kWave));
  const int t = uniform(blockIdx.x * kTok + wave / kWpt);
  const int part = wave % kWpt;
  // No early return before the barrier below: inactive waves skip the work.
  const bool active = t < a.bs;
  const int chunks = a.hidden >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<size_t>(active ? t : 0) * a.hidden);

  uint4 v[kVpl];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const int c = lane + (i * kWpt + part) * kWave;
    if (active && c < chunks) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c));
      v[i] = make_uint4(w.x, w.y, w.z, w.w);
    } else {
      v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  if constexpr (!kQuant) {
    if (!active) return;
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
          const int c = lane + (i * kWpt + part) * kWave;
          if (c < chunks) put<kNt>(dst + c, v[i]);
        }
      }
    }
  } else {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < kVpl; ++i) m2 = max_magnitude(m2, v[i]);
    uint32_t m = wave_max_u32(m2.x > m2.y ? m2.x : m2.y);
    if constexpr (kWpt > 1) {
      __shared__ uint32_t part_max[kDispatchThreads / kWave];
      if (lane == 0) part_max[wave] = m;
      __syncthreads();
      const int first = (wave / kWpt) * kWpt;
#pragma unroll
      for (int q = 0; q < kWpt; ++q) m = m > part_max[first + q] ? m : part_max[first + q];
    }
    if (!active) return;
    const float amax = half_to_f32<kFp16>(m);
    const float s = 127.0f / (amax + 1e-12f);
    const float inv = 1.0f / s;
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
          const int c = lane + (i * kWpt + part) * kWave;
          if (c < chunks) put<kNt>(reinterpret_cast<uint2*>(base) + c, q[i]);
        }
        if (part == 0 && lane == 0) *reinterpret_cast<float*>(base + a.scale_off) = inv;
      }
    }
  }
}

template <bool kFp16, bool kQuant>
hipError_t launch_vpl(const RouteArgs& a, const uint16_t* x, uint8_t* recv, hipStream_t stream) {
  constexpr int kWpt = 1;
  constexpr int kTok = kDispatchThreads / kWave / kWpt;
  const int chunks = a.hidden / 8;
  const int per_lane = (chunks + kWave * kWpt - 1) / (kWave * kWpt);
  const dim3 grid((a.bs + kTok - 1) / kTok);
  const dim3 block(kDispatchThreads);
#define MOE_DISPATCH_CASE(V)                                                                             \
  if (per_lane <= V) {                                                                                   \
    hipLaunchKernelGGL((dispatch_kernel<kFp16, kQuant, V, kWpt, false>), grid, block, 0, stream, a, x, recv); \
    return hipGetLastError();                                                                            \
  }
  MOE_DISPATCH_CASE(1)
  MOE_DISPATCH_CASE(2)
  MOE_DISPATCH_CASE(4)
  MOE_DISPATCH_CASE(8)
  MOE_DISPATCH_CASE(16)
  MOE_DISPATCH_CASE(32)
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
