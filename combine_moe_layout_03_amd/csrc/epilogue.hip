// Expert-side epilogue between dispatch and combine: dequantise the int32
// output of the first expert GEMM, SwiGLU, requantise to int8
// ("UMDK/CAM communication acceleration library deep analysis v2", section
// 4.3, stage 2 DeqSwigluQuant, and section 4.8.1, the GMM1 epilogue
// PerTokenDequantSwiGLU).
//
// Each row is one wave's work (up to n = 1024) or two or four waves' (up to
// 2048, 4096); lanes own 4-column chunks of the n output columns.  For each
// column i:
//   g = (float(acc[i])     * ws[i])     * ts      gate (int32 -> binary32 RNE)
//   u = (float(acc[n + i]) * ws[n + i]) * ts      up
//   a = (g / (1 + e^-g)) * u                      Swish(gate) * up
// each operation rounded on its own (this file is compiled with contraction
// off, and binary32 division is correctly rounded).  The row's activations
// stay in registers; the wave reduces their largest magnitude, and the row
// is quantised exactly as dispatch quantises a token row, into the same
// int8 row format (codes, then the inverse scale at byte align32(n)).
//
// e^x and the activation: swiglu.h.
#include "device_util.h"
#include "launch.h"
#include "quant.h"
#include "swiglu.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kEpiThreads = 256;
constexpr int kEpiRows = kEpiThreads / kWave;  // rows per workgroup

#define MOE_GLOBAL __attribute__((address_space(1)))
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// kW waves per row (a workgroup holds kEpiRows / kW rows); wave part p of a
// row owns the chunks lane + 64 (i kW + p), i < kIt, so each load
// instruction of a wave covers 64 consecutive chunks (1 KB of int32).  With
// kW > 1 the parts combine their largest magnitudes through LDS.
template <int kIt, int kW>
__global__ __launch_bounds__(kEpiThreads) void deq_swiglu_quant_kernel(EpilogueArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(static_cast<int>(threadIdx.x / kWave));
  const int part = wave % kW;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * (kEpiRows / kW) + wave / kW;
  // No early return before the barrier below: a wave past the last row
  // works on the last row and stores nothing.
  const bool active = m < a.rows;
  const int64_t mr = active ? m : a.rows - 1;
  const int chunks = a.n >> 2;
  // Global-address-space pointers: plain global loads, waited for by vmcnt alone.
  const MOE_GLOBAL int32_t* row = (const MOE_GLOBAL int32_t*)(a.acc) + mr * 2 * a.n;
  const MOE_GLOBAL float* ws = (const MOE_GLOBAL float*)(a.weight_scale);
  const float ts = *(const MOE_GLOBAL float*)((const MOE_GLOBAL uint8_t*)(a.token_scale) + mr * a.ts_stride);

  // Loads of every chunk first (clamped index past the row's end: the data
  // is loaded but not used), then the arithmetic.  The accumulators are
  // loaded and the codes stored non-temporally (each is touched once): at
  // 32768 rows x n 2048 that measured 102.3 us against 105.6 us with
  // ordinary loads and stores, and 109.5 us with non-temporal loads alone.
  i32x4 cg[kIt], cu[kIt];
  f32x4 wg[kIt], wu[kIt];
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int c = min(lane + (i * kW + part) * kWave, chunks - 1);
    cg[i] = __builtin_nontemporal_load(reinterpret_cast<const MOE_GLOBAL i32x4*>(row + 4 * c));
    cu[i] = __builtin_nontemporal_load(reinterpret_cast<const MOE_GLOBAL i32x4*>(row + a.n + 4 * c));
    wg[i] = *reinterpret_cast<const MOE_GLOBAL f32x4*>(ws + 4 * c);
    wu[i] = *reinterpret_cast<const MOE_GLOBAL f32x4*>(ws + a.n + 4 * c);
  }
  float act[kIt][4];
  uint32_t mag = 0;
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) act[i][q] = swiglu(cg[i][q], cu[i][q], wg[i][q], wu[i][q], ts);
    if (lane + (i * kW + part) * kWave < chunks) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t b = __float_as_uint(act[i][q]) & 0x7fffffffu;  // |a| orders as an integer
        mag = mag > b ? mag : b;
      }
    }
  }
  mag = wave_max_u32(mag);
  if constexpr (kW > 1) {
    __shared__ uint32_t part_max[kEpiRows];
    if (lane == 0) part_max[wave] = mag;
    __syncthreads();
    const int first = (wave / kW) * kW;
#pragma unroll
    for (int q = 0; q < kW; ++q) mag = mag > part_max[first + q] ? mag : part_max[first + q];
  }
  if (!active) return;
  const float amax = __uint_as_float(mag);
  const float s = 127.0f / (amax + 1e-12f);
  const float inv = 1.0f / s;
  uint8_t* out = a.out + m * a.out_row_bytes;
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int c = lane + (i * kW + part) * kWave;
    if (c < chunks) {
      const uint32_t b0 = code_bits(act[i][0], s) & 0xffu;
      const uint32_t b1 = code_bits(act[i][1], s) & 0xffu;
      const uint32_t b2 = code_bits(act[i][2], s) & 0xffu;
      const uint32_t b3 = code_bits(act[i][3], s);
      __builtin_nontemporal_store(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24), reinterpret_cast<uint32_t*>(out) + c);
    }
  }
  if (part == 0 && lane == 0) *reinterpret_cast<float*>(out + a.scale_off) = inv;
}

template <int kIt, int kW>
hipError_t launch_shape(const EpilogueArgs& a, hipStream_t stream) {
  constexpr int rows_per_group = kEpiRows / kW;
  const dim3 grid(static_cast<unsigned>((a.rows + rows_per_group - 1) / rows_per_group));
  hipLaunchKernelGGL((deq_swiglu_quant_kernel<kIt, kW>), grid, dim3(kEpiThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// The shape of select::kEpilogueShapes for n columns (one case per entry).
hipError_t launch_deq_swiglu_quant(const EpilogueArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int i = select::epilogue_shape_index(a.n);
  if (i < 0) return hipErrorInvalidValue;
  const select::EpilogueShape sh = select::kEpilogueShapes[i];
#define MOE_EPI_CASE(IT, W) \
  if (sh.it == (IT) && sh.waves == (W)) return launch_shape<IT, W>(a, stream);
  MOE_EPI_CASE(1, 1)
  MOE_EPI_CASE(2, 1)
  MOE_EPI_CASE(4, 1)
  MOE_EPI_CASE(4, 2)
  MOE_EPI_CASE(4, 4)
#undef MOE_EPI_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
