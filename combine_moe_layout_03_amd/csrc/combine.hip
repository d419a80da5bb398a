// Stage 4, combine ("UMDK/CAM communication acceleration library deep
// analysis v2", section 2.6, moe_combine_normal_zb::ReadBufferAndWeightedSum).
//
// One wave per token.  The wave first resolves, in scalar registers, the
// receive row, weight and (int8) inverse scale of each of the token's k
// entries.  Then each lane walks chunks of eight elements: it issues the k
// row loads of a chunk together, and folds them into eight binary32
// accumulators in entry order j = 0..k-1, exactly as the page does:
//   acc = +0; acc = acc + v_j * w_j  (v_j = float(row) or float(q) * inv)
// with every multiply and add rounded separately (this file is compiled with
// floating-point contraction off), so the result is bit-identical to the
// sequential binary32 definition.  The sum is rounded half-even to the
// output type.
#include "device_util.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kTokensPerBlock = kCombineThreads / kWave;

template <Recv kRecv>
struct ChunkOf;
template <>
struct ChunkOf<Recv::kBf16> { using T = uint4; static constexpr int kBytes = 16; };
template <>
struct ChunkOf<Recv::kFp16> { using T = uint4; static constexpr int kBytes = 16; };
template <>
struct ChunkOf<Recv::kInt8> { using T = uint2; static constexpr int kBytes = 8; };

// Element e (0..7) of a loaded chunk, widened to binary32 (before the weight).
template <Recv kRecv>
__device__ __forceinline__ float element(const typename ChunkOf<kRecv>::T& c, int e, float inv) {
  if constexpr (kRecv == Recv::kInt8) {
    const uint32_t w = e < 4 ? c.x : c.y;
    const int8_t q = static_cast<int8_t>((w >> (8 * (e & 3))) & 0xffu);
    return static_cast<float>(q) * inv;
  } else {
    const uint32_t w = e < 2 ? c.x : e < 4 ? c.y : e < 6 ? c.z : c.w;
    const uint32_t b = (e & 1) ? (w >> 16) : (w & 0xffffu);
    return half_to_f32<kRecv == Recv::kFp16>(b);
  }
}

template <Out kOut>
__device__ __forceinline__ void store_out(void* out, size_t elem_offset, const float (&acc)[8]) {
  if constexpr (kOut == Out::kF32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + elem_offset);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = kOut == Out::kBf16 ? f32_to_bf16(acc[2 * d]) : f32_to_f16(acc[2 * d]);
      const uint32_t hi = kOut == Out::kBf16 ? f32_to_bf16(acc[2 * d + 1]) : f32_to_f16(acc[2 * d + 1]);
      w[d] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + elem_offset) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <Recv kRecv, Out kOut, int kMaxK>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(RouteArgs a,
                                                                  const uint8_t* __restrict__ recv,
                                                                  const float* __restrict__ topk_w,
                                                                  void* __restrict__ out) {
  using Chunk = typename ChunkOf<kRecv>::T;
  constexpr int kChunkBytes = ChunkOf<kRecv>::kBytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = uniform(blockIdx.x * kTokensPerBlock + static_cast<int>(threadIdx.x / kWave));
  if (t >= a.bs) return;

  // Wave-uniform prologue: row, weight and inverse scale of every entry.
  const uint8_t* row_ptr[kMaxK];
  float wj[kMaxK];
  float invj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    row_ptr[j] = nullptr;
    wj[j] = 0.0f;
    invj[j] = 1.0f;
    if (j < a.k) {
      const int e = a.topk_idx[t * a.k + j];
      const int slot = a.send_token_idx[t * a.k + j];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(a.num_experts) && slot >= 0) {
        const int64_t row = static_cast<int64_t>(a.recv_base[e / a.epr]) + a.put_offset[e] + slot;
        if (row >= 0 && row < a.cap_rows) {
          row_ptr[j] = recv + row * a.row_bytes;
          wj[j] = topk_w[t * a.k + j];
          if constexpr (kRecv == Recv::kInt8)
            invj[j] = *reinterpret_cast<const float*>(row_ptr[j] + a.scale_off);
        }
      }
    }
  }

  const int chunks = a.hidden >> 3;
  const size_t out_base = static_cast<size_t>(t) * a.hidden;
  for (int c = lane; c < chunks; c += kWave) {
    Chunk raw[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (row_ptr[j] != nullptr)
        raw[j] = *reinterpret_cast<const Chunk*>(row_ptr[j] + static_cast<size_t>(c) * kChunkBytes);
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (row_ptr[j] == nullptr) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = element<kRecv>(raw[j], e, invj[j]);
        const float p = v * wj[j];
        acc[e] = acc[e] + p;
      }
    }
    store_out<kOut>(out, out_base + static_cast<size_t>(c) * 8, acc);
  }
}

template <Recv kRecv, Out kOut>
hipError_t launch_k(const RouteArgs& a, const uint8_t* recv, const float* w, void* out,
                    hipStream_t stream) {
  const dim3 grid((a.bs + kTokensPerBlock - 1) / kTokensPerBlock);
  const dim3 block(kCombineThreads);
  if (a.k <= 4) {
    hipLaunchKernelGGL((combine_kernel<kRecv, kOut, 4>), grid, block, 0, stream, a, recv, w, out);
  } else if (a.k <= 8) {
    hipLaunchKernelGGL((combine_kernel<kRecv, kOut, 8>), grid, block, 0, stream, a, recv, w, out);
  } else {
    hipLaunchKernelGGL((combine_kernel<kRecv, kOut, 32>), grid, block, 0, stream, a, recv, w, out);
  }
  return hipGetLastError();
}

template <Recv kRecv>
hipError_t launch_out(const RouteArgs& a, const uint8_t* recv, const float* w, void* out,
                      Out out_type, hipStream_t stream) {
  switch (out_type) {
    case Out::kBf16: return launch_k<kRecv, Out::kBf16>(a, recv, w, out, stream);
    case Out::kFp16: return launch_k<kRecv, Out::kFp16>(a, recv, w, out, stream);
    case Out::kF32: return launch_k<kRecv, Out::kF32>(a, recv, w, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_combine(const RouteArgs& r, const void* recv_x, Recv recv_type,
                          const float* topk_w, void* out, Out out_type, hipStream_t stream) {
  const uint8_t* recv = static_cast<const uint8_t*>(recv_x);
  switch (recv_type) {
    case Recv::kBf16: return launch_out<Recv::kBf16>(r, recv, topk_w, out, out_type, stream);
    case Recv::kFp16: return launch_out<Recv::kFp16>(r, recv, topk_w, out, out_type, stream);
    case Recv::kInt8: return launch_out<Recv::kInt8>(r, recv, topk_w, out, out_type, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
