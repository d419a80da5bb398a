// Stage 4, combine ("UMDK/CAM communication acceleration library deep
// analysis v2", section 2.6, moe_combine_normal_zb::ReadBufferAndWeightedSum).
//
// Every output element is the page's sum in entry order j = 0..k-1:
//   acc = +0; acc = acc + v_j * w_j  (v_j = float(row) or float(q) * inv)
// with every multiply and add rounded separately (this file is compiled with
// floating-point contraction off), so the result is bit-identical to the
// sequential binary32 definition.  The sum is rounded half-even to the
// output type (bf16: the hardware v_cvt_pk_bf16_f32 pair conversion) and
// stored with 16-byte stores.  Two kernels, four waves per token in both:
//
// combine_rows_kernel (k <= 8): wave p owns, in every row, the chunks (8
// elements each) lane + 64 (p kC + i), i < kC, and reads the token's rows
// one after another in entry order -- the order it adds in -- with the loads
// of row j + 2 in flight while row j is added into accumulators held in
// registers.  Each wave's share of a row is kC contiguous 512-byte (int8)
// or 1024-byte (16-bit) pieces.  At h = 7168, k = 8 this measured 2-4 us
// faster than reading a slice of all k rows at once, for int8 and bf16 rows.
//
// combine_kernel (k > 8): each wave owns every fourth group of 64 chunks and
// walks its chunks, software-pipelined: the k row loads of the next chunk
// are issued before the current chunk is summed.
#include "device_util.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kCombineThreads = 256;

template <Recv kRecv>
constexpr int elem_bytes() {
  return kRecv == Recv::kInt8 ? 1 : 2;
}

// kElems elements of one row, as 32-bit words.
template <Recv kRecv, int kElems>
struct Chunk {
  static constexpr int kWords = kElems * elem_bytes<kRecv>() / 4;
  uint32_t w[kWords];
};

// Element e of a chunk, widened to binary32 and dequantised (before the weight).
template <Recv kRecv, int kElems>
__device__ __forceinline__ float element(const Chunk<kRecv, kElems>& c, int e, float inv) {
  if constexpr (kRecv == Recv::kInt8) {
    const uint32_t w = c.w[e >> 2];
    const int8_t q = static_cast<int8_t>((w >> (8 * (e & 3))) & 0xffu);
    return static_cast<float>(q) * inv;
  } else {
    const uint32_t w = c.w[e >> 1];
    const uint32_t b = (e & 1) ? (w >> 16) : (w & 0xffffu);
    return half_to_f32<kRecv == Recv::kFp16>(b);
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two binary32 values -> two 16-bit patterns, round half to even.  For bf16
// this is one v_cvt_pk_bf16_f32 (rounds in the default nearest-even mode).
template <Out kOut>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (kOut == Out::kBf16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  } else {
    return f32_to_f16(a) | (f32_to_f16(b) << 16);
  }
}

typedef uint32_t o32x4 __attribute__((ext_vector_type(4)));

template <bool kNt>
__device__ __forceinline__ void put16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  if constexpr (kNt) {
    __builtin_nontemporal_store(o32x4{a, b, c, d}, reinterpret_cast<o32x4*>(p));
  } else {
    *reinterpret_cast<uint4*>(p) = make_uint4(a, b, c, d);
  }
}

template <Out kOut, int kElems, bool kNt>
__device__ __forceinline__ void store_out(void* out, size_t elem_offset, const float (&acc)[kElems]) {
  if constexpr (kOut == Out::kF32) {
    float* p = static_cast<float*>(out) + elem_offset;
#pragma unroll
    for (int q = 0; q < kElems / 4; ++q)
      put16<kNt>(p + 4 * q, __float_as_uint(acc[4 * q]), __float_as_uint(acc[4 * q + 1]),
                 __float_as_uint(acc[4 * q + 2]), __float_as_uint(acc[4 * q + 3]));
  } else {
    uint16_t* p = static_cast<uint16_t*>(out) + elem_offset;
#pragma unroll
    for (int q = 0; q < kElems / 8; ++q)
      put16<kNt>(p + 8 * q, pack2<kOut>(acc[8 * q + 0], acc[8 * q + 1]), pack2<kOut>(acc[8 * q + 2], acc[8 * q + 3]),
                 pack2<kOut>(acc[8 * q + 4], acc[8 * q + 5]), pack2<kOut>(acc[8 * q + 6], acc[8 * q + 7]));
  }
}

// Global-memory pointers: loads through them compile to global_load (vmcnt
// only), which lets the compiler wait for exactly the loads a chunk needs.
#define MOE_GLOBAL __attribute__((address_space(1)))
typedef const MOE_GLOBAL uint8_t* gbytes;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <Recv kRecv, int kElems, bool kNt>
__device__ __forceinline__ void load_chunk(Chunk<kRecv, kElems>& c, gbytes p) {
  constexpr int kWords = Chunk<kRecv, kElems>::kWords;
  if constexpr (kWords == 2) {
    const u32x2 v = kNt ? __builtin_nontemporal_load(reinterpret_cast<const MOE_GLOBAL u32x2*>(p))
                        : *reinterpret_cast<const MOE_GLOBAL u32x2*>(p);
    c.w[0] = v.x;
    c.w[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < kWords / 4; ++q) {
      const u32x4 v = kNt ? __builtin_nontemporal_load(reinterpret_cast<const MOE_GLOBAL u32x4*>(p + 16 * q))
                          : *reinterpret_cast<const MOE_GLOBAL u32x4*>(p + 16 * q);
      c.w[4 * q + 0] = v.x;
      c.w[4 * q + 1] = v.y;
      c.w[4 * q + 2] = v.z;
      c.w[4 * q + 3] = v.w;
    }
  }
}

// The chunk c of all kMaxK rows (entries that are not dispatched point at
// row 0 and are skipped when summing): no branches, so no waits between.
template <Recv kRecv, int kMaxK, int kElems, bool kNt>
__device__ __forceinline__ void load_rows(Chunk<kRecv, kElems> (&raw)[kMaxK], gbytes base,
                                          const int64_t (&row_off)[kMaxK], int c) {
  constexpr int kChunkBytes = kElems * elem_bytes<kRecv>();
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    load_chunk<kRecv, kElems, kNt>(raw[j], base + row_off[j] + static_cast<int64_t>(c) * kChunkBytes);
}

// Weighted sum of one chunk in entry order, then the store.
template <Recv kRecv, Out kOut, int kMaxK, int kElems, bool kNtStore>
__device__ __forceinline__ void fold_and_store(const Chunk<kRecv, kElems> (&raw)[kMaxK],
                                               const bool (&valid)[kMaxK], const float (&wj)[kMaxK],
                                               const float (&invj)[kMaxK], void* out,
                                               size_t elem_offset) {
  float acc[kElems];
#pragma unroll
  for (int e = 0; e < kElems; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (!valid[j]) continue;
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      const float v = element<kRecv, kElems>(raw[j], e, invj[j]);
      const float p = v * wj[j];
      acc[e] = acc[e] + p;
    }
  }
  store_out<kOut, kElems, kNtStore>(out, elem_offset, acc);
}

template <Recv kRecv, Out kOut, int kMaxK, int kElems, int kWpt, bool kNtLoad = false,
          bool kNtStore = false>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(RouteArgs a,
                                                                  const uint8_t* __restrict__ recv,
                                                                  const float* __restrict__ topk_w,
                                                                  void* __restrict__ out) {
  using C = Chunk<kRecv, kElems>;
  constexpr int kTokensPerBlock = kCombineThreads / kWave / kWpt;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(static_cast<int>(threadIdx.x / kWave));
  const int t = uniform(blockIdx.x * kTokensPerBlock + wave / kWpt);
  const int part = wave % kWpt;
  if (t >= a.bs) return;
  const gbytes base = (gbytes)(recv);

  // Wave-uniform prologue: row offset, weight and inverse scale of every
  // entry, resolved one entry per lane and broadcast (see resolve_rows).
  int64_t row_off[kMaxK];
  bool valid[kMaxK];
  int64_t my_off = 0;
  resolve_rows<kMaxK>(a, t, 0, lane, row_off, valid, &my_off);
  const int my_j = min(lane, kMaxK - 1);
  const float my_w = topk_w[min(t * a.k + my_j, a.bs * a.k - 1)];
  float my_inv = 1.0f;
  if constexpr (kRecv == Recv::kInt8)
    my_inv = *reinterpret_cast<const MOE_GLOBAL float*>(base + my_off + a.scale_off);
  float wj[kMaxK];
  float invj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    wj[j] = lane_float(my_w, j);
    invj[j] = lane_float(my_inv, j);
  }

  // Software pipeline over this lane's chunks c, c + S, c + 2S, ...: the k
  // loads of the next chunk are issued before the current one is summed.
  // `iters` counts the rounds in which this wave has at least one chunk (a
  // wave-uniform bound, so no load is issued for a round the wave does not
  // sum); lanes past the row's end inside such a round load its last chunk
  // (clamped index, data unused), so the loads of a round need no branches.
  const int chunks = a.hidden / kElems;
  constexpr int kStride = kWave * kWpt;
  const int first = part * kWave;
  const int iters = chunks > first ? (chunks - first + kStride - 1) / kStride : 0;
  const size_t out_base = static_cast<size_t>(t) * a.hidden;
  int c = lane + first;
  if (iters == 0) return;
  C buf_a[kMaxK], buf_b[kMaxK];
  load_rows<kRecv, kMaxK, kElems, kNtLoad>(buf_a, base, row_off, min(c, chunks - 1));
  for (int it = 0; it < iters; it += 2) {
    if (it + 1 < iters)
      load_rows<kRecv, kMaxK, kElems, kNtLoad>(buf_b, base, row_off, min(c + kStride, chunks - 1));
    if (c < chunks)
      fold_and_store<kRecv, kOut, kMaxK, kElems, kNtStore>(buf_a, valid, wj, invj, out,
                                                 out_base + static_cast<size_t>(c) * kElems);
    c += kStride;
    if (it + 1 >= iters) break;
    if (it + 2 < iters)
      load_rows<kRecv, kMaxK, kElems, kNtLoad>(buf_a, base, row_off, min(c + kStride, chunks - 1));
    if (c < chunks)
      fold_and_store<kRecv, kOut, kMaxK, kElems, kNtStore>(buf_b, valid, wj, invj, out,
                                                 out_base + static_cast<size_t>(c) * kElems);
    c += kStride;
  }
}

// Launch shape (swept at h = 7168, k = 8 with caches flushed, before the
// row-at-a-time kernel took k <= 8): four waves per token, 8-element chunks;
// 16-bit rows are read with non-temporal loads (streamed past the caches),
// int8 rows with ordinary loads.
template <Recv kRecv, Out kOut, int kMaxK>
hipError_t launch_shape(const RouteArgs& a, const uint8_t* recv, const float* w, void* out,
                        hipStream_t stream) {
  constexpr int kWpt = 4;
  constexpr bool kNtLoad = kRecv != Recv::kInt8;
  constexpr int kTokensPerBlock = kCombineThreads / kWave / kWpt;
  const dim3 block(kCombineThreads);
  const dim3 grid((a.bs + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL((combine_kernel<kRecv, kOut, kMaxK, 8, kWpt, kNtLoad, false>), grid, block, 0, stream,
                     a, recv, w, out);
  return hipGetLastError();
}

// k <= kMaxK: the token's rows one at a time (see the file
// header).  Lane j resolves entry j; lanes j >= k take entry k - 1's row (so
// the loads of rows past k re-read a row this wave has just read, from L2)
// but are never added.  Rows are read with no branches around the loads:
// skipping the rows past k with a branch measured 1.4 us slower.
template <Recv kRecv, Out kOut, int kC, int kMaxK>
__global__ __launch_bounds__(kCombineThreads) void combine_rows_kernel(RouteArgs a,
                                                                       const uint8_t* __restrict__ recv,
                                                                       const float* __restrict__ topk_w,
                                                                       void* __restrict__ out) {
  constexpr int kElems = 8;
  constexpr int kChunkBytes = kElems * elem_bytes<kRecv>();
  // Rows are loaded and the output stored non-temporally (streamed past the
  // caches: every row is read once and the output is not read here).  At
  // h = 7168, k = 8 that measured 1.5-2 us faster than ordinary loads and
  // stores for int8 rows at bs 4096, and 24 us at bs 16384; non-temporal
  // loads or stores alone were slower.
  constexpr bool kNt = true;
  constexpr int kD = 2;  // rows in flight ahead of the one being added
  using C = Chunk<kRecv, kElems>;
  const int lane = threadIdx.x & (kWave - 1);
  const int part = uniform(static_cast<int>(threadIdx.x / kWave));
  const int t = blockIdx.x;
  if (t >= a.bs) return;
  const gbytes base = (gbytes)(recv);

  const int k = a.k;
  const int i_e = t * k + min(lane, k - 1);
  const int e = a.topk_idx[i_e];
  const int slot = a.send_token_idx[i_e];
  const float my_w = topk_w[i_e];
  const int ec = min(max(e, 0), a.num_experts - 1);
  const int rank = static_cast<int>((static_cast<uint64_t>(ec) * a.epr_magic) >> 32);
  const int64_t row = static_cast<int64_t>(a.recv_base[rank]) + a.put_offset[ec * a.put_stride] + slot;
  const bool ok = static_cast<unsigned>(e) < static_cast<unsigned>(a.num_experts) && slot >= 0 && row >= 0 &&
                  row < a.cap_rows;
  const int64_t my_off = ok ? row * a.row_bytes : 0;  // not dispatched: row 0, read but not added
  float my_inv = 1.0f;
  if constexpr (kRecv == Recv::kInt8)
    my_inv = *reinterpret_cast<const MOE_GLOBAL float*>(base + my_off + a.scale_off);
  const int off_lo = static_cast<int>(static_cast<uint64_t>(my_off) & 0xffffffffu);
  const int off_hi = static_cast<int>(static_cast<uint64_t>(my_off) >> 32);
  const int addv = (ok && lane < k) ? 1 : 0;
  int64_t row_off[kMaxK];
  bool add[kMaxK];
#pragma unroll
  for (int q = 0; q < kMaxK; ++q) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(off_lo, q));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(off_hi, q));
    row_off[q] = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    add[q] = __builtin_amdgcn_readlane(addv, q) != 0;
  }

  const int chunks = a.hidden / kElems;
  int cidx[kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) cidx[i] = lane + (part * kC + i) * kWave;
  auto load_row = [&](C (&r)[kC], int j) {
#pragma unroll
    for (int i = 0; i < kC; ++i)
      load_chunk<kRecv, kElems, kNt>(r[i], base + row_off[j] + static_cast<int64_t>(min(cidx[i], chunks - 1)) * kChunkBytes);
  };
  float acc[kC][kElems];
#pragma unroll
  for (int i = 0; i < kC; ++i)
#pragma unroll
    for (int q = 0; q < kElems; ++q) acc[i][q] = 0.0f;
  C buf[kD + 1][kC];
#pragma unroll
  for (int j = 0; j < kD && j < kMaxK; ++j) load_row(buf[j], j);
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j + kD < kMaxK) load_row(buf[(j + kD) % (kD + 1)], j + kD);
    if (add[j]) {
      const float w = lane_float(my_w, j);
      const float inv = lane_float(my_inv, j);
#pragma unroll
      for (int i = 0; i < kC; ++i)
#pragma unroll
        for (int q = 0; q < kElems; ++q) {
          const float v = element<kRecv, kElems>(buf[j % (kD + 1)][i], q, inv);
          const float p = v * w;
          acc[i][q] = acc[i][q] + p;
        }
    }
  }
  const size_t out_base = static_cast<size_t>(t) * a.hidden;
#pragma unroll
  for (int i = 0; i < kC; ++i)
    if (cidx[i] < chunks) store_out<kOut, kElems, kNt>(out, out_base + static_cast<size_t>(cidx[i]) * kElems, acc[i]);
}

// One case per entry of select::kCombineRowsChunks: kC chunks per lane, four
// waves, 256 kC chunks of 8 elements per token.
template <Recv kRecv, Out kOut, int kMaxK>
hipError_t launch_rows_c(const RouteArgs& a, const uint8_t* recv, const float* w, void* out,
                         hipStream_t stream) {
#define MOE_ROWS_CASE(C)                                                                                   \
  case C:                                                                                                  \
    hipLaunchKernelGGL((combine_rows_kernel<kRecv, kOut, C, kMaxK>), dim3(a.bs), dim3(kCombineThreads), 0, stream, \
                       a, recv, w, out);                                                                   \
    return hipGetLastError();
  switch (select::combine_rows_chunks(a.hidden)) {
    MOE_ROWS_CASE(1)
    MOE_ROWS_CASE(2)
    MOE_ROWS_CASE(4)
    MOE_ROWS_CASE(8)
  }
#undef MOE_ROWS_CASE
  return hipErrorInvalidValue;
}

// k <= 8: the row-at-a-time kernel for at most 4 or 8 entries (one case per
// entry of select::kCombineRowsMaxK); above: the chunk-parallel kernel.
template <Recv kRecv, Out kOut>
hipError_t launch_k(const RouteArgs& a, const uint8_t* recv, const float* w, void* out,
                    hipStream_t stream) {
  switch (select::combine_rows_max_k(a.k)) {
    case 4: return launch_rows_c<kRecv, kOut, 4>(a, recv, w, out, stream);
    case 8: return launch_rows_c<kRecv, kOut, 8>(a, recv, w, out, stream);
  }
  return launch_shape<kRecv, kOut, 32>(a, recv, w, out, stream);
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
