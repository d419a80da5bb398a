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

// Cross-lane steps through DPP (the data-parallel-primitives operand form of
// VALU instructions), not through the LDS crossbar: a shift of 1, 2, 4 and
// 8 lanes within each row of 16 lanes (a lane shifted in from outside its
// row reads 0), then row_bcast:15 (the last lane of a row, to every lane of
// the next row; applied to rows 1 and 3) and row_bcast:31 (lane 31 to rows 2
// and 3).  Run as a Hillis-Steele scan these give every lane the combination
// of all lanes up to and including itself.  The whole wave must be active.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <typename Op>
__device__ __forceinline__ int wave_scan_dpp(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false));
  return v;
}

// Largest value over the wave, in every lane (a wave-uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  const int m = wave_scan_dpp(static_cast<int>(v), [](int a, int b) {
    return static_cast<int>(static_cast<uint32_t>(a) > static_cast<uint32_t>(b) ? static_cast<uint32_t>(a)
                                                                                 : static_cast<uint32_t>(b));
  });
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(m, kWave - 1));
}

// Inclusive prefix sum over the lanes of the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  return wave_scan_dpp(v, [](int a, int b) { return a + b; });
}

// A value known to be the same in every lane, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Receive rows of kN (<= 64) consecutive entries j0 .. j0+kN-1 of token t.
// Entry j goes to row recvBase[e / EPR] + putOffset[e] + sendTokenIdx[t, j]
// (putOffset[e] is this source's column of the [E][S] offsets with S
// sources: put_offset[e * put_stride]);
// an entry that is past topk, has an id outside [0, E) or a negative slot,
// or whose row falls outside the buffer, is not dispatched (valid = false,
// offset 0).  Lane j resolves entry j0 + j with vector loads (one load
// instruction per array for all entries, every index clamped into its
// array), and readlane broadcasts the results to wave-uniform registers; so
// the whole resolution costs two rounds of memory latency.  `lane_row_off`
// returns each lane's own offset (for further per-entry gathers).
template <int kN, typename Route>
__device__ __forceinline__ void resolve_rows(const Route& a, int t, int j0, int lane,
                                             int64_t (&row_off)[kN], bool (&valid)[kN],
                                             int64_t* lane_row_off = nullptr) {
  static_assert(kN <= kWave, "one entry per lane");
  const int last = a.bs * a.k - 1;
  const int j = min(lane, kN - 1);
  const int i = min(t * a.k + j0 + j, last);
  const int e = a.topk_idx[i];
  const int slot = a.send_token_idx[i];
  const int ec = min(max(e, 0), a.num_experts - 1);
  const int rank = static_cast<int>((static_cast<uint64_t>(ec) * a.epr_magic) >> 32);
  const int64_t row = static_cast<int64_t>(a.recv_base[rank]) + a.put_offset[ec * a.put_stride] + slot;
  const bool ok = (j0 + j < a.k) && static_cast<unsigned>(e) < static_cast<unsigned>(a.num_experts) &&
                  slot >= 0 && row >= 0 && row < a.cap_rows;
  const int64_t off = ok ? row * a.row_bytes : 0;
  if (lane_row_off != nullptr) *lane_row_off = off;
  const int off_lo = static_cast<int>(static_cast<uint64_t>(off) & 0xffffffffu);
  const int off_hi = static_cast<int>(static_cast<uint64_t>(off) >> 32);
  const int okv = ok ? 1 : 0;
#pragma unroll
  for (int q = 0; q < kN; ++q) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(off_lo, q));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(off_hi, q));
    row_off[q] = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    valid[q] = __builtin_amdgcn_readlane(okv, q) != 0;
  }
}

// A lane's float broadcast from lane q.
__device__ __forceinline__ float lane_float(float v, int q) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), q));
}

}  // namespace moe
