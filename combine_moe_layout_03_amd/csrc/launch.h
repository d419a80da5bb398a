// Kernel launchers of libmoe_ep.  Arguments are validated by the C entry
// points (api.hip) before any of these is called; each launcher only
// enqueues work on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ep.h"
#include "select.h"

namespace moe {

// ---- layout -------------------------------------------------------------------
// The flat (token, k) entries are cut into tiles of 2048, one workgroup per
// tile; a workgroup's waves each own a contiguous segment of its tile,
// walked in rounds of 64 entries (shape: select::layout_waves/rounds).
struct LayoutShape {
  int waves, rounds;
  int64_t tile() const { return static_cast<int64_t>(waves) * rounds * 64; }
};
inline LayoutShape layout_shape(int64_t num_experts) {
  const int e = static_cast<int>(num_experts);
  return LayoutShape{select::layout_waves(e), select::layout_rounds(e)};
}
inline int64_t layout_num_tiles(int64_t n, int64_t num_experts) {
  return select::layout_num_tiles(n, static_cast<int>(num_experts));
}
// Workspace: per-tile expert counts plus a bad-id count for every tile but
// the last (the last tile's workgroup counts its own entries).
inline size_t layout_workspace_bytes(int64_t n, int64_t num_experts) {
  return static_cast<size_t>(layout_num_tiles(n, num_experts) - 1) *
         static_cast<size_t>(num_experts + 1) * 4u;
}

hipError_t launch_layout(const int32_t* topk_idx, int32_t n, int32_t num_experts, int32_t epr,
                         int32_t ranks, int32_t* token_per_expert, int32_t* token_per_rank,
                         int32_t* send_token_idx, int32_t* bad_count, void* workspace,
                         hipStream_t stream);

// The static layout workspace of moe_layout_no_alloc: its size, and its
// device address on the current device (looked up once per device).
constexpr size_t kLayoutScratchBytes = MOE_NO_ALLOC_SCRATCH_BYTES;
hipError_t layout_scratch_address(void** ptr);

// ---- notify -------------------------------------------------------------------
hipError_t launch_notify(const int32_t* token_per_expert, int32_t epr, int32_t ranks,
                         int32_t* put_offset, int32_t* recv_count, int32_t* recv_base,
                         int32_t* recv_token_per_expert, hipStream_t stream);
hipError_t launch_notify_multi(const int32_t* token_per_expert, int32_t num_src, int32_t epr,
                               int32_t ranks, int32_t* put_offset, int32_t* recv_count,
                               int32_t* recv_base, int32_t* recv_token_per_expert,
                               hipStream_t stream);

// ---- dispatch / combine ---------------------------------------------------------
struct RouteArgs {
  const int32_t* topk_idx;        // [bs, k]
  const int32_t* send_token_idx;  // [bs, k]
  const int32_t* put_offset;      // column of [E][put_stride]: putOffset[e] at put_offset[e * put_stride]
  const int32_t* recv_base;       // [R]
  int32_t bs, hidden, k, epr, num_experts;
  int32_t put_stride;  // number of source ranks (1: a single source)
  int64_t row_bytes;   // bytes per receive row
  int64_t cap_rows;    // rows that fit in the receive buffer
  int32_t scale_off;   // byte offset of the inverse scale in an int8 row
  uint64_t epr_magic;  // ceil(2^32 / epr): e / epr == (e * epr_magic) >> 32 for e < 2^21
};

inline uint64_t div_magic(int32_t d) { return ((uint64_t(1) << 32) + uint64_t(d) - 1) / uint64_t(d); }

enum class Half { kBf16 = 0, kFp16 = 1 };
enum class Recv { kBf16 = 0, kFp16 = 1, kInt8 = 2 };
enum class Out { kBf16 = 0, kFp16 = 1, kF32 = 2 };

hipError_t launch_dispatch(const RouteArgs& r, const void* x, Half x_type, bool quant,
                           void* recv_x, hipStream_t stream);

hipError_t launch_combine(const RouteArgs& r, const void* recv_x, Recv recv_type,
                          const float* topk_w, void* out, Out out_type, hipStream_t stream);

// ---- fused layout + notify + dispatch ------------------------------------------
constexpr int kFusedWaves = 16;                 // waves per workgroup
constexpr int kFusedMaxHidden = select::kFusedMaxHidden;     // row held in registers
constexpr int64_t kFusedMaxEntries = select::kFusedMaxEntries;  // bs * k: every workgroup counts all ids
constexpr size_t kFusedMaxLds = 64 * 1024;
constexpr int kFusedMaxCopiesLog2 = 3;          // up to 8 copies of each LDS histogram

struct FusedArgs {
  const uint16_t* x;
  const int32_t* topk_idx;
  int32_t bs, hidden, k, epr, ranks, num_experts, id_bits;
  int32_t tokens_per_group;  // T: workgroup g owns tokens [g*T, (g+1)*T)
  int32_t ids_aligned16;     // topk_idx is 16-byte aligned
  int32_t copies_log2;       // log2 of the LDS histogram copies
  int32_t* token_per_expert;
  int32_t* token_per_rank;
  int32_t* send_token_idx;
  int32_t* bad_count;
  int32_t* put_offset;
  int32_t* recv_count;
  int32_t* recv_base;
  int32_t* recv_token_per_expert;
  uint8_t* recv;
  int64_t row_bytes, cap_rows;
  int32_t scale_off;
};

// ---- expert-side epilogue: dequantise, SwiGLU, requantise ------------------------
struct EpilogueArgs {
  const int32_t* acc;          // [rows][2n]: gate columns 0..n-1, up columns n..2n-1
  const float* weight_scale;   // [2n]
  const void* token_scale;     // float of row m at byte m * ts_stride
  int64_t rows, ts_stride;
  int32_t n;
  uint8_t* out;                // int8 rows: codes [0, n), inverse scale at scale_off
  int64_t out_row_bytes;
  int32_t scale_off;
};
constexpr int kEpilogueMaxN = MOE_EPILOGUE_MAX_N;

hipError_t launch_deq_swiglu_quant(const EpilogueArgs& a, hipStream_t stream);

size_t fused_lds_bytes(int32_t num_experts, int32_t tokens_per_group, int32_t topk, int32_t copies);
hipError_t launch_fused(const FusedArgs& a, Half x_type, bool quant, int groups, hipStream_t stream);

}  // namespace moe
