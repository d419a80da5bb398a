// Which compiled instance of each kernel a call runs: plain C++ functions of
// the call's sizes, with no HIP types, so that host code other than the
// launchers (a coverage check compiled with the system C++ compiler) can
// evaluate exactly the rules the launchers use.
//
// Every kernel that keeps a token's row in registers is compiled for a fixed
// set of register-array widths; a call takes the narrowest width that holds
// its row.  The tables below are those sets, and each launcher has one case
// per table entry.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {
namespace select {

constexpr int kLanes = 64;     // lanes of a wave
constexpr int kChunkElems = 8;  // 16-bit elements per 16-byte chunk

template <size_t N>
constexpr int first_at_least(const int (&table)[N], int need) {
  for (size_t i = 0; i < N; ++i)
    if (table[i] >= need) return table[i];
  return 0;  // no instance holds it
}

// Chunks of 8 elements per lane when one wave holds a row of `hidden`.
constexpr int chunks_per_lane(int hidden) { return (hidden / kChunkElems + kLanes - 1) / kLanes; }

// ---- layout: (waves, rounds of 64 entries) of a 2048-entry tile ----------
// Up to 512 experts 16 waves of 2 rounds, beyond that 4 waves of 8 rounds
// (the per-wave LDS counters, waves x E ints, must fit).
constexpr int kLayoutBigGroupMaxExperts = 512;
constexpr int layout_waves(int num_experts) { return num_experts <= kLayoutBigGroupMaxExperts ? 16 : 4; }
constexpr int layout_rounds(int num_experts) { return num_experts <= kLayoutBigGroupMaxExperts ? 2 : 8; }
// Tiles of n entries (at least one); a count kernel runs when there are several.
constexpr int64_t layout_num_tiles(int64_t n, int num_experts) {
  const int64_t tile = int64_t(layout_waves(num_experts)) * layout_rounds(num_experts) * kLanes;
  return n <= 0 ? 1 : (n + tile - 1) / tile;
}

// ---- fused layout + notify + dispatch ------------------------------------
constexpr int kFusedVpl[] = {1, 2, 4, 8, 12, 14, 16};
constexpr int kFusedMaxHidden = 16 * kLanes * kChunkElems;  // 8192: the row in registers
constexpr int64_t kFusedMaxEntries = int64_t(1) << 16;       // bs * k: every workgroup counts all ids
// Whether the one kernel applies; otherwise the entry point runs the three stages.
constexpr bool fused_applies(int bs, int hidden, int topk) {
  return bs >= 1 && hidden <= kFusedMaxHidden && int64_t(bs) * topk <= kFusedMaxEntries;
}
constexpr int fused_vpl(int hidden) { return first_at_least(kFusedVpl, chunks_per_lane(hidden)); }

// ---- dispatch: one wave per token ------------------------------------------
constexpr int kDispatchVpl[] = {1, 2, 4, 8, 16, 32};
constexpr int dispatch_vpl(int hidden) { return first_at_least(kDispatchVpl, chunks_per_lane(hidden)); }

// ---- combine ----------------------------------------------------------------
// k <= 8: the row-at-a-time kernel, compiled for at most 4 or 8 entries and
// kC chunks per lane over four waves (256 kC chunks of a row); k > 8: the
// chunk-parallel kernel (any k up to 32, any hidden).
constexpr int kCombineRowsMaxK[] = {4, 8};
constexpr int kCombineRowsChunks[] = {1, 2, 4, 8};
constexpr int kCombineWaves = 4;
constexpr int combine_rows_max_k(int topk) { return first_at_least(kCombineRowsMaxK, topk); }  // 0: k > 8
constexpr int combine_rows_chunks(int hidden) {
  return first_at_least(kCombineRowsChunks,
                        (hidden / kChunkElems + kCombineWaves * kLanes - 1) / (kCombineWaves * kLanes));
}

// ---- expert-side epilogue: (chunks of 4 columns per lane, waves per row) --
// Up to 1024 columns one wave per row with 1, 2 or 4 chunks per lane; up to
// 2048 two waves and up to 4096 four waves per row, 4 chunks per lane.
struct EpilogueShape {
  int max_chunks, it, waves;
};
constexpr EpilogueShape kEpilogueShapes[] = {{64, 1, 1}, {128, 2, 1}, {256, 4, 1}, {512, 4, 2}, {1024, 4, 4}};
constexpr int epilogue_shape_index(int n) {
  for (size_t i = 0; i < sizeof(kEpilogueShapes) / sizeof(kEpilogueShapes[0]); ++i)
    if (n / 4 <= kEpilogueShapes[i].max_chunks) return static_cast<int>(i);
  return -1;
}

// ---- first expert matmul: k is walked in 128-byte LDS stages ----------------
// A k that ends inside a stage runs the instance that masks the tail.
constexpr int kGemmStageK = 128;
constexpr bool gemm_k_tail(int k) { return k % kGemmStageK != 0; }

}  // namespace select
}  // namespace moe
