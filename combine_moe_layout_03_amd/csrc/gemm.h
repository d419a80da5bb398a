// Launcher of the first expert matmul (int8 x int8 -> int32 over per-expert
// row ranges).  Arguments are validated by moe_grouped_gemm_i8 (api.hip)
// before the launcher is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "select.h"

namespace moe {

struct GemmArgs {
  const int8_t* a;             // receive rows: row m at a + m * a_stride, k int8 codes
  int64_t a_stride;            // bytes between rows (a multiple of 16)
  int64_t rows;                // rows of a and of out
  int32_t k;                   // a multiple of 16
  const int32_t* group_count;  // [groups]: rows of each expert, in order
  int32_t groups;
  const int8_t* w;             // [groups][n][k]
  int32_t n;
  int32_t* out;                // [rows][n]
};
// Workgroup tile (rows x output columns), its waves, the LDS slots, and the
// XCD-aware tile order (see gemm.hip).
constexpr int kGemmTileM = 256, kGemmTileN = 256;
constexpr int kGemmWavesM = 4, kGemmWavesN = 2;
constexpr int kGemmStageK = select::kGemmStageK;  // bytes of k per LDS stage
constexpr int kGemmSlotsA = 2, kGemmSlotsB = 3;    // LDS slots of a stage's A and B rows
constexpr int kGemmXcdColGroups = 4;               // column groups of the tile order
constexpr int kGemmXcdRows = 8;                    // row slots per XCD block
constexpr int64_t kGemmMaxBlocks = int64_t(1) << 24;
// Workgroups of one launch (row slots x column tiles).
int64_t grouped_gemm_blocks(int64_t rows, int32_t groups, int32_t n);
hipError_t launch_grouped_gemm_i8(const GemmArgs& a, hipStream_t stream);

}  // namespace moe
