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
  int32_t n;                   // weight rows per expert (output columns of the plain form)
  int32_t* out;                // [rows][n] (the plain form)
  // The fused form: the SwiGLU epilogue on the accumulators (weights hold 2 sn
  // rows per expert: gate rows 0 .. sn-1, then up rows sn .. 2 sn - 1).
  int32_t sn;                  // activation columns
  const float* weight_scale;   // [groups][2 sn]
  const uint8_t* token_scale;  // float of row m at byte m * ts_stride
  int64_t ts_stride;
  float* act;                  // [rows][sn] activations (workspace)
  uint32_t* amax;              // [rows] largest |activation| of each row, as bits (workspace)
  uint8_t* q_out;              // int8 rows: codes [0, sn), inverse scale at q_scale_off
  int64_t q_row_bytes;
  int32_t q_scale_off;
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
// Workgroups of one launch (row slots x column tiles), plain and fused.
int64_t grouped_gemm_blocks(int64_t rows, int32_t groups, int32_t n);
int64_t grouped_gemm_swiglu_blocks(int64_t rows, int32_t groups, int32_t sn);
hipError_t launch_grouped_gemm_i8(const GemmArgs& a, hipStream_t stream);
// The fused form: clears the row maxima, runs the matmul with the SwiGLU
// epilogue into the workspace, then quantises the owned rows.
hipError_t launch_grouped_gemm_swiglu_quant(const GemmArgs& a, hipStream_t stream);

}  // namespace moe
