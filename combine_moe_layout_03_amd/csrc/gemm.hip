// First expert matmul of the MoE layer's expert side (GMM1): the dispatched
// int8 receive rows times each expert's int8 weights, summed exactly in
// int32 ("UMDK/CAM communication acceleration library deep analysis v2",
// section 4.3, stage 2, and section 4.6, where the per-expert cumulative
// token counts delimit each expert's rows).
//
// Expert g owns the receive rows [S_g, S_g + c_g), c_g = max(count_g, 0) and
// S_g the sum of the counts before g, cut at `rows`; for those rows
//   out[m][j] = sum over i < k of a[m][i] * w[g][j][i]
// with w stored [groups][n][k].  Every partial sum is bounded by
// k * 2^14 < 2^31, so the int32 accumulation is exact in any order.
//
// Tiling (gfx950, wave64, v_mfma_i32_16x16x64_i8): a workgroup of WM x WN
// waves computes a TM x TN tile of one expert's output; each wave owns a
// (TM/WM) x (TN/WN) block of 16 x 16 MFMA tiles (the library launches
// 128 x 128 tiles of 2 x 2 waves, two workgroups per CU).  K is walked in
// stages of SK = 256 bytes: every thread loads its 16-byte pieces of the
// next stage's A rows and B rows (weight rows, k contiguous) into registers
// while the waves run the current stage's MFMAs out of LDS.  In LDS a row's
// 16-byte pieces are XOR-swizzled by the row index (piece p of row r at
// position p ^ (r % 16)), so the 16 rows one fragment read touches hit 16
// different positions: no bank conflicts (the hardware counter reads zero;
// rows padded to 272 bytes instead conflicted on a third of the LDS cycles).
// A lane's fragment of A and of B takes the same 16 bytes of k (logical
// piece kk / 16 + lane / 16 of the stage), so each product pairs a[m][i]
// with w[g][j][i].
//
// The counts live on the device and the host does not read them, so the
// launch has ceil(rows / TM) + groups row slots (enough for any counts whose
// total is at most rows: expert g needs at most c_g / TM + 1 tiles) times
// the column tiles.  A workgroup finds its expert and first row by a prefix
// sum over the counts; slots past the last tile exit at once.  Rows past an
// expert's end are loaded from its last row and never stored; weight rows
// past n repeat row n - 1 and are never stored.
#include "device_util.h"
#include "launch.h"
#include "gemm.h"

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct TileSlot {
  int32_t group, row0, row_end;
};

__device__ __forceinline__ int64_t wave_scan_i64(int64_t v, int lane) {
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

// Expert and rows of row slot `slot` (one wave; the whole wave active).  The
// lane whose expert holds the slot writes it; `out->group` stays -1 if none.
template <int TM>
__device__ void find_slot(const GemmArgs& a, int64_t slot, int lane, TileSlot* out) {
  int64_t row_base = 0, tile_base = 0;
  for (int g0 = 0; g0 < a.groups; g0 += kWave) {
    const int g = g0 + lane;
    int64_t c = g < a.groups ? a.group_count[g] : 0;
    c = c > 0 ? c : 0;
    const int64_t incl = wave_scan_i64(c, lane);
    const int64_t s = min(row_base + incl - c, a.rows);
    const int64_t e = min(row_base + incl, a.rows);
    const int64_t tiles = (e - s + TM - 1) / TM;
    const int64_t tincl = wave_scan_i64(tiles, lane);
    const int64_t t0 = tile_base + tincl - tiles;
    if (g < a.groups && slot >= t0 && slot < t0 + tiles) {
      out->group = g;
      out->row0 = static_cast<int32_t>(s + (slot - t0) * TM);
      out->row_end = static_cast<int32_t>(e);
    }
    row_base = min(row_base + __shfl(incl, kWave - 1, kWave), a.rows);
    tile_base += __shfl(tincl, kWave - 1, kWave);
    if (tile_base > slot) break;
  }
}

template <int TM, int TN, int WM, int WN, int SK, int kDepth>
__global__ __launch_bounds__(kWave * WM * WN) void grouped_gemm_kernel(GemmArgs a) {
  static_assert(kDepth == 1 || kDepth == 2, "stages held in registers ahead of the LDS stage");
  constexpr int kStageK = SK;              // bytes of k per stage
  constexpr int kPieces = kStageK / 16;    // 16-byte pieces of a row per stage
  // LDS rows are kStageK bytes apart; the 16-byte piece p of tile row r
  // sits at position p ^ (r % kPieces) of its row
  constexpr bool kSwizzle = true;
  constexpr int kLdsPitch = kStageK + (kSwizzle ? 0 : 16);
  constexpr int kSwz = kSwizzle ? kPieces - 1 : 0;
  static_assert(kPieces <= 16, "a fragment's 16 rows cover every swizzle position");
  constexpr int kThreads = kWave * WM * WN;
  constexpr int kWaveM = TM / WM, kWaveN = TN / WN;
  constexpr int kMI = kWaveM / 16, kNI = kWaveN / 16;
  constexpr int kRowsPerPass = kThreads / kPieces;  // tile rows one load pass covers
  constexpr int kAPasses = TM / kRowsPerPass, kBPasses = TN / kRowsPerPass;
  static_assert(kWaveM % 16 == 0 && kWaveN % 16 == 0, "wave tile of whole MFMA tiles");
  static_assert(kThreads % kPieces == 0 && TM % kRowsPerPass == 0 && TN % kRowsPerPass == 0,
                "load passes cover the tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[TM * kLdsPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[TN * kLdsPitch];
  __shared__ TileSlot slot_info;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  // workgroup -> (row slot, column tile), column tiles innermost.  The
  // hardware deals consecutive workgroups round-robin to the 8 XCDs, so with
  // 32 column tiles each XCD holds the same 4 column tiles of every row slot
  // it runs: their weight rows (4 x 0.9 MB at k = 7168) stay in its L2 while
  // the whole GPU works through one expert's row slots.  (A contiguous range
  // of the order per XCD, or bands of several row slots, measured 6-15 %
  // slower at the benchmark shape.)
  const int64_t n_tiles = (a.n + TN - 1) / TN;
  const int64_t slot = blockIdx.x / n_tiles;
  const int64_t col_tile = blockIdx.x - slot * n_tiles;

  if (wave == 0) {
    if (lane == 0) slot_info.group = -1;
    find_slot<TM>(a, slot, lane, &slot_info);
  }
  __syncthreads();
  const int group = slot_info.group;
  if (group < 0) return;  // the same for every thread of the workgroup
  const int row0 = slot_info.row0, row_end = slot_info.row_end;
  const int col0 = static_cast<int>(col_tile) * TN;

  // this thread's 16-byte pieces: piece `piece` of tile rows r0 + p * kRowsPerPass
  const int piece = tid % kPieces, r0 = tid / kPieces;
  const int8_t* a_src[kAPasses];
  const int8_t* b_src[kBPasses];
#pragma unroll
  for (int p = 0; p < kAPasses; ++p) {
    const int row = min(row0 + r0 + p * kRowsPerPass, row_end - 1);
    a_src[p] = a.a + static_cast<int64_t>(row) * a.a_stride + piece * 16;
  }
#pragma unroll
  for (int p = 0; p < kBPasses; ++p) {
    const int col = min(col0 + r0 + p * kRowsPerPass, a.n - 1);
    b_src[p] = a.w + (static_cast<int64_t>(group) * a.n + col) * a.k + piece * 16;
  }

  using ARegs = i32x4[kAPasses];
  using BRegs = i32x4[kBPasses];
  auto load_stage = [&](int k0, ARegs& ra, BRegs& rb) {
    if (k0 + piece * 16 < a.k) {
#pragma unroll
      for (int p = 0; p < kAPasses; ++p) ra[p] = *reinterpret_cast<const i32x4*>(a_src[p] + k0);
#pragma unroll
      for (int p = 0; p < kBPasses; ++p) rb[p] = *reinterpret_cast<const i32x4*>(b_src[p] + k0);
    } else {
#pragma unroll
      for (int p = 0; p < kAPasses; ++p) ra[p] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < kBPasses; ++p) rb[p] = i32x4{0, 0, 0, 0};
    }
  };
  auto store_stage = [&](const ARegs& ra, const BRegs& rb) {
#pragma unroll
    for (int p = 0; p < kAPasses; ++p) {
      const int r = r0 + p * kRowsPerPass;
      *reinterpret_cast<i32x4*>(lds_a + r * kLdsPitch + ((piece ^ (r & kSwz)) * 16)) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < kBPasses; ++p) {
      const int r = r0 + p * kRowsPerPass;
      *reinterpret_cast<i32x4*>(lds_b + r * kLdsPitch + ((piece ^ (r & kSwz)) * 16)) = rb[p];
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  // a fragment's rows are 16-aligned, so row % kPieces is lane % kPieces
  const uint8_t* fa = lds_a + (wm * kWaveM + lane % 16) * kLdsPitch;
  const uint8_t* fb = lds_b + (wn * kWaveN + lane % 16) * kLdsPitch;
  const int lane_swz = lane & kSwz;
  i32x4 acc[kMI][kNI];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  auto compute_stage = [&]() {
#pragma unroll
    for (int kk = 0; kk < kStageK; kk += 64) {
      const int pos = ((kk / 16 + lane / 16) ^ lane_swz) * 16;
      i32x4 af[kMI], bf[kNI];
#pragma unroll
      for (int i = 0; i < kMI; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(fa + i * 16 * kLdsPitch + pos);
#pragma unroll
      for (int j = 0; j < kNI; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(fb + j * 16 * kLdsPitch + pos);
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // One LDS stage; the next kDepth stages are in flight into registers while
  // it is computed.  The barrier before a store waits for every wave to be
  // done reading the stage it replaces.
  const int stages = (a.k + kStageK - 1) / kStageK;
  ARegs ra0, ra1;
  BRegs rb0, rb1;
  load_stage(0, ra0, rb0);
  if (kDepth == 1) {
    for (int s = 0; s < stages; ++s) {
      if (s) __syncthreads();
      store_stage(ra0, rb0);
      __syncthreads();
      if (s + 1 < stages) load_stage((s + 1) * kStageK, ra0, rb0);
      compute_stage();
    }
  } else {
    if (stages > 1) load_stage(kStageK, ra1, rb1);
    for (int s = 0; s < stages; s += 2) {
      if (s) __syncthreads();
      store_stage(ra0, rb0);
      __syncthreads();
      if (s + 2 < stages) load_stage((s + 2) * kStageK, ra0, rb0);
      compute_stage();
      if (s + 1 < stages) {
        __syncthreads();
        store_stage(ra1, rb1);
        __syncthreads();
        if (s + 3 < stages) load_stage((s + 3) * kStageK, ra1, rb1);
        compute_stage();
      }
    }
  }

  // 16 x 16 result tile: lane l holds column l % 16 of rows 4 * (l / 16) + 0..3
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
#pragma unroll
    for (int j = 0; j < kNI; ++j) {
      const int col = col0 + wn * kWaveN + j * 16 + lane % 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wm * kWaveM + i * 16 + (lane / 16) * 4 + r;
        if (row < row_end && col < a.n) a.out[static_cast<int64_t>(row) * a.n + col] = acc[i][j][r];
      }
    }
  }
}

template <int TM, int TN, int WM, int WN, int SK, int kDepth>
hipError_t launch_shape(const GemmArgs& a, hipStream_t stream) {
  const int64_t slots = (a.rows + TM - 1) / TM + a.groups;
  const int64_t n_tiles = (a.n + TN - 1) / TN;
  const int64_t blocks = slots * n_tiles;
  if (blocks > kGemmMaxBlocks) return hipErrorInvalidValue;
  grouped_gemm_kernel<TM, TN, WM, WN, SK, kDepth>
      <<<dim3(static_cast<uint32_t>(blocks)), dim3(kWave * WM * WN), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

int64_t grouped_gemm_blocks(int64_t rows, int32_t groups, int32_t n) {
  return ((rows + kGemmTileM - 1) / kGemmTileM + groups) * ((n + kGemmTileN - 1) / kGemmTileN);
}

hipError_t launch_grouped_gemm_i8(const GemmArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  return launch_shape<kGemmTileM, kGemmTileN, 2, 2, 256, 1>(a, stream);
}

}  // namespace moe
