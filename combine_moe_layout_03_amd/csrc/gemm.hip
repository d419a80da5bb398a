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
// Tiling (gfx950, wave64, v_mfma_i32_16x16x64_i8): a workgroup of 4 x 2
// waves computes a 256 x 256 tile of one expert's output, each wave a
// 64 x 128 block of 16 x 16 MFMA tiles.  K is walked in stages of 64 bytes
// held in a ring of four LDS buffers (32 KB each), filled straight from
// global memory by the LDS-destination form of the global load (16 bytes per
// lane; lane l of one load writes bytes [16 l, 16 l + 16) of a 1 KB block, at
// the address the wave puts in M0): no register holds the data on the way.
// Each ring buffer is its own LDS array, so the compiler's wait analysis
// tells them apart, and every step issues exactly one stage (past the last
// stage it re-loads the last stage into a buffer that is not read again), so
// the explicit vmcnt waits are the same on every path and the compiler adds
// none of its own.
//
// Schedule (ping-pong): the waves 0-3 and 4-7 (one of each per SIMD)
// alternate between a memory phase (start the loads of stage j + 3 into the
// buffer stage j - 1 used, wait for this wave's loads of stage j + 1, read
// the fragments of stage j into registers) and a compute phase (the stage's
// 32 MFMAs), the two groups half a step apart, with a workgroup barrier
// between phases.  While one wave of a SIMD multiplies, the other issues its
// loads and LDS reads.  The barriers make it safe: a wave reads stage j only
// after a barrier that every wave reached after waiting for its own loads of
// stage j (one memory phase earlier), and refills a buffer only after a
// barrier that every wave reached after its last read of it.  The barrier is
// the plain s_barrier (the fence that __syncthreads adds would wait for
// every load in flight), and scheduling barriers keep the compiler from
// moving work across it.
//
// In LDS a stage row (A rows, then B rows) is 4 pieces of 16 bytes; piece p
// of row r sits at position p ^ ((r / 4) % 4).  A fragment read touches 16
// consecutive rows at one piece, 4 rows to a 256-byte LDS line; that swizzle
// puts them in all 16 16-byte bank groups of the line (no bank conflicts).
// The loads apply it on the global side: lane l of a load fetches the piece
// that belongs at LDS position l.  When k ends inside a stage (a separate
// instance), the pieces past k are loaded from the row's first piece (a
// valid address) and their A fragments are zeroed in registers; that
// instance also runs whole rounds of the ring, the steps past the last
// stage multiplying zeros (it serves every k that is not a multiple of
// four stages).
//
// Tile order: the hardware deals workgroup g to XCD g % 8.  With the column
// tiles in groups of 4, XCD x takes column group x % 4 of every other block
// of 8 row slots (x / 4 picks which), so each XCD's L2 serves an 8 x
// (n_tiles / 4) block of tiles and each row tile is fetched by two XCDs
// rather than all eight (at n_tiles % 4 != 0: row slots in order, column
// tiles innermost).
//
// The counts live on the device and the host does not read them, so the
// launch has ceil(rows / 256) + groups row slots (enough for any counts whose
// total is at most rows: expert g needs at most c_g / 256 + 1 tiles), rounded
// up to the tile order's blocks, times the column tiles.  A workgroup finds
// its expert and first row by a prefix sum over the counts; slots past the
// last tile exit at once.  Rows past an expert's end are loaded from its last
// row and never stored; weight rows past n repeat row n - 1 and are never
// stored.
#include "device_util.h"
#include "launch.h"
#include "gemm.h"

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
#define MOE_LDS __attribute__((address_space(3)))

constexpr int kSK = kGemmStageK;               // bytes of k per stage
constexpr int kPieces = kSK / 16;              // 16-byte pieces of a row per stage
constexpr int kRowsPerLoad = kWave / kPieces;  // stage rows one load instruction fills
constexpr int kSwzRows = 16 / kPieces;         // rows of one 256-byte LDS line
static_assert(kPieces == 4, "the LDS swizzle and the k step are written for 64-byte stages");

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

// s_waitcnt with vmcnt(n) (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_wait(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }
// s_waitcnt with lgkmcnt(0) (vmcnt and expcnt left at their maxima).
constexpr int kLgkmWait0 = 0xc07f;

// Row slots of one launch: enough for any counts, rounded up to whole pairs
// of XCD blocks when the XCD-aware order applies.
int64_t launch_slots(int64_t rows, int32_t groups, int64_t n_tiles) {
  int64_t slots = (rows + kGemmTileM - 1) / kGemmTileM + groups;
  if (n_tiles % kGemmXcdColGroups == 0)
    slots = (slots + 2 * kGemmXcdRows - 1) / (2 * kGemmXcdRows) * (2 * kGemmXcdRows);
  return slots;
}

template <int TM, int TN, int WM, int WN, int NS, bool kTail>
__global__ __launch_bounds__(kWave * WM * WN) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int kWaves = WM * WN;
  constexpr int kWaveM = TM / WM, kWaveN = TN / WN;
  constexpr int kMI = kWaveM / 16, kNI = kWaveN / 16;
  constexpr int kStageBytes = (TM + TN) * kSK;
  constexpr int kLoadsA = TM / kRowsPerLoad / kWaves;  // load instructions per thread and stage
  constexpr int kLoadsB = TN / kRowsPerLoad / kWaves;
  constexpr int kLoads = kLoadsA + kLoadsB;
  static_assert(TM % (kRowsPerLoad * kWaves) == 0 && TN % (kRowsPerLoad * kWaves) == 0,
                "every wave issues whole loads of A and of B");
  static_assert(kWaveM % 16 == 0 && kWaveN % 16 == 0, "wave tile of whole MFMA tiles");
  static_assert(NS == 4, "a ring of four stages");
  static_assert(kWaves == 8, "two groups of four waves, one wave of each per SIMD");
  static_assert((NS - 2) * kLoads < 64, "vmcnt counts the loads in flight");
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[kStageBytes];
  __shared__ TileSlot slot_info;

  const int tid = threadIdx.x, lane = tid % kWave, wave = uniform(tid / kWave);

  // workgroup -> (row slot, column tile)
  const int64_t n_tiles = (a.n + TN - 1) / TN;
  int64_t slot, col_tile;
  if (n_tiles % kGemmXcdColGroups == 0) {
    const int64_t g = blockIdx.x, x = g % 8, l = g / 8;
    const int64_t cols = n_tiles / kGemmXcdColGroups;
    const int64_t per_block = kGemmXcdRows * cols;
    const int64_t b = 2 * (l / per_block) + x / kGemmXcdColGroups;
    const int64_t w = l % per_block;
    slot = b * kGemmXcdRows + w / cols;
    col_tile = (x % kGemmXcdColGroups) * cols + w % cols;
  } else {
    slot = blockIdx.x / n_tiles;
    col_tile = blockIdx.x - slot * n_tiles;
  }

  if (wave == 0) {
    if (lane == 0) slot_info.group = -1;
    find_slot<TM>(a, slot, lane, &slot_info);
  }
  __syncthreads();
  const int group = slot_info.group;
  if (group < 0) return;  // the same for every thread of the workgroup
  const int row0 = slot_info.row0, row_end = slot_info.row_end;
  const int col0 = static_cast<int>(col_tile) * TN;

  // This lane's piece of each of its loads: load q of this wave fills stage
  // rows [kRowsPerLoad * (q * kWaves + wave), + kRowsPerLoad); lane l writes
  // position l % 4 of row l / 4, which holds piece (l % 4) ^ ((row / 4) % 4).
  const int8_t* src_a[kLoadsA];
  const int8_t* src_b[kLoadsB];
  int piece_a[kLoadsA], piece_b[kLoadsB];
#pragma unroll
  for (int q = 0; q < kLoadsA; ++q) {
    const int r = kRowsPerLoad * (q * kWaves + wave) + lane / kPieces;
    const int p = (lane % kPieces) ^ ((r / kSwzRows) & (kPieces - 1));
    const int row = min(row0 + r, row_end - 1);
    piece_a[q] = p;
    src_a[q] = a.a + static_cast<int64_t>(row) * a.a_stride + p * 16;
  }
#pragma unroll
  for (int q = 0; q < kLoadsB; ++q) {
    const int r = kRowsPerLoad * (q * kWaves + wave) + lane / kPieces;
    const int p = (lane % kPieces) ^ ((r / kSwzRows) & (kPieces - 1));
    const int col = min(col0 + r, a.n - 1);
    piece_b[q] = p;
    src_b[q] = a.w + (static_cast<int64_t>(group) * a.n + col) * a.k + p * 16;
  }

  // The loads of stage s into ring buffer `buf` (stages past the last one
  // load the last stage again).
  const int stages = (a.k + kSK - 1) / kSK;
  auto issue = [&](int s, uint8_t* buf) {
    const int k0 = min(s, stages - 1) * kSK;
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) {
      int off = k0;
      if constexpr (kTail) off = (k0 + piece_a[q] * 16 < a.k) ? off : -piece_a[q] * 16;
      const int8_t* src = src_a[q] + off;
      __builtin_amdgcn_global_load_lds(src, (MOE_LDS void*)(buf + (q * kWaves + wave) * kRowsPerLoad * kSK), 16,
                                       0, 0);
    }
#pragma unroll
    for (int q = 0; q < kLoadsB; ++q) {
      int off = k0;
      if constexpr (kTail) off = (k0 + piece_b[q] * 16 < a.k) ? off : -piece_b[q] * 16;
      const int8_t* src = src_b[q] + off;
      __builtin_amdgcn_global_load_lds(src, (MOE_LDS void*)(buf + (TM + (q * kWaves + wave) * kRowsPerLoad) * kSK),
                                       16, 0, 0);
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  // a fragment's 16 rows start at a multiple of 16, so the row's swizzle is the lane's
  const int lane_swz = ((lane % 16) / kSwzRows) & (kPieces - 1);
  const int frag_a = (wm * kWaveM + lane % 16) * kSK;
  const int frag_b = (TM + wn * kWaveN + lane % 16) * kSK;
  i32x4 acc[kMI][kNI];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Step j: the memory phase, a barrier, the compute phase, a barrier.
  auto step = [&](int j, const uint8_t* cur, uint8_t* refill) {
    issue(j + NS - 1, refill);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait((NS - 2) * kLoads));  // this wave's loads of stage j + 1
    const int pos = ((lane / 16) ^ lane_swz) * 16;
    i32x4 af[kMI], bf[kNI];
#pragma unroll
    for (int i = 0; i < kMI; ++i) af[i] = *reinterpret_cast<const i32x4*>(cur + frag_a + i * 16 * kSK + pos);
#pragma unroll
    for (int q = 0; q < kNI; ++q) bf[q] = *reinterpret_cast<const i32x4*>(cur + frag_b + q * 16 * kSK + pos);
    if constexpr (kTail) {
      // this lane's 16 bytes of k in the fragments; past k the A side is zero
      const bool live = j * kSK + (lane / 16) * 16 < a.k;
#pragma unroll
      for (int i = 0; i < kMI; ++i) af[i] = live ? af[i] : i32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);  // the fragments are in registers
    barrier();
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int q = 0; q < kNI; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[q], acc[i][q], 0, 0, 0);
    barrier();
  };
  issue(0, lds0);
  issue(1, lds1);
  issue(2, lds2);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait((NS - 2) * kLoads));  // this wave's loads of stage 0
  barrier();
  const int grp = wave / 4;
  if (grp == 1) barrier();  // the second group runs half a step behind
  // Whole rounds of the ring: without the tail, k is a multiple of NS
  // stages; with it, the steps past the last stage multiply zeros.
  const int rounds = (stages + NS - 1) / NS;
  for (int r = 0; r < rounds; ++r) {
    step(NS * r, lds0, lds3);
    step(NS * r + 1, lds1, lds0);
    step(NS * r + 2, lds2, lds1);
    step(NS * r + 3, lds3, lds2);
  }
  if (grp == 0) barrier();  // every wave passes the same number of barriers
  // no load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));

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

}  // namespace

int64_t grouped_gemm_blocks(int64_t rows, int32_t groups, int32_t n) {
  const int64_t n_tiles = (n + kGemmTileN - 1) / kGemmTileN;
  return launch_slots(rows, groups, n_tiles) * n_tiles;
}

// One case per value of select::gemm_k_tail.
hipError_t launch_grouped_gemm_i8(const GemmArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int64_t blocks = grouped_gemm_blocks(a.rows, a.groups, a.n);
  if (blocks > kGemmMaxBlocks) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kWave * kGemmWavesM * kGemmWavesN);
  if (select::gemm_k_tail(a.k)) {
    grouped_gemm_kernel<kGemmTileM, kGemmTileN, kGemmWavesM, kGemmWavesN, kGemmRing, true>
        <<<grid, block, 0, stream>>>(a);
  } else {
    grouped_gemm_kernel<kGemmTileM, kGemmTileN, kGemmWavesM, kGemmWavesN, kGemmRing, false>
        <<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
