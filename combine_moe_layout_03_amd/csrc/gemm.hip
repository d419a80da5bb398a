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
// 64 x 128 block of 16 x 16 MFMA tiles.  K is walked in stages of 128 bytes:
// the A rows of a stage (32 KB) go to one of two LDS slots, its B rows
// (32 KB) to one of three, filled straight from global memory by the
// LDS-destination form of the global load (16 bytes per lane; lane l of one
// load writes bytes [16 l, 16 l + 16) of a 1 KB block, at the address the
// wave puts in M0): no register holds the data on the way, and every load
// covers 8 rows x 128 bytes, whole cache lines (loads of half lines move
// about half as many bytes per CU and cycle).  Each slot is its own LDS
// array, so the compiler's wait analysis tells them apart, and every step
// issues the same loads (past the last stage it re-loads the last stage
// into a slot that is not read again), so the explicit vmcnt waits are the
// same on every path and the compiler adds none of its own.
//
// Schedule (ping-pong): the waves 0-3 and 4-7 (one of each per SIMD) run
// half a step apart and alternate, between workgroup barriers, a memory
// phase (fragment reads into registers) and a compute phase (32 MFMAs).  A
// stage is consumed in two such steps, k bytes [0, 64) and [64, 128) of its
// rows.  The memory phase of the first step of stage S starts the loads of
// A(S + 1), into the slot A(S - 1) used; that of the second step starts the
// loads of B(S + 2), into the slot B(S - 1) used, and then waits for this
// wave's loads of A(S + 1) and B(S + 1).  (Issuing all of a stage's loads in
// one memory phase was 8 % slower.)  While one wave of a SIMD multiplies,
// the other reads and loads.  The barriers
// make it safe: a wave reads a stage only after a barrier that every wave
// reached after waiting for its own loads of it, and refills a slot only
// after a barrier that every wave reached after its last read of it.  The
// barrier is the plain s_barrier (the fence that __syncthreads adds would
// wait for every load in flight), and scheduling barriers keep the compiler
// from moving work across it.  The five slots fill the 160 KB of LDS, so
// the tile's slot record lives in the third B slot until its first load.
//
// In LDS a stage row is 8 pieces of 16 bytes; piece p of row r sits at
// position p ^ ((r / 2) % 8).  A fragment read touches 16 consecutive rows
// at one piece, 2 rows to a 256-byte LDS line; that swizzle puts them in all
// 16 16-byte bank groups of the 8 lines (no bank conflicts).  The loads
// apply it on the global side: lane l of a load fetches the piece that
// belongs at LDS position l.  When k ends inside a stage (a separate
// instance), the pieces past k are loaded from the row's first piece (a
// valid address) and their A fragments are zeroed in registers.
//
// Tile order: the hardware deals workgroup g to XCD g % 8.  With the column
// tiles in groups of 4, XCD x takes column group x % 4 of every other block
// of 8 row slots (x / 4 picks which), so each XCD's L2 serves an 8 x
// (n_tiles / 4) block of tiles: each row tile is fetched by four XCDs and
// each weight column tile by two, rather than all eight (at n_tiles % 4 !=
// 0: row slots in order, column tiles innermost).
//
// The fused form (section 4.8.1: GMM1 with its PerTokenDequantSwiGLU
// epilogue on the accumulators) reads each expert's weights as 2 sn rows,
// gate rows then up rows; its column tile j covers gate rows [128 j, 128 j +
// 128) and the up rows sn above them, so the waves wn = 0 hold gate sums and
// wn = 1 the up sums of the same rows and activation columns.  After the k
// loop the two waves of a pair swap half their sums through LDS, compute the
// activations of their rows with the epilogue kernel's arithmetic (swiglu.h),
// store them as floats to the caller's workspace and fold each row's largest
// magnitude into a per-row word with an atomic max (an integer max of the
// sign-cleared bit patterns, exact in any order).  A second kernel then
// quantises every owned row from its maximum exactly as the epilogue kernel
// does.  The activation arithmetic is bound by the vector ALU; here it runs
// while the matrix cores wait, which is why the two separate calls are the
// faster path at the benchmarked shape (the fused one needs half the
// intermediate memory).
//
// The counts live on the device and the host does not read them, so the
// launch has ceil(rows / 256) + groups row slots (enough for any counts whose
// total is at most rows: expert g needs at most c_g / 256 + 1 tiles), rounded
// up to the tile order's blocks, times the column tiles.  A workgroup finds
// its expert and first row by a prefix sum over the counts; slots past the
// last tile exit at once.  Rows past an expert's end are loaded from its last
// row and never stored; weight rows past n repeat row n - 1 and are never
// stored.
#include <type_traits>

#include "device_util.h"
#include "launch.h"
#include "gemm.h"
#include "quant.h"
#include "swiglu.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define MOE_LDS __attribute__((address_space(3)))

constexpr int kSK = kGemmStageK;               // bytes of k per stage
constexpr int kPieces = kSK / 16;              // 16-byte pieces of a row per stage
constexpr int kRowsPerLoad = kWave / kPieces;  // stage rows one load instruction fills
constexpr int kSwzRows = 16 / kPieces;         // rows of one 256-byte LDS line
static_assert(kPieces == 8, "the LDS swizzle and the two k steps are written for 128-byte stages");

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

template <int TM, int TN, int WM, int WN, bool kTail, bool kFused>
__global__ __launch_bounds__(kWave * WM * WN) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int kWaves = WM * WN;
  constexpr int kWaveM = TM / WM, kWaveN = TN / WN;
  constexpr int kMI = kWaveM / 16, kNI = kWaveN / 16;
  constexpr int kLoadsA = TM / kRowsPerLoad / kWaves;  // load instructions per thread and stage
  constexpr int kLoadsB = TN / kRowsPerLoad / kWaves;
  static_assert(TM % (kRowsPerLoad * kWaves) == 0 && TN % (kRowsPerLoad * kWaves) == 0,
                "every wave issues whole loads of A and of B");
  static_assert(kWaveM % 16 == 0 && kWaveN % 16 == 0, "wave tile of whole MFMA tiles");
  static_assert(kWaves == 8, "two groups of four waves, one wave of each per SIMD");
  static_assert(kGemmSlotsA == 2 && kGemmSlotsB == 3, "the slot rotation below");
  static_assert(kLoadsA + 2 * kLoadsB < 64, "vmcnt counts the loads in flight");
  static_assert(sizeof(TileSlot) <= TN * kSK, "the slot record fits in a B slot");
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[TM * kSK];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[TM * kSK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[TN * kSK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[TN * kSK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb2[TN * kSK];
  // read by every wave before the workgroup barrier that precedes sb2's first load
  TileSlot& slot_info = *reinterpret_cast<TileSlot*>(sb2);

  const int tid = threadIdx.x, lane = tid % kWave, wave = uniform(tid / kWave);

  // workgroup -> (row slot, column tile)
  // The fused form's column tile j covers gate rows [j TN/2, (j+1) TN/2) of
  // the weights and the up rows sn above them.
  const int64_t n_tiles = kFused ? (a.sn + TN / 2 - 1) / (TN / 2) : (a.n + TN - 1) / TN;
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
  // position l % 8 of row l / 8, which holds piece (l % 8) ^ ((row / 2) % 8).
  // The first row of every load of a wave is the same modulo 16, so the
  // piece is the same for all of them.
  static_assert(kRowsPerLoad * kWaves % (kSwzRows * kPieces) == 0, "one piece per lane for all loads");
  const int piece = (lane % kPieces) ^ (((kRowsPerLoad * wave + lane / kPieces) / kSwzRows) & (kPieces - 1));
  const int8_t* src_a[kLoadsA];
  const int8_t* src_b[kLoadsB];
#pragma unroll
  for (int q = 0; q < kLoadsA; ++q) {
    const int r = kRowsPerLoad * (q * kWaves + wave) + lane / kPieces;
    const int row = min(row0 + r, row_end - 1);
    src_a[q] = a.a + static_cast<int64_t>(row) * a.a_stride + piece * 16;
  }
#pragma unroll
  for (int q = 0; q < kLoadsB; ++q) {
    const int r = kRowsPerLoad * (q * kWaves + wave) + lane / kPieces;
    int col = min(col0 + r, a.n - 1);
    if constexpr (kFused) {
      const int j = static_cast<int>(col_tile) * (TN / 2) + r % (TN / 2);
      col = (r < TN / 2 ? 0 : a.sn) + min(j, a.sn - 1);
    }
    src_b[q] = a.w + (static_cast<int64_t>(group) * a.n + col) * a.k + piece * 16;
  }
  const int stages = (a.k + kSK - 1) / kSK;
  // Byte offset of stage s in every source row; where this lane's piece of
  // the stage lies past k it reads the row's first piece instead.
  auto stage_offset = [&](int s) {
    const int k0 = min(s, stages - 1) * kSK;
    if constexpr (kTail) return (k0 + piece * 16 < a.k) ? k0 : -piece * 16;
    return k0;
  };

  // The loads of stage s's A rows (B rows) into slot `buf` (stages past the
  // last one load the last stage again).
  auto issue_a = [&](int s, uint8_t* buf) {
    const int off = stage_offset(s);
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) {
      const int8_t* src = src_a[q] + off;
      __builtin_amdgcn_global_load_lds(src, (MOE_LDS void*)(buf + (q * kWaves + wave) * kRowsPerLoad * kSK), 16,
                                       0, 0);
    }
  };
  auto issue_b = [&](int s, uint8_t* buf) {
    const int off = stage_offset(s);
#pragma unroll
    for (int q = 0; q < kLoadsB; ++q) {
      const int8_t* src = src_b[q] + off;
      __builtin_amdgcn_global_load_lds(src, (MOE_LDS void*)(buf + (q * kWaves + wave) * kRowsPerLoad * kSK), 16,
                                       0, 0);
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  // a fragment's 16 rows start at a multiple of 16, so the row's swizzle is the lane's
  const int lane_swz = ((lane % 16) / kSwzRows) & (kPieces - 1);
  const int frag_a = (wm * kWaveM + lane % 16) * kSK;
  const int frag_b = (wn * kWaveN + lane % 16) * kSK;
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
  // Step h (k bytes [64 h, 64 h + 64)) of stage S, its A rows in `ca` and B
  // rows in `cb`: the memory phase, a barrier, the compute phase, a barrier.
  auto step = [&](int S, int h, const uint8_t* ca, const uint8_t* cb, uint8_t* fill_a, uint8_t* fill_b) {
    if (h == 0) issue_a(S + 1, fill_a);  // into the slot A(S - 1) used
    else issue_b(S + 2, fill_b);         // into the slot B(S - 1) used
    const int pos = ((4 * h + lane / 16) ^ lane_swz) * 16;
    i32x4 af[kMI], bf[kNI];
#pragma unroll
    for (int i = 0; i < kMI; ++i) af[i] = *reinterpret_cast<const i32x4*>(ca + frag_a + i * 16 * kSK + pos);
#pragma unroll
    for (int q = 0; q < kNI; ++q) bf[q] = *reinterpret_cast<const i32x4*>(cb + frag_b + q * 16 * kSK + pos);
    if constexpr (kTail) {
      // this lane's 16 bytes of k in the fragments; past k the A side is zero
      const int keep = S * kSK + h * 64 + (lane / 16) * 16 < a.k ? -1 : 0;
#pragma unroll
      for (int i = 0; i < kMI; ++i) af[i] &= keep;
    }
    // this wave's loads of A(S + 1) and B(S + 1); those of B(S + 2) may still run
    if (h == 1) __builtin_amdgcn_s_waitcnt(vmcnt_wait(kLoadsB));
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);  // the fragments are in registers
    barrier();
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int q = 0; q < kNI; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[q], acc[i][q], 0, 0, 0);
    barrier();
  };
  // Stage S: A in sa[S % 2] (refilling sa[(S + 1) % 2]), B in sb[S % 3]
  // (refilling sb[(S + 2) % 3]).
  auto stage = [&](int S, const uint8_t* ca, const uint8_t* cb, uint8_t* fill_a, uint8_t* fill_b) {
    step(S, 0, ca, cb, fill_a, fill_b);
    step(S, 1, ca, cb, fill_a, fill_b);
  };
  issue_b(0, sb0);
  issue_a(0, sa0);
  issue_b(1, sb1);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(kLoadsB));  // this wave's loads of stage 0
  barrier();
  const int grp = wave / 4;
  if (grp == 1) barrier();  // the second group runs half a step behind
  // Whole rounds of the rotation (its period is six stages), then the rest.
  const int rounds = stages / 6;
  for (int r = 0; r < rounds; ++r) {
    stage(6 * r, sa0, sb0, sa1, sb2);
    stage(6 * r + 1, sa1, sb1, sa0, sb0);
    stage(6 * r + 2, sa0, sb2, sa1, sb1);
    stage(6 * r + 3, sa1, sb0, sa0, sb2);
    stage(6 * r + 4, sa0, sb1, sa1, sb0);
    stage(6 * r + 5, sa1, sb2, sa0, sb1);
  }
  {
    const int rest = stages - rounds * 6;
    if (rest > 0) stage(6 * rounds, sa0, sb0, sa1, sb2);
    if (rest > 1) stage(6 * rounds + 1, sa1, sb1, sa0, sb0);
    if (rest > 2) stage(6 * rounds + 2, sa0, sb2, sa1, sb1);
    if (rest > 3) stage(6 * rounds + 3, sa1, sb0, sa0, sb2);
    if (rest > 4) stage(6 * rounds + 4, sa0, sb1, sa1, sb0);
  }
  if (grp == 0) barrier();  // every wave passes the same number of barriers
  // no load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));

  // 16 x 16 result tile: lane l holds column l % 16 of rows 4 * (l / 16) + 0..3
  if constexpr (!kFused) {
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
  } else {
    // The waves wn = 0 hold gate sums and wn = 1 the up sums of the same
    // rows and activation columns.  Each wave of such a pair (wave ^ 1)
    // finishes half the pair's row tiles: it hands the other half of its
    // sums to its partner through LDS (free once every wave is past this
    // barrier), then computes the activations of its rows, folds their
    // magnitudes into the rows' maxima and stores them.
    static_assert(WN == 2 && kMI % 2 == 0, "gate and up halves of a pair of waves");
    constexpr int kHalf = kMI / 2;
    static_assert(2 * kHalf * kNI * kWave * 16 <= TM * kSK, "a pair's exchange fits in one slot");
    // the scales first, so their loads overlap the exchange below
    const int j_base = static_cast<int>(col_tile) * (TN / 2) + lane % 16;
    const float* ws = a.weight_scale + static_cast<int64_t>(group) * 2 * a.sn;
    float wg[kNI], wu[kNI];
#pragma unroll
    for (int j = 0; j < kNI; ++j) {
      const int jo = min(j_base + j * 16, a.sn - 1);
      wg[j] = ws[jo];
      wu[j] = ws[a.sn + jo];
    }
    const int row_base = row0 + wm * kWaveM + wn * kHalf * 16 + (lane / 16) * 4;  // this wave's first row
    float ts[kHalf][4];
#pragma unroll
    for (int ii = 0; ii < kHalf; ++ii)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rs = min(row_base + ii * 16 + r, row_end - 1);
        ts[ii][r] = *reinterpret_cast<const float*>(a.token_scale + static_cast<int64_t>(rs) * a.ts_stride);
      }
    barrier();
    uint8_t* const pool = wave < 2 ? sa0 : wave < 4 ? sa1 : wave < 6 ? sb0 : sb1;
    uint8_t* const mine = pool + (wave % 2) * (kHalf * kNI * kWave * 16);
    const uint8_t* const theirs = pool + ((wave % 2) ^ 1) * (kHalf * kNI * kWave * 16);
    // kKeep: the first row tile this wave finishes (0 for the gate wave); a
    // compile-time index, so the accumulators stay in registers
    auto finish = [&](auto keep_c) {
      constexpr int kKeep = decltype(keep_c)::value;
      constexpr int kGive = kHalf - kKeep;
#pragma unroll
      for (int ii = 0; ii < kHalf; ++ii)
#pragma unroll
        for (int j = 0; j < kNI; ++j)
          *reinterpret_cast<i32x4*>(mine + ((ii * kNI + j) * kWave + lane) * 16) = acc[kGive + ii][j];
      barrier();
#pragma unroll
      for (int ii = 0; ii < kHalf; ++ii) {
        float y[kNI][4];
#pragma unroll
        for (int j = 0; j < kNI; ++j) {
          const i32x4 other = *reinterpret_cast<const i32x4*>(theirs + ((ii * kNI + j) * kWave + lane) * 16);
          const i32x4 gate = kKeep == 0 ? acc[kKeep + ii][j] : other;
          const i32x4 up = kKeep == 0 ? other : acc[kKeep + ii][j];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[j][r] = swiglu(gate[r], up[r], wg[j], wu[j], ts[ii][r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row_base + ii * 16 + r;
          uint32_t mag = 0;
#pragma unroll
          for (int j = 0; j < kNI; ++j) {
            const int jo = j_base + j * 16;
            const uint32_t b = jo < a.sn ? __float_as_uint(y[j][r]) & 0x7fffffffu : 0u;  // |y| orders as an integer
            mag = mag > b ? mag : b;
          }
          // the row's maximum over its 16 lanes (the tile's columns), then
          // over the launch's column tiles through the global maximum
#pragma unroll
          for (int d = 1; d < 16; d <<= 1) {
            const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(mag), d, kWave));
            mag = mag > o ? mag : o;
          }
          if (row < row_end) {
            if (lane % 16 == 0) atomicMax(a.amax + row, mag);
            float* dst = a.act + static_cast<int64_t>(row) * a.sn;
#pragma unroll
            for (int j = 0; j < kNI; ++j)
              if (j_base + j * 16 < a.sn) dst[j_base + j * 16] = y[j][r];
          }
        }
      }
    };
    if (wn == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, kHalf>{});
  }
}

// Clears the row maxima of the fused form.
__global__ __launch_bounds__(256) void clear_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0;
}

// Quantises the activations of the rows an expert owns, one wave per row,
// exactly as the epilogue kernel quantises a row: s = 127 / (max|a| +
// 1e-12f), codes rint(a * s), inverse scale 1 / s.  Rows past the owned
// total are not written.
constexpr int kQuantRows = 4;  // waves (rows) per workgroup
__global__ __launch_bounds__(kWave * kQuantRows) void act_quant_kernel(GemmArgs a) {
  const int lane = threadIdx.x % kWave, wave = uniform(static_cast<int>(threadIdx.x / kWave));
  // the counts' total in 64 bits, as the matmul finds its rows (the counts
  // are the caller's, and several near 2^31 would wrap a 32-bit sum)
  int64_t owned = 0;
  for (int g0 = 0; g0 < a.groups; g0 += kWave) {
    const int g = g0 + lane;
    const int64_t c = g < a.groups ? max(a.group_count[g], 0) : 0;
    owned += __shfl(wave_scan_i64(c, lane), kWave - 1, kWave);
    if (owned >= a.rows) break;
  }
  owned = min(owned, a.rows);
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kQuantRows + wave;
  if (m >= owned) return;
  const float amax = __uint_as_float(a.amax[m]);
  const float s = 127.0f / (amax + 1e-12f);
  const float inv = 1.0f / s;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.act + m * a.sn);
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.q_out + m * a.q_row_bytes);
  for (int c = lane; c < a.sn / 4; c += kWave) {
    const f32x4 v = __builtin_nontemporal_load(src + c);
    const uint32_t b0 = code_bits(v[0], s) & 0xffu;
    const uint32_t b1 = code_bits(v[1], s) & 0xffu;
    const uint32_t b2 = code_bits(v[2], s) & 0xffu;
    const uint32_t b3 = code_bits(v[3], s);
    dst[c] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  if (lane == 0) *reinterpret_cast<float*>(a.q_out + m * a.q_row_bytes + a.q_scale_off) = inv;
}

}  // namespace

int64_t grouped_gemm_blocks(int64_t rows, int32_t groups, int32_t n) {
  const int64_t n_tiles = (n + kGemmTileN - 1) / kGemmTileN;
  return launch_slots(rows, groups, n_tiles) * n_tiles;
}

int64_t grouped_gemm_swiglu_blocks(int64_t rows, int32_t groups, int32_t sn) {
  const int64_t n_tiles = (sn + kGemmTileN / 2 - 1) / (kGemmTileN / 2);
  return launch_slots(rows, groups, n_tiles) * n_tiles;
}

// One case per value of select::gemm_k_tail.
hipError_t launch_grouped_gemm_i8(const GemmArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int64_t blocks = grouped_gemm_blocks(a.rows, a.groups, a.n);
  if (blocks > kGemmMaxBlocks) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kWave * kGemmWavesM * kGemmWavesN);
  if (select::gemm_k_tail(a.k)) {
    grouped_gemm_kernel<kGemmTileM, kGemmTileN, kGemmWavesM, kGemmWavesN, true, false>
        <<<grid, block, 0, stream>>>(a);
  } else {
    grouped_gemm_kernel<kGemmTileM, kGemmTileN, kGemmWavesM, kGemmWavesN, false, false>
        <<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_swiglu_quant(const GemmArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int64_t blocks = grouped_gemm_swiglu_blocks(a.rows, a.groups, a.sn);
  if (blocks > kGemmMaxBlocks) return hipErrorInvalidValue;
  const int64_t clear_blocks = (a.rows + 255) / 256;
  clear_u32_kernel<<<dim3(static_cast<uint32_t>(clear_blocks < 4096 ? clear_blocks : 4096)), dim3(256), 0, stream>>>(
      a.amax, a.rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kWave * kGemmWavesM * kGemmWavesN);
  if (select::gemm_k_tail(a.k)) {
    grouped_gemm_kernel<kGemmTileM, kGemmTileN, kGemmWavesM, kGemmWavesN, true, true>
        <<<grid, block, 0, stream>>>(a);
  } else {
    grouped_gemm_kernel<kGemmTileM, kGemmTileN, kGemmWavesM, kGemmWavesN, false, true>
        <<<grid, block, 0, stream>>>(a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  act_quant_kernel<<<dim3(static_cast<uint32_t>((a.rows + kQuantRows - 1) / kQuantRows)), dim3(kWave * kQuantRows), 0,
                     stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
