// Stage 1, dispatch layout ("UMDK/CAM communication acceleration library deep
// analysis v2", section 2.3, moe_dispatch_layout_zb): per-expert and per-rank
// counts and the send slot of every (token, k) entry.
//
// The page counts in rounds with cross-core atomics and a SyncAll per round,
// then computes send indices.  Here the flat entry list is cut into tiles
// (see LayoutShape):
//   layout_count_kernel  one workgroup per tile except the last, only when
//                        there are several tiles: an LDS histogram of the
//                        tile (order-free atomics), written to the workspace;
//   layout_rank_kernel   one workgroup per tile: the tile's starting count per
//                        expert (sum over earlier tiles' histograms), then the
//                        stable rank of every entry among equal ids, wave by
//                        wave, in flat order.  The last tile's workgroup also
//                        writes the totals.
// Inside a wave, lanes holding the same expert id find each other with one
// ballot per id bit (a match-any built from ballots); a lane's rank in its
// group is the number of group lanes below it.  The group's highest lane
// adds the group size to a wave-private LDS counter of the expert with an
// atomic that returns the old value; LDS executes one wave's operations in
// order, so that value is the count of the expert in the wave's earlier
// rounds.  Up to eight rounds' atomics are issued back to back before their
// results are shuffled to the group members, so the rounds do not wait on
// each other.  A scan over the waves and the tile base turn wave-local ranks
// into global slots.  No result depends on scheduling.
#include <mutex>

#include "device_util.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBatch = 8;  // rounds whose counter atomics are in flight together

template <int kWaves, int kRounds>
__global__ __launch_bounds__(kWaves * kWave) void layout_count_kernel(
    const int32_t* __restrict__ topk_idx, int32_t n, int32_t num_experts,
    int32_t* __restrict__ tile_count, int32_t* __restrict__ tile_bad) {
  constexpr int kThreads = kWaves * kWave;
  constexpr int kTile = kThreads * kRounds;
  extern __shared__ int32_t hist[];  // [E + 1]; hist[E] counts bad ids
  const int tile = blockIdx.x;
  // All of this thread's ids are loaded before the first LDS update.
  const int64_t begin = static_cast<int64_t>(tile) * kTile + threadIdx.x;
  int ids[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = begin + r * kThreads;
    ids[r] = i < n ? topk_idx[i] : 0;
  }
  for (int e = threadIdx.x; e <= num_experts; e += kThreads) hist[e] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (begin + r * kThreads >= n) continue;
    const int e = ids[r];
    atomicAdd(&hist[static_cast<unsigned>(e) < static_cast<unsigned>(num_experts) ? e : num_experts], 1);
  }
  __syncthreads();
  int32_t* row = tile_count + static_cast<size_t>(tile) * num_experts;
  for (int e = threadIdx.x; e < num_experts; e += kThreads) row[e] = hist[e];
  if (threadIdx.x == 0) tile_bad[tile] = hist[num_experts];
}

template <int kWaves, int kRounds>
__global__ __launch_bounds__(kWaves * kWave) void layout_rank_kernel(
    const int32_t* __restrict__ topk_idx, int32_t n, int32_t num_experts, int32_t epr,
    int32_t ranks, int32_t id_bits, int32_t num_tiles, const int32_t* __restrict__ tile_count,
    const int32_t* __restrict__ tile_bad, int32_t* __restrict__ token_per_expert,
    int32_t* __restrict__ token_per_rank, int32_t* __restrict__ send_token_idx,
    int32_t* __restrict__ bad_count) {
  constexpr int kThreads = kWaves * kWave;
  constexpr int kSegment = kRounds * kWave;
  constexpr int kTile = kWaves * kSegment;
  constexpr int kB = kRounds < kBatch ? kRounds : kBatch;
  static_assert(kRounds % kB == 0, "rounds come in batches");
  extern __shared__ int32_t lds[];
  int32_t* wave_cnt = lds;                     // [kWaves][E]
  int32_t* base = lds + kWaves * num_experts;  // [E]
  __shared__ int32_t block_bad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid / kWave);
  const int tile = blockIdx.x;

  // This wave's ids, loaded first so they are in flight meanwhile.
  const int64_t seg_begin = static_cast<int64_t>(tile) * kTile + static_cast<int64_t>(wave) * kSegment;
  int ids[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = seg_begin + r * kWave + lane;
    ids[r] = i < n ? topk_idx[i] : -1;
  }

  // Starting count of every expert for this tile: the sum of the earlier
  // tiles' histograms, 16 independent loads in flight per thread per batch.
  for (int e = tid; e < num_experts; e += kThreads) {
    int s = 0;
    for (int t0 = 0; t0 < tile; t0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = (t0 + u < tile) ? tile_count[static_cast<size_t>(t0 + u) * num_experts + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) s += v[u];
    }
    base[e] = s;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wave_cnt[w * num_experts + e] = 0;
  }
  if (tid == 0) block_bad = 0;
  __syncthreads();

  // Per wave: stable rank of each entry among earlier entries of this wave's
  // segment with the same expert id.  Invalid entries get rank -1.
  int32_t* my_cnt = wave_cnt + wave * num_experts;
  int local[kRounds];
  int my_bad = 0;
#pragma unroll
  for (int b0 = 0; b0 < kRounds; b0 += kB) {
    int ret[kB];
    int leader[kB];
    int below[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int r = b0 + u;
      const int64_t i = seg_begin + r * kWave + lane;
      const int e = ids[r];
      const bool in_range = i < n;
      const bool valid = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(num_experts);
      my_bad += (in_range && !valid) ? 1 : 0;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < id_bits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t set = __ballot(bit);
        peers &= bit ? set : ~set;
      }
      // For a valid lane, `peers` is the set of valid lanes with the same id;
      // its highest lane is the group's leader.
      below[u] = valid ? lanes_below(peers) : -1;
      leader[u] = valid ? 63 - __builtin_clzll(peers) : lane;
      ret[u] = 0;
      if (valid && leader[u] == lane) ret[u] = atomicAdd(&my_cnt[e], __popcll(peers));
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int start = __shfl(ret[u], leader[u], kWave);
      local[b0 + u] = below[u] < 0 ? -1 : start + below[u];
    }
  }
  if (my_bad) atomicAdd(&block_bad, my_bad);
  __syncthreads();

  // Exclusive scan over the waves, on top of the tile base.
  for (int e = tid; e < num_experts; e += kThreads) {
    int s = base[e];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = wave_cnt[w * num_experts + e];
      wave_cnt[w * num_experts + e] = s;
      s += c;
    }
    base[e] = s;  // count of expert e over tiles 0..tile
  }
  __syncthreads();

#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i = seg_begin + r * kWave + lane;
    if (i < n) send_token_idx[i] = local[r] >= 0 ? my_cnt[ids[r]] + local[r] : -1;
  }

  if (tile == num_tiles - 1) {
    for (int e = tid; e < num_experts; e += kThreads) token_per_expert[e] = base[e];
    for (int r = tid; r < ranks; r += kThreads) {
      int s = 0;
      for (int j = 0; j < epr; ++j) s += base[r * epr + j];
      token_per_rank[r] = s;
    }
    if (bad_count != nullptr && tid == 0) {
      int b = block_bad;
      for (int t = 0; t < num_tiles - 1; ++t) b += tile_bad[t];
      *bad_count = b;
    }
  }
}

template <int kWaves, int kRounds>
hipError_t launch_shape(const int32_t* topk_idx, int32_t n, int32_t num_experts, int32_t epr,
                        int32_t ranks, int32_t* token_per_expert, int32_t* token_per_rank,
                        int32_t* send_token_idx, int32_t* bad_count, void* workspace,
                        hipStream_t stream) {
  constexpr int kThreads = kWaves * kWave;
  constexpr int64_t kTile = static_cast<int64_t>(kThreads) * kRounds;
  const int num_tiles = n <= 0 ? 1 : static_cast<int>((n + kTile - 1) / kTile);
  int32_t* tile_count = static_cast<int32_t*>(workspace);
  int32_t* tile_bad =
      tile_count == nullptr ? nullptr : tile_count + static_cast<size_t>(num_tiles - 1) * num_experts;
  if (num_tiles > 1) {
    const size_t lds = static_cast<size_t>(num_experts + 1) * sizeof(int32_t);
    hipLaunchKernelGGL((layout_count_kernel<kWaves, kRounds>), dim3(num_tiles - 1), dim3(kThreads), lds,
                       stream, topk_idx, n, num_experts, tile_count, tile_bad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  int id_bits = 0;
  while ((1 << id_bits) < num_experts) ++id_bits;
  const size_t lds = static_cast<size_t>(kWaves + 1) * num_experts * sizeof(int32_t);
  hipLaunchKernelGGL((layout_rank_kernel<kWaves, kRounds>), dim3(num_tiles), dim3(kThreads), lds, stream,
                     topk_idx, n, num_experts, epr, ranks, id_bits, num_tiles, tile_count, tile_bad,
                     token_per_expert, token_per_rank, send_token_idx, bad_count);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layout(const int32_t* topk_idx, int32_t n, int32_t num_experts, int32_t epr,
                         int32_t ranks, int32_t* token_per_expert, int32_t* token_per_rank,
                         int32_t* send_token_idx, int32_t* bad_count, void* workspace,
                         hipStream_t stream) {
  const LayoutShape shape = layout_shape(num_experts);
  if (shape.waves == 16 && shape.rounds == 2) {
    return launch_shape<16, 2>(topk_idx, n, num_experts, epr, ranks, token_per_expert, token_per_rank,
                               send_token_idx, bad_count, workspace, stream);
  }
  if (shape.waves == 4 && shape.rounds == 8) {
    return launch_shape<4, 8>(topk_idx, n, num_experts, epr, ranks, token_per_expert, token_per_rank,
                              send_token_idx, bad_count, workspace, stream);
  }
  return hipErrorInvalidValue;
}

// ---- the layout workspace without allocation --------------------------------
// For callers that cannot allocate: a file-scope device array serves as the
// per-tile count table.  In host code `layout_scratch` names a host-side
// stand-in, not device memory; its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to a kernel.  Every call on a device shares
// the device's array (calls that overlap on one device race).  Nothing in it
// needs clearing: the count kernel writes every entry the rank kernel reads.
namespace {
static __device__ __align__(256) int32_t layout_scratch[kLayoutScratchBytes / sizeof(int32_t)];

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchMaxDevices];  // device address of layout_scratch on each device
}  // namespace

hipError_t layout_scratch_address(void** ptr) {
  int device = 0;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return err;
  if (device < 0 || device >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(layout_scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace moe
