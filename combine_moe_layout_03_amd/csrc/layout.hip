// Stage 1, dispatch layout ("UMDK/CAM communication acceleration library deep
// analysis v2", section 2.3, moe_dispatch_layout_zb): per-expert and per-rank
// counts and the send slot of every (token, k) entry.
//
// The page counts in rounds with cross-core atomics and a SyncAll per round,
// then computes send indices.  Here the flat entry list is cut into tiles of
// kLayoutTile entries:
//   layout_count_kernel  one workgroup per tile except the last: an LDS
//                        histogram of the tile (order-free atomics), written
//                        to the workspace;
//   layout_rank_kernel   one workgroup per tile: the tile's starting count per
//                        expert (sum over earlier tiles), then the stable rank
//                        of every entry among equal ids, wave by wave, in flat
//                        order.  The last tile's workgroup also writes the
//                        totals.
// Inside a wave, lanes holding the same expert id find each other with one
// ballot per id bit (a match-any built from ballots); a lane's rank in its
// group is the number of group lanes below it.  A per-wave LDS counter per
// expert carries the rank across rounds; a scan over the four waves and the
// tile base turn it into the global slot.  No result depends on scheduling.
#include "device_util.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int32_t* __restrict__ topk_idx, int32_t n, int32_t num_experts,
    int32_t* __restrict__ tile_count, int32_t* __restrict__ tile_bad) {
  extern __shared__ int32_t hist[];  // [E + 1]; hist[E] counts bad ids
  const int tile = blockIdx.x;
  for (int e = threadIdx.x; e <= num_experts; e += kLayoutThreads) hist[e] = 0;
  __syncthreads();
  // All of this thread's ids are loaded before the first LDS update, so the
  // loads are in flight together.
  constexpr int kPer = kLayoutTile / kLayoutThreads;
  const int begin = tile * kLayoutTile + threadIdx.x;
  int ids[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = begin + r * kLayoutThreads;
    ids[r] = i < n ? topk_idx[i] : -2;
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if (ids[r] == -2 && begin + r * kLayoutThreads >= n) continue;
    const int e = ids[r];
    const int key = static_cast<unsigned>(e) < static_cast<unsigned>(num_experts) ? e : num_experts;
    atomicAdd(&hist[key], 1);
  }
  __syncthreads();
  int32_t* row = tile_count + static_cast<size_t>(tile) * num_experts;
  for (int e = threadIdx.x; e < num_experts; e += kLayoutThreads) row[e] = hist[e];
  if (threadIdx.x == 0) tile_bad[tile] = hist[num_experts];
}

__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const int32_t* __restrict__ topk_idx, int32_t n, int32_t num_experts, int32_t epr,
    int32_t ranks, int32_t id_bits, int32_t num_tiles, const int32_t* __restrict__ tile_count,
    const int32_t* __restrict__ tile_bad, int32_t* __restrict__ token_per_expert,
    int32_t* __restrict__ token_per_rank, int32_t* __restrict__ send_token_idx,
    int32_t* __restrict__ bad_count) {
  extern __shared__ int32_t lds[];
  constexpr int kWaves = kLayoutThreads / kWave;
  int32_t* wave_cnt = lds;                       // [kWaves][E]
  int32_t* base = lds + kWaves * num_experts;    // [E]
  __shared__ int32_t block_bad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid / kWave);
  const int tile = blockIdx.x;

  // Starting count of every expert for this tile: the sum over earlier
  // tiles, 16 independent loads in flight per thread per batch.
  for (int e = tid; e < num_experts; e += kLayoutThreads) {
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
  // segment with the same expert id.
  int32_t* my_cnt = wave_cnt + wave * num_experts;
  const int seg_begin = tile * kLayoutTile + wave * kLayoutSegment;
  int local[kLayoutRounds];
  int key[kLayoutRounds];
  int ids[kLayoutRounds];
  int my_bad = 0;
  // All rounds' ids are loaded first (in flight together); the rounds then
  // only touch LDS.
#pragma unroll
  for (int r = 0; r < kLayoutRounds; ++r) {
    const int i = seg_begin + r * kWave + lane;
    ids[r] = i < n ? topk_idx[i] : -1;
  }
#pragma unroll
  for (int r = 0; r < kLayoutRounds; ++r) {
    const int i = seg_begin + r * kWave + lane;
    const bool in_range = i < n;
    const int e = ids[r];
    const bool valid = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(num_experts);
    my_bad += (in_range && !valid) ? 1 : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(bit);
      peers &= bit ? set : ~set;
    }
    // For a valid lane, `peers` is the set of valid lanes with the same id.
    const int below = lanes_below(peers);
    const int group = __popcll(peers);
    const int prev = valid ? my_cnt[e] : 0;
    local[r] = prev + below;
    key[r] = valid ? e : -1;
    // The group's highest lane advances the counter; the wave's LDS reads of
    // this round are issued before this write.
    if (valid && below == group - 1) my_cnt[e] = prev + group;
  }
  if (my_bad) atomicAdd(&block_bad, my_bad);
  __syncthreads();

  // Exclusive scan over the waves, on top of the tile base.
  for (int e = tid; e < num_experts; e += kLayoutThreads) {
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
  for (int r = 0; r < kLayoutRounds; ++r) {
    const int i = seg_begin + r * kWave + lane;
    if (i < n) send_token_idx[i] = key[r] >= 0 ? my_cnt[key[r]] + local[r] : -1;
  }

  if (tile == num_tiles - 1) {
    for (int e = tid; e < num_experts; e += kLayoutThreads) token_per_expert[e] = base[e];
    for (int r = tid; r < ranks; r += kLayoutThreads) {
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

}  // namespace

hipError_t launch_layout(const int32_t* topk_idx, int32_t n, int32_t num_experts, int32_t epr,
                         int32_t ranks, int32_t* token_per_expert, int32_t* token_per_rank,
                         int32_t* send_token_idx, int32_t* bad_count, void* workspace,
                         hipStream_t stream) {
  const int num_tiles = static_cast<int>(layout_num_tiles(n));
  int32_t* tile_count = static_cast<int32_t*>(workspace);
  int32_t* tile_bad =
      tile_count == nullptr ? nullptr : tile_count + static_cast<size_t>(num_tiles - 1) * num_experts;
  if (num_tiles > 1) {
    const size_t lds = static_cast<size_t>(num_experts + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_count_kernel, dim3(num_tiles - 1), dim3(kLayoutThreads), lds, stream,
                       topk_idx, n, num_experts, tile_count, tile_bad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  int id_bits = 0;
  while ((1 << id_bits) < num_experts) ++id_bits;
  const size_t lds = static_cast<size_t>(kLayoutThreads / kWave + 1) * num_experts * sizeof(int32_t);
  hipLaunchKernelGGL(layout_rank_kernel, dim3(num_tiles), dim3(kLayoutThreads), lds, stream,
                     topk_idx, n, num_experts, epr, ranks, id_bits, num_tiles, tile_count, tile_bad,
                     token_per_expert, token_per_rank, send_token_idx, bad_count);
  return hipGetLastError();
}

}  // namespace moe
