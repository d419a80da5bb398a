// Stage 2, notify ("UMDK/CAM communication acceleration library deep analysis
// v2", section 2.4, moe_notify_dispatch_zb).  On one device the all-gather of
// every rank's tokenPerExpert has a single source, so what remains is the
// prefix sum.  One workgroup computes the global exclusive scan G over the
// experts in LDS; then
//   recvBase[r]  = G[r * EPR]                       (rank regions in order)
//   recvCount[r] = G[(r + 1) * EPR] - G[r * EPR]
//   putOffset[e] = G[e] - G[(e / EPR) * EPR]        (offset inside the rank)
#include "device_util.h"
#include "launch.h"
#include "moe_ep.h"

namespace moe {
namespace {

constexpr int kNotifyThreads = 256;
constexpr int kNotifyPerThread = (MOE_MAX_EXPERTS + kNotifyThreads - 1) / kNotifyThreads;

__global__ __launch_bounds__(kNotifyThreads) void notify_kernel(
    const int32_t* __restrict__ token_per_expert, int32_t num_experts, int32_t epr, int32_t ranks,
    int32_t* __restrict__ put_offset, int32_t* __restrict__ recv_count,
    int32_t* __restrict__ recv_base, int32_t* __restrict__ recv_token_per_expert) {
  __shared__ int32_t g[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t wave_sum[kNotifyThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int per = (num_experts + kNotifyThreads - 1) / kNotifyThreads;
  const int first = tid * per;

  int cnt[kNotifyPerThread];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kNotifyPerThread; ++j) {
    const int e = first + j;
    cnt[j] = (j < per && e < num_experts) ? token_per_expert[e] : 0;
    sum += cnt[j];
  }
  const int incl = wave_inclusive_scan(sum);
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kNotifyThreads / kWave; ++w) {
    if (w < wave) run += wave_sum[w];
    total += wave_sum[w];
  }
#pragma unroll
  for (int j = 0; j < kNotifyPerThread; ++j) {
    const int e = first + j;
    if (j < per && e < num_experts) {
      g[e] = run;
      recv_token_per_expert[e] = cnt[j];
    }
    run += cnt[j];
  }
  if (tid == 0) g[num_experts] = total;
  __syncthreads();
  for (int e = tid; e < num_experts; e += kNotifyThreads) put_offset[e] = g[e] - g[(e / epr) * epr];
  for (int r = tid; r < ranks; r += kNotifyThreads) {
    recv_base[r] = g[r * epr];
    recv_count[r] = g[(r + 1) * epr] - g[r * epr];
  }
}

// Several source ranks (section 2.4's all-gather of every rank's
// tokenPerExpert, with section 2.6's index expertId * epWorldSize + srcRank):
// the count matrix count[s][e] is scanned in the order f = e * S + s
// (expert-major, source-minor).  With G the global exclusive scan over f:
//   putOffset[e][s] = G[e*S + s] - G[rank(e) * EPR * S]
//   recvBase[r]     = G[r * EPR * S]
//   recvCount[r]    = G[(r + 1) * EPR * S] - G[r * EPR * S]
//   recvTokenPerExpert[e] = sum over s of count[s][e]
// One workgroup; thread t owns the contiguous range [t * per, (t + 1) * per)
// of f.  Its first kCache values are loaded once, together, and kept in
// registers (the rest, only for count matrices above 8 Ki entries, are
// re-read).  Pass 1 sums the range (and adds each value to its expert's
// total in LDS); a workgroup scan gives each thread its start, and the
// thread owning a rank's first f records the rank's base.  Pass 2 writes
// the offsets.
constexpr int kMultiThreads = 1024;
constexpr int kCache = 8;

__global__ __launch_bounds__(kMultiThreads) void notify_multi_kernel(
    const int32_t* __restrict__ count, int32_t num_src, int32_t num_experts, int32_t epr,
    int32_t ranks, int32_t* __restrict__ put_offset, int32_t* __restrict__ recv_count,
    int32_t* __restrict__ recv_base, int32_t* __restrict__ recv_token_per_expert) {
  __shared__ int32_t rank_base[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t expert_total[MOE_MAX_EXPERTS];
  __shared__ int32_t wave_sum[kMultiThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = num_experts * num_src;  // at most MOE_MAX_EXPERTS * MOE_MAX_SOURCES
  const int per = (n + kMultiThreads - 1) / kMultiThreads;
  const int f0 = min(tid * per, n);
  const int f1 = min(f0 + per, n);
  for (int e = tid; e < num_experts; e += kMultiThreads) expert_total[e] = 0;
  // (expert, source) of f0; the walks below step s, then e
  const int e0 = f0 / num_src;
  const int s0 = f0 - e0 * num_src;
  auto at = [&](int e, int src) { return count[static_cast<int64_t>(src) * num_experts + e]; };
  int cache[kCache];
  {
    int e = e0, src = s0;
#pragma unroll
    for (int c = 0; c < kCache; ++c) {
      const bool in = f0 + c < f1;
      cache[c] = in ? at(e, src) : 0;
      if (in && ++src == num_src) { src = 0; ++e; }
    }
  }
  __syncthreads();  // expert_total cleared
  int sum = 0;
  {
    int e = e0, src = s0;
    for (int f = f0; f < f1; ++f) {
      const int c = f - f0 < kCache ? cache[f - f0] : at(e, src);
      sum += c;
      if (c != 0) atomicAdd(&expert_total[e], c);
      if (++src == num_src) { src = 0; ++e; }
    }
  }
  const int incl = wave_inclusive_scan(sum);
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  int total = 0;
  for (int w = 0; w < kMultiThreads / kWave; ++w) {
    if (w < wave) run += wave_sum[w];
    total += wave_sum[w];
  }
  // rank bases: rank r starts at f = r * EPR * S, i.e. at (e = r * EPR, s = 0)
  {
    int acc = run;
    int e = e0, src = s0;
    for (int f = f0; f < f1; ++f) {
      if (src == 0 && e % epr == 0) rank_base[e / epr] = acc;
      acc += f - f0 < kCache ? cache[f - f0] : at(e, src);
      if (++src == num_src) { src = 0; ++e; }
    }
  }
  if (tid == 0) rank_base[ranks] = total;
  __syncthreads();
  {
    int acc = run;
    int e = e0, src = s0;
    for (int f = f0; f < f1; ++f) {
      put_offset[f] = acc - rank_base[e / epr];
      acc += f - f0 < kCache ? cache[f - f0] : at(e, src);
      if (++src == num_src) { src = 0; ++e; }
    }
  }
  for (int r = tid; r < ranks; r += kMultiThreads) {
    recv_base[r] = rank_base[r];
    recv_count[r] = rank_base[r + 1] - rank_base[r];
  }
  for (int e = tid; e < num_experts; e += kMultiThreads) recv_token_per_expert[e] = expert_total[e];
}

}  // namespace

hipError_t launch_notify_multi(const int32_t* token_per_expert, int32_t num_src, int32_t epr,
                               int32_t ranks, int32_t* put_offset, int32_t* recv_count,
                               int32_t* recv_base, int32_t* recv_token_per_expert,
                               hipStream_t stream) {
  hipLaunchKernelGGL(notify_multi_kernel, dim3(1), dim3(kMultiThreads), 0, stream, token_per_expert,
                     num_src, epr * ranks, epr, ranks, put_offset, recv_count, recv_base,
                     recv_token_per_expert);
  return hipGetLastError();
}

hipError_t launch_notify(const int32_t* token_per_expert, int32_t epr, int32_t ranks,
                         int32_t* put_offset, int32_t* recv_count, int32_t* recv_base,
                         int32_t* recv_token_per_expert, hipStream_t stream) {
  hipLaunchKernelGGL(notify_kernel, dim3(1), dim3(kNotifyThreads), 0, stream, token_per_expert,
                     epr * ranks, epr, ranks, put_offset, recv_count, recv_base,
                     recv_token_per_expert);
  return hipGetLastError();
}

}  // namespace moe
