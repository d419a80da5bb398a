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
  const int incl = wave_inclusive_scan(sum, lane);
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

}  // namespace

hipError_t launch_notify(const int32_t* token_per_expert, int32_t epr, int32_t ranks,
                         int32_t* put_offset, int32_t* recv_count, int32_t* recv_base,
                         int32_t* recv_token_per_expert, hipStream_t stream) {
  hipLaunchKernelGGL(notify_kernel, dim3(1), dim3(kNotifyThreads), 0, stream, token_per_expert,
                     epr * ranks, epr, ranks, put_offset, recv_count, recv_base,
                     recv_token_per_expert);
  return hipGetLastError();
}

}  // namespace moe
