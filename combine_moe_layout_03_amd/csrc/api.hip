// C entry points of libmoe_ep: argument checks on the host, then kernel
// launches on the caller's stream.  Every check runs before anything is
// enqueued, so a call that returns an error has enqueued nothing.  No call
// allocates, frees or waits.
#include <hip/hip_runtime.h>

#include <atomic>
#include <limits>

#include "launch.h"
#include "gemm.h"
#include "moe_ep.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t err) {
  if (err == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(err);
  return MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Compute units of the current device, queried once per device (the fused
// kernel's grid is one workgroup per CU); later calls only read the cache.
constexpr int kMaxCachedDevices = 64;
std::atomic<int> g_device_cus[kMaxCachedDevices];  // 0: not queried yet

hipError_t current_device_cus(int* cus) {
  int device = 0;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return err;
  const bool cached = device >= 0 && device < kMaxCachedDevices;
  int c = cached ? g_device_cus[device].load(std::memory_order_relaxed) : 0;
  if (c == 0) {
    err = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, device);
    if (err != hipSuccess) return err;
    if (cached) g_device_cus[device].store(c, std::memory_order_relaxed);
  }
  *cus = c;
  return hipSuccess;
}

size_t align32(int64_t v) { return static_cast<size_t>((v + 31) / 32 * 32); }

// An int8 receive row: h codes, the float inverse scale at byte align32(h)
// (the page's hUBAlignSize with UB_ALIGN_SIZE = 32) in a 32-byte block, and
// the row stride rounded up to whole 128-byte cache lines.  The page fixes
// where the scale goes but not the row stride; with rows that start on a
// line boundary no two rows share a line, which dispatch writes and combine
// reads at different times (at h = 7168: 7296-byte rows; with 7200-byte
// rows the back-to-back step took 108.6 instead of 92.9 us).
constexpr size_t kRecvLine = 128;
size_t int8_row_bytes(int64_t hidden) { return (align32(hidden) + 32u + kRecvLine - 1) / kRecvLine * kRecvLine; }

// Shared checks on the routing scalars.
int check_experts(int32_t epr, int32_t ranks) {
  if (epr < 1 || ranks < 1) return MOE_ERR_BAD_SHAPE;
  const int64_t e = static_cast<int64_t>(epr) * ranks;
  if (e > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_tokens(int32_t bs, int32_t topk) {
  if (bs < 0 || topk < 1) return MOE_ERR_BAD_SHAPE;
  if (topk > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(bs) * topk > std::numeric_limits<int32_t>::max()) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_hidden(int32_t hidden) {
  if (hidden < 1) return MOE_ERR_BAD_SHAPE;
  if (hidden % 8 != 0 || hidden > MOE_MAX_HIDDEN) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int row_bytes(int32_t hidden, moe_dtype recv, size_t* bytes) {
  switch (recv) {
    case MOE_BF16:
    case MOE_FP16:
      *bytes = static_cast<size_t>(hidden) * 2u;
      return MOE_OK;
    case MOE_INT8_ROWSCALE:
      *bytes = int8_row_bytes(hidden);
      return MOE_OK;
    default:
      return MOE_ERR_BAD_DTYPE;
  }
}

// Source count and index of a multi-source call.
int check_sources(int32_t num_src, int32_t src_rank) {
  if (num_src < 1 || src_rank < 0 || src_rank >= num_src) return MOE_ERR_BAD_SHAPE;
  if (num_src > MOE_MAX_SOURCES) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Routing arguments common to dispatch and combine; source src_rank of
// num_src reads column src_rank of putOffset [E][num_src].
int make_route(int32_t bs, int32_t hidden, int32_t topk, const int32_t* topk_idx,
               const int32_t* send_token_idx, const int32_t* put_offset, const int32_t* recv_base,
               int32_t epr, int32_t ranks, int32_t num_src, int32_t src_rank, moe_dtype recv_type,
               size_t recv_bytes, moe::RouteArgs* r) {
  int st = check_tokens(bs, topk);
  if (st) return st;
  if ((st = check_experts(epr, ranks))) return st;
  if ((st = check_sources(num_src, src_rank))) return st;
  if ((st = check_hidden(hidden))) return st;
  size_t rb = 0;
  if ((st = row_bytes(hidden, recv_type, &rb))) return st;
  if (bs == 0) return MOE_OK;  // nothing to move; empty tensors may have NULL data
  if (!topk_idx || !send_token_idx || !put_offset || !recv_base) return MOE_ERR_NULL_PTR;
  if (!aligned(topk_idx, 4) || !aligned(send_token_idx, 4) || !aligned(put_offset, 4) ||
      !aligned(recv_base, 4))
    return MOE_ERR_BAD_ALIGN;
  const size_t need = rb * static_cast<size_t>(bs) * static_cast<size_t>(topk);
  if (recv_bytes < need) return MOE_ERR_BUFFER_TOO_SMALL;
  r->topk_idx = topk_idx;
  r->send_token_idx = send_token_idx;
  r->put_offset = put_offset + src_rank;
  r->put_stride = num_src;
  r->recv_base = recv_base;
  r->bs = bs;
  r->hidden = hidden;
  r->k = topk;
  r->epr = epr;
  r->num_experts = epr * ranks;
  r->row_bytes = static_cast<int64_t>(rb);
  r->cap_rows = static_cast<int64_t>(recv_bytes / rb);
  r->scale_off = static_cast<int32_t>(align32(hidden));
  r->epr_magic = moe::div_magic(epr);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_recv_row_bytes(int32_t hidden, moe_dtype recv, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL_PTR;
  if (hidden < 1) return MOE_ERR_BAD_SHAPE;
  return row_bytes(hidden, recv, bytes);
}

int moe_layout_workspace_bytes(int32_t bs, int32_t topk, int32_t num_experts, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL_PTR;
  int st = check_tokens(bs, topk);
  if (st) return st;
  if (num_experts < 1) return MOE_ERR_BAD_SHAPE;
  if (num_experts > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  *bytes = moe::layout_workspace_bytes(static_cast<int64_t>(bs) * topk, num_experts);
  return MOE_OK;
}

int moe_layout(const int32_t* topk_idx, int32_t bs, int32_t topk, int32_t epr, int32_t ranks,
               int32_t* token_per_expert, int32_t* token_per_rank, int32_t* send_token_idx,
               int32_t* bad_id_count, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_tokens(bs, topk);
  if (st) return st;
  if ((st = check_experts(epr, ranks))) return st;
  if (!token_per_expert || !token_per_rank) return MOE_ERR_NULL_PTR;
  if (bs > 0 && (!topk_idx || !send_token_idx)) return MOE_ERR_NULL_PTR;
  const int32_t e = epr * ranks;
  const int64_t n = static_cast<int64_t>(bs) * topk;
  const size_t need = moe::layout_workspace_bytes(n, e);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return MOE_ERR_NULL_PTR;
  if (!aligned(workspace, 4) || !aligned(token_per_expert, 4) || !aligned(token_per_rank, 4) ||
      !aligned(send_token_idx, 4) || !aligned(topk_idx, 4) || !aligned(bad_id_count, 4))
    return MOE_ERR_BAD_ALIGN;
  return hip_status(moe::launch_layout(topk_idx, static_cast<int32_t>(n), e, epr, ranks,
                                       token_per_expert, token_per_rank, send_token_idx,
                                       bad_id_count, workspace, static_cast<hipStream_t>(stream)));
}

int moe_layout_no_alloc(const int32_t* topk_idx, int32_t bs, int32_t topk, int32_t epr, int32_t ranks,
                        int32_t* token_per_expert, int32_t* token_per_rank, int32_t* send_token_idx,
                        int32_t* bad_id_count, void* stream) {
  int st = check_tokens(bs, topk);
  if (st) return st;
  if ((st = check_experts(epr, ranks))) return st;
  if (!token_per_expert || !token_per_rank) return MOE_ERR_NULL_PTR;
  if (bs > 0 && (!topk_idx || !send_token_idx)) return MOE_ERR_NULL_PTR;
  if (!aligned(token_per_expert, 4) || !aligned(token_per_rank, 4) || !aligned(send_token_idx, 4) ||
      !aligned(topk_idx, 4) || !aligned(bad_id_count, 4))
    return MOE_ERR_BAD_ALIGN;
  const int32_t e = epr * ranks;
  const int64_t n = static_cast<int64_t>(bs) * topk;
  const size_t need = moe::layout_workspace_bytes(n, e);
  if (need > moe::kLayoutScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  void* scratch = nullptr;
  const hipError_t err = moe::layout_scratch_address(&scratch);
  if (err != hipSuccess) return hip_status(err);
  return hip_status(moe::launch_layout(topk_idx, static_cast<int32_t>(n), e, epr, ranks, token_per_expert,
                                       token_per_rank, send_token_idx, bad_id_count, scratch,
                                       static_cast<hipStream_t>(stream)));
}

int moe_notify(const int32_t* token_per_expert, int32_t epr, int32_t ranks, int32_t* put_offset,
               int32_t* recv_count, int32_t* recv_base, int32_t* recv_token_per_expert,
               void* stream) {
  int st = check_experts(epr, ranks);
  if (st) return st;
  if (!token_per_expert || !put_offset || !recv_count || !recv_base || !recv_token_per_expert)
    return MOE_ERR_NULL_PTR;
  if (!aligned(token_per_expert, 4) || !aligned(put_offset, 4) || !aligned(recv_count, 4) ||
      !aligned(recv_base, 4) || !aligned(recv_token_per_expert, 4))
    return MOE_ERR_BAD_ALIGN;
  return hip_status(moe::launch_notify(token_per_expert, epr, ranks, put_offset, recv_count,
                                       recv_base, recv_token_per_expert,
                                       static_cast<hipStream_t>(stream)));
}

int moe_notify_multi(const int32_t* token_per_expert, int32_t num_src, int32_t epr, int32_t ranks,
                     int32_t* put_offset, int32_t* recv_count, int32_t* recv_base,
                     int32_t* recv_token_per_expert, void* stream) {
  int st = check_experts(epr, ranks);
  if (st) return st;
  if ((st = check_sources(num_src, 0))) return st;
  if (!token_per_expert || !put_offset || !recv_count || !recv_base || !recv_token_per_expert)
    return MOE_ERR_NULL_PTR;
  if (!aligned(token_per_expert, 4) || !aligned(put_offset, 4) || !aligned(recv_count, 4) ||
      !aligned(recv_base, 4) || !aligned(recv_token_per_expert, 4))
    return MOE_ERR_BAD_ALIGN;
  return hip_status(moe::launch_notify_multi(token_per_expert, num_src, epr, ranks, put_offset,
                                             recv_count, recv_base, recv_token_per_expert,
                                             static_cast<hipStream_t>(stream)));
}

int moe_dispatch(const void* x, moe_dtype x_type, int32_t bs, int32_t hidden, int32_t topk,
                 const int32_t* topk_idx, const int32_t* send_token_idx, const int32_t* put_offset,
                 const int32_t* recv_base, int32_t epr, int32_t ranks, int quant_int8,
                 void* recv_x, size_t recv_x_bytes, void* stream) {
  return moe_dispatch_src(x, x_type, bs, hidden, topk, topk_idx, send_token_idx, put_offset, recv_base,
                          epr, ranks, 1, 0, quant_int8, recv_x, recv_x_bytes, stream);
}

int moe_dispatch_src(const void* x, moe_dtype x_type, int32_t bs, int32_t hidden, int32_t topk,
                     const int32_t* topk_idx, const int32_t* send_token_idx, const int32_t* put_offset,
                     const int32_t* recv_base, int32_t epr, int32_t ranks, int32_t num_src,
                     int32_t src_rank, int quant_int8, void* recv_x, size_t recv_x_bytes, void* stream) {
  if (x_type != MOE_BF16 && x_type != MOE_FP16) return MOE_ERR_BAD_DTYPE;
  if (quant_int8 != 0 && quant_int8 != 1) return MOE_ERR_BAD_DTYPE;
  const moe_dtype recv_type = quant_int8 ? MOE_INT8_ROWSCALE : x_type;
  moe::RouteArgs r{};
  int st = make_route(bs, hidden, topk, topk_idx, send_token_idx, put_offset, recv_base, epr, ranks,
                      num_src, src_rank, recv_type, recv_x_bytes, &r);
  if (st) return st;
  if (bs == 0) return MOE_OK;
  if (!x || !recv_x) return MOE_ERR_NULL_PTR;
  if (!aligned(x, 16) || !aligned(recv_x, 16)) return MOE_ERR_BAD_ALIGN;
  return hip_status(moe::launch_dispatch(r, x, x_type == MOE_FP16 ? moe::Half::kFp16 : moe::Half::kBf16,
                                         quant_int8 != 0, recv_x, static_cast<hipStream_t>(stream)));
}

int moe_combine(const void* recv_x, moe_dtype recv_type, size_t recv_x_bytes, int32_t bs,
                int32_t hidden, int32_t topk, const int32_t* topk_idx, const float* topk_weights,
                const int32_t* send_token_idx, const int32_t* put_offset, const int32_t* recv_base,
                int32_t epr, int32_t ranks, void* out, moe_dtype out_type, void* stream) {
  return moe_combine_src(recv_x, recv_type, recv_x_bytes, bs, hidden, topk, topk_idx, topk_weights,
                         send_token_idx, put_offset, recv_base, epr, ranks, 1, 0, out, out_type, stream);
}

int moe_combine_src(const void* recv_x, moe_dtype recv_type, size_t recv_x_bytes, int32_t bs,
                    int32_t hidden, int32_t topk, const int32_t* topk_idx, const float* topk_weights,
                    const int32_t* send_token_idx, const int32_t* put_offset, const int32_t* recv_base,
                    int32_t epr, int32_t ranks, int32_t num_src, int32_t src_rank, void* out,
                    moe_dtype out_type, void* stream) {
  if (recv_type != MOE_BF16 && recv_type != MOE_FP16 && recv_type != MOE_INT8_ROWSCALE)
    return MOE_ERR_BAD_DTYPE;
  if (out_type != MOE_BF16 && out_type != MOE_FP16 && out_type != MOE_FP32) return MOE_ERR_BAD_DTYPE;
  moe::RouteArgs r{};
  int st = make_route(bs, hidden, topk, topk_idx, send_token_idx, put_offset, recv_base, epr, ranks,
                      num_src, src_rank, recv_type, recv_x_bytes, &r);
  if (st) return st;
  if (bs == 0) return MOE_OK;
  if (!recv_x || !out || !topk_weights) return MOE_ERR_NULL_PTR;
  if (!aligned(recv_x, 16) || !aligned(out, 16) || !aligned(topk_weights, 4)) return MOE_ERR_BAD_ALIGN;
  const moe::Recv rt = recv_type == MOE_INT8_ROWSCALE ? moe::Recv::kInt8
                       : recv_type == MOE_FP16        ? moe::Recv::kFp16
                                                      : moe::Recv::kBf16;
  const moe::Out ot = out_type == MOE_FP32 ? moe::Out::kF32
                      : out_type == MOE_FP16 ? moe::Out::kFp16
                                             : moe::Out::kBf16;
  return hip_status(moe::launch_combine(r, recv_x, rt, topk_weights, out, ot,
                                        static_cast<hipStream_t>(stream)));
}

namespace {

// Whether the one-kernel form applies (host logic only).
bool fused_applies(int32_t bs, int32_t hidden, int32_t topk) { return moe::select::fused_applies(bs, hidden, topk); }

// Tokens per workgroup, LDS histogram copies and workgroups of the one
// kernel: one workgroup per CU (fewer for small batches); as many histogram
// copies (up to 8) as leave room in kFusedMaxLds for 8 KiB of per-token
// state; more workgroups when the per-token state of one would not fit.
int fused_grid(int32_t bs, int32_t topk, int32_t num_experts, int cus, int32_t* tokens_per_group,
               int32_t* copies_log2) {
  int lg = moe::kFusedMaxCopiesLog2;
  while (lg > 0 && moe::fused_lds_bytes(num_experts, 0, topk, 1 << lg) + 8192 > moe::kFusedMaxLds) --lg;
  const size_t fixed = moe::fused_lds_bytes(num_experts, 0, topk, 1 << lg);
  const size_t per_token = moe::fused_lds_bytes(num_experts, 1, topk, 1 << lg) - fixed;
  const int64_t t_max = static_cast<int64_t>((moe::kFusedMaxLds - fixed) / per_token);
  int64_t groups = bs < cus ? bs : cus;
  if (groups < 1) groups = 1;
  int64_t tpg = (bs + groups - 1) / groups;
  if (tpg > t_max) tpg = t_max;
  groups = (bs + tpg - 1) / tpg;
  *tokens_per_group = static_cast<int32_t>(tpg);
  *copies_log2 = lg;
  return static_cast<int>(groups);
}

}  // namespace

int moe_fused_supported(int32_t bs, int32_t hidden, int32_t topk, int32_t expert_num_per_rank, int32_t ranks,
                        moe_dtype x_type, int quant_int8, int* supported) {
  if (!supported) return MOE_ERR_NULL_PTR;
  int st = check_tokens(bs, topk);
  if (st) return st;
  if ((st = check_experts(expert_num_per_rank, ranks))) return st;
  if ((st = check_hidden(hidden))) return st;
  if (x_type != MOE_BF16 && x_type != MOE_FP16) return MOE_ERR_BAD_DTYPE;
  if (quant_int8 != 0 && quant_int8 != 1) return MOE_ERR_BAD_DTYPE;
  *supported = fused_applies(bs, hidden, topk) ? 1 : 0;
  return MOE_OK;
}

int moe_layout_notify_dispatch(const void* x, moe_dtype x_type, int32_t bs, int32_t hidden, int32_t topk,
                               const int32_t* topk_idx, int32_t epr, int32_t ranks, int quant_int8,
                               int32_t* token_per_expert, int32_t* token_per_rank, int32_t* send_token_idx,
                               int32_t* bad_id_count, int32_t* put_offset, int32_t* recv_count,
                               int32_t* recv_base, int32_t* recv_token_per_expert, void* recv_x,
                               size_t recv_x_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  if (x_type != MOE_BF16 && x_type != MOE_FP16) return MOE_ERR_BAD_DTYPE;
  if (quant_int8 != 0 && quant_int8 != 1) return MOE_ERR_BAD_DTYPE;
  const moe_dtype recv_type = quant_int8 ? MOE_INT8_ROWSCALE : x_type;
  int st = check_tokens(bs, topk);
  if (st) return st;
  if ((st = check_experts(epr, ranks))) return st;
  if ((st = check_hidden(hidden))) return st;
  if (!token_per_expert || !token_per_rank || !put_offset || !recv_count || !recv_base ||
      !recv_token_per_expert)
    return MOE_ERR_NULL_PTR;
  if (bs > 0 && (!x || !topk_idx || !send_token_idx || !recv_x)) return MOE_ERR_NULL_PTR;
  const int64_t n = static_cast<int64_t>(bs) * topk;
  const bool one_kernel = fused_applies(bs, hidden, topk);
  if (!one_kernel) {
    const size_t need_ws = moe::layout_workspace_bytes(n, epr * ranks);
    if (workspace_bytes < need_ws) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (need_ws > 0 && !workspace) return MOE_ERR_NULL_PTR;
  }
  size_t rb = 0;
  if ((st = row_bytes(hidden, recv_type, &rb))) return st;
  if (recv_x_bytes < rb * static_cast<size_t>(bs) * static_cast<size_t>(topk)) return MOE_ERR_BUFFER_TOO_SMALL;
  if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 4) || !aligned(send_token_idx, 4) ||
      !aligned(workspace, 4) || !aligned(token_per_expert, 4) || !aligned(token_per_rank, 4) ||
      !aligned(bad_id_count, 4) || !aligned(put_offset, 4) || !aligned(recv_count, 4) ||
      !aligned(recv_base, 4) || !aligned(recv_token_per_expert, 4))
    return MOE_ERR_BAD_ALIGN;

  if (!one_kernel) {
    if ((st = moe_layout(topk_idx, bs, topk, epr, ranks, token_per_expert, token_per_rank, send_token_idx,
                         bad_id_count, workspace, workspace_bytes, stream)))
      return st;
    if ((st = moe_notify(token_per_expert, epr, ranks, put_offset, recv_count, recv_base,
                         recv_token_per_expert, stream)))
      return st;
    return moe_dispatch(x, x_type, bs, hidden, topk, topk_idx, send_token_idx, put_offset, recv_base, epr,
                        ranks, quant_int8, recv_x, recv_x_bytes, stream);
  }

  int cus = 0;
  const hipError_t err = current_device_cus(&cus);
  if (err != hipSuccess) return hip_status(err);
  moe::FusedArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.topk_idx = topk_idx;
  a.bs = bs;
  a.hidden = hidden;
  a.k = topk;
  a.epr = epr;
  a.ranks = ranks;
  a.num_experts = epr * ranks;
  int id_bits = 0;
  while ((1 << id_bits) < a.num_experts) ++id_bits;
  a.id_bits = id_bits;
  const int groups = fused_grid(bs, topk, a.num_experts, cus, &a.tokens_per_group, &a.copies_log2);
  a.ids_aligned16 = aligned(topk_idx, 16) ? 1 : 0;
  a.token_per_expert = token_per_expert;
  a.token_per_rank = token_per_rank;
  a.send_token_idx = send_token_idx;
  a.bad_count = bad_id_count;
  a.put_offset = put_offset;
  a.recv_count = recv_count;
  a.recv_base = recv_base;
  a.recv_token_per_expert = recv_token_per_expert;
  a.recv = static_cast<uint8_t*>(recv_x);
  a.row_bytes = static_cast<int64_t>(rb);
  a.cap_rows = static_cast<int64_t>(recv_x_bytes / rb);
  a.scale_off = static_cast<int32_t>(align32(hidden));
  const moe::Half xt = x_type == MOE_FP16 ? moe::Half::kFp16 : moe::Half::kBf16;
  return hip_status(moe::launch_fused(a, xt, quant_int8 != 0, groups, static_cast<hipStream_t>(stream)));
}

int moe_deq_swiglu_quant(const int32_t* acc, int32_t rows, int32_t n, const float* weight_scale,
                         const void* token_scale, int64_t token_scale_stride, void* out, size_t out_bytes,
                         void* stream) {
  if (rows < 0 || n < 1 || token_scale_stride < 4 || token_scale_stride % 4 != 0) return MOE_ERR_BAD_SHAPE;
  if (n % 4 != 0 || n > moe::kEpilogueMaxN) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!acc || !weight_scale || !token_scale || !out) return MOE_ERR_NULL_PTR;
  if (!aligned(acc, 16) || !aligned(weight_scale, 16) || !aligned(out, 16) || !aligned(token_scale, 4))
    return MOE_ERR_BAD_ALIGN;
  size_t rb = 0;
  int st = row_bytes(n, MOE_INT8_ROWSCALE, &rb);
  if (st) return st;
  if (out_bytes / rb < static_cast<size_t>(rows)) return MOE_ERR_BUFFER_TOO_SMALL;
  moe::EpilogueArgs a{};
  a.acc = acc;
  a.weight_scale = weight_scale;
  a.token_scale = token_scale;
  a.rows = rows;
  a.ts_stride = token_scale_stride;
  a.n = n;
  a.out = static_cast<uint8_t*>(out);
  a.out_row_bytes = static_cast<int64_t>(rb);
  a.scale_off = static_cast<int32_t>(align32(n));
  return hip_status(moe::launch_deq_swiglu_quant(a, static_cast<hipStream_t>(stream)));
}

int moe_grouped_gemm_i8(const void* a, int64_t a_row_bytes, int32_t rows, int32_t k,
                        const int32_t* group_count, int32_t groups, const void* w, int32_t n,
                        int32_t* out, size_t out_bytes, void* stream) {
  if (rows < 0 || k < 1 || n < 1 || groups < 1 || a_row_bytes < k) return MOE_ERR_BAD_SHAPE;
  if (k % 16 != 0 || k > MOE_GEMM_MAX_K || n > MOE_GEMM_MAX_N || groups > MOE_GEMM_MAX_GROUPS)
    return MOE_ERR_UNSUPPORTED;
  if (a_row_bytes % 16 != 0) return MOE_ERR_BAD_ALIGN;
  if (rows == 0) return MOE_OK;
  if (!a || !group_count || !w || !out) return MOE_ERR_NULL_PTR;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(group_count, 4) || !aligned(out, 4))
    return MOE_ERR_BAD_ALIGN;
  if (out_bytes / 4u / static_cast<size_t>(n) < static_cast<size_t>(rows)) return MOE_ERR_BUFFER_TOO_SMALL;
  if (moe::grouped_gemm_blocks(rows, groups, n) > moe::kGemmMaxBlocks) return MOE_ERR_UNSUPPORTED;
  moe::GemmArgs g{};
  g.a = static_cast<const int8_t*>(a);
  g.a_stride = a_row_bytes;
  g.rows = rows;
  g.k = k;
  g.group_count = group_count;
  g.groups = groups;
  g.w = static_cast<const int8_t*>(w);
  g.n = n;
  g.out = out;
  return hip_status(moe::launch_grouped_gemm_i8(g, static_cast<hipStream_t>(stream)));
}

namespace {
constexpr size_t align256(size_t v) { return (v + 255) / 256 * 256; }
size_t swiglu_act_bytes(int32_t rows, int32_t n) {
  return align256(static_cast<size_t>(rows) * static_cast<size_t>(n) * 4u);
}
}  // namespace

int moe_gemm_swiglu_quant_workspace_bytes(int32_t rows, int32_t n, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL_PTR;
  if (rows < 0 || n < 1) return MOE_ERR_BAD_SHAPE;
  *bytes = swiglu_act_bytes(rows, n) + align256(static_cast<size_t>(rows) * 4u);
  return MOE_OK;
}

int moe_grouped_gemm_swiglu_quant_i8(const void* a, int64_t a_row_bytes, int32_t rows, int32_t k,
                                     const int32_t* group_count, int32_t groups, const void* w, int32_t n,
                                     const float* weight_scale, const void* token_scale,
                                     int64_t token_scale_stride, void* out, size_t out_bytes, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (rows < 0 || k < 1 || n < 1 || groups < 1 || a_row_bytes < k || token_scale_stride < 4 ||
      token_scale_stride % 4 != 0)
    return MOE_ERR_BAD_SHAPE;
  if (k % 16 != 0 || k > MOE_GEMM_MAX_K || n % 4 != 0 || n > MOE_GEMM_MAX_N / 2 || groups > MOE_GEMM_MAX_GROUPS)
    return MOE_ERR_UNSUPPORTED;
  if (a_row_bytes % 16 != 0) return MOE_ERR_BAD_ALIGN;
  if (rows == 0) return MOE_OK;
  if (!a || !group_count || !w || !weight_scale || !token_scale || !out || !workspace) return MOE_ERR_NULL_PTR;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(group_count, 4) || !aligned(weight_scale, 4) ||
      !aligned(token_scale, 4) || !aligned(out, 16) || !aligned(workspace, 16))
    return MOE_ERR_BAD_ALIGN;
  size_t rb = 0;
  int st = row_bytes(n, MOE_INT8_ROWSCALE, &rb);
  if (st) return st;
  if (out_bytes / rb < static_cast<size_t>(rows)) return MOE_ERR_BUFFER_TOO_SMALL;
  size_t need = 0;
  st = moe_gemm_swiglu_quant_workspace_bytes(rows, n, &need);
  if (st) return st;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (moe::grouped_gemm_swiglu_blocks(rows, groups, n) > moe::kGemmMaxBlocks) return MOE_ERR_UNSUPPORTED;
  moe::GemmArgs g{};
  g.a = static_cast<const int8_t*>(a);
  g.a_stride = a_row_bytes;
  g.rows = rows;
  g.k = k;
  g.group_count = group_count;
  g.groups = groups;
  g.w = static_cast<const int8_t*>(w);
  g.n = 2 * n;
  g.sn = n;
  g.weight_scale = weight_scale;
  g.token_scale = static_cast<const uint8_t*>(token_scale);
  g.ts_stride = token_scale_stride;
  g.act = static_cast<float*>(workspace);
  g.amax = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + swiglu_act_bytes(rows, n));
  g.q_out = static_cast<uint8_t*>(out);
  g.q_row_bytes = static_cast<int64_t>(rb);
  g.q_scale_off = static_cast<int32_t>(align32(n));
  return hip_status(moe::launch_grouped_gemm_swiglu_quant(g, static_cast<hipStream_t>(stream)));
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_PTR: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "bad shape (a size is out of range)";
    case MOE_ERR_BAD_ALIGN: return "pointer or row stride not aligned as the entry point requires";
    case MOE_ERR_BAD_DTYPE: return "unsupported element type for this argument";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than its size query returns";
    case MOE_ERR_BUFFER_TOO_SMALL: return "receive or output buffer smaller than the call needs";
    case MOE_ERR_UNSUPPORTED: return "size outside the library's limits (MOE_MAX_*, MOE_GEMM_MAX_*, divisibility)";
    case MOE_ERR_HIP: return "HIP launch failed (see moe_last_hip_error)";
    case MOE_ERR_SCRATCH_LIMIT:
      return "shape needs more workspace than the static scratch of the no-alloc entry point "
             "(MOE_NO_ALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
