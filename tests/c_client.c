/*
 * A plain C client of libmoe_ep.so: the four stages of the EP-normal
 * pipeline ("UMDK/CAM communication acceleration library deep analysis v2",
 * section 2: layout 2.3, notify 2.4, dispatch with dynamic int8 2.5,
 * combine 2.6) and their one-launch form (section 3.2), then the expert side
 * on the receive buffer in place (section 4.3 stage 2: the grouped int8
 * matmul GMM1 over the received experts' rows, and the same matmul with its
 * section 4.8.1 dequant + SwiGLU + int8 epilogue fused), driven through the
 * C ABI with the HIP runtime alone -- no Python, no torch -- and every output
 * compared bit for bit with the CPU oracle (liboracle.so, test
 * infrastructure) on the same inputs; the oracle's expert side reads the
 * oracle's own receive rows.
 *
 * Inputs come from splitmix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014) as raw bit patterns: bf16 rows with
 * exponents spread over 2^-7 .. 2^3 and one all-zero row, k distinct expert
 * ids per token with about 2 % of the entries replaced by ids outside
 * [0, E), and routing weights in (0, 1); int8 expert weights uniform, and
 * column scales near 2^-13 so that the gate values come out of order 1.
 *
 * Exit status 0 when every comparison holds, 1 on a mismatch, 2 on a call
 * that fails.  Test program only.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"

/* The oracle's entry points (oracle/moe_oracle.c). */
#define KIND_BF16 0
#define KIND_INT8 3
int oracle_layout(const int32_t *topk_idx, int64_t bs, int64_t k, int64_t epr, int64_t ranks,
                  int32_t *token_per_expert, int32_t *token_per_rank, int32_t *send_token_idx,
                  int64_t *bad_count);
int oracle_notify(const int32_t *token_per_expert, int64_t epr, int64_t ranks, int32_t *put_offset,
                  int32_t *recv_count, int32_t *recv_base, int32_t *recv_token_per_expert);
int oracle_dispatch(const uint16_t *x, int x_kind, int64_t bs, int64_t h, int64_t k, const int32_t *topk_idx,
                    const int32_t *send_token_idx, const int32_t *put_offset, const int32_t *recv_base,
                    int64_t epr, int64_t ranks, int quant, int64_t rows, uint16_t *recv_rows, int8_t *codes,
                    float *inv);
int oracle_grouped_gemm_i8(const int8_t *a, int64_t a_stride, int64_t rows, int64_t k,
                           const int32_t *group_count, int64_t groups, const int8_t *w, int64_t n,
                           const int64_t *row_list, int64_t nlist, int32_t *out, int32_t *row_group);
int oracle_swiglu_quant_row(const int32_t *acc, int64_t n, const float *weight_scale, float token_scale,
                            int8_t *codes, float *inv, float *act_out);
int oracle_combine(const uint16_t *recv_rows, const int8_t *codes, const float *inv, int recv_kind, int64_t bs,
                   int64_t h, int64_t k, const int32_t *topk_idx, const float *topk_w,
                   const int32_t *send_token_idx, const int32_t *put_offset, const int32_t *recv_base,
                   int64_t epr, int64_t ranks, int64_t rows, void *out, int out_kind, float *acc_scratch);

/* H % 16 == 0 (the matmul's k) but not a multiple of 32 (a ragged scale
 * offset); NA activation columns from 2 NA gate and up columns per expert. */
enum { BS = 300, H = 528, K = 6, EPR = 4, R = 8, E = EPR * R, N = BS * K, NA = 64 };

static uint64_t rng_state = 0x5eed0c11e47ULL;
static uint64_t splitmix64(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ULL);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

#define HIP_OK(call)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(2);                                                                            \
    }                                                                                     \
  } while (0)

#define MOE_OK_(call)                                                                     \
  do {                                                                                    \
    int s_ = (call);                                                                      \
    if (s_ != MOE_OK) {                                                                   \
      fprintf(stderr, "%s:%d: %s -> status %d (%s)\n", __FILE__, __LINE__, #call, s_,     \
              moe_status_str(s_));                                                        \
      exit(2);                                                                            \
    }                                                                                     \
  } while (0)

static void *dev_alloc(size_t bytes) {
  void *p = NULL;
  HIP_OK(hipMalloc(&p, bytes ? bytes : 4));
  HIP_OK(hipMemset(p, 0, bytes ? bytes : 4));
  return p;
}

static void *dev_copy(const void *host, size_t bytes) {
  void *p = dev_alloc(bytes);
  HIP_OK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
  return p;
}

static void *host_copy(const void *dev, size_t bytes) {
  void *p = malloc(bytes);
  if (!p) exit(2);
  HIP_OK(hipMemcpy(p, dev, bytes, hipMemcpyDeviceToHost));
  return p;
}

static int failures = 0;
static void expect_equal(const char *what, const void *got, const void *want, size_t bytes) {
  if (memcmp(got, want, bytes) != 0) {
    const uint8_t *g = (const uint8_t *)got, *w = (const uint8_t *)want;
    size_t i = 0;
    while (g[i] == w[i]) ++i;
    fprintf(stderr, "MISMATCH %s at byte %zu of %zu\n", what, i, bytes);
    ++failures;
  }
}

/* Receive rows of the GPU buffer (codes at [0, H), inverse scale at
 * align32(H)) against the oracle's codes and inverse scales. */
static void expect_rows(const char *what, const uint8_t *recv, size_t row_bytes, const int8_t *codes,
                        const float *inv) {
  const size_t scale_off = (H + 31) / 32 * 32;
  for (int r = 0; r < N; ++r) {
    const uint8_t *row = recv + (size_t)r * row_bytes;
    if (memcmp(row, codes + (size_t)r * H, H) != 0 || memcmp(row + scale_off, inv + r, 4) != 0) {
      fprintf(stderr, "MISMATCH %s: receive row %d\n", what, r);
      ++failures;
      return;
    }
  }
}

/* The expert side on the receive buffer in place: the grouped matmul to
 * int32, and the fused matmul + epilogue to int8 rows, against the oracle's
 * matmul and row epilogue over the oracle's receive rows. */
static void expert_side(const void *d_recv, size_t row_bytes, const int32_t *d_counts, const int8_t *o_codes,
                        const float *o_inv, const int32_t *o_counts) {
  const size_t wbytes = (size_t)E * 2 * NA * H;
  int8_t *w = malloc(wbytes);
  float *ws = malloc(sizeof(float) * E * 2 * NA);
  if (!w || !ws) exit(2);
  for (size_t i = 0; i < wbytes; ++i) w[i] = (int8_t)(splitmix64() >> 56);
  for (int i = 0; i < E * 2 * NA; ++i) {
    const uint64_t u = splitmix64();
    const uint32_t bits = (uint32_t)(112 + u % 4) << 23 | (uint32_t)((u >> 8) & 0x7fffff);
    memcpy(&ws[i], &bits, 4);
  }
  void *d_w = dev_copy(w, wbytes);
  void *d_ws = dev_copy(ws, sizeof(float) * E * 2 * NA);
  int32_t *d_acc = NULL;
  HIP_OK(hipMalloc((void **)&d_acc, sizeof(int32_t) * N * 2 * NA));
  HIP_OK(hipMemset(d_acc, 0x5a, sizeof(int32_t) * N * 2 * NA));
  size_t q_bytes = 0, wsp_bytes = 0;
  MOE_OK_(moe_recv_row_bytes(NA, MOE_INT8_ROWSCALE, &q_bytes));
  MOE_OK_(moe_gemm_swiglu_quant_workspace_bytes(N, NA, &wsp_bytes));
  uint8_t *d_q = NULL;
  HIP_OK(hipMalloc((void **)&d_q, q_bytes * N));
  HIP_OK(hipMemset(d_q, 0xa5, q_bytes * N));
  void *d_wsp = dev_alloc(wsp_bytes);
  const size_t scale_off = (H + 31) / 32 * 32;
  MOE_OK_(moe_grouped_gemm_i8(d_recv, (int64_t)row_bytes, N, H, d_counts, E, d_w, 2 * NA, d_acc,
                              sizeof(int32_t) * N * 2 * NA, NULL));
  MOE_OK_(moe_grouped_gemm_swiglu_quant_i8(d_recv, (int64_t)row_bytes, N, H, d_counts, E, d_w, NA, d_ws,
                                           (const uint8_t *)d_recv + scale_off, (int64_t)row_bytes, d_q,
                                           q_bytes * N, d_wsp, wsp_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());
  int32_t *acc = host_copy(d_acc, sizeof(int32_t) * N * 2 * NA);
  uint8_t *q = host_copy(d_q, q_bytes * N);

  int32_t *o_acc = calloc((size_t)N * 2 * NA, sizeof(int32_t));
  int32_t *o_grp = malloc(sizeof(int32_t) * N);
  if (!o_acc || !o_grp) exit(2);
  if (oracle_grouped_gemm_i8(o_codes, H, N, H, o_counts, E, w, 2 * NA, NULL, N, o_acc, o_grp)) {
    fprintf(stderr, "oracle matmul failed\n");
    exit(2);
  }
  int owned = 0, bad_acc = -1, bad_q = -1;
  for (int m = 0; m < N; ++m) {
    const uint8_t *row = q + (size_t)m * q_bytes;
    if (o_grp[m] < 0) {
      /* rows of no expert: neither call writes them */
      for (int j = 0; j < 2 * NA; ++j)
        if (acc[(size_t)m * 2 * NA + j] != 0x5a5a5a5a && bad_acc < 0) bad_acc = m;
      for (size_t b = 0; b < q_bytes; ++b)
        if (row[b] != 0xa5 && bad_q < 0) bad_q = m;
      continue;
    }
    ++owned;
    if (memcmp(acc + (size_t)m * 2 * NA, o_acc + (size_t)m * 2 * NA, sizeof(int32_t) * 2 * NA) && bad_acc < 0)
      bad_acc = m;
    int8_t codes[NA];
    float inv = 0;
    if (oracle_swiglu_quant_row(o_acc + (size_t)m * 2 * NA, NA, ws + (size_t)o_grp[m] * 2 * NA, o_inv[m], codes,
                                &inv, NULL)) {
      fprintf(stderr, "oracle epilogue failed on row %d\n", m);
      exit(2);
    }
    if ((memcmp(row, codes, NA) || memcmp(row + (NA + 31) / 32 * 32, &inv, 4)) && bad_q < 0) bad_q = m;
  }
  if (bad_acc >= 0) fprintf(stderr, "MISMATCH grouped matmul: row %d\n", bad_acc);
  if (bad_q >= 0) fprintf(stderr, "MISMATCH fused matmul + epilogue: row %d\n", bad_q);
  failures += (bad_acc >= 0) + (bad_q >= 0);
  printf("c client, expert side on the receive buffer: %s (%d owned rows of %d, %d experts, k %d, "
         "%d gate + %d up columns)\n",
         bad_acc < 0 && bad_q < 0 ? "bit-exact" : "MISMATCH", owned, N, E, H, NA, NA);
  free(w); free(ws); free(acc); free(q); free(o_acc); free(o_grp);
  HIP_OK(hipFree(d_w)); HIP_OK(hipFree(d_ws)); HIP_OK(hipFree(d_acc)); HIP_OK(hipFree(d_q));
  HIP_OK(hipFree(d_wsp));
}

int main(void) {
  /* inputs */
  uint16_t *x = malloc(sizeof(uint16_t) * BS * H);
  int32_t *idx = malloc(sizeof(int32_t) * N);
  float *w = malloc(sizeof(float) * N);
  if (!x || !idx || !w) return 2;
  for (int t = 0; t < BS; ++t)
    for (int i = 0; i < H; ++i) {
      const uint64_t u = splitmix64();
      const uint16_t sign = (uint16_t)((u & 1u) << 15);
      const uint16_t expo = (uint16_t)(120 + (u >> 1) % 11);
      const uint16_t mant = (uint16_t)((u >> 8) & 0x7f);
      x[(size_t)t * H + i] = t == 7 ? 0 : (uint16_t)(sign | (expo << 7) | mant);
    }
  for (int t = 0; t < BS; ++t)
    for (int j = 0; j < K; ++j) {
      int e, again;
      do {
        e = (int)(splitmix64() % E);
        again = 0;
        for (int q = 0; q < j; ++q) again |= idx[t * K + q] == e;
      } while (again);
      idx[t * K + j] = e;
      const uint64_t u = splitmix64();
      if (u % 50 == 0) idx[t * K + j] = (u >> 8) % 2 ? -1 : E + 5;
      const uint32_t bits = (uint32_t)(120 + (u >> 16) % 7) << 23 | (uint32_t)((u >> 24) & 0x7fffff);
      memcpy(&w[t * K + j], &bits, 4);
    }

  size_t row_bytes = 0, ws_bytes = 0;
  MOE_OK_(moe_recv_row_bytes(H, MOE_INT8_ROWSCALE, &row_bytes));
  MOE_OK_(moe_layout_workspace_bytes(BS, K, E, &ws_bytes));

  /* the oracle */
  int32_t o_tpe[E], o_tpr[R], o_po[E], o_rc[R], o_rb[R], o_rtpe[E];
  int32_t *o_sti = malloc(sizeof(int32_t) * N);
  int8_t *o_codes = calloc((size_t)N * H, 1);
  float *o_inv = calloc(N, sizeof(float));
  uint16_t *o_out = malloc(sizeof(uint16_t) * BS * H);
  float *acc = malloc(sizeof(float) * H);
  int64_t o_bad = 0;
  if (!o_sti || !o_codes || !o_inv || !o_out || !acc) return 2;
  if (oracle_layout(idx, BS, K, EPR, R, o_tpe, o_tpr, o_sti, &o_bad) ||
      oracle_notify(o_tpe, EPR, R, o_po, o_rc, o_rb, o_rtpe) ||
      oracle_dispatch(x, KIND_BF16, BS, H, K, idx, o_sti, o_po, o_rb, EPR, R, 1, N, NULL, o_codes, o_inv) ||
      oracle_combine(NULL, o_codes, o_inv, KIND_INT8, BS, H, K, idx, w, o_sti, o_po, o_rb, EPR, R, N, o_out,
                     KIND_BF16, acc)) {
    fprintf(stderr, "oracle call failed\n");
    return 2;
  }

  /* the library: four calls on one stream, then the one-launch form */
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void *d_x = dev_copy(x, sizeof(uint16_t) * BS * H);
  void *d_idx = dev_copy(idx, sizeof(int32_t) * N);
  void *d_w = dev_copy(w, sizeof(float) * N);
  void *d_ws = dev_alloc(ws_bytes);
  for (int form = 0; form < 2; ++form) {
    int32_t *d_tpe = dev_alloc(4 * E), *d_tpr = dev_alloc(4 * R), *d_sti = dev_alloc(4 * N);
    int32_t *d_bad = dev_alloc(4), *d_po = dev_alloc(4 * E), *d_rc = dev_alloc(4 * R);
    int32_t *d_rb = dev_alloc(4 * R), *d_rtpe = dev_alloc(4 * E);
    void *d_recv = dev_alloc((size_t)N * row_bytes);
    void *d_out = dev_alloc(sizeof(uint16_t) * BS * H);
    if (form == 0) {
      MOE_OK_(moe_layout(d_idx, BS, K, EPR, R, d_tpe, d_tpr, d_sti, d_bad, d_ws, ws_bytes, stream));
      MOE_OK_(moe_notify(d_tpe, EPR, R, d_po, d_rc, d_rb, d_rtpe, stream));
      MOE_OK_(moe_dispatch(d_x, MOE_BF16, BS, H, K, d_idx, d_sti, d_po, d_rb, EPR, R, 1, d_recv,
                           (size_t)N * row_bytes, stream));
    } else {
      int one = 0;
      MOE_OK_(moe_fused_supported(BS, H, K, EPR, R, MOE_BF16, 1, &one));
      if (!one) {
        fprintf(stderr, "expected the one-kernel form at this shape\n");
        return 1;
      }
      MOE_OK_(moe_layout_notify_dispatch(d_x, MOE_BF16, BS, H, K, d_idx, EPR, R, 1, d_tpe, d_tpr, d_sti, d_bad,
                                         d_po, d_rc, d_rb, d_rtpe, d_recv, (size_t)N * row_bytes, d_ws,
                                         ws_bytes, stream));
    }
    MOE_OK_(moe_combine(d_recv, MOE_INT8_ROWSCALE, (size_t)N * row_bytes, BS, H, K, d_idx, d_w, d_sti, d_po,
                        d_rb, EPR, R, d_out, MOE_BF16, stream));
    HIP_OK(hipStreamSynchronize(stream));

    const char *name = form == 0 ? "four calls" : "one launch + combine";
    int32_t *g;
    expect_equal("tokenPerExpert", g = host_copy(d_tpe, 4 * E), o_tpe, 4 * E); free(g);
    expect_equal("tokenPerRank", g = host_copy(d_tpr, 4 * R), o_tpr, 4 * R); free(g);
    expect_equal("sendTokenIdx", g = host_copy(d_sti, 4 * N), o_sti, 4 * N); free(g);
    g = host_copy(d_bad, 4);
    if ((int64_t)g[0] != o_bad) {
      fprintf(stderr, "MISMATCH badIdCount %d vs %lld\n", g[0], (long long)o_bad);
      ++failures;
    }
    free(g);
    expect_equal("putOffset", g = host_copy(d_po, 4 * E), o_po, 4 * E); free(g);
    expect_equal("recvCount", g = host_copy(d_rc, 4 * R), o_rc, 4 * R); free(g);
    expect_equal("recvBase", g = host_copy(d_rb, 4 * R), o_rb, 4 * R); free(g);
    expect_equal("recvTokenPerExpert", g = host_copy(d_rtpe, 4 * E), o_rtpe, 4 * E); free(g);
    uint8_t *recv = host_copy(d_recv, (size_t)N * row_bytes);
    expect_rows(name, recv, row_bytes, o_codes, o_inv);
    free(recv);
    uint16_t *out = host_copy(d_out, sizeof(uint16_t) * BS * H);
    expect_equal("combine output", out, o_out, sizeof(uint16_t) * BS * H);
    free(out);
    if (form == 0) expert_side(d_recv, row_bytes, d_rtpe, o_codes, o_inv, o_rtpe);
    printf("c client, %s: %s (bs %d, h %d, topk %d, %d experts, %d ranks, %lld bad ids)\n", name,
           failures ? "MISMATCH" : "bit-exact", BS, H, K, E, R, (long long)o_bad);
    HIP_OK(hipFree(d_tpe)); HIP_OK(hipFree(d_tpr)); HIP_OK(hipFree(d_sti)); HIP_OK(hipFree(d_bad));
    HIP_OK(hipFree(d_po)); HIP_OK(hipFree(d_rc)); HIP_OK(hipFree(d_rb)); HIP_OK(hipFree(d_rtpe));
    HIP_OK(hipFree(d_recv)); HIP_OK(hipFree(d_out));
  }
  HIP_OK(hipFree(d_x)); HIP_OK(hipFree(d_idx)); HIP_OK(hipFree(d_w)); HIP_OK(hipFree(d_ws));
  HIP_OK(hipStreamDestroy(stream));
  free(x); free(idx); free(w); free(o_sti); free(o_codes); free(o_inv); free(o_out); free(acc);
  return failures ? 1 : 0;
}
