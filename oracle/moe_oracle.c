/*
 * CPU oracle for the MoE expert-parallel "EP normal" dispatch/combine
 * pipeline: layout -> notify -> dispatch (optional dynamic int8 quant) ->
 * combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source
 * with the HIP library and the HIP library never calls it.
 *
 * Source of the method: the page "UMDK/CAM communication acceleration library
 * deep analysis v2" (backyes.github.io, CAM v2 analysis), section 2 "EP Normal
 * communication operators":
 *   2.1  the four stages and their order,
 *   2.2.1 comm_args.h (UB_ALIGN_SIZE = 32 bytes; the CommArgs scalars),
 *   2.3  moe_dispatch_layout_zb (per-expert counts, per-(token,k) send index),
 *   2.4  moe_notify_dispatch_zb (prefix sums: putOffset, receive counts; with
 *        several source ranks, over the all-gathered count matrix),
 *   2.5  moe_dispatch_normal_zb / QuantProcess (row scatter, dynamic int8),
 *   2.6  moe_combine_normal_zb / ReadBufferAndWeightedSum (weighted gather),
 *   2.8  the per-rank zero-buffer layout (token region read by combine).
 * and, for the expert side between dispatch and combine, section 4
 * "Fused Deep MoE": 4.3 (stage 2: GMM1, int8 x int8 -> int32, then
 * DeqSwigluQuant), 4.6 (the per-expert cumulative token counts, gmGroupList)
 * and 4.8.1 (the GMM1 epilogue PerTokenDequantSwiGLU).
 *
 * Everything here is the plain definition, in the order the page gives,
 * single-threaded, in IEEE binary32 where the page fixes float (the quantiser
 * and the combine accumulator are float on the page).  Build with
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 * so that every multiply and every add is rounded on its own.
 *
 * Readings taken where the page leaves a step open:
 *  - send slots are the stable counting-sort rank: entries of one expert are
 *    numbered in flat (token, k) order, token-ascending;
 *  - per-rank counts count rows (one per (token, k) entry), since combine
 *    reads one row per entry;
 *  - on one device the logical ranks' receive regions are concatenated in
 *    rank order with no gaps, and inside a rank the experts' rows are
 *    contiguous in expert order; with several sources, an expert's rows are
 *    ordered by source rank, then by send slot;
 *  - the quantiser stores the inverse scale 1/s; combine dequantises with
 *    (float)q * inv before the weight multiply;
 *  - combine sums j = 0..k-1 from +0.0f, multiply then add, each rounded;
 *  - expert ids outside [0, E) are counted as bad, get slot -1, are not
 *    dispatched and add nothing in combine;
 *  - the epilogue's SwiGLU is Swish(gate) * up with the gate in the first
 *    half of the accumulator row (the page shows x*sigmoid(x) on the left
 *    half and the right half passed through, but not the product), and its
 *    output row is quantised like a dispatched row; e^x is computed by a
 *    named published method, written out (exp_cw);
 *  - the first expert matmul (GMM1) gives expert g the rows [S_g, S_g + c_g)
 *    of the receive buffer, S_g the sum of the counts before g (a negative
 *    count counts as 0), takes its weights as [groups][n][k] (one k-vector
 *    per output column) and sums the int8 products exactly into int32.
 *
 * Parity pins live in tests/ (brute force, stable-sort and prefix-sum
 * equivalence, hand-worked quantiser rows, order-sensitive combine rows,
 * float64 error bounds, exhaustive conversion checks).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_INTERNAL (-2)

/* Element kinds used by the oracle's entry points. */
#define KIND_BF16 0
#define KIND_FP16 1
#define KIND_FP32 2
#define KIND_INT8 3

/* ------------------------------------------------------------------------ */
/* Scalar conversions, written from the IEEE 754 / bfloat16 definitions.     */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t f32_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* bfloat16 is the upper half of a binary32: widening is exact. */
static float bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/* binary16 -> binary32, exact: value = (-1)^s * m * 2^(exp-25) for normal
 * numbers with implicit bit, m * 2^-24 for subnormals. */
static float f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1F;
  int man = h & 0x3FF;
  float mag;
  if (exp == 0) {
    mag = ldexpf((float)man, -24);
  } else if (exp == 31) {
    mag = man ? NAN : INFINITY;
  } else {
    mag = ldexpf((float)(1024 + man), exp - 25);
  }
  return sign ? -mag : mag;
}

/* binary32 -> bfloat16 with round-half-to-even.  The two candidates are the
 * truncation T (upper 16 bits) and T + 1; the discarded low half decides:
 * above 0x8000 rounds up, below rounds down, exactly 0x8000 picks the even
 * one.  Carries ripple into the exponent, which is the correct result
 * (including rounding up to infinity). */
static uint16_t f32_to_bf16(float f) {
  uint32_t u = f32_to_bits(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, keep sign */
  }
  uint32_t upper = u >> 16;
  uint32_t lower = u & 0xFFFFu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* binary32 -> binary16 with round-half-to-even, from the definition: find
 * the binade of |f|, scale the significand to an integer count of binary16
 * ulps in double (exact), round that count to nearest-even, re-encode. */
static uint16_t f32_to_f16(float f) {
  uint16_t sign = (f32_to_bits(f) >> 16) & 0x8000u;
  if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
  double a = fabs((double)f);
  if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: ulp is 2^-24; a count of 1024 is the smallest normal,
     * whose encoding 0x0400 is the same integer. */
    double m = nearbyint(a * ldexp(1.0, 24));
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e2;
  (void)frexp(a, &e2); /* a = fr * 2^e2, fr in [0.5, 1) */
  int e = e2 - 1;      /* a in [2^e, 2^(e+1)) */
  double m = nearbyint(ldexp(a, 10 - e)); /* in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
}

static float to_f32(uint16_t v, int kind) {
  return kind == KIND_FP16 ? f16_to_f32(v) : bf16_to_f32(v);
}

/* Array forms, exported so the tests can pin the conversions exhaustively. */
int oracle_bf16_to_f32(const uint16_t *in, float *out, int64_t n) {
  if ((n && (!in || !out)) || n < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
  return ORACLE_OK;
}
int oracle_f16_to_f32(const uint16_t *in, float *out, int64_t n) {
  if ((n && (!in || !out)) || n < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f32(in[i]);
  return ORACLE_OK;
}
int oracle_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
  if ((n && (!in || !out)) || n < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
  return ORACLE_OK;
}
int oracle_f32_to_f16(const float *in, uint16_t *out, int64_t n) {
  if ((n && (!in || !out)) || n < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16(in[i]);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Stage 1: dispatch layout (page section 2.3).                              */
/* ------------------------------------------------------------------------ */

/* tokenPerExpert[e] = number of (t, j) with topkIdx[t, j] == e.
 * sendTokenIdx[t, j] = how many earlier entries (in flat t*k + j order) went
 * to the same expert -- the entry's position inside its expert's region.
 * tokenPerRank[r] = sum of tokenPerExpert over rank r's experts
 * e in [r*EPR, (r+1)*EPR).  Ids outside [0, E) are bad: slot -1. */
int oracle_layout(const int32_t *topk_idx, int64_t bs, int64_t k, int64_t epr,
                  int64_t ranks, int32_t *token_per_expert, int32_t *token_per_rank,
                  int32_t *send_token_idx, int64_t *bad_count) {
  if (bs < 0 || k < 1 || epr < 1 || ranks < 1) return ORACLE_BAD_ARG;
  if (!token_per_expert || !token_per_rank || !bad_count) return ORACLE_BAD_ARG;
  if (bs > 0 && (!topk_idx || !send_token_idx)) return ORACLE_BAD_ARG;
  int64_t num_experts = epr * ranks;

  for (int64_t e = 0; e < num_experts; ++e) token_per_expert[e] = 0;
  int64_t bad = 0;
  for (int64_t t = 0; t < bs; ++t) {
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < 0 || e >= num_experts) {
        send_token_idx[t * k + j] = -1;
        bad += 1;
        continue;
      }
      send_token_idx[t * k + j] = token_per_expert[e];
      token_per_expert[e] += 1;
    }
  }
  for (int64_t r = 0; r < ranks; ++r) {
    int32_t sum = 0;
    for (int64_t e = r * epr; e < (r + 1) * epr; ++e) sum += token_per_expert[e];
    token_per_rank[r] = sum;
  }
  *bad_count = bad;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Stage 2: notify (page section 2.4).                                       */
/* ------------------------------------------------------------------------ */

/* With one source the all-gather of tokenPerExpert is the identity.  Inside
 * each destination rank r the experts' regions follow each other in expert
 * order: putOffset[e] = sum of the counts of r's earlier experts, and
 * recvCount[r] = the total of r's experts.  The ranks' regions follow each
 * other in rank order: recvBase[r] = sum of recvCount[r'] for r' < r.
 * recvTokenPerExpert is the per-expert receive count (one source: the same
 * numbers as the input). */
int oracle_notify(const int32_t *token_per_expert, int64_t epr, int64_t ranks,
                  int32_t *put_offset, int32_t *recv_count, int32_t *recv_base,
                  int32_t *recv_token_per_expert) {
  if (epr < 1 || ranks < 1) return ORACLE_BAD_ARG;
  if (!token_per_expert || !put_offset || !recv_count || !recv_base || !recv_token_per_expert)
    return ORACLE_BAD_ARG;
  int32_t base = 0;
  for (int64_t r = 0; r < ranks; ++r) {
    int32_t acc = 0;
    for (int64_t e = r * epr; e < (r + 1) * epr; ++e) {
      put_offset[e] = acc;
      acc += token_per_expert[e];
      recv_token_per_expert[e] = token_per_expert[e];
    }
    recv_count[r] = acc;
    recv_base[r] = base;
    base += acc;
  }
  return ORACLE_OK;
}

/* Stage 2 with several source ranks (page section 2.4: every rank's
 * tokenPerExpert is all-gathered, then prefix sums give the write offsets;
 * section 2.6 reads the offset of (expert e, source s) at index
 * e * epWorldSize + s).  Input: token_per_expert[s][e] for num_src sources.
 * Inside destination rank r the rows are ordered by expert, then by source:
 *   for r: acc = 0
 *     for e of r ascending, for s = 0 .. num_src-1:
 *       put_offset[e][s] = acc; acc += count[s][e]
 *     recv_count[r] = acc
 * recv_base[r] concatenates the ranks' regions in rank order, and
 * recv_token_per_expert[e] = sum over s of count[s][e].  With one source this
 * is oracle_notify. */
int oracle_notify_multi(const int32_t *token_per_expert, int64_t num_src, int64_t epr,
                        int64_t ranks, int32_t *put_offset, int32_t *recv_count,
                        int32_t *recv_base, int32_t *recv_token_per_expert) {
  if (num_src < 1 || epr < 1 || ranks < 1) return ORACLE_BAD_ARG;
  if (!token_per_expert || !put_offset || !recv_count || !recv_base || !recv_token_per_expert)
    return ORACLE_BAD_ARG;
  int64_t num_experts = epr * ranks;
  int32_t base = 0;
  for (int64_t r = 0; r < ranks; ++r) {
    int32_t acc = 0;
    for (int64_t e = r * epr; e < (r + 1) * epr; ++e) {
      int32_t sum = 0;
      for (int64_t src = 0; src < num_src; ++src) {
        int32_t c = token_per_expert[src * num_experts + e];
        put_offset[e * num_src + src] = acc;
        acc += c;
        sum += c;
      }
      recv_token_per_expert[e] = sum;
    }
    recv_count[r] = acc;
    recv_base[r] = base;
    base += acc;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Stage 3: dispatch (page section 2.5).                                     */
/* ------------------------------------------------------------------------ */

/* QuantProcess for one row of h elements:
 *   f_i  = float(x_i)                          (exact widening)
 *   amax = max_i |f_i|
 *   s    = 127.0f / (amax + 1e-12f)            (binary32 add, then divide)
 *   q_i  = round-half-even(f_i * s)            (one binary32 multiply)
 *   inv  = 1.0f / s                            (stored after the row)
 * The page's cast chain int32 -> half -> int8 is exact here: |f_i * s| can
 * not reach 127.5, so q_i is already in [-127, 127]. */
int oracle_quant_row(const uint16_t *x, int x_kind, int64_t h, int8_t *codes, float *inv,
                     float *scale_out) {
  if (!x || !codes || !inv || h < 1) return ORACLE_BAD_ARG;
  if (x_kind != KIND_BF16 && x_kind != KIND_FP16) return ORACLE_BAD_ARG;
  float amax = 0.0f;
  for (int64_t i = 0; i < h; ++i) {
    float a = fabsf(to_f32(x[i], x_kind));
    if (a > amax) amax = a;
  }
  float denom = amax + 1e-12f;
  float s = 127.0f / denom;
  for (int64_t i = 0; i < h; ++i) {
    float y = to_f32(x[i], x_kind) * s;
    float r = nearbyintf(y); /* default rounding mode: to nearest, ties even */
    if (r > 127.0f || r < -127.0f) return ORACLE_INTERNAL;
    codes[i] = (int8_t)(int32_t)r;
  }
  *inv = 1.0f / s;
  if (scale_out) *scale_out = s;
  return ORACLE_OK;
}

/* Destination row of entry (t, j), or -1 if the entry is not dispatched. */
static int64_t dest_row(const int32_t *topk_idx, const int32_t *send_token_idx,
                        const int32_t *put_offset, const int32_t *recv_base, int64_t k,
                        int64_t epr, int64_t num_experts, int64_t t, int64_t j) {
  int32_t e = topk_idx[t * k + j];
  int32_t slot = send_token_idx[t * k + j];
  if (e < 0 || e >= num_experts || slot < 0) return -1;
  return (int64_t)recv_base[e / epr] + put_offset[e] + slot;
}

/* Scatter: row dst(t, j) of the receive buffer gets token t's row, either as
 * is (quant == 0: recv_rows[rows][h], 16-bit patterns of x's type) or as
 * int8 codes plus inverse scale (quant == 1: codes[rows][h], inv[rows]).
 * Every one of a token's k copies carries the same bytes.  Rows never
 * written are left as the caller initialised them. */
int oracle_dispatch(const uint16_t *x, int x_kind, int64_t bs, int64_t h, int64_t k,
                    const int32_t *topk_idx, const int32_t *send_token_idx,
                    const int32_t *put_offset, const int32_t *recv_base, int64_t epr,
                    int64_t ranks, int quant, int64_t rows, uint16_t *recv_rows,
                    int8_t *codes, float *inv) {
  if (bs < 0 || h < 1 || k < 1 || epr < 1 || ranks < 1 || rows < 0) return ORACLE_BAD_ARG;
  if (x_kind != KIND_BF16 && x_kind != KIND_FP16) return ORACLE_BAD_ARG;
  if (bs == 0) return ORACLE_OK;
  if (!x || !topk_idx || !send_token_idx || !put_offset || !recv_base) return ORACLE_BAD_ARG;
  if (quant ? (!codes || !inv) : !recv_rows) return ORACLE_BAD_ARG;
  int64_t num_experts = epr * ranks;
  for (int64_t t = 0; t < bs; ++t) {
    const uint16_t *src = x + t * h;
    for (int64_t j = 0; j < k; ++j) {
      int64_t dst = dest_row(topk_idx, send_token_idx, put_offset, recv_base, k, epr,
                             num_experts, t, j);
      if (dst < 0) continue;
      if (dst >= rows) return ORACLE_INTERNAL;
      if (!quant) {
        for (int64_t i = 0; i < h; ++i) recv_rows[dst * h + i] = src[i];
      } else {
        /* each copy is quantised from the source row on its own; the result
         * only depends on the row, so all k copies carry the same bytes */
        int rc = oracle_quant_row(src, x_kind, h, codes + dst * h, &inv[dst], NULL);
        if (rc) return rc;
      }
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Stage 4: combine (page section 2.6).                                      */
/* ------------------------------------------------------------------------ */

/* For each token t and element i:
 *   acc = +0.0f
 *   for j = 0 .. k-1 (dispatched entries only):
 *       v   = float(row[dst(t,j)][i])            (bf16 / fp16 rows)
 *          or float(code) * inv[dst(t,j)]         (int8 rows; dequantise)
 *       p   = v * topkWeights[t, j]              (rounded)
 *       acc = acc + p                            (rounded)
 *   out[t, i] = acc rounded half-even to the output type (or acc for fp32).
 * recv_kind: KIND_BF16 / KIND_FP16 with recv_rows, or KIND_INT8 with codes
 * and inv.  out_kind: KIND_BF16, KIND_FP16 (uint16 patterns) or KIND_FP32. */
int oracle_combine(const uint16_t *recv_rows, const int8_t *codes, const float *inv,
                   int recv_kind, int64_t bs, int64_t h, int64_t k, const int32_t *topk_idx,
                   const float *topk_w, const int32_t *send_token_idx,
                   const int32_t *put_offset, const int32_t *recv_base, int64_t epr,
                   int64_t ranks, int64_t rows, void *out, int out_kind, float *acc_scratch) {
  if (bs < 0 || h < 1 || k < 1 || epr < 1 || ranks < 1 || rows < 0) return ORACLE_BAD_ARG;
  if (recv_kind != KIND_BF16 && recv_kind != KIND_FP16 && recv_kind != KIND_INT8)
    return ORACLE_BAD_ARG;
  if (out_kind != KIND_BF16 && out_kind != KIND_FP16 && out_kind != KIND_FP32)
    return ORACLE_BAD_ARG;
  if (bs == 0) return ORACLE_OK;
  if (!topk_idx || !topk_w || !send_token_idx || !put_offset || !recv_base || !out ||
      !acc_scratch)
    return ORACLE_BAD_ARG;
  if (recv_kind == KIND_INT8 ? (!codes || !inv) : !recv_rows) return ORACLE_BAD_ARG;
  int64_t num_experts = epr * ranks;
  float *acc = acc_scratch; /* h floats, supplied by the caller */
  for (int64_t t = 0; t < bs; ++t) {
    for (int64_t i = 0; i < h; ++i) acc[i] = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      int64_t dst = dest_row(topk_idx, send_token_idx, put_offset, recv_base, k, epr,
                             num_experts, t, j);
      if (dst < 0) continue;
      if (dst >= rows) return ORACLE_INTERNAL;
      float w = topk_w[t * k + j];
      for (int64_t i = 0; i < h; ++i) {
        float v;
        if (recv_kind == KIND_INT8) {
          v = (float)codes[dst * h + i] * inv[dst];
        } else {
          v = to_f32(recv_rows[dst * h + i], recv_kind);
        }
        float p = v * w;
        acc[i] = acc[i] + p;
      }
    }
    for (int64_t i = 0; i < h; ++i) {
      if (out_kind == KIND_FP32) {
        ((float *)out)[t * h + i] = acc[i];
      } else if (out_kind == KIND_BF16) {
        ((uint16_t *)out)[t * h + i] = f32_to_bf16(acc[i]);
      } else {
        ((uint16_t *)out)[t * h + i] = f32_to_f16(acc[i]);
      }
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert-side epilogue between dispatch and combine: dequantise the int32   */
/* accumulators of the first expert GEMM, SwiGLU, requantise to int8 (the    */
/* same page, section 4 "Fused Deep MoE": section 4.3 stage 2,               */
/* DeqSwigluQuant, and section 4.8.1, the GMM1 epilogue PerTokenDequantSwiGLU).*/
/* ------------------------------------------------------------------------ */

/* e^x in binary32 by a named published method, written out step by step so
 * that it can be reproduced exactly: Cody and Waite's argument reduction
 * (W. J. Cody, W. Waite, "Software Manual for the Elementary Functions",
 * 1980), x = k ln2 + r with ln 2 split as C1 + C2, C1 = 355/512 exact in nine
 * bits (so k*C1 is exact for |k| < 2^15) and C2 = ln 2 - C1 rounded to
 * binary32; then e^r by its Taylor series to degree 7 in Horner form
 * (|r| <= ln2/2, truncation below 2^-27 relative); then the scale by 2^k.
 *   k  = round-half-even(x * log2(e))          (log2(e) rounded to binary32)
 *   r  = (x - k*C1) - k*C2                     (each operation rounded)
 *   p  = 1 + r(1 + r(1/2 + r(1/6 + r(1/24 + r(1/120 + r(1/720 + r/5040))))))
 *        (each coefficient 1/n! rounded to binary32; multiply, then add)
 *   result = p * 2^k, as p * 2^127 * 2 for k = 128 and as (p * 2^(k+64)) * 2^-64
 *   for k < -126 (a subnormal result, rounded once by the last multiply).
 * Inputs above 89 give +inf and below -104 give +0 (e^89 exceeds the largest
 * binary32 and e^-104 is below half the smallest subnormal); NaN stays NaN. */
static float pow2i(int k) { /* 2^k for -126 <= k <= 127 */
  return bits_to_f32((uint32_t)(k + 127) << 23);
}

static float exp_cw(float x) {
  if (x != x) return x;
  if (x > 89.0f) return INFINITY;
  if (x < -104.0f) return 0.0f;
  const float log2e = 1.44269502162933349609375f; /* 0x3FB8AA3B */
  const float c1 = 0.693359375f;                  /* 355/512 */
  const float c2 = -2.12194440e-4f;               /* ln 2 - 355/512 */
  float kf = nearbyintf(x * log2e);
  int k = (int)kf;
  float r = x - kf * c1;
  r = r - kf * c2;
  float p = 1.0f / 5040.0f;
  p = p * r + 1.0f / 720.0f;
  p = p * r + 1.0f / 120.0f;
  p = p * r + 1.0f / 24.0f;
  p = p * r + 1.0f / 6.0f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  if (k > 127) return (p * pow2i(127)) * 2.0f;
  if (k < -126) return (p * pow2i(k + 64)) * pow2i(-64);
  return p * pow2i(k);
}

int oracle_exp_f32(const float *in, float *out, int64_t n) {
  if ((n && (!in || !out)) || n < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = exp_cw(in[i]);
  return ORACLE_OK;
}

/* One row of the first expert GEMM's output: acc[0 .. 2n), the gate half
 * (columns 0 .. n-1) followed by the up half (columns n .. 2n-1).
 *   v_c   = (float(acc_c) * weight_scale[c]) * token_scale
 *           (page 4.8.1 steps 4-6: int32 -> fp32 round-half-even, times the
 *           column's weight scale, times the token's scale; each rounded)
 *   act_i = (g / (1 + e^-g)) * u,   g = v_i, u = v_(n+i)
 *           (steps 7: -g, Exp, +1, Div on the gate half; the up half passes
 *           through; the two are multiplied, SwiGLU = Swish(gate) * up)
 *   then the row act[0 .. n) is quantised exactly like a dispatched row:
 *   amax = max |act_i|, s = 127 / (amax + 1e-12f), q_i = rint(act_i * s),
 *   inv = 1 / s   (section 4.3 stage 2: "Quantize FP32 -> INT8").
 * act_out (optional) receives the binary32 activations before quantisation. */
static float swiglu_act(const int32_t *acc, int64_t n, const float *weight_scale,
                        float token_scale, int64_t i) {
  float g = (float)acc[i] * weight_scale[i];
  g = g * token_scale;
  float u = (float)acc[n + i] * weight_scale[n + i];
  u = u * token_scale;
  float e = exp_cw(-g);
  float d = e + 1.0f;
  float y = g / d;
  return y * u;
}

int oracle_swiglu_quant_row(const int32_t *acc, int64_t n, const float *weight_scale,
                            float token_scale, int8_t *codes, float *inv, float *act_out) {
  if (!acc || !weight_scale || !codes || !inv || n < 1) return ORACLE_BAD_ARG;
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = swiglu_act(acc, n, weight_scale, token_scale, i);
    if (act_out) act_out[i] = a;
    float m = fabsf(a);
    if (m > amax) amax = m;
  }
  float den = amax + 1e-12f;
  float s = 127.0f / den;
  for (int64_t i = 0; i < n; ++i) {
    float a = swiglu_act(acc, n, weight_scale, token_scale, i);
    float r = nearbyintf(a * s);
    if (!(r <= 127.0f && r >= -127.0f)) return ORACLE_INTERNAL;
    codes[i] = (int8_t)(int32_t)r;
  }
  inv[0] = 1.0f / s;
  return ORACLE_OK;
}

/* All rows: acc [rows][2n], token scale of row m at
 * token_scale[m * ts_stride] (in floats), codes [rows][n], inv [rows]. */
int oracle_swiglu_quant(const int32_t *acc, int64_t rows, int64_t n, const float *weight_scale,
                        const float *token_scale, int64_t ts_stride, int8_t *codes, float *inv) {
  if (rows < 0 || n < 1 || ts_stride < 1) return ORACLE_BAD_ARG;
  if (rows == 0) return ORACLE_OK;
  if (!acc || !weight_scale || !token_scale || !codes || !inv) return ORACLE_BAD_ARG;
  for (int64_t m = 0; m < rows; ++m) {
    int rc = oracle_swiglu_quant_row(acc + m * 2 * n, n, weight_scale, token_scale[m * ts_stride],
                                     codes + m * n, &inv[m], NULL);
    if (rc) return rc;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* First expert matmul (GMM1): section 4.3, stage 2 -- the dispatched int8    */
/* rows times each expert's int8 weights, accumulated in int32 -- with the    */
/* experts' row ranges given by per-expert token counts (section 4.6,         */
/* gmGroupList holds their running sums).                                     */
/* ------------------------------------------------------------------------ */

/* Row m of the receive buffer is a[m * a_stride .. + k) (int8 codes); the
 * weights of expert g are w[(g * n + j) * k + i] for output column j.
 * Expert g owns rows [S_g, S_g + c_g), c_g = max(group_count[g], 0) and S_g
 * the sum of c over the experts before g.  For the rows listed in row_list
 * (all rows 0 .. rows-1 in order when row_list is NULL; then nlist = rows):
 *   out[q][j] = sum over i of a[m][i] * w[g][j][i]   (exact, in int64)
 * and row_group[q] = g; a row that no expert owns gets row_group -1 and its
 * out row is left as it is.  A sum outside int32 is an error (it cannot
 * happen for k <= 2^17). */
int oracle_grouped_gemm_i8(const int8_t *a, int64_t a_stride, int64_t rows, int64_t k,
                           const int32_t *group_count, int64_t groups, const int8_t *w,
                           int64_t n, const int64_t *row_list, int64_t nlist, int32_t *out,
                           int32_t *row_group) {
  if (rows < 0 || k < 1 || n < 1 || groups < 1 || a_stride < k || nlist < 0) return ORACLE_BAD_ARG;
  if (!row_list && nlist != rows) return ORACLE_BAD_ARG;
  if (nlist == 0) return ORACLE_OK;
  if (!a || !group_count || !w || !out || !row_group) return ORACLE_BAD_ARG;
  for (int64_t q = 0; q < nlist; ++q) {
    int64_t m = row_list ? row_list[q] : q;
    if (m < 0 || m >= rows) return ORACLE_BAD_ARG;
    int64_t owner = -1, start = 0;
    for (int64_t g = 0; g < groups; ++g) {
      int64_t c = group_count[g] > 0 ? group_count[g] : 0;
      if (m >= start && m < start + c) {
        owner = g;
        break;
      }
      start += c;
    }
    row_group[q] = (int32_t)owner;
    if (owner < 0) continue;
    for (int64_t j = 0; j < n; ++j) {
      int64_t acc = 0;
      for (int64_t i = 0; i < k; ++i)
        acc += (int64_t)a[m * a_stride + i] * (int64_t)w[(owner * n + j) * k + i];
      if (acc > INT32_MAX || acc < INT32_MIN) return ORACLE_INTERNAL;
      out[q * n + j] = (int32_t)acc;
    }
  }
  return ORACLE_OK;
}
