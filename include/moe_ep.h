/*
 * moe_ep.h -- C ABI of the MoE expert-parallel dispatch/combine library
 * (libmoe_ep.so, HIP kernels for gfx950 / MI355X).
 *
 * The four entry points are the four stages of the "EP normal" pipeline
 * described on the page "UMDK/CAM communication acceleration library deep
 * analysis v2", section 2 (2.1 gives the stage order):
 *
 *   moe_layout   -- 2.3 moe_dispatch_layout_zb
 *   moe_notify   -- 2.4 moe_notify_dispatch_zb
 *   moe_dispatch -- 2.5 moe_dispatch_normal_zb (with QuantProcess)
 *   moe_combine  -- 2.6 moe_combine_normal_zb (ReadBufferAndWeightedSum)
 *
 * Scalars follow the page's CommArgs (2.2.1): batch size bs, hidden size h,
 * topk k, expertNumPerRank EPR and rankSize R; E = R * EPR experts and the
 * destination rank of expert e is e / EPR.
 *
 * Single device.  The R ranks are logical: their receive regions are
 * concatenated, in rank order, inside one device buffer.  Region r starts at
 * row recvBase[r]; inside it expert e's rows start at putOffset[e] and are
 * ordered by send slot (token order).  Row r of the receive buffer lives at
 * byte offset r * moe_recv_row_bytes(h, type).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to device memory (or to
 *    memory the device can address); the library never allocates, frees or
 *    keeps device memory.  Between calls it keeps only the compute-unit
 *    count of each device it has launched the fused kernel on (read once,
 *    the one device-property query) and, per thread, the last HIP error.
 *  - Arrays are dense, row-major, in the element types given below.
 *  - Work is only enqueued on `stream` (a hipStream_t; NULL means the null
 *    stream) and the call returns without waiting.  Stage order on one stream
 *    replaces the page's SyncAll / BarrierAll between stages.
 *  - Argument errors (NULL pointer, bad shape, alignment, dtype, buffer too
 *    small, unsupported size) are found on the host before anything is
 *    enqueued; the call then returns the error code and enqueues nothing.
 *    MOE_ERR_HIP means a launch failed (see moe_last_hip_error()).
 *  - Calls on different streams that share output buffers race; calls on
 *    different buffers may run concurrently.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
  MOE_BF16 = 0,          /* bfloat16 */
  MOE_FP16 = 1,          /* IEEE binary16 */
  MOE_FP32 = 2,          /* IEEE binary32 (combine output only) */
  MOE_INT8_ROWSCALE = 3  /* int8 codes + float inverse scale per row (receive buffer) */
} moe_dtype;

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_NULL_PTR = 1,
  MOE_ERR_BAD_SHAPE = 2,
  MOE_ERR_BAD_ALIGN = 3,
  MOE_ERR_BAD_DTYPE = 4,
  MOE_ERR_WORKSPACE_TOO_SMALL = 5,
  MOE_ERR_BUFFER_TOO_SMALL = 6,
  MOE_ERR_UNSUPPORTED = 7,
  MOE_ERR_HIP = 8,
  MOE_ERR_SCRATCH_LIMIT = 9
};

/* Limits of the library. */
#define MOE_MAX_EXPERTS 2048   /* E = R * EPR */
#define MOE_MAX_HIDDEN 16384   /* h */
#define MOE_MAX_TOPK 32        /* k */
#define MOE_MAX_SOURCES 384    /* source ranks sharing one receive buffer (the
                                  page's CAM_MAX_RANK_SIZE) */
#define MOE_EPILOGUE_MAX_N 4096 /* n, the epilogue's output columns (2n inputs) */
#define MOE_GEMM_MAX_K 65536    /* k of the first expert matmul: sums stay below 2^31 */
#define MOE_GEMM_MAX_N 65536    /* n of the first expert matmul */
#define MOE_GEMM_MAX_GROUPS 65536 /* experts of one first-expert-matmul call */
#define MOE_NO_ALLOC_SCRATCH_BYTES (1u << 20) /* moe_layout_no_alloc's static workspace */

/* Bytes of one receive-buffer row for hidden size `hidden` and receive type
 * `recv` (page 2.5 and 2.2.1):
 *   MOE_BF16, MOE_FP16:   2 * hidden (the row as is);
 *   MOE_INT8_ROWSCALE:    align32(hidden) + 32 rounded up to a multiple of
 *                         128 -- int8 codes at bytes [0, hidden), the float
 *                         inverse scale 1/s at byte align32(hidden)
 *                         (UB_ALIGN_SIZE = 32); the other bytes are padding
 *                         with unspecified contents.  The page places the
 *                         scale but leaves the row stride open; rows here
 *                         start on 128-byte cache-line boundaries (7296 bytes
 *                         at hidden = 7168).
 * Host only; writes *bytes.  Errors: NULL_PTR, BAD_SHAPE (hidden < 1),
 * BAD_DTYPE. */
int moe_recv_row_bytes(int32_t hidden, moe_dtype recv, size_t* bytes);

/* Device workspace that moe_layout needs for `bs` tokens, `topk` entries per
 * token and `numExperts` experts (a per-tile count table).  This follows the
 * page's operator-call convention (section 6.7, EXEC_NPU_CMD: ask the
 * operator for its workspace size, let the caller allocate that many bytes,
 * then submit the operator with the workspace on a stream); here the caller
 * allocates through its own allocator (torch) and passes the pointer.  May
 * be 0, in which case moe_layout accepts a NULL workspace.  Host only. */
int moe_layout_workspace_bytes(int32_t bs, int32_t topk, int32_t numExperts, size_t* bytes);

/* Stage 1, dispatch layout (page 2.3).
 * In:  topkIdx        device int32 [bs, topk], expert id of each (token, k)
 *                     entry; ids outside [0, E) are "bad".
 * Out: tokenPerExpert device int32 [E]: entries routed to each expert.
 *      tokenPerRank   device int32 [R]: rows each logical rank receives
 *                     (sum of tokenPerExpert over its EPR experts).
 *      sendTokenIdx   device int32 [bs, topk]: the entry's slot inside its
 *                     expert's region = the number of earlier entries (flat
 *                     t*topk + j order) with the same expert; -1 for bad ids.
 *      badIdCount     device int32 [1] or NULL: number of bad entries.
 * workspace: device memory of at least moe_layout_workspace_bytes(...) bytes,
 * 4-byte aligned; contents on entry do not matter.
 * bs may be 0 (outputs are still written).  Deterministic: the result does
 * not depend on scheduling. */
int moe_layout(const int32_t* topkIdx, int32_t bs, int32_t topk, int32_t expertNumPerRank,
               int32_t rankSize, int32_t* tokenPerExpert, int32_t* tokenPerRank,
               int32_t* sendTokenIdx, int32_t* badIdCount, void* workspace,
               size_t workspaceBytes, void* stream);

/* moe_layout for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same stage, the same outputs bit for bit, with no workspace argument.
 * The per-tile count table lives in a static device array of
 * MOE_NO_ALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends; the call allocates and frees nothing.  Shapes
 * whose table (moe_layout_workspace_bytes) would exceed it return
 * MOE_ERR_SCRATCH_LIMIT before anything is enqueued (1 MiB: bs * topk up to
 * about 2.09 million entries at 256 experts, 262144 at 2048).  Every call on
 * one device shares that device's array: calls that overlap in time on one
 * device (other streams, other threads) race and must be serialised by the
 * caller.  The first call on a device looks up the array's device address
 * (a runtime symbol query, no allocation).  Other arguments and errors as
 * moe_layout. */
int moe_layout_no_alloc(const int32_t* topkIdx, int32_t bs, int32_t topk, int32_t expertNumPerRank,
                        int32_t rankSize, int32_t* tokenPerExpert, int32_t* tokenPerRank,
                        int32_t* sendTokenIdx, int32_t* badIdCount, void* stream);

/* Stage 2, notify (page 2.4).  With a single source the page's all-gather of
 * tokenPerExpert is the identity and the prefix sums remain:
 * In:  tokenPerExpert     device int32 [E] (from moe_layout).
 * Out: putOffset          device int32 [E]: start of expert e's rows inside
 *                         its rank's region (exclusive scan over the rank's
 *                         experts in id order).
 *      recvCount          device int32 [R]: rows in rank r's region.
 *      recvBase           device int32 [R]: first row of rank r's region
 *                         (exclusive scan of recvCount).
 *      recvTokenPerExpert device int32 [E]: rows each expert receives.
 * The counts are moe_layout's: non-negative, with a total that fits in
 * int32.  Other counts give unspecified offsets; dispatch and combine still
 * touch no row outside their receive buffer. */
int moe_notify(const int32_t* tokenPerExpert, int32_t expertNumPerRank, int32_t rankSize,
               int32_t* putOffset, int32_t* recvCount, int32_t* recvBase,
               int32_t* recvTokenPerExpert, void* stream);

/* Stage 3, dispatch (page 2.5).  Entry (t, j) with a valid id e and slot
 * s >= 0 writes token t's row to receive row
 *     recvBase[e / EPR] + putOffset[e] + s.
 * In:  x         device [bs, hidden] of xType (MOE_BF16 or MOE_FP16), 16-byte
 *                aligned.
 *      topkIdx, sendTokenIdx  device int32 [bs, topk] (from moe_layout).
 *      putOffset device int32 [E], recvBase device int32 [R] (from moe_notify).
 *      quantInt8 0: rows are copied as is (receive type = xType);
 *                1: rows are quantised (receive type MOE_INT8_ROWSCALE):
 *                   s = 127 / (max|x_t| + 1e-12), codes = round-half-even
 *                   (x * s) in binary32, inverse scale 1/s stored after the
 *                   codes (correctly rounded binary32 divisions).
 * Out: recvX     device buffer of recvXBytes bytes, 16-byte aligned; needs
 *                bs * topk rows of moe_recv_row_bytes(hidden, recvType).
 * Entries whose row would fall outside recvXBytes are skipped.  Requires
 * hidden % 8 == 0 and hidden <= MOE_MAX_HIDDEN (else MOE_ERR_UNSUPPORTED). */
int moe_dispatch(const void* x, moe_dtype xType, int32_t bs, int32_t hidden, int32_t topk,
                 const int32_t* topkIdx, const int32_t* sendTokenIdx, const int32_t* putOffset,
                 const int32_t* recvBase, int32_t expertNumPerRank, int32_t rankSize,
                 int quantInt8, void* recvX, size_t recvXBytes, void* stream);

/* Stage 4, combine (page 2.6).  For each token t and element i:
 *     acc = +0.0f
 *     for j = 0 .. topk-1 with a valid id and slot (row as in dispatch):
 *         v   = float(row[i])                (MOE_BF16 / MOE_FP16 rows)
 *            or float(code[i]) * inv(row)    (MOE_INT8_ROWSCALE rows)
 *         acc = acc + v * topkWeights[t, j]  (multiply and add rounded apart)
 *     out[t, i] = acc, rounded half-even to outType.
 * The result is bit-identical to that sequential binary32 definition.
 * In:  recvX       device receive buffer of recvType, recvXBytes bytes,
 *                  16-byte aligned; rows outside it contribute nothing.
 *      topkIdx, sendTokenIdx device int32 [bs, topk]; topkWeights device
 *                  float [bs, topk]; putOffset [E], recvBase [R] as above.
 * Out: out         device [bs, hidden] of outType (MOE_BF16, MOE_FP16 or
 *                  MOE_FP32), 16-byte aligned.
 * Requires hidden % 8 == 0 and hidden <= MOE_MAX_HIDDEN. */
int moe_combine(const void* recvX, moe_dtype recvType, size_t recvXBytes, int32_t bs,
                int32_t hidden, int32_t topk, const int32_t* topkIdx, const float* topkWeights,
                const int32_t* sendTokenIdx, const int32_t* putOffset, const int32_t* recvBase,
                int32_t expertNumPerRank, int32_t rankSize, void* out, moe_dtype outType,
                void* stream);

/* ---- Several source ranks sharing one receive buffer -------------------- */

/* Stage 2 with S = numSrc source ranks (page 2.4: every rank's
 * tokenPerExpert is all-gathered before the prefix sums; page 2.6: combine
 * reads the base of (expert, source) at index expertId * epWorldSize +
 * srcRank).  Inside destination rank r the rows are ordered by expert
 * (ascending), then by source (ascending), then by send slot; the ranks'
 * regions are concatenated in rank order.
 * In:  tokenPerExpert     device int32 [S][E]: row s is source s's
 *                         moe_layout output.
 * Out: putOffset          device int32 [E][S]: start of the rows of
 *                         (expert e, source s) inside e's rank region.
 *      recvCount          device int32 [R]: rows in rank r's region.
 *      recvBase           device int32 [R]: first row of rank r's region.
 *      recvTokenPerExpert device int32 [E]: rows expert e receives from all
 *                         sources.
 * Requires 1 <= numSrc <= MOE_MAX_SOURCES; the total row count must fit in
 * int32.  With numSrc == 1 the outputs equal moe_notify's. */
int moe_notify_multi(const int32_t* tokenPerExpert, int32_t numSrc, int32_t expertNumPerRank,
                     int32_t rankSize, int32_t* putOffset, int32_t* recvCount, int32_t* recvBase,
                     int32_t* recvTokenPerExpert, void* stream);

/* moe_dispatch (page section 2.5) for source srcRank of numSrc, at the
 * offsets of section 2.6's index: entry (t, j) with a valid id e
 * and slot s >= 0 writes to receive row
 *     recvBase[e / EPR] + putOffset[e][srcRank] + s
 * with putOffset [E][numSrc] and recvBase from moe_notify_multi.  The
 * receive buffer is shared by all sources; it must hold at least this
 * source's bs * topk rows (the sum over sources for all rows to land; rows
 * past recvXBytes are skipped).  Other arguments as moe_dispatch.  Calls for
 * different sources write disjoint rows and may run concurrently. */
int moe_dispatch_src(const void* x, moe_dtype xType, int32_t bs, int32_t hidden, int32_t topk,
                     const int32_t* topkIdx, const int32_t* sendTokenIdx, const int32_t* putOffset,
                     const int32_t* recvBase, int32_t expertNumPerRank, int32_t rankSize,
                     int32_t numSrc, int32_t srcRank, int quantInt8, void* recvX,
                     size_t recvXBytes, void* stream);

/* moe_combine (page section 2.6) for source srcRank of numSrc: reads the
 * rows moe_dispatch_src wrote for that source (same row formula), with the
 * same arithmetic and bit-exactness as moe_combine.  Other arguments as
 * moe_combine. */
int moe_combine_src(const void* recvX, moe_dtype recvType, size_t recvXBytes, int32_t bs,
                    int32_t hidden, int32_t topk, const int32_t* topkIdx, const float* topkWeights,
                    const int32_t* sendTokenIdx, const int32_t* putOffset, const int32_t* recvBase,
                    int32_t expertNumPerRank, int32_t rankSize, int32_t numSrc, int32_t srcRank,
                    void* out, moe_dtype outType, void* stream);

/* ---- Fused layout + notify + dispatch ------------------------------------ */

/* *supported = 1 if moe_layout_notify_dispatch (the single-kernel form of
 * section 3.2) runs as one kernel for this shape, 0 if it runs the three
 * stages one after another (bs == 0, hidden above 8192, or bs * topk above
 * 2^16: every workgroup of the one kernel reads all bs * topk ids).  Host
 * only; the answer does not depend on the device. */
int moe_fused_supported(int32_t bs, int32_t hidden, int32_t topk, int32_t expertNumPerRank,
                        int32_t rankSize, moe_dtype xType, int quantInt8, int* supported);

/* Stages 1-3 in one launch: the single-kernel low-latency form of the
 * pipeline ("UMDK/CAM communication acceleration library deep analysis v2",
 * section 3.2, moe_dispatch_lowlatency_zb: local expert counts, count
 * exchange, global count matrix and prefix sum, then the token writes in one
 * kernel).  Every output is identical to moe_layout, moe_notify and
 * moe_dispatch called in turn with the same arguments, which is also what
 * this call does when the one kernel does not apply (moe_fused_supported).
 * Arguments as in those three calls; workspace and workspaceBytes are
 * moe_layout's (moe_layout_workspace_bytes) and are used only by the
 * three-stage form.
 * The one kernel needs no inter-workgroup synchronisation: each workgroup
 * counts all ids itself, ranks its own tokens' entries and writes their
 * rows; workgroup 0 writes the layout and notify outputs. */
int moe_layout_notify_dispatch(const void* x, moe_dtype xType, int32_t bs, int32_t hidden,
                               int32_t topk, const int32_t* topkIdx, int32_t expertNumPerRank,
                               int32_t rankSize, int quantInt8, int32_t* tokenPerExpert,
                               int32_t* tokenPerRank, int32_t* sendTokenIdx, int32_t* badIdCount,
                               int32_t* putOffset, int32_t* recvCount, int32_t* recvBase,
                               int32_t* recvTokenPerExpert, void* recvX, size_t recvXBytes,
                               void* workspace, size_t workspaceBytes, void* stream);

/* Expert-side epilogue between dispatch and combine: dequantise the int32
 * output of the first expert GEMM, SwiGLU, and requantise to int8 -- page
 * section 4.3 (Fused Deep MoE, stage 2 "DeqSwigluQuant") and section 4.8.1
 * (the GMM1 epilogue PerTokenDequantSwiGLU).
 *
 * acc        [rows][2n] int32, device, 16-byte aligned: row m is the GEMM
 *            output of receive row m, gate columns 0 .. n-1 then up columns
 *            n .. 2n-1.
 * weightScale [2n] float, device, 16-byte aligned: per-column dequant scale.
 * tokenScale  device bytes, 4-byte aligned: the float scale of row m is at
 *            byte offset m * tokenScaleStride (a multiple of 4, >= 4).  A dense
 *            float array has stride 4; the int8 receive buffer's inverse
 *            scales are used in place with tokenScale = recvX + align32(h)
 *            and tokenScaleStride = moe_recv_row_bytes(h, MOE_INT8_ROWSCALE).
 * out        device, 16-byte aligned, outBytes >= rows * moe_recv_row_bytes(n,
 *            MOE_INT8_ROWSCALE): int8 rows in the receive-buffer format.
 *
 * For every row m and column i, each operation rounded to binary32:
 *   g = (float(acc[m][i]) * weightScale[i]) * ts_m            (int32 -> float
 *   u = (float(acc[m][n+i]) * weightScale[n+i]) * ts_m         rounds half-even)
 *   a_i = (g / (1 + e^-g)) * u                                 (Swish(g) * u)
 * then the row a is quantised like a dispatched row: s = 127 / (max|a| +
 * 1e-12f), codes rint(a_i * s) (half-even) at bytes [0, n), inv = 1/s as a
 * float at byte align32(n).  e^x is binary32 Cody-Waite reduction with
 * ln 2 = 355/512 + (ln 2 - 355/512) and the degree-7 Taylor polynomial,
 * +inf above 89, +0 below -104.  Activations must be finite (scales and
 * accumulators that overflow binary32 are outside the contract).
 *
 * Requires rows >= 0 and n >= 1 (else MOE_ERR_BAD_SHAPE), n % 4 == 0 and
 * n <= MOE_EPILOGUE_MAX_N (else MOE_ERR_UNSUPPORTED).  rows == 0 enqueues
 * nothing. */
int moe_deq_swiglu_quant(const int32_t* acc, int32_t rows, int32_t n, const float* weightScale,
                         const void* tokenScale, int64_t tokenScaleStride, void* out, size_t outBytes,
                         void* stream);

/* First expert matmul (GMM1) of the expert side: the dispatched int8 rows
 * times each expert's int8 weights, summed exactly in int32 -- page section
 * 4.3 (Fused Deep MoE, stage 2: "GMM1 (INT8 x INT8 -> INT32)") with the
 * experts' row ranges given by per-expert token counts (section 4.6, the
 * cumulative counts gmGroupList).  Its output is moe_deq_swiglu_quant's acc.
 *
 * a          device, 16-byte aligned: row m at a + m * aRowBytes holds k int8
 *            codes in its first k bytes (the rest of the row is not read).
 *            The int8 receive buffer is used in place with aRowBytes =
 *            moe_recv_row_bytes(k, MOE_INT8_ROWSCALE).  It must hold
 *            (rows - 1) * aRowBytes + k bytes.
 * groupCount [groups] int32, device, 4-byte aligned: expert g owns rows
 *            [S_g, S_g + c_g) with c_g = max(groupCount[g], 0) and S_g the
 *            sum of c over the experts before g; rows at or past `rows` are
 *            owned by nobody.  moe_notify's recvTokenPerExpert (one source)
 *            or a rank's slice of it are such counts.  Not read by the host.
 * w          [groups][n][k] int8, device, 16-byte aligned: the weights of
 *            expert g for output column j are the k bytes at (g * n + j) * k.
 * out        [rows][n] int32, device, 4-byte aligned, outBytes >= rows * n * 4:
 *            out[m][j] = sum over i < k of a[m][i] * w[g][j][i] for each row m
 *            owned by expert g (exact: every partial sum is below 2^31 in
 *            magnitude).  Rows that no expert owns are not written.
 *
 * Requires rows >= 0, k >= 1, n >= 1, groups >= 1, aRowBytes >= k (else
 * MOE_ERR_BAD_SHAPE); k % 16 == 0, k <= MOE_GEMM_MAX_K, n <= MOE_GEMM_MAX_N,
 * groups <= MOE_GEMM_MAX_GROUPS, and at most 2^24 workgroups in the launch
 * (row slots ceil(rows / 256) + groups, rounded up to a multiple of 16 when
 * ceil(n / 256) % 4 == 0, times ceil(n / 256)) (else MOE_ERR_UNSUPPORTED);
 * aRowBytes a multiple of 16 (else MOE_ERR_BAD_ALIGN); outBytes as above
 * (else MOE_ERR_BUFFER_TOO_SMALL).  rows == 0 enqueues nothing. */
int moe_grouped_gemm_i8(const void* a, int64_t aRowBytes, int32_t rows, int32_t k,
                        const int32_t* groupCount, int32_t groups, const void* w, int32_t n,
                        int32_t* out, size_t outBytes, void* stream);

/* Bytes of workspace that moe_grouped_gemm_swiglu_quant_i8 needs for `rows`
 * rows and n activation columns (the query-size, caller-allocates convention
 * of page section 6.7): the activations as floats [rows][n] and one word per
 * row.  Requires rows >= 0 and n >= 1 (else MOE_ERR_BAD_SHAPE). */
int moe_gemm_swiglu_quant_workspace_bytes(int32_t rows, int32_t n, size_t* bytes);

/* The first expert matmul with its epilogue fused -- page section 4.8.1
 * (GMM1 with the PerTokenDequantSwiGLU epilogue on its accumulators) and
 * section 4.3 (stage 2, GMM1 then DeqSwigluQuant): the int32 sums never
 * reach memory.  For every row m owned by expert g (as moe_grouped_gemm_i8
 * defines ownership), out row m is bit for bit what moe_deq_swiglu_quant
 * writes for row m of moe_grouped_gemm_i8's output with expert g's scales:
 *   acc[j] = sum over i < k of a[m][i] * w[g][j][i], j < 2n (gate j < n, up n + j)
 *   act_j  = Swish((float(acc[j]) * ws[g][j]) * ts_m) * ((float(acc[n+j]) * ws[g][n+j]) * ts_m)
 *   codes rint(act_j * s), s = 127 / (max_j |act_j| + 1e-12f), inverse 1/s.
 *
 * a, aRowBytes, rows, k, groupCount, groups: as moe_grouped_gemm_i8.
 * w          [groups][2n][k] int8, device, 16-byte aligned: expert g's gate
 *            weights (output columns 0 .. n-1), then its up weights.
 * weightScale [groups][2n] float, device, 4-byte aligned: per-expert,
 *            per-column dequant scales.
 * tokenScale, tokenScaleStride: as moe_deq_swiglu_quant (the int8 receive
 *            buffer's inverse scales in place, or a dense float array).
 * out        device, 16-byte aligned, outBytes >= rows * moe_recv_row_bytes(n,
 *            MOE_INT8_ROWSCALE): int8 rows in the receive-buffer format.
 *            Rows that no expert owns are not written.
 * workspace  device, 16-byte aligned, workspaceBytes >=
 *            moe_gemm_swiglu_quant_workspace_bytes(rows, n); caller-owned,
 *            contents on return unspecified.
 *
 * Requires rows >= 0, k >= 1, n >= 1, groups >= 1, aRowBytes >= k,
 * tokenScaleStride a multiple of 4 and >= 4 (else MOE_ERR_BAD_SHAPE);
 * k % 16 == 0, k <= MOE_GEMM_MAX_K, n % 4 == 0, 2n <= MOE_GEMM_MAX_N, groups
 * <= MOE_GEMM_MAX_GROUPS, and at most 2^24 workgroups in the matmul launch
 * (moe_grouped_gemm_i8's count with ceil(n / 128) column tiles) (else
 * MOE_ERR_UNSUPPORTED); aRowBytes a multiple of 16 (else MOE_ERR_BAD_ALIGN);
 * a small out buffer gives MOE_ERR_BUFFER_TOO_SMALL, a small workspace
 * MOE_ERR_WORKSPACE_TOO_SMALL.  rows == 0 enqueues nothing.  Enqueues three
 * kernels (clear the row maxima, the matmul with the activation, the
 * quantisation). */
int moe_grouped_gemm_swiglu_quant_i8(const void* a, int64_t aRowBytes, int32_t rows, int32_t k,
                                     const int32_t* groupCount, int32_t groups, const void* w, int32_t n,
                                     const float* weightScale, const void* tokenScale,
                                     int64_t tokenScaleStride, void* out, size_t outBytes, void* workspace,
                                     size_t workspaceBytes, void* stream);

/* Diagnostics.  No counterpart on the pages (their operator calls report
 * failure through the framework's own status; section 6.7 does not show it):
 * the text of one of this library's status codes (static storage). */
const char* moe_status_str(int status);

/* Diagnostics, no counterpart on the pages: the hipError_t value of the last
 * MOE_ERR_HIP returned on this thread (0 if none). */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
