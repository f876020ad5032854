/*
 * awq.h -- C ABI of libawq: AWQ activation-aware INT4 weight quantization, the
 * data-parallel hot path (statistic, 20-candidate scale search, pack) on one MI355X, the
 * clipping search that follows the scale search, the folding of the chosen scales and the
 * W4A16 product over the packed artefact.
 *
 * Sources (cited by page title and section):
 *   [EXPLAINER] "AWQ：为什么 4-bit 权重量化要先观察 Activation" (charlestar.github.io)
 *   [DREAMVFIA] "AWQ salient weight / GGUF compilation" report (dreamvfia.cn)
 *   [MODULES]   "5. 核心模块：校准器、压缩算法、格式封装与 kernel 后端" (ai-infra.cypggs.com)
 *
 * Conventions shared by every entry point
 *   - Orientation: X is [M, K] (M calibration tokens, K input channels), row-major with
 *     row stride ldx elements (ldx >= K).  W is a PyTorch Linear weight [N, K] (N output
 *     channels), row-major with row stride ldw (ldw >= K).  Groups of `group` consecutive k
 *     along a row of W are quantized together ([EXPLAINER §7]: the source groups along the
 *     last, input, dimension of the [N, K] tensor).
 *   - Every pointer argument is DEVICE memory owned by the caller; buffers must stay alive
 *     until the work queued on `stream` has finished.  The library allocates no device
 *     memory, keeps no mutable global state and is reentrant; every call is asynchronous on
 *     `stream` (a hipStream_t; NULL is the default stream).  The one exception is
 *     awq_search_static, whose workspace is a static device array (see there).
 *   - Argument errors are returned synchronously as an awq_status before anything is
 *     queued; no kernel is launched in that case.
 *   - Data errors can only be seen on the device: kernels OR AWQ_FLAG_* bits into *flags.
 *     The caller clears *flags before the call.  When a bit is set after the stream work
 *     finished, the outputs of that call are undefined.
 *   - Fixed quantization contract ([EXPLAINER §7]; quant config zero_point = True,
 *     w_bit = 4, q_group_size = 128 in [DREAMVFIA §四]): asymmetric 4-bit codes 0..15,
 *     group = 128 along K.  K must be a multiple of 128.
 */
#ifndef AWQ_H
#define AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AWQ_ABI_VERSION 8

#if defined(__GNUC__)
#define AWQ_API __attribute__((visibility("default")))
#else
#define AWQ_API
#endif

/* Status codes returned synchronously. */
typedef enum {
  AWQ_OK = 0,
  AWQ_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, ld < K, n_grid outside [1, 64],
                              n_clip outside [1, 20] */
  AWQ_ERR_SHAPE = 2,       /* K not a multiple of the group size, 64-bit size overflow,
                              awq_search / awq_clip: 512 rows of X or 128 rows of W span 2^31
                              bytes or more; awq_search: one candidate's group ranges
                              (8 N K / 128 bytes) do; awq_w4a16: 512 rows of X or of Y do */
  AWQ_ERR_UNSUPPORTED = 3, /* dtype other than F32/BF16, group other than 128 */
  AWQ_ERR_WORKSPACE = 4,   /* workspace pointer null or smaller than the size function says */
  AWQ_ERR_HIP = 5,         /* a HIP launch or runtime call failed */
  AWQ_ERR_SCRATCH = 6      /* awq_search_static: the call needs more workspace than
                              AWQ_STATIC_SCRATCH_BYTES */
} awq_status;

/* Element types of X and W. */
typedef enum { AWQ_DTYPE_F32 = 0, AWQ_DTYPE_BF16 = 1 } awq_dtype;

/* Data-error bits OR-ed into *flags by the kernels. */
#define AWQ_FLAG_NONFINITE_X 0x1u    /* awq_stats: X holds NaN or Inf */
#define AWQ_FLAG_NONFINITE_W 0x2u    /* awq_pack: W holds NaN or Inf, or W*s overflows fp32 */
#define AWQ_FLAG_SCALE_RANGE 0x4u    /* a scale candidate is not finite and positive in fp32,
                                        or the statistic a is negative or not finite; awq_clip,
                                        awq_pack*: a given scale is not finite and positive;
                                        awq_pack_clipped: a threshold is negative or not finite */
#define AWQ_FLAG_F16_RANGE 0x8u      /* awq_pack: a group step does not fit fp16 */
#define AWQ_FLAG_NONFINITE_LOSS 0x10u /* awq_search / awq_clip: a candidate loss is not finite
                                         (NaN/Inf in X or W reach the losses through the
                                         product) */

typedef struct ihipStream_t* awq_stream_t; /* the same type as hipStream_t */
typedef struct ihipEvent_t* awq_event_t;   /* the same type as hipEvent_t */

/* ABI version of the loaded library (AWQ_ABI_VERSION). */
AWQ_API int awq_abi_version(void);

/* Static, NUL-terminated description of a status code. */
AWQ_API const char* awq_status_string(int status);

/* ---------------------------------------------------------------------------------------
 * Step 1: activation statistic  ([EXPLAINER §1]; [DREAMVFIA §二] writes it (1/B) sum |X|)
 *   a[j] = (1/M) * sum_m |X[m, j]|  for j < K
 * Arithmetic: every term is accumulated in fp64 (exact for bf16 inputs in practice), a
 * fixed-order reduction, one rounding to fp32 at the end; bitwise reproducible.
 *   X       [M, K] of x_dtype, row stride ldx
 *   a_out   fp32 [K]
 *   ws      workspace of at least awq_stats_workspace_bytes(M, K) bytes (device)
 *   flags   device uint32; AWQ_FLAG_NONFINITE_X if X holds NaN/Inf
 * ------------------------------------------------------------------------------------- */
AWQ_API size_t awq_stats_workspace_bytes(int64_t M, int64_t K);
AWQ_API int awq_stats(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                      float* a_out, void* ws, size_t ws_bytes, uint32_t* flags,
                      awq_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Steps 2-4 and the argmin of step 5: the candidate scale search ([EXPLAINER §3, §4]).
 *   For i < n_grid, alpha_i = i / n_grid (n_grid = 20 gives 0, 0.05, ..., 0.95):
 *     r_j = max(a_j ^ alpha_i, 1e-4)          (fp64; 0^0 = 1)
 *     s_j = fp32(r_j / sqrt(max_k r_k * min_k r_k)),  rs_j = fp32(1 / s_j)
 *   For every group g of 128 k in row n of W:  v = W[n,k] * s_k (fp32),
 *     Delta = max(max v - min v, 1e-5) / 15,  z = clamp(rne(-min v / Delta), 0, 15),
 *     q = clamp(rne(v / Delta) + z, 0, 15),   E[n,k] = W[n,k] - Delta (q - z) / s_k
 *   loss_i = sum_{m,n} (X E^T)[m,n]^2 / (M N)      ([EXPLAINER §4]: module-output MSE)
 *   best = first index attaining min loss           (earliest candidate wins ties)
 * The quantized weights never leave the chip: each tile is quantized in registers and fed
 * to a bf16 matrix-core product whose squared output error is reduced in the same kernel.
 * Inside the search the code uses v * (1/Delta); awq_pack always divides exactly.
 *   X, W           as above (both F32 or BF16; F32 X is split into two bf16 terms)
 *   a              fp32 [K]: the statistic (normally awq_stats' output)
 *   group, n_grid  128 and 1..64 (20 in the method)
 *   losses_out     fp64 [n_grid];  best_out int32 [1];  s_best_out fp32 [K] = s of the winner
 *   s_table_out    fp32 [n_grid, K] or NULL: the whole scale table
 *   ws             workspace of at least awq_search_workspace_bytes(...) bytes (device).
 *                  When K is a multiple of 256 and at least 512, that size ends with room for
 *                  a copy of X in matrix-core operand order, xcopy = round_up(2 * round_up(M, 32)
 *                  * K, 256) bytes, which the fastest kernel (bf16 X and W) reads X from.  A
 *                  workspace at least xcopy bytes short of the full size still works: it runs
 *                  a kernel that stages X itself, with bit-identical results.
 *   flags          AWQ_FLAG_SCALE_RANGE, AWQ_FLAG_NONFINITE_LOSS
 * ------------------------------------------------------------------------------------- */
AWQ_API size_t awq_search_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group,
                                          int32_t n_grid);
AWQ_API int awq_search(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                       const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                       int32_t group, int32_t n_grid, double* losses_out, int32_t* best_out,
                       float* s_best_out, float* s_table_out, void* ws, size_t ws_bytes,
                       uint32_t* flags, awq_stream_t stream);

/* The same search with two caller-created events (hipEventCreate; either may be NULL)
 * recorded on `stream` immediately before and after the fused quantize + product + squared
 * error kernel, so that a caller can time that kernel alone with hipEventElapsedTime (the
 * scale table, group-range and select launches fall outside the pair).  Arguments, results
 * and errors as awq_search; a failed hipEventRecord returns AWQ_ERR_HIP. */
AWQ_API int awq_search_timed(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                             int32_t group, int32_t n_grid, double* losses_out,
                             int32_t* best_out, float* s_best_out, float* s_table_out, void* ws,
                             size_t ws_bytes, uint32_t* flags, awq_stream_t stream,
                             awq_event_t fused_begin, awq_event_t fused_end);

/* The same search without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It calls no hipMalloc, hipFree or allocating library routine: its workspace
 * is a static device array of AWQ_STATIC_SCRATCH_BYTES (128 MiB) inside the library, one
 * copy on each GPU the library runs on, held until the process ends.  The current device
 * must be the device of `stream`.
 *   Limit: a call whose workspace less the copy of X (awq_search_workspace_bytes minus
 *          xcopy, see awq_search) exceeds AWQ_STATIC_SCRATCH_BYTES returns AWQ_ERR_SCRATCH
 *          before any HIP call (for n_grid = 20 that part is about 1.25 N K bytes: K = N =
 *          4096 needs 21 MB, K = 14336 with N = 4096 needs 74 MB; N = 28672 with K = 4096
 *          does not fit).  The copy of X is used when the whole workspace fits (K = N = M =
 *          4096: 55 MB), else the kernel that stages X itself runs.
 *   Sharing: every call on one GPU uses that GPU's single copy and leaves its contents
 *          behind; nothing in it has to start at zero.  Calls that overlap on one GPU (two
 *          streams, or two host threads) race on it and must be serialised by the caller.
 * Arguments, results and other errors as awq_search (no ws, ws_bytes). */
#define AWQ_STATIC_SCRATCH_BYTES (128u * 1024u * 1024u)
AWQ_API int awq_search_static(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                              const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                              int32_t group, int32_t n_grid, double* losses_out, int32_t* best_out,
                              float* s_best_out, float* s_table_out, uint32_t* flags,
                              awq_stream_t stream);

/* The same search for projections that read one X and must share one scale vector
 * ([EXPLAINER §6]: Q, K and V all consume the normalized input, so s applies to all of them
 * together), given as a list of weights instead of one concatenated W: the layer's output
 * channels are the rows of Ws[0], then Ws[1], ..., and
 *   loss_i = sum over all weights and m, n of (X E^T)[m,n]^2 / (M * sum_w N_w).
 * Each weight's rows are padded to a multiple of 128 inside the search, so with every N_w a
 * multiple of 128 the losses are bit-identical to awq_search on the concatenated W.
 *   Ws, Ns, ldws   host arrays of n_weights (1..8) entries: device pointer, rows and row
 *                  stride of each weight [N_w, K] (all of dtype w_dtype); read during the
 *                  call only
 *   ws             workspace of at least awq_search_multi_workspace_bytes(...) bytes
 * Other arguments, results and errors as awq_search. */
AWQ_API size_t awq_search_multi_workspace_bytes(int64_t M, int64_t K, const int64_t* Ns,
                                                int32_t n_weights, int32_t group, int32_t n_grid);
AWQ_API int awq_search_multi(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const void* const* Ws, int w_dtype, const int64_t* Ns,
                             const int64_t* ldws, int32_t n_weights, const float* a,
                             int32_t group, int32_t n_grid, double* losses_out,
                             int32_t* best_out, float* s_best_out, float* s_table_out, void* ws,
                             size_t ws_bytes, uint32_t* flags, awq_stream_t stream);

/* The same search with the loss in its Gram form ([EXPLAINER §1]: the exact layer-output
 * squared error carries the cross terms of X^T X):
 *   sum_{m,n} (X E^T)[m,n]^2 = sum_n E[n,:] G E[n,:]^T,   G = X^T X,
 * with G formed once on the matrix cores (fp32 sums per 1024 tokens, then across blocks) and
 * kept as G_hi + G_lo, two bf16 matrices (16 significand bits of G) interleaved in one
 * [K, 2K] matrix.  Every candidate then multiplies both with E^T into the same outputs
 * (2 * 2 K^2 N flop instead of 2 M K N) and dots each output with E[n, k'], both E rounded to
 * bf16 as the direct form's product operand is.  For K > 512 the
 * matrix holds T = diag(G) + 2 triu(G, 1) instead (the same quadratic form, zero below the
 * diagonal), and each 512-row block of the product skips the columns left of its first row:
 * about 2 K (K + 512) N flop per candidate, less work than the direct form when
 * M > K + 512 (the cost of G aside).  The losses differ
 * from awq_search's only by rounding: G's representation (2^-16 relative per entry) and its
 * sums, and the sums over k of products that cancel (the quadratic form), where the direct
 * form sums squares.  Candidates, codes, tie rule and outputs as awq_search.
 *   X, W   AWQ_DTYPE_BF16 only (AWQ_ERR_UNSUPPORTED otherwise); 512 x 2K bf16 must span less
 *          than 2^31 bytes (K < 2^20)
 *   ws     workspace of at least awq_search_gram_workspace_bytes(...) bytes: the search
 *          workspace for K rows (without a copy of X), the K x 2K bf16 matrix (stored in
 *          matrix-core operand order), and fp32 sums of the G tiles that are split along the
 *          tokens to fill the last round of blocks (at most 64 MiB)
 * Other arguments, results and errors as awq_search. */
AWQ_API size_t awq_search_gram_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group,
                                               int32_t n_grid);
AWQ_API int awq_search_gram(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                            const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                            int32_t group, int32_t n_grid, double* losses_out, int32_t* best_out,
                            float* s_best_out, float* s_table_out, void* ws, size_t ws_bytes,
                            uint32_t* flags, awq_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Step 5: real quantization and packing of S W ([EXPLAINER §7, §8]; [MODULES §5.3]:
 * INT4 codes eight per int32).  Exact fp32 contract: v = W*s, Delta = max(max-min,1e-5)/15
 * and q use correctly rounded division and ties-to-even rounding, bit-identical to the
 * definition above.
 *   qweight  int32 [N, K/8]: nibble i (bits 4i..4i+3) of word j holds the code of k = 8j+i
 *   scales   fp16 [N, K/128] (uint16 storage): Delta rounded to nearest even
 *   zeros    fp16 [N, K/128] (uint16 storage): the integer zero point z (never -0)
 * The dequantized weight is scales * (q - zeros) / s[k]; the caller folds 1/s into the
 * producer of X ([EXPLAINER §6]).  4.25 bits per weight ([EXPLAINER §8]).
 *   flags    AWQ_FLAG_NONFINITE_W, AWQ_FLAG_SCALE_RANGE, AWQ_FLAG_F16_RANGE
 * ------------------------------------------------------------------------------------- */
AWQ_API int awq_pack(const void* W, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                     const float* s, int32_t group, int32_t* qweight, uint16_t* scales,
                     uint16_t* zeros, uint32_t* flags, awq_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * After the scale search: the clipping search ([EXPLAINER §5]).  With the scales s (normally
 * awq_search's s_best_out), v = W*s (fp32); for every row n and group g of 128 k,
 * absmax = max |v| over the group, and for i < n_clip (10 in the method):
 *   f_i = fp32(1 - i/20)  (1, 0.95, ..., 0.55),   c_i = fp32(absmax * f_i)
 *   the clipped group clamp(v, -c_i, c_i) is quantized with the contract of awq_search
 *   (Delta and z from the clipped group's own max and min, exact fp32 division), and
 *   err_i[n, g] = (1/M) sum_m ( sum_{k in g} X[m, k] E_i[n, k] )^2,
 *   E_i[n, k] = W[n, k] - Delta (q - z) / s_k:
 * the mean squared error of the group's partial output over the M given tokens.  The caller
 * passes the calibration tokens to score as X (a row stride ldx = r K takes every r-th row
 * of a larger X).  Each (n, g) keeps the first i with the least error.  The products run on
 * the bf16 matrix cores as in awq_search; the codes inside them use the exact contract.
 *   s             fp32 [K], finite and positive
 *   group, n_clip 128 and 1..20
 *   max_val_out   fp32 [N, K/128]: c of the chosen candidate (the clamp of awq_pack_clipped)
 *   best_out      int32 [N, K/128] or NULL: the chosen i
 *   err_out       fp64 [n_clip, N, K/128] or NULL: every candidate's error
 *   ws            workspace of at least awq_clip_workspace_bytes(...) bytes (device)
 *   flags         AWQ_FLAG_NONFINITE_W, AWQ_FLAG_SCALE_RANGE, AWQ_FLAG_NONFINITE_LOSS
 * ------------------------------------------------------------------------------------- */
AWQ_API size_t awq_clip_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group,
                                        int32_t n_clip);
AWQ_API int awq_clip(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                     const void* W, int w_dtype, int64_t N, int64_t ldw, const float* s,
                     int32_t group, int32_t n_clip, float* max_val_out, int32_t* best_out,
                     double* err_out, void* ws, size_t ws_bytes, uint32_t* flags,
                     awq_stream_t stream);

/* awq_pack of the clipped weight clamp(W*s, -max_val, max_val) ([EXPLAINER §5]: the chosen
 * thresholds apply to the real quantization).  max_val: fp32 [N, K/128] (normally
 * awq_clip's max_val_out); NULL gives awq_pack.  Outputs, contract and flags as awq_pack. */
AWQ_API int awq_pack_clipped(const void* W, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                             const float* s, const float* max_val, int32_t group,
                             int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                             uint32_t* flags, awq_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Applying the chosen scales ([EXPLAINER §6]).  The inverse scaling goes into the producer of
 * X and every projection that reads X takes s on its input columns (all of them: Q, K and V
 * share one X).  Each result is the exact quotient or product rounded once to the operand's
 * type (fp32 correctly rounded; bf16 round to nearest even).  In place unless noted; dtype
 * AWQ_DTYPE_F32 or AWQ_DTYPE_BF16; no group constraint on the sizes; elementwise and
 * bandwidth-bound (16-byte accesses when every row start is 16-byte aligned).
 *   awq_fold_rows   A [rows, cols], row stride lda: A[r, c] /= s[r].  A producer's output
 *                   channel r feeds input channel r of the scaled layer: a LayerNorm's gamma
 *                   and beta (rows = K, cols = lda = 1; both must be folded), an RMSNorm's
 *                   gamma, or a preceding Linear's weight [K, K_in] and bias [K].
 *   awq_scale_cols  W [N, K], row stride ldw: W[n, k] *= s[k] (a consuming Linear).
 *   awq_scaled_act  Y[m, k] = act(X[m, k]) / s[k], X and Y [M, K] with row stride ld (Y may be
 *                   X): the runtime form after a non-linearity, where nothing can absorb S^-1;
 *                   the division follows the activation.  act: AWQ_ACT_GELU (exact,
 *                   0.5 x (1 + erf(x / sqrt 2))) or AWQ_ACT_SILU (x / (1 + exp(-x))), in fp32
 *                   with the device erfc / exp, so within a few fp32 ulps of the exact value.
 *   s               fp32 [rows] (fold) or [K], 4-byte aligned
 *   flags           AWQ_FLAG_SCALE_RANGE if a scale is not finite and positive
 * ------------------------------------------------------------------------------------- */
#define AWQ_ACT_GELU 0
#define AWQ_ACT_SILU 1
AWQ_API int awq_fold_rows(void* A, int dtype, int64_t rows, int64_t cols, int64_t lda, const float* s,
                          uint32_t* flags, awq_stream_t stream);
AWQ_API int awq_scale_cols(void* W, int dtype, int64_t N, int64_t K, int64_t ldw, const float* s,
                           uint32_t* flags, awq_stream_t stream);
AWQ_API int awq_scaled_act(const void* X, void* Y, int dtype, int64_t M, int64_t K, int64_t ld, int act,
                           const float* s, uint32_t* flags, awq_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Using the artefact: the W4A16 product ([EXPLAINER §7]: decode Delta (q - z); §8: 4-bit
 * weights with 16-bit activations, the weight decoded on the fly and never written back).
 *   Y[m, n] = sum_k X'[m, k] * scales[n, k/128] * (q[n, k] - zeros[n, k/128])
 * with the artefact of awq_pack / awq_pack_clipped (qweight int32 [N, K/8], nibble i of word j
 * = code of k = 8j+i; scales, zeros fp16 [N, K/128]) and activations X' that already carry
 * S^-1 (folded into their producer, awq_fold_rows, or awq_scaled_act).
 *   X        [M, K], AWQ_DTYPE_BF16 or AWQ_DTYPE_F32, row stride ldx (16-byte aligned rows)
 *   Y        fp32 [M, N], row stride ldy >= N
 * Up to 8 bf16 tokens (any number of fp32 tokens, 8 per launch) take the decode kernel:
 * products exact in fp32, the group scale applied per 32 channels, fp32 sums.  More bf16
 * tokens take the prefill kernel on the bf16 matrix cores, which rounds the decoded weight
 * Delta (q - z) once to bf16 (relative 2^-8) and accumulates in fp32.
 * qweight must be 16-byte aligned.  No data-error flags: non-finite X reaches Y.
 * ------------------------------------------------------------------------------------- */
AWQ_API int awq_w4a16(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                      const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group, float* Y,
                      int64_t ldy, awq_stream_t stream);

/* The same product with a workspace.  The prefill (bf16 X, more than 8 tokens) then first
 * copies X into matrix-core operand order in the workspace (the layout of awq_search's copy of
 * X) and reads its matrix operand from there straight into registers, instead of staging X
 * through on-chip memory: the same products in the same order, so Y is identical bit for bit.
 *   awq_w4a16_workspace_bytes: the bytes that copy needs, 2 * round_up(M, 32) * K for bf16 X
 *              with more than 8 tokens, else 0 (no workspace used; 0 also for invalid sizes)
 *   ws         device memory of at least that size, 16-byte aligned, or NULL; a smaller
 *              workspace (or NULL) runs the product as awq_w4a16 does
 * Other arguments, results and errors as awq_w4a16. */
AWQ_API size_t awq_w4a16_workspace_bytes(int64_t M, int64_t K, int x_dtype);
AWQ_API int awq_w4a16_ws(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                         const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group, float* Y,
                         int64_t ldy, void* ws, size_t ws_bytes, awq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_H */
