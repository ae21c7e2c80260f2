/*
 * w8a8.h -- guarded W8A8 block-quantized linear layer for AMD MI355X (gfx950).
 *
 * The operation (Y = X * W^T for a linear layer, X[M,K] activations, W[N,K]
 * output-channel weight rows) is the guarded INT8 linear of the TurboT2VA
 * inference stack, in the 128x128 block form:
 *
 *   - weights and activations are quantized to INT8 per 128x128 block
 *     (TurboDiffusion news article, bjdmk.com.cn: quantization section and
 *     inference list -- linear weights at 128x128 block granularity,
 *     activations at the same granularity during inference, INT8 GEMM);
 *   - each block's scale is its max-abs value divided by 127, weights are
 *     quantized once ("static"), activations on every call ("dynamic"),
 *     products accumulate in INT32 and scales/bias are applied in the
 *     epilogue (TurboT2VA paper, arXiv 2608.24674, architecture-aware
 *     inference stack, W8A8 linear paragraph -- there per row/channel; here
 *     per block, so the INT32 sum is exact within each 128-deep K-block and
 *     the block scales are applied once per K-block);
 *   - the guard: only a bf16 input whose M, K and N are multiples of 128
 *     goes to INT8; any other call is computed in bf16 from the bf16 weight
 *     the layer keeps beside its INT8 copy (TurboT2VA paper, same section,
 *     guard paragraph; pchao.org summary, method overview and caveats).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE memory (HIP), row-major and contiguous.
 *     bf16 and fp16 tensors are arrays of 16-bit words.  A host pointer, or
 *     any pointer HIP does not know as device-accessible, is rejected with
 *     W8A8_ERR_INVALID_ARG before anything is enqueued.
 *   - Quantized tensors: q int8 [R, C] with the same layout as the source,
 *     scales fp32 [R/128, C/128] row-major (block (i, j) covers rows
 *     128i..128i+127 and columns 128j..128j+127).
 *   - Quantization: a = max |v| over the block (exact), s = fl32(a / 127),
 *     q = rint(fl32(v / s)) (ties to even, correctly rounded division),
 *     clamped to [-127, 127]; an all-zero block has s = 0 and q = 0.
 *     Inputs must be finite.
 *   - Ownership: the caller allocates every buffer (including the
 *     workspace) and keeps it alive until the enqueued work completes.  The
 *     library never allocates, frees, copies to or from the host, or
 *     synchronizes; all work is enqueued on `stream` (0 = null stream).
 *   - Errors: integer status, nothing thrown.  On an error detected before a
 *     launch nothing is enqueued.  W8A8_ERR_HIP means a HIP call failed; the
 *     HIP error code is kept per thread (w8a8_last_hip_error).
 *   - The library is stateless apart from that per-thread slot: calls are
 *     reentrant; calls on different streams may run concurrently.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { W8A8_OK = 0, W8A8_ERR_INVALID_ARG = 1, W8A8_ERR_UNSUPPORTED = 2, W8A8_ERR_HIP = 3 };
enum { W8A8_DTYPE_BF16 = 0, W8A8_DTYPE_FP16 = 1, W8A8_DTYPE_FP32 = 2 };
enum { W8A8_PATH_INT8 = 0, W8A8_PATH_BF16 = 1 };
#define W8A8_BLOCK 128

/* Largest K of the block-scale GEMM: it addresses a 256-row operand tile
 * with 32-bit byte offsets (256 * K < 2^31). */
#define W8A8_BLOCK_MAX_K 4194304
/* Largest row stride (in elements) of the rotary embedding's fused Q/K entry,
 * whose per-block buffer offsets are 32-bit. */
#define W8A8_ROPE_MAX_LD 4194304

/*
 * Static weight quantization (done once, at load): w_bf16 [N, K] ->
 * qw int8 [N, K] and sw fp32 [N/128, K/128].
 * Strict: N or K not a multiple of 128, or w_bf16/qw not 16-byte aligned ->
 * W8A8_ERR_UNSUPPORTED.  Null pointers or N, K <= 0 -> W8A8_ERR_INVALID_ARG.
 */
int w8a8_quantize_weight(const void *w_bf16, int64_t N, int64_t K, int8_t *qw, float *sw,
                         hipStream_t stream);

/*
 * Dynamic activation quantization (every call): x_bf16 [M, K] ->
 * qx int8 [M, K] and sx fp32 [M/128, K/128].  Same rule and errors as
 * w8a8_quantize_weight.
 */
int w8a8_quantize_act(const void *x_bf16, int64_t M, int64_t K, int8_t *qx, float *sx,
                      hipStream_t stream);

/*
 * INT8 GEMM on already-quantized operands with per-K-block dequantization:
 *   Y[m, n] = bf16( sum_kb  P[m, n, kb] * sx[m/128, kb] * sw[n/128, kb]
 *                   (+ bias[n]) ),
 *   P[m, n, kb] = exact int32 sum over the 128 k of K-block kb of
 *                 qx[m, k] * qw[n, k].
 * The sum over K-blocks is carried in fp32; bias (bf16 [N], nullable) is
 * added in fp32; Y is bf16 [M, N], rounded to nearest even.
 * Strict: M, N, K multiples of 128, K <= W8A8_BLOCK_MAX_K and qx, qw, y
 * 16-byte aligned, else W8A8_ERR_UNSUPPORTED.
 */
int w8a8_gemm_blockscale(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                         const void *bias_bf16, int64_t M, int64_t N, int64_t K, void *y_bf16,
                         hipStream_t stream);

/*
 * Bytes of workspace w8a8_linear needs for the INT8 path: qx [M, K] plus sx
 * [M/128, K/128], each 256-byte aligned inside the workspace.  0 when M or K
 * is not a multiple of 128 (such calls always take the fallback).
 */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * Guarded linear: Y[M, N] (bf16) = X[M, K] * W[N, K]^T (+ bias).
 *   x        : [M, K], dtype x_dtype (W8A8_DTYPE_*), M = flattened leading dims
 *   w_bf16   : the layer's bf16 weight [N, K] (required: the fallback uses it)
 *   qw, sw   : w8a8_quantize_weight outputs for w_bf16 (both null -> no
 *              INT8 path; exactly one null -> W8A8_ERR_INVALID_ARG)
 *   bias_bf16: [N] or null
 *   y_bf16   : [M, N] output
 *   workspace: >= w8a8_linear_workspace_bytes(M, K) bytes when the INT8
 *              path is taken (may be null/0 otherwise)
 *   path_out : if not null, receives the W8A8_PATH_* taken
 * INT8 path iff w8a8_route(...) == W8A8_PATH_INT8, K <= W8A8_BLOCK_MAX_K,
 * x, y and qw are 16-byte aligned, sw 4-byte and bias 8-byte aligned, and
 * the workspace is 16-byte aligned: then the activation is quantized into
 * the workspace and w8a8_gemm_blockscale's computation runs.  Otherwise the
 * bf16 fallback runs: Y = bf16( sum_k bf16(x[m,k]) * w[n,k] (+ bias[n]) )
 * with fp32 accumulation; fp16/fp32 x is rounded to bf16 (nearest even) on
 * load.  The path is decided from dtype, shapes, qw and the operands'
 * alignment first; only a call that takes the INT8 path needs the
 * workspace.  Never fails on dtype or shape: returns W8A8_ERR_INVALID_ARG
 * only for null required pointers, sizes <= 0, an unknown dtype, a host
 * pointer, or (INT8 path) a missing or too small workspace.
 */
int w8a8_linear(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16,
                void *workspace, size_t workspace_bytes, hipStream_t stream, int *path_out);

/* Size of the device array that w8a8_linear_noalloc uses as its workspace:
 * 32 MiB + 64 KiB, enough for M*K up to 2^25 (e.g. 8192 x 4096). */
#define W8A8_NOALLOC_SCRATCH_BYTES (33554432 + 65536)

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): w8a8_linear with no
 * workspace argument.  The INT8 path's qx and sx go to a fixed device array
 * of W8A8_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; this entry never allocates or frees memory.
 * Same guard, arguments, results and errors as w8a8_linear, plus:
 * W8A8_ERR_UNSUPPORTED when the call takes the INT8 path and
 * w8a8_linear_workspace_bytes(M, K) exceeds the array (use w8a8_linear with
 * a caller workspace then; a call that the guard sends to the fallback runs
 * at any size);
 * W8A8_ERR_HIP if the array's device address cannot be obtained.  The array
 * belongs to the stream's device (the current device for the null stream).
 * Calls share it: calls that overlap in time on one GPU (several streams,
 * several threads) race on its contents and must be ordered by the caller.
 */
int w8a8_linear_noalloc(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                        const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16, hipStream_t stream,
                        int *path_out);

/*
 * The guard alone (host only, pure, touches no device): W8A8_PATH_INT8 iff
 * x_dtype is bf16, M, K and N are multiples of 128 and has_qweight != 0;
 * W8A8_PATH_BF16 for every other valid call; -1 for sizes <= 0 or an
 * unknown dtype.  w8a8_linear additionally sends misaligned pointers to the
 * fallback.
 */
int w8a8_route(int x_dtype, int64_t M, int64_t K, int64_t N, int has_qweight);

/*
 * Test hook: the INT8 GEMM's main loop with an epilogue that stores the
 * exact int32 per-K-block partials instead of dequantizing them.
 * Window rows [m0, m0+mt) of qx and [n0, n0+nt) of qw; m0, mt, n0, nt
 * multiples of 128 inside the matrices; partials int32 [mt, nt, K/128].
 * Strict shape/alignment rules (and K limit) as w8a8_gemm_blockscale.
 */
int w8a8_debug_kblock_partials(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N, int64_t K,
                               int64_t m0, int64_t mt, int64_t n0, int64_t nt, int32_t *partials,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Post-scale form (TurboT2VA paper, architecture-aware inference stack, W8A8
 * paragraph): static per-output-channel weight scales and dynamic per-row
 * activation scales, s = max(max-abs, 1e-4) / 127 (eps = fl32(1e-4)), INT32
 * accumulation over the whole of K, both scales and the bias applied once in
 * the epilogue.  The guard is the same as for the block form.
 * ------------------------------------------------------------------------- */

/* Largest K the post-scale GEMM accepts: K * 127^2 must fit in int32. */
#define W8A8_POSTSCALE_MAX_K 133120

/*
 * Row-wise quantization: x_bf16 [R, K] -> q int8 [R, K] and s fp32 [R],
 * s_i = fl32(max(max_k |x_ik|, eps) / 127), q = rint(fl32(x / s)) ties to
 * even, clamp [-127, 127].  Used for activations (rows = tokens) and weights
 * (rows = output channels).  Strict: K % 8 != 0 or x/q not 16-byte aligned
 * -> W8A8_ERR_UNSUPPORTED; null pointers or R, K <= 0 -> W8A8_ERR_INVALID_ARG.
 */
int w8a8_quantize_rows(const void *x_bf16, int64_t R, int64_t K, int8_t *q, float *s,
                       hipStream_t stream);

/*
 * Post-scale INT8 GEMM:
 *   Y[m, n] = bf16( float(sum_k qx[m, k] * qw[n, k]) * sx[m] * sw[n] (+ bias[n]) ),
 * the sum exact in int32 over all K.  qx [M,K], sx [M], qw [N,K], sw [N].
 * Strict: M, N, K multiples of 128, K <= W8A8_POSTSCALE_MAX_K, qx/qw/y
 * 16-byte aligned, sw 16-byte aligned, else W8A8_ERR_UNSUPPORTED.
 */
int w8a8_gemm_postscale(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                        const void *bias_bf16, int64_t M, int64_t N, int64_t K, void *y_bf16,
                        hipStream_t stream);

/* Workspace of w8a8_linear_postscale: qx [M, K] + sx [M], each 256-byte
 * aligned; 0 when M or K is not a multiple of 128. */
size_t w8a8_linear_postscale_workspace_bytes(int64_t M, int64_t K);

/*
 * Guarded post-scale linear: same arguments, guard and fallback as
 * w8a8_linear, with qw/sw from w8a8_quantize_rows (sw [N]).  INT8 path iff
 * w8a8_route(...) == W8A8_PATH_INT8, K <= W8A8_POSTSCALE_MAX_K and the
 * pointers are 16-byte aligned; otherwise the bf16 fallback.
 */
int w8a8_linear_postscale(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N,
                          const void *w_bf16, const int8_t *qw, const float *sw,
                          const void *bias_bf16, void *y_bf16, void *workspace,
                          size_t workspace_bytes, hipStream_t stream, int *path_out);

/* ---------------------------------------------------------------------------
 * Producer fused with the activation quantization (TurboT2VA paper,
 * architecture-aware inference stack: memory-bound elementwise work is fused
 * into neighbouring kernels).  The producer here is the MLP's activation
 * between its two linears: exact GELU, x * Phi(x) with Phi the standard
 * normal CDF (Hendrycks and Gimpel), rounded once to bf16 (nearest, ties to
 * even).  Results equal an fp64 evaluation of x * erfc(-x / sqrt 2) / 2
 * rounded once to bf16, for every finite bf16 x.  Inputs must be finite.
 * ------------------------------------------------------------------------- */

/* Largest K of w8a8_gelu_quantize_act (a 128-row tile must span < 2^31 bytes). */
#define W8A8_GELU_QUANT_MAX_K 8388480

/*
 * Elementwise GELU: y[i] = bf16(GELU(x[i])) for i < n (bf16 in, bf16 out).
 * Any n >= 0 (n = 0 enqueues nothing and accepts null pointers); y may equal
 * x (in place).  Pointers must be 2-byte aligned device memory, else
 * W8A8_ERR_UNSUPPORTED / W8A8_ERR_INVALID_ARG; n < 0 -> W8A8_ERR_INVALID_ARG.
 */
int w8a8_gelu_bf16(const void *x_bf16, int64_t n, void *y_bf16, hipStream_t stream);

/*
 * Fused producer + quantize: X' = bf16(GELU(y)) elementwise on y_bf16 [M, K],
 * then X' is quantized by the block rule of w8a8_quantize_act into qx int8
 * [M, K] and sx fp32 [M/128, K/128].  X' itself is never written: the codes
 * and scales equal w8a8_quantize_act applied to w8a8_gelu_bf16(y), bit for
 * bit.  Strict like w8a8_quantize_act (M, K multiples of 128, y and qx
 * 16-byte aligned, else W8A8_ERR_UNSUPPORTED), and K <= W8A8_GELU_QUANT_MAX_K.
 */
int w8a8_gelu_quantize_act(const void *y_bf16, int64_t M, int64_t K, int8_t *qx, float *sx,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The other producer the TurboT2VA paper fuses (architecture-aware inference
 * stack, fused-kernels paragraph): RMS normalization combined with a
 * timestep-dependent scale and shift, the input of a transformer block's
 * projections.  For row i = b*L + l of x_bf16 [B*L, K] (L tokens per batch
 * entry b; scale_bf16 and shift_bf16 are [B, K]):
 *   r_i  = fl32( 1 / sqrt(sum_k x_ik^2 / K + eps) )   (fp64, rounded once),
 *   y_ik = bf16( fl32(fl32(fl32(x_ik * r_i) * fl32(1 + scale[b,k])) + shift[b,k]) )
 * each fl32 one IEEE fp32 operation, bf16 rounding to nearest even.  The sum
 * of squares is an fp64 sum in the kernel's order; another order can move
 * it by a few fp64 ulps, which changes r only when r lies within ~2^-50 of
 * an fp32 rounding boundary.  eps must be finite and > 0, inputs finite;
 * B*L < 2^31.  Errors: null pointers, sizes <= 0 or a bad eps ->
 * W8A8_ERR_INVALID_ARG; K % 8 != 0 or x, scale, shift (and y or qx) not
 * 16-byte aligned -> W8A8_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */

/* y_bf16 [B*L, K] = the modulated normalization of x (any B*L >= 1); r_ws is
 * a caller-provided workspace of B*L floats (4-byte aligned, else
 * W8A8_ERR_UNSUPPORTED) that receives r. */
int w8a8_rmsnorm_modulate_bf16(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                               const void *shift_bf16, double eps, float *r_ws, void *y_bf16, hipStream_t stream);

/* Bytes of workspace w8a8_rmsnorm_modulate_quantize_act needs for M = B*L
 * rows of width K (0 when M or K <= 0). */
size_t w8a8_rmsnorm_quantize_workspace_bytes(int64_t M, int64_t K);

/*
 * Fused producer + quantize: y as above, quantized by the block rule of
 * w8a8_quantize_act into qx int8 [B*L, K] and sx fp32 [B*L/128, K/128]
 * without ever being written (equal, bit for bit, to w8a8_quantize_act
 * applied to w8a8_rmsnorm_modulate_bf16's output).  B*L and K must be
 * multiples of 128 (else W8A8_ERR_UNSUPPORTED).
 *
 * When K % 256 == 0 and the K/256 workgroups of a band need at most half of
 * what the current device holds of them at once (K up to 98304 on a whole
 * MI355X), x is read once: the workgroups of each 128-row band hold
 * 256-column slices in registers and exchange fp64 row partials through the
 * workspace, waiting for one another (bounded: a wait that does not
 * complete in ~1 s gives up and leaves the codes of its slice wrong; the
 * workspace's first 32-bit word is cleared at the start of such a call and
 * set nonzero by a wait that gives up).  Other widths take two reads of x
 * and do not touch that word.  workspace: device memory,
 * 16-byte aligned (else W8A8_ERR_UNSUPPORTED), at least
 * w8a8_rmsnorm_quantize_workspace_bytes(B*L, K) bytes (else
 * W8A8_ERR_INVALID_ARG); its contents on return are scratch apart from that
 * first word.  Calls that share a workspace must not overlap in time.
 */
int w8a8_rmsnorm_modulate_quantize_act(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                       const void *shift_bf16, double eps, void *workspace, size_t workspace_bytes,
                                       int8_t *qx, float *sx, hipStream_t stream);

/*
 * The layer-normalization form of the producer (the fused-kernels paragraph
 * replaces LayerNorm modules as well as RMSNorm ones), no affine weight; for
 * row i = b*L + l:
 *   m_i  = fl32(mean_k x_ik),   r_i = fl32( 1 / sqrt(var_k x_ik + eps) )
 *          (mean and variance in fp64, the variance over the deviations
 *          from the fp64 mean)
 *   y_ik = bf16( fl32( fl32( fl32( fl32(x_ik - m_i) * r_i ) * fl32(1 + scale[b,k]) ) + shift[b,k] ) )
 * Arguments, layouts and errors as for the RMS entries, except the caller's
 * workspace stats_ws: 2*B*L floats, 8-byte aligned (else
 * W8A8_ERR_UNSUPPORTED), left holding (m_i, r_i) per row.  The fused entry
 * equals, bit for bit, w8a8_quantize_act applied to the bf16 entry's y.
 */
int w8a8_layernorm_modulate_bf16(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                 const void *shift_bf16, double eps, float *stats_ws, void *y_bf16,
                                 hipStream_t stream);
int w8a8_layernorm_modulate_quantize_act(const void *x_bf16, int64_t B, int64_t L, int64_t K,
                                         const void *scale_bf16, const void *shift_bf16, double eps,
                                         float *stats_ws, int8_t *qx, float *sx, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Guarded linears with their producer in front (the TurboT2VA paper's guard
 * paragraph and fused-kernels paragraph together: the fused kernel runs when
 * the INT8 path applies, else the unfused producer and the bf16 linear).
 * The route is w8a8_linear's, taken on the producer's bf16 output [M, K]:
 * INT8 iff M, K, N are multiples of 128, a quantized weight is given, K is
 * within the fused quantizer's and the GEMM's limits and the input, y, qw
 * (16 bytes), sw (4) and bias (8) are aligned.  The INT8 path runs the fused
 * producer + block quantization into the workspace and the block GEMM (the
 * result equals w8a8_linear on the producer's bf16 output, bit for bit); the
 * fallback writes the producer's bf16 output into the workspace and runs the
 * bf16 GEMM on it.  Both paths need the workspace (device memory, 16-byte
 * aligned, w8a8_linear_producer_workspace_bytes(M, K) bytes, else
 * W8A8_ERR_INVALID_ARG / W8A8_ERR_UNSUPPORTED).  path_out (nullable)
 * receives the W8A8_PATH_* taken.
 * ------------------------------------------------------------------------- */

/* Workspace of the producer linears: the larger of qx + sx and a bf16 [M, K]
 * copy, plus 8 bytes of statistics per row, each part 256-byte aligned. */
size_t w8a8_linear_producer_workspace_bytes(int64_t M, int64_t K);

/*
 * Y[M, N] = bf16(GELU(u)) [M, K] * W^T (+ bias): the MLP's second linear with
 * the exact GELU of w8a8_gelu_bf16 in front; u bf16 [M, K] (2-byte aligned).
 */
int w8a8_linear_gelu(const void *u_bf16, int64_t M, int64_t K, int64_t N, const void *w_bf16, const int8_t *qw,
                     const float *sw, const void *bias_bf16, void *y_bf16, void *workspace, size_t workspace_bytes,
                     hipStream_t stream, int *path_out);

/*
 * Y[B*L, N] = w8a8_rmsnorm_modulate_bf16(x, scale, shift, eps) * W^T (+ bias)
 * (and the layer-normalization form): x bf16 [B*L, K], scale and shift
 * [B, K], eps and the normalization's own requirements as documented for
 * w8a8_rmsnorm_modulate_bf16 (K % 8 == 0 and 16-byte aligned x, scale and
 * shift on both paths, else W8A8_ERR_UNSUPPORTED).
 */
int w8a8_linear_rmsnorm_modulate(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                 const void *shift_bf16, double eps, int64_t N, const void *w_bf16, const int8_t *qw,
                                 const float *sw, const void *bias_bf16, void *y_bf16, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream, int *path_out);
int w8a8_linear_layernorm_modulate(const void *x_bf16, int64_t B, int64_t L, int64_t K, const void *scale_bf16,
                                   const void *shift_bf16, double eps, int64_t N, const void *w_bf16,
                                   const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream, int *path_out);

/* ---------------------------------------------------------------------------
 * Gated residual update (TurboT2VA paper, architecture-aware inference stack,
 * fused-kernels paragraph, which lists gated residual updates among the fused
 * patterns): the residual stream h takes a linear's output o scaled by a
 * gate per batch entry and channel,
 *   y[i, n] = bf16( fl32( h[i, n] + fl32( gate[i / L, n] * o[i, n] ) ) )
 * each fl32 one IEEE fp32 operation, bf16 to nearest even.  h, o, y are bf16
 * [B*L, N] = [M, N] row-major; gate bf16 [B, N]; L = rows (tokens) per batch
 * entry.  N must be a multiple of 8 and h, o, gate, y 16-byte aligned (else
 * W8A8_ERR_UNSUPPORTED); null pointers, sizes <= 0, M not a multiple of L, or
 * a y that overlaps h (or o) without coinciding -> W8A8_ERR_INVALID_ARG.
 * All buffers are the caller's device memory; calls are asynchronous on
 * `stream`.  Inputs must be finite (a sum may round to +-Inf).
 * ------------------------------------------------------------------------- */

/* The update alone: y may be h or o itself (in place). */
int w8a8_gated_residual(const void *h_bf16, const void *o_bf16, const void *gate_bf16, int64_t B, int64_t L,
                        int64_t N, void *y_bf16, hipStream_t stream);

/*
 * w8a8_gemm_blockscale whose bf16 output o (bias included) feeds the update
 * in the GEMM's epilogue: o is rounded to bf16 exactly as w8a8_gemm_blockscale
 * writes it and never reaches memory, so the result equals, bit for bit,
 * w8a8_gated_residual applied to w8a8_gemm_blockscale's output.  Requirements
 * of both, plus M <= INT32_MAX; y may be h itself (in place).
 */
int w8a8_gemm_blockscale_gated_residual(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                                        const void *bias_bf16, int64_t M, int64_t N, int64_t K,
                                        const void *h_bf16, const void *gate_bf16, int64_t L, void *y_bf16,
                                        hipStream_t stream);

/*
 * The guarded layer followed by the update: w8a8_linear's routing, workspace
 * and errors; on the INT8 path quantize + the fused GEMM above, on the bf16
 * fallback the bf16 GEMM into y and then the update in place on y.  y must
 * not overlap h (W8A8_ERR_INVALID_ARG), since the fallback writes o into y
 * first; N a multiple of 8 and h, gate, y 16-byte aligned on both paths.
 */
int w8a8_linear_gated_residual(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                               const int8_t *qw, const float *sw, const void *bias_bf16, const void *h_bf16,
                               const void *gate_bf16, int64_t L, void *y_bf16, void *workspace,
                               size_t workspace_bytes, hipStream_t stream, int *path_out);

/* ---------------------------------------------------------------------------
 * INT8 query/key for the sparse attention (TurboT2VA paper, architecture-
 * aware inference stack, sparse-attention paragraph: its kernel consumes Q
 * and K as INT8 and in its own layout, not token-major).  The attention
 * kernel itself is not part of this library.
 * ------------------------------------------------------------------------- */

/*
 * Attention Q or K, quantized per block of 128 tokens x D head dims:
 *   input  x_bf16, element (b, l, h, d) at x[(b*L + l)*ld + h*D + d]
 *          (sequence-major; ld >= H*D is the row stride in elements, so x
 *          may be a column slice of a fused Q/K/V projection output);
 *   output q int8 [B, H, L, D] (head-major, contiguous) and
 *          s fp32 [B, H, ceil(L/128)], block j of (b, h) covering tokens
 *          128j .. min(128j + 127, L - 1);
 *   rule   the block rule of w8a8_quantize_act over each block's tokens and
 *          all D dims (s = fl32(max |x| / 127), q = rint(fl32(x / s)) ties
 *          to even, an all-zero block has s = 0, q = 0).
 * Any L >= 1 (the last block may be shorter).  D must be 64 or 128, x
 * 16-byte aligned with ld a multiple of 8, q 16-byte aligned, else
 * W8A8_ERR_UNSUPPORTED; null pointers, sizes <= 0 or ld < H*D ->
 * W8A8_ERR_INVALID_ARG.  Inputs must be finite.
 */
int w8a8_quantize_qk(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, int8_t *q,
                     float *s, hipStream_t stream);

/*
 * Attention V in FP8 beside the INT8 Q/K (same paragraph: the value
 * aggregation takes FP8 values), in the same blocks and layout as
 * w8a8_quantize_qk: per (b, h) and block of 128 tokens x D,
 * s = fl32(max |x| / 448) and code = E4M3(fl32(x / s)), the OCP FP8 format
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest finite 448,
 * no infinities), nearest with ties to the even code; an all-zero block has
 * s = 0 and codes 0.  q uint8 [B, H, L, D] (head-major, E4M3 bit patterns),
 * s fp32 [B, H, ceil(L/128)].  Arguments and errors as for w8a8_quantize_qk.
 */
int w8a8_quantize_v_fp8(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, uint8_t *q,
                        float *s, hipStream_t stream);

/*
 * Split-halves rotary position embedding of attention Q or K (TurboT2VA
 * paper, architecture-aware inference stack, fused-kernels paragraph, which
 * lists split rotary embeddings among the fused patterns), which precedes
 * their INT8 quantization:
 *   input  x_bf16 as for w8a8_quantize_qk (element (b, l, h, d) at
 *          x[(b*L + l)*ld + h*D + d]); cos_t and sin_t fp32 [L, D/2],
 *          row-major, row l holding the angles of token position l for
 *          pairs 0 .. D/2-1, shared by every batch entry and head;
 *   rule   for d < D/2, with c = cos_t[l*D/2 + d], s = sin_t[l*D/2 + d]:
 *            y(d)       = bf16(fl32(fl32(x(d) * c) - fl32(x(d + D/2) * s)))
 *            y(d + D/2) = bf16(fl32(fl32(x(d + D/2) * c) + fl32(x(d) * s)))
 *          each fl32 one IEEE fp32 operation (no fused multiply-add), bf16
 *          to nearest even.
 * w8a8_rope_bf16 writes y_bf16 [B*L, H*D] (sequence-major, contiguous).
 * w8a8_rope_quantize_qk writes w8a8_quantize_qk's outputs (q [B, H, L, D],
 * s [B, H, ceil(L/128)]) for the rotated values, which never reach memory;
 * it equals, bit for bit, w8a8_quantize_qk applied to w8a8_rope_bf16's y.
 * Requirements and errors as for w8a8_quantize_qk, plus: cos_t, sin_t (and
 * y_bf16) 16-byte aligned device memory, else W8A8_ERR_UNSUPPORTED (host
 * pointers: W8A8_ERR_INVALID_ARG); w8a8_rope_quantize_qk also needs
 * ld <= W8A8_ROPE_MAX_LD (else W8A8_ERR_UNSUPPORTED).  x must not overlap y.  All buffers are
 * the caller's; the calls are asynchronous on `stream`.
 */
int w8a8_rope_bf16(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld, const float *cos_t,
                   const float *sin_t, void *y_bf16, hipStream_t stream);
int w8a8_rope_quantize_qk(const void *x_bf16, int64_t B, int64_t L, int64_t H, int64_t D, int64_t ld,
                          const float *cos_t, const float *sin_t, int8_t *q, float *s, hipStream_t stream);

/* Static, human-readable name of a W8A8_* status code. */
const char *w8a8_status_string(int status);

/* hipError_t of the last W8A8_ERR_HIP returned on this thread (0 if none). */
int w8a8_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
