/*
 * nvfp4.h - C ABI of libnvfp4.so: NVFP4 weight quantization with FourOverSix
 * block-scale selection, dequantization, and the W4A16 GEMM over the packed
 * weights, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *  [Notes07] "SOAR Weekly Champion Notes 07 | Vanilla Xiao Zhang: NVFP4
 *            Quantization Improvements and Speculative Decoding in Practice",
 *            sections "01 Background" (E2M1 value set, M=6 convention) and
 *            "02 FourOverSix" (M=4 scale = fp8(1.5 * M=6 scale), keep the
 *            scale with the strictly smaller block MSE, format unchanged).
 *  [Recap]   "SOAR 2026 Recap: From Compute Limits to the Open-Source
 *            Ecosystem", section "1. Quantization and GEMM dispatch" (all
 *            linear weights in NVFP4 at 0.5 byte per element; W4A16 kernel
 *            for small token counts M, another path for large M, chosen by
 *            latency).
 *  [Notes08] "SOAR Weekly Champion Notes 08 | Vanilla Xiao Zhang: Evolving
 *            Speculative Decoding on MiniCPM-SALA", section "01 A Brief
 *            Recap of Speculative Decoding" (decode is bandwidth bound: every
 *            generated token reads all of the weights from GPU memory).
 *
 * Format.  A weight matrix W is [n, k] row-major (k = reduction dim,
 * k % 16 == 0).  It is stored as
 *   codes  uint8 [n, k/2]   two 4-bit E2M1 codes per byte; byte j of a row
 *                           holds element 2j in bits 0-3 and 2j+1 in bits
 *                           4-7; code bit 3 = sign, bits 0-2 = magnitude
 *                           index of {0, .5, 1, 1.5, 2, 3, 4, 6};
 *   scales uint8 [n, k/16]  one E4M3 (bias 7, max 448, no inf) bit pattern
 *                           per 16 consecutive elements along k, sign bit 0;
 *   tensor_scale float32    one per matrix;
 * and W_hat[r][c] = val(code) * scale(r, c/16) * tensor_scale.
 * The block size 16, the E4M3 flavour and the fp32 tensor scale are the
 * problem statement's choices; the pages only say "FP8 block scale".
 *
 * Conventions for every entry point.
 *  - Array arguments are DEVICE pointers to caller-owned memory, 16-byte
 *    aligned; scalar arguments marked "device scalar" are device pointers to
 *    one float, 4-byte aligned.  The library never allocates, frees or
 *    retains caller memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; buffers must stay valid until the stream has passed it.
 *  - Argument checks happen on the host before anything is enqueued; on an
 *    error nothing is written and no GPU call is made.  Errors after the
 *    checks (launch failures) return NVFP4_ERR_HIP.
 *  - The last error message of the calling thread is nvfp4_last_error().
 *  - Calls are thread-safe; the library holds no mutable global state apart
 *    from a per-device cache of the device check.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_API __attribute__((visibility("default")))

/* Status codes. */
enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_VALUE = 1,     /* null required pointer, negative dims, bad enum */
  NVFP4_ERR_UNSUPPORTED_SHAPE = 2, /* k % 16 != 0, or a dimension too large */
  NVFP4_ERR_MISALIGNED = 3,        /* pointer not aligned as documented */
  NVFP4_ERR_WORKSPACE_TOO_SMALL = 4,
  NVFP4_ERR_HIP = 5,               /* HIP runtime / launch error */
  NVFP4_ERR_UNSUPPORTED_DEVICE = 6 /* current device is not gfx950 */
};

/* Output element types. */
enum { NVFP4_BF16 = 0, NVFP4_F32 = 1 };

/* GEMM paths (token-count dispatch of [Recap] section 1). */
enum { NVFP4_PATH_AUTO = 0, NVFP4_PATH_SKINNY = 1, NVFP4_PATH_TILED = 2 };

/* Conversion implementation selector for the _ex entry points. */
enum {
  NVFP4_IMPL_DEFAULT = 0,  /* fastest implementation validated for gfx950 */
  NVFP4_IMPL_PORTABLE = 1, /* plain ALU code for FP4 rounding / decoding */
  NVFP4_IMPL_HWCVT = 2     /* gfx950 scaled FP4 conversion instructions */
};

/*
 * nvfp4_quantize_fos - FourOverSix NVFP4 quantization of one fp32 matrix.
 *
 * Computes ([Notes07] sections 01-02; the per-step arithmetic is this
 * library's stated reading, one IEEE fp32 operation per step, round to
 * nearest even, no fused multiply-add):
 *   amax  = max |w| over the matrix, or *amax_in when amax_in != NULL;
 *   s_t   = amax / 2688 (2688 = 6 * 448), or 1 if that is 0;
 *   per 16-element block: a = max |w_i|; u6 = min(a / (6 s_t), 448);
 *     sigma6 = E4M3 round-to-nearest-even(u6);
 *     sigma4 = E4M3 RNE(1.5 * sigma6), not a candidate if it overflows
 *              (sigma6 >= 320);
 *     for each candidate sigma: R = sigma ? min(1/(sigma*s_t), FLT_MAX) : 0,
 *       code_i = E2M1 RNE(|w_i| * R) (saturating at 6, sign kept, also
 *       for values that round to zero), w_hat_i = val * sigma * s_t,
 *       SSE = pairwise tree sum of (w_i - w_hat_i)^2 over the 16 elements;
 *     keep sigma4 iff it is a candidate and SSE4 < SSE6 (a tie keeps M=6).
 *
 * w          device fp32 [n, k] row-major, finite values (NaN/inf input
 *            gives unspecified codes but no fault).
 * n, k       n >= 0, k >= 0, k % 16 == 0, n * k < 2^40.
 * amax_in    device scalar or NULL.  When given it must be finite and
 *            >= max |w| (e.g. the max over all row shards of a matrix);
 *            a smaller value saturates block scales at 448.
 * amax_out   device scalar (required): receives the amax that was used.
 * tensor_scale device scalar (required): receives s_t.
 * codes      device uint8 [n, k/2].
 * scales     device uint8 [n, k/16]: E4M3 bits of the chosen block scales.
 * m4_mask    device uint8 [n, k/16] or NULL: 1 where M=4 was chosen.
 *            (Diagnostic only: the NVFP4 format does not store the choice.)
 * Kernels: one fill of amax_out + one amax reduction pass (skipped when
 * amax_in is given) and one quantization pass.  Deterministic.
 */
NVFP4_API int nvfp4_quantize_fos(const float* w, int64_t n, int64_t k, const float* amax_in,
                                 float* amax_out, float* tensor_scale, uint8_t* codes,
                                 uint8_t* scales, uint8_t* m4_mask, void* stream);

/*
 * nvfp4_tensor_amax - amax_out = max |w| over an fp32 [n, k] matrix (exact).
 * The first step of nvfp4_quantize_fos, exposed so that callers can compute
 * it separately (for example per row shard, followed by a max across shards,
 * then nvfp4_quantize_fos with amax_in).  w: device fp32, 16-byte aligned;
 * amax_out: device scalar.  n, k >= 0, n * k % 4 == 0 (true when k % 16 == 0).
 * Two kernels: a fill of amax_out and the reduction (atomic max on the fp32
 * bit pattern, which orders like the value for non-negative floats).
 */
NVFP4_API int nvfp4_tensor_amax(const float* w, int64_t n, int64_t k, float* amax_out, void* stream);

/* Same as nvfp4_quantize_fos with an explicit conversion implementation
 * (NVFP4_IMPL_*).  Every implementation produces identical bits. */
NVFP4_API int nvfp4_quantize_fos_ex(const float* w, int64_t n, int64_t k, const float* amax_in,
                                    float* amax_out, float* tensor_scale, uint8_t* codes,
                                    uint8_t* scales, uint8_t* m4_mask, int impl, void* stream);

/*
 * nvfp4_quantize_fos_gptq - FourOverSix block scales fixed first, then GPTQ's
 * error-compensating column updates inside them ([Notes07] section 03 "How we
 * integrated it": scale estimation and the M=6 / M=4 choice, then the GPTQ
 * iterations; GPTQ is the published method of Frantar et al., 2022).
 *
 * Step 1 is nvfp4_quantize_fos on w (amax_in / amax_out / tensor_scale /
 * scales / m4_mask as there).  Step 2 quantizes the columns of a working
 * copy of w in order, with each block's fixed scale (the quantizer's C5-C7),
 * and after column j subtracts e_j * U[j, l] from every later column l,
 * e_j = (w_j - w_hat_j) / U[j, j]; codes receives the result.  Each element
 * gets its updates in increasing j, one fp32 product and one fp32
 * subtraction each, so the result is exactly reproducible.
 *
 * hinv_u     device fp32 [k, k] row-major: the upper Cholesky factor U of
 *            the inverse Hessian (H^-1 = U^T U; H from calibration
 *            activations X, e.g. 2 X^T X plus damping); only the upper
 *            triangle is read; diagonal > 0.
 * workspace  device buffer of >= nvfp4_quantize_fos_gptq_workspace_size(n, k)
 *            bytes, 16-byte aligned (working copy of w and two panels of
 *            errors); contents on entry do not matter.
 * k % 64 == 0 (columns are processed 64 at a time) and (k/64)(n/64) below
 * 2^24 (one launch's grid; beyond HBM capacity anyway); other arguments as
 * nvfp4_quantize_fos.  Launches: the quantizer, then one kernel per 64
 * columns (the panel and the previous panel's trailing update together).
 */
NVFP4_API size_t nvfp4_quantize_fos_gptq_workspace_size(int64_t n, int64_t k);
NVFP4_API int nvfp4_quantize_fos_gptq(const float* w, int64_t n, int64_t k, const float* hinv_u,
                                      const float* amax_in, float* amax_out, float* tensor_scale,
                                      uint8_t* codes, uint8_t* scales, uint8_t* m4_mask,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_gptq_hessian - GPTQ's damped Hessian from calibration activations:
 * H = 2 X^T X + damp * mean(diag(2 X^T X)) * I (the matrix whose inverse
 * weighs the column errors of GPTQ, Frantar et al., 2022, run inside the
 * FourOverSix scales: [Notes07] section 03 "How we integrated it").
 *
 * x          device bf16 [s, k] row-major: s calibration samples of the
 *            layer's k inputs (the activations the layer sees).
 * damp       the damping fraction (GPTQ uses 0.01); finite, >= 0.
 * h          device fp32 [k, k] row-major, written whole (symmetric).
 * workspace  device buffer of >= nvfp4_gptq_hessian_workspace_size(s, k)
 *            bytes (X^T, bf16), 16-byte aligned; contents on entry do not
 *            matter.
 * s >= 0, 0 <= k <= 65536.  Products of bf16 values are exact in fp32 and
 * summed in fp32 in a fixed order (bit-reproducible); the diagonal mean is
 * summed in float64.  s == 0 gives H = 0; k == 0 does nothing.
 * The factor nvfp4_quantize_fos_gptq takes, the upper Cholesky factor U of
 * H^-1, is left to the caller: it is a standard dense factorization
 * (Cholesky of H, its inverse, Cholesky again; O(k^3) once per layer) that
 * any linear-algebra library provides and the method does not change.
 * Launches: a transpose, the product (tiles on and above the diagonal,
 * mirrored), the damping.
 */
NVFP4_API size_t nvfp4_gptq_hessian_workspace_size(int64_t s, int64_t k);
NVFP4_API int nvfp4_gptq_hessian(const void* x, int64_t s, int64_t k, float damp, float* h, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * nvfp4_dequant - W_hat from the packed format ([Notes07] section 02:
 * "dequant" of a block with its scale).
 *
 * out_dtype NVFP4_F32: w_out[r][c] = sign * fl32(fl32(val * sigma) * s_t)
 *   (val * sigma is exact, so this is the correctly rounded W_hat; it equals
 *   the w_hat the quantizer used in its error comparison).
 * out_dtype NVFP4_BF16: the fp32 value rounded to nearest-even bfloat16.
 * codes, scales as in the format above; tensor_scale device scalar;
 * w_out device [n, k] of out_dtype.  n >= 0, k >= 0, k % 16 == 0.
 */
NVFP4_API int nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                            void* w_out, int64_t n, int64_t k, int out_dtype, void* stream);

/*
 * nvfp4_w4a16_gemm - y[m, n] = x[m, k] . W_hat[n, k]^T with bf16
 * activations and NVFP4 weights ([Recap] section 1: W4A16 for small token
 * counts; decode reads every weight from HBM once per token, so this
 * kernel is bound by HBM bandwidth, [Notes08] section 01).
 *
 * Products val * sigma are exact in bf16; accumulation is fp32; s_t is
 * applied in fp32 once per output; one final rounding to out_dtype.
 * Summation order is implementation-defined but fixed for a given
 * (m, n, k, path) (results are bit-reproducible run to run).
 *
 * x          device bf16 [m, k] row-major.
 * codes, scales  the packed weights [n, k/2], [n, k/16].
 * tensor_scale   device scalar.
 * y          device [m, n] of out_dtype (NVFP4_BF16 or NVFP4_F32).
 * m, n, k    >= 0, k % 16 == 0.  m == 0 or n == 0: nothing is done;
 *            k == 0: y = 0.
 * workspace  device buffer of at least
 *            nvfp4_w4a16_gemm_workspace_size(m, n, k) bytes, 16-byte
 *            aligned (may be NULL when that size is 0).  Scratch: its
 *            contents on entry do not matter.  Calls that may run
 *            concurrently must use distinct workspaces.  The full-K
 *            kernels (see below) need none (size 0); it holds fp32
 *            partial sums [splits, m, n] whenever a path splits K.
 * Dispatch (the lower-latency kernel for the shape, [Recap] section 1, as
 * measured on MI355X; nvfp4_w4a16_gemm_path tells which):
 *   m <= 16 -> memory-bound skinny kernel, one launch, no workspace: for
 *     m == 1 with k a multiple of 32 from 2048 to 32768 a kernel in which
 *     each wave streams whole weight rows (lanes along K, the activations
 *     staged once per workgroup: 8 rows for k = 2048 or 4096, else 4 rows,
 *     or 8 for k < 4096 on more than 8192 rows, with the activations copied
 *     by LDS DMA); for
 *     4 < m <= 16 with k % 512 == 0 and k <= 4096 a persistent kernel (a
 *     workgroup per CU walks 16-row tiles with the activations in LDS
 *     once); otherwise a workgroup per 16 weight rows over the whole K
 *     (except 8 < m <= 16 on large matrices, n > 4096 or n * k > 2^25,
 *     with k % 512 == 0, and 4 < m <= 8 there with k > 4096: the streaming
 *     split-K kernel below; and 8 < m <= 16 with n > 4096, n * k > 2^25,
 *     k % 512 != 0 and k % 64 == 0: the tiled kernel);
 *   16 < m <= 64 -> with at most 256 tiles of 16 rows, k <= 4096 (and
 *     m <= 48 unless k <= 2048) and k a multiple of 128 that 4 to 8 waves
 *     of 4 or 8 steps of 128 cover: one launch, a workgroup per 16
 *     rows over the whole K, no workspace; otherwise the split-K skinny
 *     kernel plus a reduction kernel, when k % 512 == 0, k % 64 != 0, or
 *     n * k <= 2^25; else the tiled kernel.  Within it: for k % 512 == 0
 *     the streaming kernel (an x chunk of 1024, or 512, staged once per
 *     workgroup, then many 16-row weight tiles streamed through it);
 *     otherwise activations shared through LDS by 64 weight rows;
 *   m > 64 -> the tiled kernel;
 *   n >= 2^27 -> the tiled kernel at any m (the skinny kernels' grid would
 *     pass 2^32 work-items; forcing NVFP4_PATH_SKINNY there is an error).
 * The tiled kernel (bf16 MFMA): when k % 64 == 0, one 64-token tile x 256
 * (or, for k >= 8192, 128) weight rows for m <= 64, 128 x 128 tiles for
 * m <= 128, else 256 weight rows x 128 tokens with the weights dequantized
 * in registers (128 k per barrier when k % 128 == 0); K is split over
 * workgroups (fp32 partials in the workspace, one reduction kernel) when
 * there are few tiles.  Other k: 128 x 128 single-stage tiles.
 */
NVFP4_API size_t nvfp4_w4a16_gemm_workspace_size(int64_t m, int64_t n, int64_t k);
NVFP4_API int nvfp4_w4a16_gemm(const void* x, const uint8_t* codes, const uint8_t* scales,
                               const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                               int out_dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * nvfp4_w4a16_gemm_grouped - the W4A16 GEMMs of G weight matrices that read
 * the same activations (a decoder layer's q, k and v projections, or gate
 * and up: [Recap] section 1's W4A16 kernel, decode being bound by reading
 * every weight once per token, [Notes08] section 01), in one call.
 *
 * The G packed matrices are stacked row-wise: codes [n_total, k/2] and
 * scales [n_total, k/16] hold group 0's rows, then group 1's, ... (each
 * quantized on its own: nvfp4_quantize_fos can write straight into a row
 * block of the stacked buffers); tensor_scales is a device fp32 [G] array,
 * group g's s_t; group_rows a host int64 [G] array of row counts, each a
 * positive multiple of 16, n_total their sum (< 2^27).  y [m, n_total] of
 * out_dtype: columns of group g hold x . W_hat_g^T with s_t[g] (the fused
 * output of the stacked projections; group g's result is the column block
 * starting at the sum of the earlier groups' rows).  G in 1 .. 4.
 * Everything else as nvfp4_w4a16_gemm on (m, n_total, k), including the
 * dispatch and the workspace: nvfp4_w4a16_gemm_workspace_size(m, n_total,
 * k) bytes.  One launch (or two with a K split) instead of G.
 */
NVFP4_API int nvfp4_w4a16_gemm_grouped(const void* x, const uint8_t* codes, const uint8_t* scales,
                                       const float* tensor_scales, const int64_t* group_rows, int groups,
                                       void* y, int64_t m, int64_t k, int out_dtype, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Same, with an explicit path (NVFP4_PATH_*), a split-K factor
 * (0 = automatic; skinny path: >= 1 = the split-K kernel with that many K
 * chunks, clamped to [1, 64], more when a chunk would not fit in registers
 * and LDS; tiled path with k % 64 == 0: that many K splits of whole 64-wide
 * steps (128-wide when m > 128 and k % 128 == 0), at most k / 64, fewer when
 * the steps do not divide evenly; other k ignore it) and a dequantization implementation (NVFP4_IMPL_*).  The
 * skinny path requires m <= 64.  The workspace size for these choices is
 * nvfp4_w4a16_gemm_workspace_size_ex(m, n, k, path, split_k). */
NVFP4_API size_t nvfp4_w4a16_gemm_workspace_size_ex(int64_t m, int64_t n, int64_t k, int path,
                                                    int split_k);
NVFP4_API int nvfp4_w4a16_gemm_ex(const void* x, const uint8_t* codes, const uint8_t* scales,
                                  const float* tensor_scale, void* y, int64_t m, int64_t n,
                                  int64_t k, int out_dtype, void* workspace,
                                  size_t workspace_bytes, int path, int split_k, int impl,
                                  void* stream);

/*
 * nvfp4_w4a16_gemm_noalloc - nvfp4_w4a16_gemm without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results (the same kernels: bit-identical to
 * nvfp4_w4a16_gemm) and errors otherwise.
 *
 * When the plan splits K, its fp32 partial sums go to a fixed per-GPU
 * device array of nvfp4_noalloc_scratch_bytes() bytes (32 MiB) that the
 * library holds on each GPU it runs on until the process ends; its address
 * is looked up once per device on the first call made there.  A shape whose
 * plan needs more (nvfp4_w4a16_gemm_workspace_size(m, n, k) larger than
 * that) is rejected with NVFP4_ERR_WORKSPACE_TOO_SMALL before any launch.
 * The call allocates nothing.  All calls on one GPU share the array: calls
 * that overlap on one GPU (other streams, other threads) race; serialize
 * them.  The array's contents on entry do not matter.
 */
NVFP4_API int nvfp4_w4a16_gemm_noalloc(const void* x, const uint8_t* codes, const uint8_t* scales,
                                       const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                                       int out_dtype, void* stream);
NVFP4_API size_t nvfp4_noalloc_scratch_bytes(void);

/* The path NVFP4_PATH_AUTO picks for (m, n, k): NVFP4_PATH_SKINNY or
 * NVFP4_PATH_TILED. */
NVFP4_API int nvfp4_w4a16_gemm_path(int64_t m, int64_t n, int64_t k);

/*
 * nvfp4_w4a16_gemm_dx - input gradient of an NVFP4 linear layer,
 * dx = dy @ W_hat, for quantization-aware training ([Recap] section 3,
 * "Draft training": the forward GEMM runs on the FP4 weights and gradients
 * pass straight through to the master weights; the weight gradient dy^T x
 * has no FP4 operand and is the caller's plain GEMM).
 *
 * dx[i, j] = s_t * sum over r < n of dy[i, r] * (val * sigma)[r, j]:
 * fp32 accumulation in any order, rounded once to out_dtype.
 *
 * dy         device bf16 [m, n] row-major (the forward output's gradient).
 * codes, scales, tensor_scale: the packed [n, k] weights, as nvfp4_w4a16_gemm.
 * dx         device [m, k] of out_dtype (NVFP4_BF16 or NVFP4_F32).
 * workspace  device, >= nvfp4_w4a16_gemm_dx_workspace_size(m, n, k) bytes
 *            (0 when the reduction is not split: NULL allowed), 16-byte
 *            aligned; fp32 partial sums [splits, m, k] when few 128 x 128
 *            output tiles leave the GPU idle (the reduction over n is then
 *            split over workgroups and a second kernel adds the planes in
 *            order).  Scratch; contents on entry do not matter.
 * Any m, n; k % 16 == 0; pointers 16-byte aligned.  n == 0 writes zeros.
 * Same accuracy contract as nvfp4_w4a16_gemm; deterministic.
 */
NVFP4_API size_t nvfp4_w4a16_gemm_dx_workspace_size(int64_t m, int64_t n, int64_t k);
NVFP4_API int nvfp4_w4a16_gemm_dx(const void* dy, const uint8_t* codes, const uint8_t* scales,
                                  const float* tensor_scale, void* dx, int64_t m, int64_t n, int64_t k,
                                  int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_quantize_act - bf16 activations to NVFP4 for the W4A4 product
 * ([Recap] section 1: above about 48 tokens the pages' GEMM takes NVFP4
 * activations too).  The weights' format with the standard block scale (no
 * FourOverSix choice): s_t = fl32(amax / 2688) (1 if 0) from the activations'
 * own amax (or amax_in), sigma = E4M3_RNE(min(fl32(a / fl32(6 s_t)), 448))
 * per 16 elements along k, codes = E2M1_RNE(fl32(|x| R)) with
 * R = min(1 / fl32(sigma s_t), FLT_MAX) (0 for sigma = 0), sign bit from x.
 *
 * x              device bf16 [m, k] row-major, k % 16 == 0, 16-byte aligned.
 * codes, scales  device outputs [m, k/2] and [m, k/16] as the weights'.
 * x_blockscaled  optional device bf16 [m, k]: sign * val * sigma (exact in
 *                bf16; the tensor scale not applied).
 * amax_in, amax_out, tensor_scale: as nvfp4_quantize_fos.
 * Launches: a zero fill and a max reduction (without amax_in), then one
 * quantization kernel.  Bit-exact and deterministic.
 */
NVFP4_API int nvfp4_quantize_act(const void* x, int64_t m, int64_t k, const float* amax_in,
                                 float* amax_out, float* tensor_scale, uint8_t* codes,
                                 uint8_t* scales, void* x_blockscaled, void* stream);

/*
 * nvfp4_w4a4_gemm - y = xhat @ W_hat^T with xhat the NVFP4 quantization of
 * the activations (nvfp4_quantize_act) and W_hat the packed weights
 * ([Recap] section 1, the W4A4 path).
 *
 * gfx950's scaled FP4 matrix instructions take one power-of-two scale per
 * 32 elements, so they cannot multiply NVFP4's E4M3 scale per 16 exactly;
 * this entry point quantizes the activations, writes their block-scaled
 * values (exact in bf16) to the workspace, and runs the W4A16 GEMM on them
 * (path chosen as nvfp4_w4a16_gemm does) with the product of both tensor
 * scales applied once in the epilogue.  Same accuracy contract as
 * nvfp4_w4a16_gemm, against the W4A4 reference.
 *
 * Arguments as nvfp4_w4a16_gemm; workspace: device, 16-byte aligned like
 * every other buffer, at least nvfp4_w4a4_gemm_workspace_size(m, n, k) bytes
 * (activation scalars, block-scaled values, codes and scales, then the
 * GEMM's workspace, laid out from the buffer's first 256-byte boundary; the
 * size includes the bytes skipped to reach it); caller-owned scratch;
 * contents on entry do not matter.
 */
NVFP4_API size_t nvfp4_w4a4_gemm_workspace_size(int64_t m, int64_t n, int64_t k);
NVFP4_API int nvfp4_w4a4_gemm(const void* x, const uint8_t* codes, const uint8_t* scales,
                              const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                              int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_selftest_cvt - validation of the gfx950 FP4 and FP8 (E4M3)
 * conversion instructions against the library's portable ALU rounding and
 * decoding.
 * Runs on `stream` and writes 8 uint32 counters to the device buffer
 * `counters_out`:
 *  [0] fp32 -> FP4 code mismatches over every non-NaN fp32 bit pattern
 *      (both signs, including +-inf), through each of the four byte
 *      positions the packing conversion can write,
 *  [1] FP4 byte -> 2 x fp32 decode mismatches (256 bytes, read from each
 *      of the four byte positions of a word),
 *  [2] FP4 byte -> 2 x fp32 with scale sigma, against fl32(val * sigma),
 *      for every E4M3 sigma in [0, 448],
 *  [3] FP4 byte -> 2 x bf16 with scale sigma, against val * sigma,
 *  [4] number of fp32 values tested in [0],
 *  [5] FP4 byte -> 2 x bf16 decode at unit scale (256 bytes, from each of
 *      the four byte positions),
 *  [6] E4M3 scale byte -> fp32 decode (256 bytes, sign included, from each
 *      of the four byte positions; NaN for 0x7F and 0xFF), [7] reserved (0).
 * Used by the tests to decide whether NVFP4_IMPL_HWCVT is exact.
 */
NVFP4_API int nvfp4_selftest_cvt(uint32_t* counters_out, void* stream);

/*
 * nvfp4_stream_read - measurement helper: reads `bytes` of device memory
 * once and computes nothing of the method.  Decode reads every weight from
 * HBM once per token ([Notes08] section 01), so a W4A16 GEMM at small token
 * counts is bounded by this GPU's read bandwidth; this kernel measures that
 * ceiling at the size of a weight matrix, as the reference the GEMMs'
 * throughput is reported against (beside the published 8 TB/s).
 *
 * buf: device, 16-byte aligned, `bytes` a multiple of 16 (0: no work);
 * grid: workgroups of 256 threads (1 .. 65536); loads_in_flight: 16-byte
 * loads per thread in flight (2, 4, 8 or 16); nontemporal != 0: streaming
 * (non-temporal) loads; sink: device buffer of 64 uint32 that the kernel may
 * write (only if the data folds to one fixed value: it keeps the loads from
 * being removed).  Every load is in bounds.  Asynchronous on `stream`.
 * Errors: NVFP4_ERR_INVALID_VALUE (null buf or sink, bad grid or
 * loads_in_flight), NVFP4_ERR_UNSUPPORTED_SHAPE (bytes not a multiple of 16,
 * or >= 2^40), NVFP4_ERR_MISALIGNED, NVFP4_ERR_UNSUPPORTED_DEVICE,
 * NVFP4_ERR_HIP.
 */
NVFP4_API int nvfp4_stream_read(const void* buf, size_t bytes, int grid, int loads_in_flight, int nontemporal,
                                uint32_t* sink, void* stream);

NVFP4_API const char* nvfp4_status_string(int status);
NVFP4_API const char* nvfp4_last_error(void);
/* 10000 * major + 100 * minor + patch */
NVFP4_API int nvfp4_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H_ */
