// GPTQ weight optimisation inside the FourOverSix block scales, gfx950.
//
// "SOAR Weekly Champion Notes 07 ...", section "03 How we integrated it":
// every block's scale (and with it the M=6 / M=4 choice) is estimated and
// fixed first; GPTQ's iterations then run inside those scales.  GPTQ (the
// published method of Frantar et al., 2022) quantizes the columns one after
// another and pushes each column's rounding error, scaled by the inverse
// Hessian, onto the columns not yet quantized.  With U the upper Cholesky
// factor of the inverse Hessian (an input), column j's error is
// e_j = (w_j - what_j) / U[j, j] and column l > j becomes w_l - e_j U[j, l].
//
// The fp32 steps are fixed so that the result is exactly reproducible: each
// element receives its updates in increasing j, one product and one
// subtraction each (no contraction); the quantization of an element is the
// quantizer's C5-C7 with its block's fixed sigma.  Rows are independent, so
// the column loop runs for all rows in parallel, 64 columns per panel, one
// launch (k_gptq_step) per panel L with two kinds of workgroups:
//  * panel role: applies panel L-1's errors to panel L's columns, then
//    quantizes them in order, 16 lanes per weight row (4 columns each); each
//    column's scaled error reaches the row's other lanes by one DPP row
//    broadcast; the codes and, column-major, the 64 errors are written;
//  * trailing role: applies panel L-1's errors to the columns after panel
//    L, in 64 x 64 tiles, one lane per column, j = 0 .. 63 in order.
// So the serial panel runs beside the trailing update instead of between
// two of them.  Errors are double-buffered (panel L writes one buffer while
// the trailing role reads panel L-1's); the two roles touch disjoint
// columns.  Each element still receives its updates in increasing j.
// Until the first trailing update has written them, columns are read from W
// itself; from there on the updated copy lives in the workspace.
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kGB = 64;     // columns per panel
constexpr int kPR = 16;     // weight rows per panel workgroup (16 lanes each)
constexpr int kTW = 16;     // rows per wave in the trailing update
constexpr int kTRows = 64;  // rows per trailing-update workgroup (4 waves)

// Value of lane `src` (0..15) of each row of 16 lanes, to every lane of the
// row (DPP row broadcast; `src` must fold to a constant).
__device__ __forceinline__ float row_bcast(float v, int src) {
  const int x = __float_as_int(v);
  int r;
  switch (src) {
#define NVFP4_BCAST(i) \
  case i: r = __builtin_amdgcn_update_dpp(0, x, 0x150 + i, 0xF, 0xF, false); break;
    NVFP4_BCAST(0) NVFP4_BCAST(1) NVFP4_BCAST(2) NVFP4_BCAST(3) NVFP4_BCAST(4) NVFP4_BCAST(5)
    NVFP4_BCAST(6) NVFP4_BCAST(7) NVFP4_BCAST(8) NVFP4_BCAST(9) NVFP4_BCAST(10) NVFP4_BCAST(11)
    NVFP4_BCAST(12) NVFP4_BCAST(13) NVFP4_BCAST(14)
#undef NVFP4_BCAST
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x15F, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}

// E2M1 magnitude code of v >= 0 (round to nearest, ties to even, saturating)
// and its value, by the gfx950 conversions at unit scale (the quantizer's
// default implementation; the library's self-test checks both exhaustively).
__device__ __forceinline__ uint32_t e2m1_quant(float v, float* val) {
  const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 7u;
  *val = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)[0];
  return c;
}

// Panel role: panel L (columns b0 .. b0+63, b0 = 64 L), 16 lanes per weight
// row, each holding 4 of the row's panel columns in registers.  First the
// errors of panel L-1 are applied to them (the trailing update of the
// previous launch stopped short of this panel), then the columns are
// quantized in order: column j by the lane that owns it, its scaled error
// broadcast to the row's other lanes (one DPP row broadcast), each lane
// updating its own columns.
__device__ __forceinline__ void panel_role(float* smem, const float* src, const float* __restrict__ u,
                                           const uint8_t* __restrict__ scales,
                                           const float* __restrict__ tensor_scale,
                                           uint8_t* __restrict__ codes, const float* __restrict__ err_prev,
                                           float* __restrict__ err_cur, int n, int k, int L) {
  const int b0 = L * kGB;
  float* us = smem;                   // [64][64]: U[b0 + j][b0 + l], zero below the diagonal
  float* up = smem + kGB * kGB;       // [64][64]: U[b0 - 64 + j][b0 + l]
  float* ep = smem + 2 * kGB * kGB;   // [16][64]: errors of panel L-1 for this workgroup's rows
  const int row0 = blockIdx.x * kPR;
  for (int e = threadIdx.x; e < kGB * kGB; e += blockDim.x) {
    const int j = e / kGB, l = e - j * kGB;
    // products below the diagonal only reach columns already quantized
    us[e] = l >= j ? u[(int64_t)(b0 + j) * k + b0 + l] : 0.0f;
    if (L > 0) up[e] = u[(int64_t)(b0 - kGB + j) * k + b0 + l];
  }
  if (L > 0) {
    for (int e = threadIdx.x; e < kPR * kGB; e += blockDim.x) {
      const int j = e / kPR, r = e - j * kPR;
      ep[r * kGB + j] = row0 + r < n ? err_prev[(int64_t)j * n + row0 + r] : 0.0f;
    }
  }
  __syncthreads();
  const int p = threadIdx.x & 15;  // the lane's panel columns 4p .. 4p+3 (block p / 4)
  const int rl = threadIdx.x >> 4;
  const int row = row0 + rl;
  if (row >= n) return;  // whole rows of 16 lanes leave together
  const float s_t = tensor_scale[0];

  const float4 t4 = *reinterpret_cast<const float4*>(src + (int64_t)row * k + b0 + 4 * p);
  float w[4] = {t4.x, t4.y, t4.z, t4.w};
  if (L > 0) {
    // panel L-1's 64 errors, in column order
#pragma unroll
    for (int j = 0; j < kGB; j += 4) {
      const float4 e4 = *reinterpret_cast<const float4*>(&ep[rl * kGB + j]);
      const float ev4[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float4 ur = *reinterpret_cast<const float4*>(&up[(j + d) * kGB + 4 * p]);
        w[0] = w[0] - ev4[d] * ur.x;
        w[1] = w[1] - ev4[d] * ur.y;
        w[2] = w[2] - ev4[d] * ur.z;
        w[3] = w[3] - ev4[d] * ur.w;
      }
    }
  }
  // the block's fixed sigma and the quantizer's C5 reciprocal
  // R = min(1 / fl32(sigma * s_t), FLT_MAX), 0 for sigma = 0
  const float sg = e4m3_decode(scales[(int64_t)row * (k / 16) + b0 / 16 + p / 4] & 0x7Fu);
  const float rcp = fminf(1.0f / (sg * s_t), kFltMax);
  const float R = sg == 0.0f ? 0.0f : rcp;

  // The loop is one straight-line block (selects, no branches), so the
  // scheduler can issue the reads of later columns early: the chain
  // quantize -> divide -> broadcast -> update of the next column is the
  // critical path.
  uint32_t cw = 0u;  // the lane's 4 codes
  float ev[4];       // the lane's 4 scaled errors
  // U's diagonal (uniform: scalar registers) and the lane's 4 values of the
  // next kPf rows of U, read ahead of their use
  float ud[kGB];
#pragma unroll
  for (int j = 0; j < kGB; ++j) ud[j] = u[(int64_t)(b0 + j) * k + b0 + j];
  constexpr int kPf = 4;
  float4 ub[kPf];
#pragma unroll
  for (int j = 0; j < kPf; ++j) ub[j] = *reinterpret_cast<const float4*>(&us[j * kGB + 4 * p]);
#pragma unroll
  for (int j = 0; j < kGB; ++j) {
    const int po = j / 4, t = j % 4;
    // every lane quantizes its own column t; the owner's (p == po) is column j
    float val;
    const uint32_t mag = e2m1_quant(fabsf(w[t]) * R, &val);
    const float wabs = (val * sg) * s_t;
    const bool neg = __builtin_signbit(w[t]);
    const float what = neg ? -wabs : wabs;
    const float e_own = (w[t] - what) / ud[j];
    const bool own = p == po;
    cw |= own ? (mag | (neg ? 8u : 0u)) << (4 * t) : 0u;
    ev[t] = own ? e_own : ev[t];
    const float e = row_bcast(e_own, po);
    const float4 ur = ub[j % kPf];
    if (j + kPf < kGB) ub[j % kPf] = *reinterpret_cast<const float4*>(&us[(j + kPf) * kGB + 4 * p]);
    w[0] = w[0] - e * ur.x;
    w[1] = w[1] - e * ur.y;
    w[2] = w[2] - e * ur.z;
    w[3] = w[3] - e * ur.w;
  }
  *reinterpret_cast<uint16_t*>(codes + (int64_t)row * (k / 2) + b0 / 2 + 2 * p) = (uint16_t)cw;
#pragma unroll
  for (int t = 0; t < 4; ++t) (err_cur + (int64_t)(4 * p + t) * n)[(uint32_t)row] = ev[t];  // column-major
}

// Trailing role: applies the 64 errors of panel L-1 (U rows b0 .. b0+63,
// b0 = 64 (L-1)) to one 64-column x 64-row tile of the columns after panel
// L, j = 0 .. 63 in order per element: one lane per column holding its 64
// values of U, each wave 16 rows, two at a time, the errors broadcast from
// LDS.
__device__ __forceinline__ void trail_role(float* smem, const float* src, float* dst,
                                           const float* __restrict__ u, const float* __restrict__ err_prev,
                                           int n, int k, int L, int tile, int col_blocks) {
  const int b0 = (L - 1) * kGB;
  float(*es)[kGB + 4] = reinterpret_cast<float(*)[kGB + 4]>(smem);  // +4: 4-way, not 64-way, conflicts on the fill
  const int bx = tile % col_blocks;
  const int r0 = (tile / col_blocks) * kTRows;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // col < k: the columns after panel L are a multiple of 64, col_blocks of them
  const int col = b0 + 2 * kGB + bx * 64 + lane;
  const int i0 = wv * kTW;
  const int rows = min(kTW, n - r0 - i0);  // <= 0 past the last row
  const int64_t off = (int64_t)(r0 + i0) * k + col;
  const float* sp = src + off;
  float* dp = dst + off;
  // U's column, the first two rows and the errors are all in flight at once
  float uc[kGB];
#pragma unroll
  for (int j = 0; j < kGB; ++j) uc[j] = u[(int64_t)(b0 + j) * k + col];
  float x0 = rows > 0 ? sp[0] : 0.0f;
  float x1 = rows > 1 ? sp[k] : 0.0f;
  for (int e = threadIdx.x; e < kTRows * kGB; e += blockDim.x) {
    const int j = e / kTRows, i = e - j * kTRows;
    es[i][j] = (r0 + i < n) ? err_prev[(int64_t)j * n + r0 + i] : 0.0f;
  }
  __syncthreads();
  for (int i = 0; i < rows; i += 2) {
    // next pair in flight while this one is updated
    const float n0 = i + 2 < rows ? sp[(int64_t)(i + 2) * k] : 0.0f;
    const float n1 = i + 3 < rows ? sp[(int64_t)(i + 3) * k] : 0.0f;
    const float* e0 = es[i0 + i];
    const float* e1 = es[i0 + i + 1];  // row i0 + 15 at most: rows is even when it reaches 16
#pragma unroll
    for (int j = 0; j < kGB; j += 4) {
      const float4 a = *reinterpret_cast<const float4*>(e0 + j);
      const float4 b = *reinterpret_cast<const float4*>(e1 + j);
      x0 = x0 - a.x * uc[j];
      x1 = x1 - b.x * uc[j];
      x0 = x0 - a.y * uc[j + 1];
      x1 = x1 - b.y * uc[j + 1];
      x0 = x0 - a.z * uc[j + 2];
      x1 = x1 - b.z * uc[j + 2];
      x0 = x0 - a.w * uc[j + 3];
      x1 = x1 - b.w * uc[j + 3];
    }
    dp[(int64_t)i * k] = x0;
    if (i + 1 < rows) dp[(int64_t)(i + 1) * k] = x1;
    x0 = n0;
    x1 = n1;
  }
}

// Launch L: workgroups [0, panel_blocks) quantize panel L, the rest update
// the columns after it with panel L-1's errors.  The two roles touch
// disjoint columns of the working matrix and different error buffers.
__global__ __launch_bounds__(256, 4) void k_gptq_step(const float* panel_src, const float* trail_src,
                                                   float* wc, const float* __restrict__ u,
                                                   const uint8_t* __restrict__ scales,
                                                   const float* __restrict__ tensor_scale,
                                                   uint8_t* __restrict__ codes,
                                                   const float* __restrict__ err_prev,
                                                   float* __restrict__ err_cur, int n, int k, int L,
                                                   int panel_blocks, int col_blocks) {
  __shared__ __attribute__((aligned(16))) float smem[2 * kGB * kGB + kPR * kGB];
  if ((int)blockIdx.x < panel_blocks)
    panel_role(smem, panel_src, u, scales, tensor_scale, codes, err_prev, err_cur, n, k, L);
  else
    trail_role(smem, trail_src, wc, u, err_prev, n, k, L, (int)blockIdx.x - panel_blocks, col_blocks);
}

}  // namespace

size_t gptq_workspace_bytes(int64_t n, int64_t k) {
  return (size_t)n * (size_t)k * sizeof(float) + 2 * (size_t)n * kGB * sizeof(float);
}

hipError_t launch_gptq(const float* w, int64_t n, int64_t k, const float* hinv_u,
                       const float* amax_in, float* amax_out, float* tensor_scale,
                       uint8_t* codes, uint8_t* scales, uint8_t* m4_mask, void* workspace,
                       int impl, hipStream_t stream) {
  // 1. FourOverSix: tensor scale, block scales, mask (and round-to-nearest
  //    codes, replaced below)
  hipError_t e = launch_quantize_fos(w, n, k, amax_in, amax_out, tensor_scale, codes, scales,
                                     m4_mask, impl, stream);
  if (e != hipSuccess || n == 0 || k == 0) return e;
  float* wc = reinterpret_cast<float*>(workspace);  // updated W (columns >= 128)
  float* er[2] = {wc + n * k, wc + n * k + n * kGB};  // errors of even / odd panels, [64][n]
  // 2. one launch per panel L: quantize panel L while the columns after it
  //    get panel L-1's errors
  const int N = (int)n, K = (int)k;
  const int panels = K / kGB;
  const int panel_blocks = (int)(((int64_t)N + kPR - 1) / kPR);
  const int64_t row_tiles = ((int64_t)N + kTRows - 1) / kTRows;
  for (int L = 0; L < panels; ++L) {
    // panel L's columns: only W's own values before launch 2 (the first
    // trailing update, in launch 1, starts after panel 1)
    const float* panel_src = L >= 2 ? wc : w;
    const float* trail_src = L >= 2 ? wc : w;
    const int col_blocks = L >= 1 ? panels - L - 1 : 0;
    const int64_t blocks = panel_blocks + (int64_t)col_blocks * row_tiles;
    hipLaunchKernelGGL(k_gptq_step, dim3((unsigned)blocks), dim3(256), 0, stream, panel_src, trail_src, wc,
                       hinv_u, scales, tensor_scale, codes, er[(L + 1) & 1], er[L & 1], N, K, L,
                       panel_blocks, col_blocks);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
