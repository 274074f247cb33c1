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
// the column loop runs for all rows in parallel, 64 columns per panel:
//  * k_gptq_panel: four lanes per weight row, each holding one 16-column
//    block of the panel (its fixed sigma is that lane's) in registers and
//    the panel's 64 x 64 block of U in LDS.  Column j is quantized by the
//    lane that owns it; its scaled error is broadcast to the row's other
//    three lanes (a quad DPP move), which update their own columns.  The
//    lane writes its 16 codes and, column-major, the row's 64 errors;
//  * k_gptq_trail: applies the panel's 64 errors to every later column,
//    j = 0 .. 63 in order per element: a workgroup covers 64 columns x 64
//    rows, one lane per column holding its 64 values of U in registers, each
//    wave 16 rows, two at a time, the errors broadcast from LDS.
// The first panel and the first trailing update read W itself; from there
// on the updated copy lives in the workspace.
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kGB = 64;     // columns per panel
constexpr int kTW = 16;     // rows per wave in the trailing update
constexpr int kTRows = 64;  // rows per trailing-update workgroup (4 waves)

// Value of lane `src` (0..3) of each quad, to every lane of the quad.
__device__ __forceinline__ float quad_bcast(float v, int src) {
  const int x = __float_as_int(v);
  int r;
  switch (src) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0x00, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x55, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, x, 0xFF, 0xF, 0xF, false); break;
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

__global__ __launch_bounds__(256) void k_gptq_panel(const float* __restrict__ src,
                                                    const float* __restrict__ u,
                                                    const uint8_t* __restrict__ scales,
                                                    const float* __restrict__ tensor_scale,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ err, int n, int k,
                                                    int b0) {
  // U[b0 + j][b0 + l] for l >= j; zero below the diagonal (those products
  // only reach columns that are already quantized)
  __shared__ float us[kGB][kGB];
  for (int e = threadIdx.x; e < kGB * kGB; e += blockDim.x) {
    const int j = e / kGB, l = e - j * kGB;
    us[j][l] = l >= j ? u[(int64_t)(b0 + j) * k + b0 + l] : 0.0f;
  }
  __syncthreads();
  const int q = threadIdx.x & 3;  // the lane's block: panel columns 16q .. 16q+15
  const int row = blockIdx.x * 64 + (threadIdx.x >> 2);
  if (row >= n) return;  // whole quads leave together
  const float s_t = tensor_scale[0];

  float w[16];
  const float4* wr = reinterpret_cast<const float4*>(src + (int64_t)row * k + b0 + 16 * q);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float4 t = wr[m];
    w[4 * m] = t.x;
    w[4 * m + 1] = t.y;
    w[4 * m + 2] = t.z;
    w[4 * m + 3] = t.w;
  }
  // the block's fixed sigma and the quantizer's C5 reciprocal
  // R = min(1 / fl32(sigma * s_t), FLT_MAX), 0 for sigma = 0
  const float sg = e4m3_decode(scales[(int64_t)row * (k / 16) + b0 / 16 + q] & 0x7Fu);
  const float rcp = fminf(1.0f / (sg * s_t), kFltMax);
  const float R = sg == 0.0f ? 0.0f : rcp;

  uint32_t cw0 = 0u, cw1 = 0u;
#pragma unroll
  for (int j = 0; j < kGB; ++j) {
    const int qo = j / 16, t = j % 16;
    // every lane quantizes its own column t; the owner's (q == qo) is column j
    float val;
    const uint32_t mag = e2m1_quant(fabsf(w[t]) * R, &val);
    const float wabs = (val * sg) * s_t;
    const bool neg = __builtin_signbit(w[t]);
    const float what = neg ? -wabs : wabs;
    const float e_own = (w[t] - what) / us[j][j];
    if (q == qo) {
      const uint32_t c = (mag | (neg ? 8u : 0u)) << (4 * (t % 8));
      if (t < 8) cw0 |= c; else cw1 |= c;
      (err + (int64_t)j * n)[(uint32_t)row] = e_own;  // column-major: coalesced over rows
    }
    const float e = quad_bcast(e_own, qo);
#pragma unroll
    for (int l = 0; l < 16; ++l) w[l] = w[l] - e * us[j][16 * q + l];
  }
  *reinterpret_cast<uint2*>(codes + (int64_t)row * (k / 2) + b0 / 2 + 8 * q) = make_uint2(cw0, cw1);
}

__global__ __launch_bounds__(256) void k_gptq_trail(const float* __restrict__ src,
                                                    float* __restrict__ dst,
                                                    const float* __restrict__ u,
                                                    const float* __restrict__ err, int n, int k,
                                                    int b0, int col_blocks) {
  __shared__ float es[kTRows][kGB + 4];  // +4: 4-way instead of 64-way bank conflicts on the fill
  const int bx = (int)(blockIdx.x % (unsigned)col_blocks);
  const int r0 = (int)(blockIdx.x / (unsigned)col_blocks) * kTRows;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // col < k: the columns after a panel are a multiple of 64, col_blocks of them
  const int col = b0 + kGB + bx * 64 + lane;
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
    es[i][j] = (r0 + i < n) ? err[(int64_t)j * n + r0 + i] : 0.0f;
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

}  // namespace

size_t gptq_workspace_bytes(int64_t n, int64_t k) {
  return (size_t)n * (size_t)k * sizeof(float) + (size_t)n * kGB * sizeof(float);
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
  float* wc = reinterpret_cast<float*>(workspace);  // updated W (columns >= 64)
  float* er = wc + n * k;                           // one panel's errors, [64][n]
  // 2. panels of 64 columns, each followed by the update of the later columns
  const int N = (int)n, K = (int)k;
  const unsigned row_blocks = (unsigned)(((int64_t)N + 63) / 64);
  for (int b0 = 0; b0 < K; b0 += kGB) {
    const float* src = b0 == 0 ? w : wc;
    hipLaunchKernelGGL(k_gptq_panel, dim3(row_blocks), dim3(256), 0, stream, src, hinv_u, scales, tensor_scale,
                       codes, er, N, K, b0);
    const int rest = K - b0 - kGB;  // a multiple of 64
    if (rest > 0) {
      const int col_blocks = rest / 64;
      const int64_t blocks = (int64_t)col_blocks * (((int64_t)N + kTRows - 1) / kTRows);
      hipLaunchKernelGGL(k_gptq_trail, dim3((unsigned)blocks), dim3(256), 0, stream, src, wc, hinv_u, er, N, K,
                         b0, col_blocks);
    }
  }
  return hipGetLastError();
}

}  // namespace nvfp4
