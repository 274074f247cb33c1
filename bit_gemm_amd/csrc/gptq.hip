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
// the column loop runs for all rows in parallel:
//  * k_gptq_panel: 64 columns at a time, one thread per weight row holding
//    the row's 64 values in registers and the 64 x 64 block of U in LDS;
//    quantizes the columns in order, updates the rest of the panel after
//    each, writes the codes and the 64 scaled errors (column-major);
//  * k_gptq_trail: applies the panel's 64 errors to every later column,
//    j = 0 .. 63 in order per element: one thread per column holding its 64
//    values of U, the errors of 64 rows broadcast from LDS.
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kGB = 64;   // columns per panel
constexpr int kTR = 64;   // rows per trailing-update workgroup

__global__ __launch_bounds__(256) void k_gptq_copy(const float4* __restrict__ src,
                                                   float4* __restrict__ dst, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_gptq_panel(const float* __restrict__ wc,
                                                    const float* __restrict__ u,
                                                    const uint8_t* __restrict__ scales,
                                                    const float* __restrict__ tensor_scale,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ err, int n, int k,
                                                    int b0) {
  __shared__ float us[kGB][kGB + 1];  // U[b0 + j][b0 + l]
  for (int e = threadIdx.x; e < kGB * kGB; e += blockDim.x) {
    const int j = e / kGB, l = e - j * kGB;
    us[j][l] = u[(int64_t)(b0 + j) * k + b0 + l];
  }
  __syncthreads();
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n) return;
  const float s_t = tensor_scale[0];

  float w[kGB];
  const float4* wr = reinterpret_cast<const float4*>(wc + (int64_t)row * k + b0);
#pragma unroll
  for (int q = 0; q < kGB / 4; ++q) {
    const float4 t = wr[q];
    w[4 * q] = t.x;
    w[4 * q + 1] = t.y;
    w[4 * q + 2] = t.z;
    w[4 * q + 3] = t.w;
  }
  // the fixed sigma of the 4 blocks and their reciprocals (the quantizer's
  // C5: R = min(1 / fl32(sigma * s_t), FLT_MAX), 0 for sigma = 0)
  const uint32_t sw = *reinterpret_cast<const uint32_t*>(scales + (int64_t)row * (k / 16) + b0 / 16);
  float sg[4], rr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    sg[q] = e4m3_decode((sw >> (8 * q)) & 0x7Fu);  // the quantizer writes non-negative scales
    const float r = fminf(1.0f / (sg[q] * s_t), kFltMax);
    rr[q] = sg[q] == 0.0f ? 0.0f : r;
  }

  uint32_t cw[kGB / 8];
#pragma unroll
  for (int d = 0; d < kGB / 8; ++d) cw[d] = 0u;
#pragma unroll
  for (int j = 0; j < kGB; ++j) {
    const int q = j / 16;
    const uint32_t mag = e2m1_rne_portable(fabsf(w[j]) * rr[q]);
    // magnitude of the code, both forms computed and selected (no branch)
    const float lo = 0.5f * (float)mag, hi = __uint_as_float((mag + 252u) << 22);
    const float wabs = ((mag < 2u ? lo : hi) * sg[q]) * s_t;
    const bool neg = __builtin_signbit(w[j]);
    const float what = neg ? -wabs : wabs;
    const float e = (w[j] - what) / us[j][j];
    cw[j / 8] |= (mag | (neg ? 8u : 0u)) << (4 * (j % 8));
    // column-major: coalesced over the rows (uniform base, 32-bit offset)
    (err + (int64_t)j * n)[(uint32_t)row] = e;
#pragma unroll
    for (int l = j + 1; l < kGB; ++l) w[l] = w[l] - e * us[j][l];
    // keep the compiler from hoisting later columns' LDS reads (register
    // pressure): one column's 63 values of U at a time
    asm volatile("" ::: "memory");
  }
  uint4* cdst = reinterpret_cast<uint4*>(codes + (int64_t)row * (k / 2) + b0 / 2);
  cdst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
  cdst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
}

__global__ __launch_bounds__(256) void k_gptq_trail(float* __restrict__ wc,
                                                    const float* __restrict__ u,
                                                    const float* __restrict__ err, int n, int k,
                                                    int b0, int col_blocks) {
  __shared__ float es[kTR][kGB];
  // one flat grid: col_blocks blocks of 256 columns per 64 rows
  const int bx = (int)(blockIdx.x % (unsigned)col_blocks);
  const int r0 = (int)(blockIdx.x / (unsigned)col_blocks) * kTR;
  for (int e = threadIdx.x; e < kTR * kGB; e += blockDim.x) {
    const int j = e / kTR, i = e - j * kTR;
    es[i][j] = (r0 + i < n) ? err[(int64_t)j * n + r0 + i] : 0.0f;
  }
  __syncthreads();
  const int col = b0 + kGB + bx * (int)blockDim.x + (int)threadIdx.x;
  if (col >= k) return;
  float uc[kGB];
#pragma unroll
  for (int j = 0; j < kGB; ++j) uc[j] = u[(int64_t)(b0 + j) * k + col];
  const int rows = min(kTR, n - r0);
  for (int i = 0; i < rows; ++i) {
    float* p = wc + (int64_t)(r0 + i) * k + col;
    float x = *p;
#pragma unroll
    for (int j = 0; j < kGB; ++j) x = x - es[i][j] * uc[j];
    *p = x;
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
  float* wc = reinterpret_cast<float*>(workspace);
  float* er = wc + n * k;
  // 2. working copy of W
  {
    const int64_t n4 = n * k / 4;
    int64_t grid = (n4 + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_gptq_copy, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(w), reinterpret_cast<float4*>(wc), n4);
  }
  // 3. panels of 64 columns, each followed by the update of the later columns
  const int N = (int)n, K = (int)k;
  for (int b0 = 0; b0 < K; b0 += kGB) {
    hipLaunchKernelGGL(k_gptq_panel, dim3((unsigned)(((int64_t)N + 255) / 256)), dim3(256), 0, stream, wc,
                       hinv_u, scales, tensor_scale, codes, er, N, K, b0);
    const int rest = K - b0 - kGB;
    if (rest > 0) {
      const int col_blocks = (rest + 255) / 256;
      const int64_t blocks = (int64_t)col_blocks * (((int64_t)N + kTR - 1) / kTR);
      hipLaunchKernelGGL(k_gptq_trail, dim3((unsigned)blocks), dim3(256), 0, stream, wc, hinv_u, er, N, K,
                         b0, col_blocks);
    }
  }
  return hipGetLastError();
}

}  // namespace nvfp4
