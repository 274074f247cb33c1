// NVFP4 dequantization for gfx950: W_hat = sign * fl32(fl32(val * sigma) * s_t)
// as fp32, or that value rounded to nearest-even bf16.  This is the
// "dequant(W_block, scale)" of "SOAR Weekly Champion Notes 07 ...", section
// "02 FourOverSix", with the tensor scale applied.
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

// One thread per 16 output bytes: 8 elements (bf16 output, half a block) or
// 4 elements (fp32 output, a quarter block), so the stores of a wave cover
// 1 KiB contiguously.  FP4 codes are decoded by the gfx950 conversion with
// a unit scale (exact: every code's value, checked over all 256 bytes by
// nvfp4_selftest_cvt); val * sigma is exact, then one rounding by s_t.
// The output is written with streaming stores (written once, not re-read).
template <bool F32>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ tensor_scale,
                                                 void* __restrict__ out, int64_t nthreads) {
  constexpr int E = F32 ? 4 : 8;  // elements per thread
  const float s_t = tensor_scale[0];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nthreads; t += stride) {
    const float sigma = scale_at<kConvHw, 0>(scales[t * E / 16]);
    float v[E];
    if constexpr (F32) {
      const uint32_t c = reinterpret_cast<const uint16_t*>(codes)[t];
      const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
      const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
      v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
    } else {
      const uint32_t c = reinterpret_cast<const uint32_t*>(codes)[t];
      const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
      const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
      const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
      const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
      v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
      v[4] = d[0]; v[5] = d[1]; v[6] = e[0]; v[7] = e[1];
    }
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (v[i] * sigma) * s_t;
    if constexpr (F32) {
      store_u4_stream(reinterpret_cast<float4*>(out) + t, __float_as_uint(v[0]), __float_as_uint(v[1]),
                      __float_as_uint(v[2]), __float_as_uint(v[3]));
    } else {
      uint4 u;
      u.x = bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16);
      u.y = bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16);
      u.z = bf16_rne_bits(v[4]) | (bf16_rne_bits(v[5]) << 16);
      u.w = bf16_rne_bits(v[6]) | (bf16_rne_bits(v[7]) << 16);
      store_u4_stream(reinterpret_cast<uint4*>(out) + t, u.x, u.y, u.z, u.w);
    }
  }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                          void* out, int64_t n, int64_t k, int out_f32, hipStream_t stream) {
  const int64_t count = n * k;
  if (count == 0) return hipSuccess;
  const int64_t nthreads = count / (out_f32 ? 4 : 8);
  int64_t grid = (nthreads + 255) / 256;
  if (grid > 8192) grid = 8192;  // 32 workgroups per CU, grid-stride beyond
  if (out_f32)
    hipLaunchKernelGGL(k_dequant<true>, dim3((unsigned)grid), dim3(256), 0, stream, codes, scales,
                       tensor_scale, out, nthreads);
  else
    hipLaunchKernelGGL(k_dequant<false>, dim3((unsigned)grid), dim3(256), 0, stream, codes, scales,
                       tensor_scale, out, nthreads);
  return hipGetLastError();
}

}  // namespace nvfp4
