// NVFP4 dequantization for gfx950: W_hat = sign * fl32(fl32(val * sigma) * s_t)
// as fp32, or that value rounded to nearest-even bf16.  This is the
// "dequant(W_block, scale)" of "SOAR Weekly Champion Notes 07 ...", section
// "02 FourOverSix", with the tensor scale applied.  One lane per 16-element
// block.
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

__device__ __forceinline__ float scale_value(uint32_t s) {
  const float v = e4m3_decode(s & 0x7Fu);
  return (s & 0x80u) ? -v : v;
}

template <bool F32>
__global__ __launch_bounds__(256) void k_dequant(const uint2* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ tensor_scale,
                                                 void* __restrict__ out, int64_t nblocks) {
  const float s_t = tensor_scale[0];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
    const uint2 c = codes[b];
    const float sigma = scale_value(scales[b]);
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t code = ((i < 8 ? c.x : c.y) >> (4 * (i & 7))) & 0xFu;
      v[i] = (e2m1_val_portable(code) * sigma) * s_t;
    }
    if constexpr (F32) {
      float4* o = reinterpret_cast<float4*>(out) + 4 * b;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
      uint4* o = reinterpret_cast<uint4*>(out) + 2 * b;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint4 u;
        u.x = bf16_rne_bits(v[8 * q + 0]) | (bf16_rne_bits(v[8 * q + 1]) << 16);
        u.y = bf16_rne_bits(v[8 * q + 2]) | (bf16_rne_bits(v[8 * q + 3]) << 16);
        u.z = bf16_rne_bits(v[8 * q + 4]) | (bf16_rne_bits(v[8 * q + 5]) << 16);
        u.w = bf16_rne_bits(v[8 * q + 6]) | (bf16_rne_bits(v[8 * q + 7]) << 16);
        o[q] = u;
      }
    }
  }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                          void* out, int64_t n, int64_t k, int out_f32, hipStream_t stream) {
  const int64_t nblocks = n * k / 16;
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  if (grid > (1 << 20)) grid = 1 << 20;
  if (out_f32)
    hipLaunchKernelGGL(k_dequant<true>, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint2*>(codes), scales, tensor_scale, out, nblocks);
  else
    hipLaunchKernelGGL(k_dequant<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint2*>(codes), scales, tensor_scale, out, nblocks);
  return hipGetLastError();
}

}  // namespace nvfp4
