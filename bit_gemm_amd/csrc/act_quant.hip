// Activation quantization to NVFP4 for the W4A4 product, gfx950.
//
// "SOAR 2026 Recap: From Compute Limits to the Open-Source Ecosystem",
// section "1. Quantization and GEMM dispatch": above about 48 tokens the GEMM
// switches to a W4A4 path whose activations are NVFP4 too.  The activations
// (bf16) get the weights' format with the standard block scale: tensor scale
// s_t = amax / 2688 from their own amax, block scale sigma = E4M3 of the
// block amax over 6 s_t, E2M1 codes of |x| R with R = 1 / fl32(sigma s_t)
// (the quantizer's C1, C2, C5, C6, C9 with the M=6 candidate only).
//
// gfx950's scaled FP4 matrix instructions take one power-of-two scale per 32
// elements, not an E4M3 scale per 16, so they cannot multiply this format
// exactly.  Instead the kernel also writes the block-scaled activations
// val * sigma (at most 6 significant bits: exact in bf16), which the bf16
// MFMA GEMM multiplies exactly; the tensor scales of both operands are
// applied once, in the GEMM's epilogue.
//
//  k_act_fill_zero  amax = 0 (a kernel, not a memset: capture-safe)
//  k_act_amax       grid-stride max |x| over bf16 -> atomicMax on the fp32
//                   bit pattern (non-negative floats order like their bits)
//  k_act_quant      one lane per 16-element block: scale, codes, block-scaled
//                   bf16 values; workgroup 0 writes s_t (and s_t * the
//                   weights' tensor scale for the GEMM)
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

__global__ void k_act_fill_zero(float* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0.0f;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float absmax8(const uint4& v) {
  const float a = fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))), fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  const float b = fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))), fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return fmaxf(a, b);
}

__global__ __launch_bounds__(256) void k_act_amax(const uint4* __restrict__ x, int64_t n8,
                                                  float* __restrict__ amax) {
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int U = 4;  // four independent 16-byte loads in flight
  for (; i + (U - 1) * stride < n8; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, absmax8(v[u]));
  }
  for (; i < n8; i += stride) m = fmaxf(m, absmax8(x[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
  }
}

// Block-scaled values of the 8 codes in `word` (element i at bits 4i), as
// 4 words of bf16 pairs: val * sigma is exact in fp32 and has at most 6
// significant bits, so dropping the low 16 bits is exact.
template <int J>
__device__ __forceinline__ uint32_t scaled_pair(uint32_t word, float sigma) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, J);
  return (__float_as_uint(v[0] * sigma) >> 16) | (__float_as_uint(v[1] * sigma) & 0xFFFF0000u);
}

__global__ __launch_bounds__(256) void k_act_quant(const uint4* __restrict__ x, int64_t nblocks,
                                                   const float* amax_src, float* amax_out,
                                                   float* __restrict__ tensor_scale,
                                                   const float* __restrict__ w_scale,
                                                   float* __restrict__ comb_scale,
                                                   uint2* __restrict__ codes,
                                                   uint8_t* __restrict__ scales,
                                                   uint4* __restrict__ xs) {
  const float amax = amax_src[0];
  float s_t = amax / 2688.0f;  // 2688 = 6 (FP4 max) * 448 (E4M3 max)
  s_t = (s_t == 0.0f) ? 1.0f : s_t;
  const float d6 = 6.0f * s_t;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    tensor_scale[0] = s_t;
    if (amax_out != amax_src) amax_out[0] = amax;
    if (comb_scale) comb_scale[0] = s_t * w_scale[0];
  }
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
    const uint4 p0 = x[2 * b], p1 = x[2 * b + 1];
    const uint32_t wd[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(wd[i]);
      v[2 * i + 1] = bf16_hi(wd[i]);
    }
    const float a = fmaxf(absmax8(p0), absmax8(p1));
    uint32_t c6;
    const float sg = e4m3_rne(fminf(a / d6, 448.0f), &c6);
    const float rcp = fminf(1.0f / (sg * s_t), kFltMax);
    const float R = sg == 0.0f ? 0.0f : rcp;
    // signed inputs: the conversion keeps the sign, also of values that
    // round to zero
    const uint32_t lo = e2m1_pack8_hw(v[0] * R, v[1] * R, v[2] * R, v[3] * R, v[4] * R, v[5] * R,
                                      v[6] * R, v[7] * R);
    const uint32_t hi = e2m1_pack8_hw(v[8] * R, v[9] * R, v[10] * R, v[11] * R, v[12] * R,
                                      v[13] * R, v[14] * R, v[15] * R);
    codes[b] = make_uint2(lo, hi);
    scales[b] = (uint8_t)c6;
    if (xs) {
      xs[2 * b] = make_uint4(scaled_pair<0>(lo, sg), scaled_pair<1>(lo, sg), scaled_pair<2>(lo, sg),
                             scaled_pair<3>(lo, sg));
      xs[2 * b + 1] = make_uint4(scaled_pair<0>(hi, sg), scaled_pair<1>(hi, sg),
                                 scaled_pair<2>(hi, sg), scaled_pair<3>(hi, sg));
    }
  }
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* x, int64_t m, int64_t k, const float* amax_in,
                               float* amax_out, float* tensor_scale, uint8_t* codes,
                               uint8_t* scales, uint16_t* xs, const float* w_scale,
                               float* comb_scale, hipStream_t stream) {
  const int64_t count = m * k;
  const float* amax_src = amax_in;
  if (amax_src == nullptr) {
    hipLaunchKernelGGL(k_act_fill_zero, dim3(1), dim3(64), 0, stream, amax_out);
    if (count > 0) {
      int64_t blocks = (count / 8 + 255) / 256;
      if (blocks > 256) blocks = 256;  // one device-scope atomic per workgroup
      hipLaunchKernelGGL(k_act_amax, dim3((unsigned)blocks), dim3(256), 0, stream,
                         reinterpret_cast<const uint4*>(x), count / 8, amax_out);
    }
    amax_src = amax_out;
  }
  const int64_t nblocks = count / 16;
  int64_t grid = (nblocks + 255) / 256;
  if (grid < 1) grid = 1;  // also writes the scalars for empty input
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_act_quant, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(x), nblocks, amax_src, amax_out, tensor_scale,
                     w_scale, comb_scale, reinterpret_cast<uint2*>(codes), scales,
                     reinterpret_cast<uint4*>(xs));
  return hipGetLastError();
}

}  // namespace nvfp4
