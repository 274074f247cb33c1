// W4A16 GEMM for large token counts on gfx950: bf16 MFMA tiles.
//
// The pages switch to another kernel above M ~ 48 ("SOAR 2026 Recap ...",
// section "1. Quantization and GEMM dispatch"), there an FP4 x FP4 MMA.  Here
// the activations stay bf16 (W4A16) and the weights are dequantized to bf16
// (val * sigma is exact in bf16) into LDS, because the NVFP4 block scales
// (E4M3 per 16) are not the block-scale layout of gfx950's scaled MFMA.
//
// Tile: 128 weight rows (n) x 128 token rows (m) x 64 k per step, 256
// threads = 4 waves in a 2 x 2 grid, each wave 64 x 64 = 4 x 4 MFMA
// 16x16x32 tiles.  Global loads of step s+1 are issued before the MFMAs of
// step s (register prefetch); LDS holds one step of A and B fragments.
#include "launchers.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kBN = 128, kBM = 128, kBK = 64;
// LDS fragment layout (each entry 16 bytes = 8 bf16):
//   A[kk(2)][ntile(8)][g(4)][r(16)]  = W_hat[n0 + 16 ntile + r][k0 + 32 kk + 8 g ..]
//   B[kk(2)][mtile(8)][g(4)][c(16)]  = x[m0 + 16 mtile + c][k0 + 32 kk + 8 g ..]
constexpr int kFragBytes = 2 * 8 * 4 * 16 * 16;  // 16 KiB per operand

template <int IMPL>
__device__ __forceinline__ uint4 dequant8u(uint32_t d, float sigma) {
  uint4 o;
  if constexpr (IMPL == kConvHw) {
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    o.x = pack_bf16_exact(v0[0] * sigma, v0[1] * sigma);
    o.y = pack_bf16_exact(v1[0] * sigma, v1[1] * sigma);
    o.z = pack_bf16_exact(v2[0] * sigma, v2[1] * sigma);
    o.w = pack_bf16_exact(v3[0] * sigma, v3[1] * sigma);
  } else {
    uint32_t t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t[i] = pack_bf16_exact(e2m1_val_portable((d >> (8 * i)) & 0xFu) * sigma,
                             e2m1_val_portable((d >> (8 * i + 4)) & 0xFu) * sigma);
    o = make_uint4(t[0], t[1], t[2], t[3]);
  }
  return o;
}

__device__ __forceinline__ float scale_value(uint32_t s) {
  const float v = e4m3_decode(s & 0x7Fu);
  return (s & 0x80u) ? -v : v;
}

template <int IMPL, bool K32>
__global__ __launch_bounds__(256) void k_tiled(const uint16_t* __restrict__ x,
                                               const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ scales,
                                               const float* __restrict__ tensor_scale,
                                               void* __restrict__ y, int M, int N, int K,
                                               int out_f32) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kFragBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kFragBytes];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;

  // Loader roles.  Weights: thread t loads row n0 + t/2, 32 codes at
  // k0 + 32*(t%2) (16 bytes) and their 2 scales.  x: thread t loads 4
  // 16-byte pieces p = t + 256 i: row m0 + p/8, k0 + 8*(p%8).
  const int wrow = n0 + (t >> 1), whalf = t & 1;
  const bool wrow_ok = wrow < N;
  const uint8_t* crow = codes + (int64_t)wrow * (K / 2);
  const uint8_t* srow = scales + (int64_t)wrow * (K / 16);

  uint32_t cw[4];
  uint32_t sb0, sb1;
  uint4 xv[4];
  auto load_step = [&](int k0) {
    const int kk = k0 + 32 * whalf;
    cw[0] = cw[1] = cw[2] = cw[3] = 0u;
    sb0 = sb1 = 0u;
    if constexpr (K32) {
      if (wrow_ok && kk < K) {
        const uint4 c = *reinterpret_cast<const uint4*>(crow + kk / 2);
        cw[0] = c.x; cw[1] = c.y; cw[2] = c.z; cw[3] = c.w;
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(srow + kk / 16);
        sb0 = s2 & 0xFFu;
        sb1 = s2 >> 8;
      }
    } else {
      if (wrow_ok && kk < K) {
        const uint2 a = *reinterpret_cast<const uint2*>(crow + kk / 2);
        cw[0] = a.x; cw[1] = a.y;
        sb0 = srow[kk / 16];
      }
      if (wrow_ok && kk + 16 < K) {
        const uint2 b = *reinterpret_cast<const uint2*>(crow + kk / 2 + 8);
        cw[2] = b.x; cw[3] = b.y;
        sb1 = srow[kk / 16 + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = t + 256 * i;
      const int m = m0 + (p >> 3), k = k0 + 8 * (p & 7);
      xv[i] = make_uint4(0u, 0u, 0u, 0u);
      if (m < M && k < K) xv[i] = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k);
    }
  };
  auto store_step = [&]() {
    const float sg0 = scale_value(sb0), sg1 = scale_value(sb1);
    const int rl = t >> 1, nt = rl >> 4, rr = rl & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = dequant8u<IMPL>(cw[j], j < 2 ? sg0 : sg1);
      const int off = (((whalf * 8 + nt) * 4 + j) * 16 + rr) * 16;
      *reinterpret_cast<uint4*>(sA + off) = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = t + 256 * i;
      const int ml = p >> 3, k8 = p & 7;
      const int kk = k8 >> 2, gg = k8 & 3;
      const int off = (((kk * 8 + (ml >> 4)) * 4 + gg) * 16 + (ml & 15)) * 16;
      *reinterpret_cast<uint4*>(sB + off) = xv[i];
    }
  };

  const int wn = wave >> 1, wm = wave & 1;  // wave's 64 x 64 sub-tile
  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (K + kBK - 1) / kBK;
  if (nsteps > 0) load_step(0);
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();  // previous step's fragments fully consumed
    store_step();
    __syncthreads();
    if (s + 1 < nsteps) load_step((s + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t*>(sA + (((kk * 8 + 4 * wn + i) * 4 + g) * 16 + r16) * 16);
        bfr[i] = *reinterpret_cast<const bf16x8_t*>(sB + (((kk * 8 + 4 * wm + i) * 4 + g) * 16 + r16) * 16);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  }

  // epilogue: acc[a][b] lane holds D[n = 16(4wn+a) + 4g + i][m = 16(4wm+b) + r16]
  const float s_t = tensor_scale[0];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int m = m0 + 16 * (4 * wm + b) + r16;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 16 * (4 * wn + a) + 4 * g + i;
        if (n >= N) continue;
        const int64_t idx = (int64_t)m * N + n;
        if (out_f32)
          reinterpret_cast<float*>(y)[idx] = acc[a][b][i] * s_t;
        else
          reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)bf16_rne_bits(acc[a][b][i] * s_t);
      }
    }
  }
}

}  // namespace

hipError_t launch_tiled(const void* x, const uint8_t* codes, const uint8_t* scales,
                        const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                        int out_f32, int impl, hipStream_t stream) {
  const dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  const bool k32 = (k % 32) == 0;
  if (impl == kConvHw) {
    if (k32) hipLaunchKernelGGL((k_tiled<kConvHw, true>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, (int)m, (int)n, (int)k, out_f32);
    else hipLaunchKernelGGL((k_tiled<kConvHw, false>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, (int)m, (int)n, (int)k, out_f32);
  } else {
    if (k32) hipLaunchKernelGGL((k_tiled<kConvPortable, true>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, (int)m, (int)n, (int)k, out_f32);
    else hipLaunchKernelGGL((k_tiled<kConvPortable, false>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, (int)m, (int)n, (int)k, out_f32);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
