// W4A16 GEMM for decode-sized token counts (m <= 64) on gfx950.
//
// y[m, n] = s_t * sum_k x[m, k] * (val(code[n, k]) * sigma[n, k/16]).
// The pages run a W4A16 kernel for small token counts ("SOAR 2026 Recap ...",
// section "1. Quantization and GEMM dispatch"); decode is bound by reading
// the weights from HBM ("SOAR Weekly Champion Notes 08 ...", section "01").
//
// Design (memory-bound): the packed weights are read exactly once, with
// 16-byte loads; activations are small and reused, so each workgroup stages
// its K chunk of x in LDS, already in MFMA B-operand order.  Weights are the
// MFMA A operand: each wave owns 16 weight rows; lane l holds row l%16 and 32
// consecutive codes (two 16-element blocks) per K step of 128.  val * sigma
// has at most 6 significant bits, so it is exact in bf16; the products are
// accumulated in fp32 by v_mfma_f32_16x16x32_bf16 and s_t is applied once in
// fp32 at the end.  The K dimension is split over grid.y; with more than one
// split the fp32 partial sums go to a workspace and k_reduce adds them in
// split order (deterministic).
#include "launchers.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kRowsPerWg = 16 * kWaves;
constexpr int kStepK = 128;        // K per main-loop step (4 MFMAs of K=32)

// Decode 8 codes (one dword, element i at bits 4i) scaled by sigma into an
// MFMA bf16x8 operand, element order = code order.
template <int IMPL>
__device__ __forceinline__ bf16x8_t dequant8(uint32_t d, float sigma) {
  u32x4_t o;
  if constexpr (IMPL == kConvHw) {
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    o[0] = pack_bf16_exact(v0[0] * sigma, v0[1] * sigma);
    o[1] = pack_bf16_exact(v1[0] * sigma, v1[1] * sigma);
    o[2] = pack_bf16_exact(v2[0] * sigma, v2[1] * sigma);
    o[3] = pack_bf16_exact(v3[0] * sigma, v3[1] * sigma);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = e2m1_val_portable((d >> (8 * i)) & 0xFu) * sigma;
      const float b = e2m1_val_portable((d >> (8 * i + 4)) & 0xFu) * sigma;
      o[i] = pack_bf16_exact(a, b);
    }
  }
  return __builtin_bit_cast(bf16x8_t, o);
}

__device__ __forceinline__ float scale_value(uint32_t s) {
  const float v = e4m3_decode(s & 0x7Fu);
  return (s & 0x80u) ? -v : v;
}

// out_mode: 0 = bf16 y, 1 = fp32 y, 2 = fp32 partial sums into ws[split].
template <int MT, int IMPL, bool K32>
__global__ __launch_bounds__(256) void k_skinny(const uint16_t* __restrict__ x,
                                                const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales,
                                                const float* __restrict__ tensor_scale,
                                                void* __restrict__ y, float* __restrict__ ws,
                                                int M, int N, int K, int kchunk, int out_mode) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;  // lane group: which 32 codes of the K step
  const int r16 = lane & 15;

  const int k0 = blockIdx.y * kchunk;
  const int kend = min(k0 + kchunk, K);
  const int nks = (kend - k0 + kStepK - 1) / kStepK;  // K steps in this chunk

  // ---- stage x[0:16*MT, k0:kend) into LDS in B-operand order -------------
  // piece (ks, j, mt, g, mm) = 8 bf16 of x[16 mt + mm][k0 + 128 ks + 32 g + 8 j ..]
  {
    const int pieces_per_row = nks * 16;  // 16-byte pieces per x row in the chunk
    const int total = 16 * MT * pieces_per_row;
    for (int p = threadIdx.x; p < total; p += blockDim.x) {
      const int m = p / pieces_per_row;
      const int k8 = p - m * pieces_per_row;
      const int k = k0 + 8 * k8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M && k < kend) v = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k);
      const int ks = k8 >> 4, rem = k8 & 15;
      const int pg = rem >> 2, pj = rem & 3;
      const int mt = m >> 4, mm = m & 15;
      const int off = ((((ks * 4 + pj) * MT + mt) * 4 + pg) * 16 + mm) * 16;
      *reinterpret_cast<uint4*>(lds + off) = v;
    }
  }
  __syncthreads();

  const int row = blockIdx.x * kRowsPerWg + wave * 16 + r16;
  const bool row_ok = row < N;
  const uint8_t* crow = codes + (int64_t)row * (K / 2);
  const uint8_t* srow = scales + (int64_t)row * (K / 16);

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < nks; ++ks) {
    const int kk = k0 + ks * kStepK + 32 * g;  // first of this lane's 32 codes
    u32x4_t cw = {0u, 0u, 0u, 0u};
    uint32_t sb0 = 0u, sb1 = 0u;
    if constexpr (K32) {
      if (row_ok && kk < kend) {
        cw = *reinterpret_cast<const u32x4_t*>(crow + kk / 2);
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(srow + kk / 16);
        sb0 = s2 & 0xFFu;
        sb1 = s2 >> 8;
      }
    } else {
      if (row_ok && kk < kend) {
        const uint2 a = *reinterpret_cast<const uint2*>(crow + kk / 2);
        cw[0] = a.x;
        cw[1] = a.y;
        sb0 = srow[kk / 16];
      }
      if (row_ok && kk + 16 < kend) {
        const uint2 b = *reinterpret_cast<const uint2*>(crow + kk / 2 + 8);
        cw[2] = b.x;
        cw[3] = b.y;
        sb1 = srow[kk / 16 + 1];
      }
    }
    const float sg0 = scale_value(sb0), sg1 = scale_value(sb1);
    bf16x8_t a[4];
    a[0] = dequant8<IMPL>(cw[0], sg0);
    a[1] = dequant8<IMPL>(cw[1], sg0);
    a[2] = dequant8<IMPL>(cw[2], sg1);
    a[3] = dequant8<IMPL>(cw[3], sg1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int off = ((((ks * 4 + j) * MT + mt) * 4 + g) * 16 + r16) * 16;
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(lds + off);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b, acc[mt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds D[n = 4g + i][m = r16] of each m tile --------
  const float s_t = tensor_scale[0];
  const int nbase = blockIdx.x * kRowsPerWg + wave * 16 + 4 * g;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = nbase + i;
      if (n >= N) continue;
      const int64_t idx = (int64_t)m * N + n;
      if (out_mode == 2) {
        ws[(int64_t)blockIdx.y * M * N + idx] = acc[mt][i];
      } else if (out_mode == 1) {
        reinterpret_cast<float*>(y)[idx] = acc[mt][i] * s_t;
      } else {
        reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)bf16_rne_bits(acc[mt][i] * s_t);
      }
    }
  }
}

// y = s_t * sum over splits (in split order) of the fp32 partial sums.
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ ws,
                                                const float* __restrict__ tensor_scale,
                                                void* __restrict__ y, int64_t mn, int splits,
                                                int out_f32) {
  const float s_t = tensor_scale[0];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
    float s = ws[i];
    for (int sp = 1; sp < splits; ++sp) s += ws[(int64_t)sp * mn + i];
    if (out_f32)
      reinterpret_cast<float*>(y)[i] = s * s_t;
    else
      reinterpret_cast<uint16_t*>(y)[i] = (uint16_t)bf16_rne_bits(s * s_t);
  }
}

template <int MT, int IMPL, bool K32>
void launch_mt(dim3 grid, size_t lds, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
               const uint8_t* scales, const float* ts, void* y, float* ws, int M, int N, int K,
               int kchunk, int out_mode) {
  hipLaunchKernelGGL((k_skinny<MT, IMPL, K32>), grid, dim3(256), lds, stream, x, codes, scales, ts,
                     y, ws, M, N, K, kchunk, out_mode);
}

template <int IMPL, bool K32>
void launch_impl(int mt, dim3 grid, size_t lds, hipStream_t stream, const uint16_t* x,
                 const uint8_t* codes, const uint8_t* scales, const float* ts, void* y, float* ws,
                 int M, int N, int K, int kchunk, int out_mode) {
  switch (mt) {
    case 1: launch_mt<1, IMPL, K32>(grid, lds, stream, x, codes, scales, ts, y, ws, M, N, K, kchunk, out_mode); break;
    case 2: launch_mt<2, IMPL, K32>(grid, lds, stream, x, codes, scales, ts, y, ws, M, N, K, kchunk, out_mode); break;
    case 3: launch_mt<3, IMPL, K32>(grid, lds, stream, x, codes, scales, ts, y, ws, M, N, K, kchunk, out_mode); break;
    default: launch_mt<4, IMPL, K32>(grid, lds, stream, x, codes, scales, ts, y, ws, M, N, K, kchunk, out_mode); break;
  }
}

int max_chunk(int mt) {
  // LDS per workgroup = kchunk * 32 * MT bytes; keep it <= 64 KiB
  return mt == 1 ? 2048 : (mt == 2 ? 1024 : 512);
}

}  // namespace

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int forced_splits) {
  SkinnyPlan p{1, kStepK, 0};
  const int mt = (int)((m + 15) / 16);
  const int64_t ksteps = (k + kStepK - 1) / kStepK;
  if (ksteps == 0) return p;
  int64_t splits;
  if (forced_splits > 0) {
    splits = forced_splits;
  } else {
    const int64_t wgs_n = (n + kRowsPerWg - 1) / kRowsPerWg;
    splits = (1024 + wgs_n - 1) / wgs_n;  // aim at ~4 workgroups per CU
  }
  if (splits < 1) splits = 1;
  if (splits > 64) splits = 64;
  if (splits > ksteps) splits = ksteps;
  int64_t steps_per = (ksteps + splits - 1) / splits;
  const int64_t max_steps = max_chunk(mt) / kStepK;
  if (steps_per > max_steps) steps_per = max_steps;
  p.kchunk = (int)(steps_per * kStepK);
  p.splits = (int)((ksteps + steps_per - 1) / steps_per);
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  return p;
}

hipError_t launch_skinny(const void* x, const uint8_t* codes, const uint8_t* scales,
                         const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                         int out_f32, const SkinnyPlan& plan, void* workspace, int impl,
                         hipStream_t stream) {
  const int mt = (int)((m + 15) / 16);
  const dim3 grid((unsigned)((n + kRowsPerWg - 1) / kRowsPerWg), (unsigned)plan.splits);
  const int nks = plan.kchunk / kStepK;
  const size_t lds = (size_t)nks * 4 * mt * 4 * 16 * 16;
  const int out_mode = plan.splits > 1 ? 2 : (out_f32 ? 1 : 0);
  const bool k32 = (k % 32) == 0;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  float* ws = reinterpret_cast<float*>(workspace);
  if (impl == kConvHw) {
    if (k32) launch_impl<kConvHw, true>(mt, grid, lds, stream, xp, codes, scales, tensor_scale, y, ws, (int)m, (int)n, (int)k, plan.kchunk, out_mode);
    else launch_impl<kConvHw, false>(mt, grid, lds, stream, xp, codes, scales, tensor_scale, y, ws, (int)m, (int)n, (int)k, plan.kchunk, out_mode);
  } else {
    if (k32) launch_impl<kConvPortable, true>(mt, grid, lds, stream, xp, codes, scales, tensor_scale, y, ws, (int)m, (int)n, (int)k, plan.kchunk, out_mode);
    else launch_impl<kConvPortable, false>(mt, grid, lds, stream, xp, codes, scales, tensor_scale, y, ws, (int)m, (int)n, (int)k, plan.kchunk, out_mode);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  const int64_t mn = m * n;
  int64_t blocks = (mn + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)blocks), dim3(256), 0, stream, ws, tensor_scale, y,
                     mn, plan.splits, out_f32);
  return hipGetLastError();
}

}  // namespace nvfp4
