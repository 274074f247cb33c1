// W4A16 GEMM for large token counts on gfx950: bf16 MFMA tiles.
//
// The pages switch to another kernel above M ~ 48 ("SOAR 2026 Recap ...",
// section "1. Quantization and GEMM dispatch"), there an FP4 x FP4 MMA.  Here
// the activations stay bf16 (W4A16) and the weights are dequantized to bf16
// (val * sigma is exact in bf16), because the NVFP4 block scales
// (E4M3 per 16) are not the block-scale layout of gfx950's scaled MFMA.
//
// Kernels:
//  * k_lmr (K a multiple of 64, m > 128): 256 weight rows x 128 tokens per
//    workgroup, each wave dequantizing its 64 weight rows straight into MFMA
//    A fragments (the weights never touch LDS) while the activations arrive
//    in LDS by DMA; v_mfma_f32_32x32x16_bf16, two waves per SIMD.  k_lmr2,
//    the same with 128 k per barrier, where K is a multiple of 128.
//  * k_lm (K a multiple of 64, m <= 128): BN weight rows x BM tokens per
//    workgroup, v_mfma_f32_32x32x16_bf16 (the 32x32 shape keeps the matrix
//    cores busy with few independent accumulators; the 16x16x32 shape needs
//    more than a wave holds here), 64 k per step, two LDS stages (the next
//    step's weights are dequantized and its activations stored while the
//    current step's MFMAs run, one barrier per step), global loads two steps
//    ahead.  Configurations: m <= 64: one 64-token tile x 256 weight rows
//    (4 waves), or x 128 rows for long K; 64 < m <= 128: 128 x 128.
//  With few tiles the K loop is split over workgroups (fp32 partials, then
//  a reduction kernel adds them in split order).
//  * k_tiled (any K): 128 x 128 x 64 tiles, 4 waves of 4 x 4
//    v_mfma_f32_16x16x32_bf16, one LDS stage.
#include "launchers.h"
#include "nvfp4_device.h"

namespace nvfp4 {
NVFP4_VARIANT_BEGIN
namespace {


constexpr int kBN = 128, kBM = 128, kBK = 64;
// LDS fragment layout (each entry 16 bytes = 8 bf16):
//   A[kk(2)][ntile(8)][g(4)][r(16)]  = W_hat[n0 + 16 ntile + r][k0 + 32 kk + 8 g ..]
//   B[kk(2)][mtile(8)][g(4)][c(16)]  = x[m0 + 16 mtile + c][k0 + 32 kk + 8 g ..]
constexpr int kFragBytes = 2 * 8 * 4 * 16 * 16;  // 16 KiB per operand

template <int IMPL>
__device__ __forceinline__ uint4 dequant8u(uint32_t d, float sigma) {
  const u32x4_t o = dequant8_bf16<IMPL>(d, sigma);
  return make_uint4(o[0], o[1], o[2], o[3]);
}


template <int IMPL, bool K32>
__global__ __launch_bounds__(256) void k_tiled(const uint16_t* __restrict__ x,
                                               const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ scales,
                                               const KScale tensor_scale,
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
    const float sg0 = scale_at<IMPL, 0>(sb0), sg1 = scale_at<IMPL, 0>(sb1);
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
  const float s_t0 = first_scale(tensor_scale);
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
        const float s_t = col_scale(tensor_scale, n, s_t0);
        const int64_t idx = (int64_t)m * N + n;
        if (out_f32)
          reinterpret_cast<float*>(y)[idx] = acc[a][b][i] * s_t;
        else
          reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)bf16_rne_bits(acc[a][b][i] * s_t);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// k_lm.  A fragment (ks, T) is 32 rows x 16 k in LDS, entry l (16 bytes) =
// (h = l / 32, r = l % 32) holds row r of tile T at k = k0 + 8 (4 h + ks)
// .. +8: the loader lane (h, r) owns the contiguous k0 + 32 h .. +32 of its
// row (16 bytes of codes, 2 scales; 64 bytes of activations), and the MFMA
// reads entry `lane` - the same k order on both operands, so the products
// pair up.  Every LDS store and load is one contiguous 1 KiB per wave.
// blockIdx.z = K split: steps [z * steps_per, min(K / 64, (z + 1) * steps_per)).
template <int BN, int BM, int WGN, int WGM, int IMPL>
__global__ __launch_bounds__(64 * WGN * WGM) void k_lm(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const KScale tensor_scale,
                                                       void* __restrict__ y, float* __restrict__ ws,
                                                       int M, int N, int K, int steps_per,
                                                       int out_f32) {
  constexpr int NW = WGN * WGM;
  constexpr int NT = BN / 32, MT = BM / 32;    // 32-row tiles per workgroup
  constexpr int WNT = NT / WGN, WMT = MT / WGM;  // per wave
  constexpr int A_BYTES = 4 * NT * 1024, B_BYTES = 4 * MT * 1024;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int WA = (NT + NW - 1) / NW, WB = (MT + NW - 1) / NW;  // loader tiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int wn = wave / WGM, wm = wave % WGM;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;

  // one step of loader data in registers (codes, scales, activations)
  struct Regs {
    u32x4_t cv[WA];
    uint32_t sv[WA];
    u32x4_t xv[WB][4];
  };
  auto load_step = [&](Regs& R, int k0) {
#pragma unroll
    for (int i = 0; i < WA; ++i) {
      const int tile = WA * wave + i;
      if (tile >= NT) break;
      const int row = n0 + 32 * tile + r32;
      const int rowc = min(row, N - 1);
      R.cv[i] = *reinterpret_cast<const u32x4_t*>(codes + (int64_t)rowc * (K / 2) + k0 / 2 + 16 * h);
      const uint32_t s2 = *reinterpret_cast<const uint16_t*>(scales + (int64_t)rowc * (K / 16) + k0 / 16 + 2 * h);
      R.sv[i] = row < N ? s2 : 0u;  // sigma 0: rows past N contribute zeros
    }
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      const int tile = WB * wave + j;
      if (tile >= MT) break;
      // rows past M read row M - 1 (finite values); their outputs are not stored
      const int m = min(m0 + 32 * tile + r32, M - 1);
      const uint16_t* xp = x + (int64_t)m * K + k0 + 32 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) R.xv[j][q] = *reinterpret_cast<const u32x4_t*>(xp + 8 * q);
    }
  };
  auto store_step = [&](const Regs& R, uint8_t* st) {
    uint8_t* sA = st;
    uint8_t* sB = st + A_BYTES;
#pragma unroll
    for (int i = 0; i < WA; ++i) {
      const int tile = WA * wave + i;
      if (tile >= NT) break;
      const float sg0 = scale_at<IMPL, 0>(R.sv[i]), sg1 = scale_at<IMPL, 1>(R.sv[i]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 o = dequant8u<IMPL>(R.cv[i][ks], ks < 2 ? sg0 : sg1);
        *reinterpret_cast<uint4*>(sA + ((ks * NT + tile) * 64 + lane) * 16) = o;
      }
    }
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      const int tile = WB * wave + j;
      if (tile >= MT) break;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        *reinterpret_cast<u32x4_t*>(sB + ((ks * MT + tile) * 64 + lane) * 16) = R.xv[j][ks];
    }
  };

  f32x16_t acc[WNT][WMT];
#pragma unroll
  for (int a = 0; a < WNT; ++a)
#pragma unroll
    for (int b = 0; b < WMT; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  const int s0 = blockIdx.z * steps_per;
  const int nsteps = min(K / 64 - s0, steps_per);  // >= 1 (the plan has no empty split)
  const int kbase = s0 * 64;

  // One step: MFMAs on LDS stage s % 2 while stage (s + 1) % 2 is filled
  // from R (step s + 1) and R is reloaded with step s + 2.  (Two register
  // sets, loads three steps ahead, measured slower: the extra VGPRs cost
  // more occupancy than the longer prefetch gains.)
  auto iter = [&](int s, Regs& R) {
    __syncthreads();  // stage s % 2 complete; nobody reads stage (s + 1) % 2 any more
    const uint8_t* sA = lds + (s & 1) * STAGE;
    const uint8_t* sB = sA + A_BYTES;
    bf16x8_t af[2][WNT], bfr[2][WMT];
#pragma unroll
    for (int i = 0; i < WNT; ++i)
      af[0][i] = *reinterpret_cast<const bf16x8_t*>(sA + ((WNT * wn + i) * 64 + lane) * 16);
#pragma unroll
    for (int j = 0; j < WMT; ++j)
      bfr[0][j] = *reinterpret_cast<const bf16x8_t*>(sB + ((WMT * wm + j) * 64 + lane) * 16);
    if (s + 1 < nsteps) {
      store_step(R, lds + ((s + 1) & 1) * STAGE);
      if (s + 2 < nsteps) load_step(R, kbase + (s + 2) * 64);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < 4) {
#pragma unroll
        for (int i = 0; i < WNT; ++i)
          af[c ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(sA + (((ks + 1) * NT + WNT * wn + i) * 64 + lane) * 16);
#pragma unroll
        for (int j = 0; j < WMT; ++j)
          bfr[c ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(sB + (((ks + 1) * MT + WMT * wm + j) * 64 + lane) * 16);
      }
#pragma unroll
      for (int a = 0; a < WNT; ++a)
#pragma unroll
        for (int b = 0; b < WMT; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c][a], bfr[c][b], acc[a][b], 0, 0, 0);
    }
  };

  Regs R;
  load_step(R, kbase);
  store_step(R, lds);
  if (nsteps > 1) load_step(R, kbase + 64);
  for (int s = 0; s < nsteps; ++s) iter(s, R);  // stores step s + 1, loads step s + 2

  // D of a 32 x 32 tile: lane l, value v -> weight row 8 (v / 4) + 4 (l / 32)
  // + v % 4, token l % 32.  With a K split: raw fp32 partials to plane z.
  const bool partial = gridDim.z > 1;
  float* plane = ws + (int64_t)blockIdx.z * M * N;
  const float s_t0 = first_scale(tensor_scale);
#pragma unroll
  for (int b = 0; b < WMT; ++b) {
    const int m = m0 + 32 * (WMT * wm + b) + r32;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < WNT; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 32 * (WNT * wn + a) + 8 * q + 4 * h;
        const float s_t = partial ? 1.0f : col_scale(tensor_scale, n, s_t0);  // n .. n + 3: one group
        const float v0 = acc[a][b][4 * q] * s_t, v1 = acc[a][b][4 * q + 1] * s_t;
        const float v2 = acc[a][b][4 * q + 2] * s_t, v3 = acc[a][b][4 * q + 3] * s_t;
        const int64_t idx = (int64_t)m * N + n;
        if (partial) {
          if ((N & 3) == 0 && n + 3 < N) {
            *reinterpret_cast<float4*>(plane + idx) = make_float4(v0, v1, v2, v3);
          } else {
            const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) plane[idx + i] = vv[i];
          }
        } else if ((N & 3) == 0 && n + 3 < N) {  // 4 outputs, 16- or 8-byte aligned
          if (out_f32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + idx) = make_float4(v0, v1, v2, v3);
          } else {
            uint2 v;
            v.x = bf16_rne_bits(v0) | (bf16_rne_bits(v1) << 16);
            v.y = bf16_rne_bits(v2) | (bf16_rne_bits(v3) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) = v;
          }
        } else {
          const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (n + i >= N) continue;
            if (out_f32)
              reinterpret_cast<float*>(y)[idx + i] = vv[i];
            else
              reinterpret_cast<uint16_t*>(y)[idx + i] = (uint16_t)bf16_rne_bits(vv[i]);
          }
        }
      }
    }
  }
}

// Epilogue of the weights-in-registers kernels: wave `wave`'s 64 weight rows
// x MTILES 32-token tiles.  D of a 32 x 32 tile: lane l, value v -> weight
// row 8 (v / 4) + 4 (l / 32) + v % 4, token l % 32.  With a K split (more
// than one plane): raw fp32 partials to plane blockIdx.z.
template <int MTILES>
__device__ __forceinline__ void store_lmr(const f32x16_t (&acc)[2][MTILES], const KScale tensor_scale, void* y,
                                          float* ws, int M, int N, int n0, int m0, int wave, int out_f32) {
  const int lane = threadIdx.x & 63, h = lane >> 5, r32 = lane & 31;
  const bool partial = gridDim.z > 1;
  float* plane = ws + (int64_t)blockIdx.z * M * N;
  const float s_t0 = first_scale(tensor_scale);
#pragma unroll
  for (int b = 0; b < MTILES; ++b) {
    const int m = m0 + 32 * b + r32;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 64 * wave + 32 * a + 8 * q + 4 * h;
        const float s_t = partial ? 1.0f : col_scale(tensor_scale, n, s_t0);  // n .. n + 3: one group
        const float v0 = acc[a][b][4 * q] * s_t, v1 = acc[a][b][4 * q + 1] * s_t;
        const float v2 = acc[a][b][4 * q + 2] * s_t, v3 = acc[a][b][4 * q + 3] * s_t;
        const int64_t idx = (int64_t)m * N + n;
        if (partial) {
          if ((N & 3) == 0 && n + 3 < N) {
            *reinterpret_cast<float4*>(plane + idx) = make_float4(v0, v1, v2, v3);
          } else {
            const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) plane[idx + i] = vv[i];
          }
        } else if ((N & 3) == 0 && n + 3 < N) {
          if (out_f32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + idx) = make_float4(v0, v1, v2, v3);
          } else {
            uint2 v;
            v.x = bf16_rne_bits(v0) | (bf16_rne_bits(v1) << 16);
            v.y = bf16_rne_bits(v2) | (bf16_rne_bits(v3) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) = v;
          }
        } else {
          const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (n + i >= N) continue;
            if (out_f32)
              reinterpret_cast<float*>(y)[idx + i] = vv[i];
            else
              reinterpret_cast<uint16_t*>(y)[idx + i] = (uint16_t)bf16_rne_bits(vv[i]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_lmr: large-M kernel with the weights in registers.  A workgroup covers
// 256 weight rows x BM tokens with 4 waves; wave w owns rows 64 w .. +64 (two
// 32-row MFMA A tiles) against all BM tokens.  Per 64-k step:
//  * each lane loads, for each of its two rows, the 32 codes (16 bytes) and
//    the 2 scale bytes of its k half (h = lane / 32: k0 + 32 h .. +32), and
//    dequantizes them straight into A fragments - the weights never touch
//    LDS (in k_lm their dequantized stores and fragment loads were most of
//    the LDS traffic);
//  * the step's activations (BM rows x 128 bytes) arrive in LDS by DMA,
//    shared by the 4 waves: DMA instruction c copies token rows 8 c .. +8,
//    whole cache lines, lane l -> row 8 c + l / 8, 16-byte piece
//    (l % 8) ^ ((row / 2) % 8), so piece q of row r lands at slot
//    q ^ ((r / 2) % 8) and the B fragment reads of 16 rows hit 16 bank
//    groups.
// k order: MFMA ks of a step pairs logical k 0..7 with physical k 8 ks .. +8
// and logical k 8..15 with 32 + 8 ks .. +8, on both operands.
// Pipeline: weights two steps ahead (two register sets), activations one
// step ahead (two LDS stages).  The loads are inline asm with counted waits
// (the compiler cannot count LDS DMA and plain loads together); every step
// issues the same loads (addresses clamped to the last step at the end), so
// the wait count is the same at every step.
// blockIdx.z = K split as in k_lm.
template <int BM, int IMPL>
__global__ __launch_bounds__(256, 2) void k_lmr(const uint16_t* __restrict__ x,
                                             const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ scales,
                                             const KScale tensor_scale,
                                             void* __restrict__ y, float* __restrict__ ws, int M,
                                             int N, int K, int steps_per, int out_f32) {
  constexpr int MTILES = BM / 32;  // 32-token MFMA B tiles
  constexpr int NDMA = BM / 32;    // DMA instructions per wave per step (BM rows x 128 B / 4 waves)
  constexpr int STAGE = BM * 128;
  constexpr int WOPS = 4;          // weight loads per step: 2 x codes, 2 x scales
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int n0 = blockIdx.x * 256, m0 = blockIdx.y * BM;
  const int s0 = blockIdx.z * steps_per;
  const int nsteps = min(K / 64 - s0, steps_per);  // >= 1 (the plan has no empty split)
  const int kbase = s0 * 64;

  // weight rows of this lane (rows past N read row N - 1; not stored)
  const uint8_t* cp[2];
  const uint8_t* sp[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = min(n0 + 64 * wave + 32 * a + r32, N - 1);
    cp[a] = codes + (int64_t)row * (K / 2) + kbase / 2 + 16 * h;
    sp[a] = scales + (int64_t)row * (K / 16) + kbase / 16 + 2 * h;
  }
  // activation pieces this lane copies (token rows past M read row M - 1)
  const uint16_t* xp[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int rho = 8 * (wave + 4 * i) + (lane >> 3);
    const int m = min(m0 + rho, M - 1);
    xp[i] = x + (int64_t)m * K + kbase + 8 * ((lane & 7) ^ ((rho >> 1) & 7));
  }

  struct WRegs {
    u32x4_t c[2];
    uint32_t s[2];
  };
  auto issue_w = [&](WRegs& W, int step) {
    step = min(step, nsteps - 1);
#pragma unroll
    for (int a = 0; a < 2; ++a) load_b128_async<0>(W.c[a], cp[a] + 32 * step);
#pragma unroll
    for (int a = 0; a < 2; ++a) load_u16_async<0>(W.s[a], sp[a] + 4 * step);
  };
  auto issue_x = [&](int step) {
    const int st = step & 1;
    step = min(step, nsteps - 1);
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      copy16_to_lds(xp[i] + 64 * step, lds + st * STAGE + 1024 * (wave + 4 * i));
    asm volatile("" ::: "memory");
  };

  f32x16_t acc[2][MTILES];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < MTILES; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // One step: wait for its weights (set W) and activations (stage s % 2) -
  // only the weights issued one step earlier may still be in flight - then
  // a barrier (every wave's copies have landed, and every wave is done with
  // stage (s + 1) % 2), dequantize, issue the loads of steps s + 1 (copies)
  // and s + 2 (weights, into W), and run the MFMAs.
  auto step = [&](int s, WRegs& W) {
    wait_vm4<WOPS>(W.c[0], W.c[1], W.s[0], W.s[1]);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8_t af[4][2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float sg0 = scale_at<IMPL, 0>(W.s[a]), sg1 = scale_at<IMPL, 1>(W.s[a]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        af[ks][a] = __builtin_bit_cast(bf16x8_t, dequant8u<IMPL>(W.c[a][ks], ks < 2 ? sg0 : sg1));
    }
    issue_x(s + 1);
    issue_w(W, s + 2);
    const uint8_t* st = lds + (s & 1) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int b = 0; b < MTILES; ++b) {
        const int rho = 32 * b + r32;
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(
            st + 128 * rho + 16 * ((4 * h + ks) ^ ((rho >> 1) & 7)));
#pragma unroll
        for (int a = 0; a < 2; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][a], bv, acc[a][b], 0, 0, 0);
      }
    }
  };

  WRegs W0, W1;
  issue_w(W0, 0);
  issue_x(0);
  issue_w(W1, 1);
  for (int s = 0; s < nsteps; s += 2) {
    step(s, W0);
    if (s + 1 < nsteps) step(s + 1, W1);
  }
  wait_vm_all();  // the tail's clamped copies must land before the workgroup's LDS is released
  store_lmr<MTILES>(acc, tensor_scale, y, ws, M, N, n0, m0, wave, out_f32);
}

// ---------------------------------------------------------------------------
// k_lmr2: k_lmr with 128 k per barrier (K a multiple of 128).  The same
// workgroup tile, lane roles and per-64-k MFMA order as k_lmr; a double step
// is two 64-k halves, each laid out in LDS as one k_lmr stage (two stages of
// 2 x BM x 128 bytes).  Per double step each lane loads, for each of its two
// rows, the 64 bytes of codes its halves need as two back-to-back 16-byte
// loads from one 64-byte segment (the second is served by the L1), and the 8
// scale bytes of the row in one 8-byte load (lane half h uses bytes 2h, 2h+1
// of each 4-byte word, word j for half j).  Against k_lmr: half the barriers
// and half the weight requests to the L2 per k.
// Pipeline: activations one double step ahead (two LDS stages), weights
// one double step ahead in one register set, reloaded after the second
// half's dequantization; every double step waits for all of its loads.
// blockIdx.z = K split: steps_per (64-k steps) is even.
template <int BM, int IMPL>
__global__ __launch_bounds__(256, 2) void k_lmr2(const uint16_t* __restrict__ x,
                                              const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales,
                                              const KScale tensor_scale,
                                              void* __restrict__ y, float* __restrict__ ws, int M,
                                              int N, int K, int steps_per, int out_f32) {
  constexpr int MTILES = BM / 32;  // 32-token MFMA B tiles
  constexpr int NDMA = BM / 32;    // DMA instructions per wave per half
  constexpr int HALF = BM * 128;   // one 64-k half of a stage
  constexpr int STAGE = 2 * HALF;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int n0 = blockIdx.x * 256, m0 = blockIdx.y * BM;
  const int s0 = blockIdx.z * steps_per;                  // even
  const int nd = min(K / 64 - s0, steps_per) / 2;         // >= 1 double steps
  const int kbase = s0 * 64;

  // weight rows of this lane (rows past N read row N - 1; not stored)
  const uint8_t* cp[2];
  const uint8_t* sp[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = min(n0 + 64 * wave + 32 * a + r32, N - 1);
    cp[a] = codes + (int64_t)row * (K / 2) + kbase / 2 + 16 * h;
    sp[a] = scales + (int64_t)row * (K / 16) + kbase / 16;
  }
  // activation pieces this lane copies, as in k_lmr (token rows past M read row M - 1)
  const uint16_t* xp[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int rho = 8 * (wave + 4 * i) + (lane >> 3);
    const int m = min(m0 + rho, M - 1);
    xp[i] = x + (int64_t)m * K + kbase + 8 * ((lane & 7) ^ ((rho >> 1) & 7));
  }

  struct WRegs {
    u32x4_t c[2][2];  // [row][half]: 32 codes of the lane's k quarter of the half
    u32x2_t s[2];     // [row]: the double step's 8 scale bytes
  };
  auto issue_w = [&](WRegs& W, int d) {
    d = min(d, nd - 1);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      load_b128_async<0>(W.c[a][0], cp[a] + 64 * d);
      load_b128_async<32>(W.c[a][1], cp[a] + 64 * d);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) load_b64_async<0>(W.s[a], sp[a] + 8 * d);
  };
  auto issue_x = [&](int d) {
    const int st = d & 1;
    d = min(d, nd - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < NDMA; ++i)
        copy16_to_lds(xp[i] + 128 * d + 64 * j, lds + st * STAGE + j * HALF + 1024 * (wave + 4 * i));
    asm volatile("" ::: "memory");
  };

  f32x16_t acc[2][MTILES];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < MTILES; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  WRegs W;
  issue_x(0);
  issue_w(W, 0);
  for (int d = 0; d < nd; ++d) {
    // every load of double step d has landed (this wave's), then the
    // barrier: every wave's copies have landed and every wave is done with
    // stage (d + 1) % 2
    asm volatile("s_waitcnt vmcnt(0)"
                 : "+v"(W.c[0][0]), "+v"(W.c[0][1]), "+v"(W.c[1][0]), "+v"(W.c[1][1]), "+v"(W.s[0]), "+v"(W.s[1])
                 :
                 : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint8_t* st = lds + (d & 1) * STAGE;
    issue_x(d + 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // the second half's dequantization stays after the first half's MFMAs
      // (hoisted, both halves' fragments would not fit two waves per SIMD)
      if (j == 1) __builtin_amdgcn_sched_barrier(0);
      bf16x8_t af[4][2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const uint32_t w = W.s[a][j] >> (16 * h);
        const float sg0 = scale_at<IMPL, 0>(w), sg1 = scale_at<IMPL, 1>(w);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          af[ks][a] = __builtin_bit_cast(bf16x8_t, dequant8u<IMPL>(W.c[a][j][ks], ks < 2 ? sg0 : sg1));
      }
      if (j == 1) issue_w(W, d + 1);  // the weight registers are free again
      const uint8_t* sh = st + j * HALF;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int b = 0; b < MTILES; ++b) {
          const int rho = 32 * b + r32;
          const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(
              sh + 128 * rho + 16 * ((4 * h + ks) ^ ((rho >> 1) & 7)));
#pragma unroll
          for (int a = 0; a < 2; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][a], bv, acc[a][b], 0, 0, 0);
        }
      }
    }
  }
  wait_vm_all();  // the tail's clamped loads must land before the workgroup's LDS is released
  store_lmr<MTILES>(acc, tensor_scale, y, ws, M, N, n0, m0, wave, out_f32);
}

template <int BM, int IMPL>
hipError_t launch_lmr(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                      KScale ts, void* y, float* ws, int M, int N, int K, int splits,
                      int steps_per, int out_f32, hipStream_t stream) {
  constexpr size_t lds = 2 * (size_t)BM * 128;
  hipError_t e = set_lds_limit<k_lmr<BM, IMPL>>(lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)((M + BM - 1) / BM), (unsigned)splits);
  hipLaunchKernelGGL((k_lmr<BM, IMPL>), grid, dim3(256), lds, stream, x, codes, scales, ts, y, ws,
                     M, N, K, steps_per, out_f32);
  e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return split_reduce(ws, ts, y, (int64_t)M * N, N, splits, out_f32, stream);
}

template <int BM, int IMPL>
hipError_t launch_lmr2(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                       KScale ts, void* y, float* ws, int M, int N, int K, int splits,
                       int steps_per, int out_f32, hipStream_t stream) {
  constexpr size_t lds = 4 * (size_t)BM * 128;
  hipError_t e = set_lds_limit<k_lmr2<BM, IMPL>>(lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)((M + BM - 1) / BM), (unsigned)splits);
  hipLaunchKernelGGL((k_lmr2<BM, IMPL>), grid, dim3(256), lds, stream, x, codes, scales, ts, y, ws,
                     M, N, K, steps_per, out_f32);
  e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return split_reduce(ws, ts, y, (int64_t)M * N, N, splits, out_f32, stream);
}

template <int BN, int BM, int WGN, int WGM, int IMPL>
hipError_t launch_lm(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                     KScale ts, void* y, float* ws, int M, int N, int K, int splits,
                     int steps_per, int out_f32, hipStream_t stream) {
  constexpr size_t lds = 2 * (4 * (BN / 32) * 1024 + 4 * (BM / 32) * 1024);
  hipError_t e = set_lds_limit<k_lm<BN, BM, WGN, WGM, IMPL>>(lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)splits);
  hipLaunchKernelGGL((k_lm<BN, BM, WGN, WGM, IMPL>), grid, dim3(64 * WGN * WGM), lds, stream, x,
                     codes, scales, ts, y, ws, M, N, K, steps_per, out_f32);
  e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return split_reduce(ws, ts, y, (int64_t)M * N, N, splits, out_f32, stream);
}

template <int IMPL>
hipError_t launch_lm_plan(const TiledPlan& p, const uint16_t* x, const uint8_t* codes,
                          const uint8_t* scales, KScale ts, void* y, float* ws, int M, int N,
                          int K, int out_f32, hipStream_t stream) {
  switch (p.kernel) {
    case 3:
      return launch_lm<128, 64, 2, 2, IMPL>(x, codes, scales, ts, y, ws, M, N, K, p.splits,
                                            p.steps_per_split, out_f32, stream);
    case 4:
      return launch_lm<256, 64, 4, 1, IMPL>(x, codes, scales, ts, y, ws, M, N, K, p.splits,
                                            p.steps_per_split, out_f32, stream);
    case 5:
      return launch_lmr<128, IMPL>(x, codes, scales, ts, y, ws, M, N, K, p.splits,
                                   p.steps_per_split, out_f32, stream);
    case 6:
      return launch_lmr2<128, IMPL>(x, codes, scales, ts, y, ws, M, N, K, p.splits,
                                    p.steps_per_split, out_f32, stream);
    default:
      return launch_lm<128, 128, 2, 2, IMPL>(x, codes, scales, ts, y, ws, M, N, K, p.splits,
                                             p.steps_per_split, out_f32, stream);
  }
}

}  // namespace

TiledPlan plan_tiled(int64_t m, int64_t n, int64_t k, int forced_splits) {
  TiledPlan p{0, 1, 0, 0};
  if (k < 64 || k % 64 != 0) return p;  // single-stage kernel, no split
  const int64_t nsteps = k / 64;
  const int64_t cap = nsteps / 4 > 0 ? nsteps / 4 : 1;  // >= 4 steps per split
  int64_t splits = 1;
  if (m <= 64) {
    // one 64-token tile: 128 weight rows per workgroup for long K, else
    // 256; K split to about 450 workgroups
    p.kernel = nsteps >= 128 ? 3 : 4;
    const int64_t bn = p.kernel == 3 ? 128 : 256;
    const int64_t tiles = (n + bn - 1) / bn;
    splits = (448 + tiles / 2) / tiles;
  } else if (m > 128) {
    // k_lmr (weights in registers, 256 x 128 tiles, two waves per SIMD):
    // measured faster than the LDS-staged kernels from m = 256 on every
    // decoder shape (e.g. 4096 x 4096 x 4096: 142 us against 181 us; 4096 x
    // 14336 at m = 1024: 149 against 212 us), K split to about 256
    // workgroups with at least 16 steps of 64 per split; k_lmr2 (128 k per
    // barrier) where K allows it, 5-9 % faster on the decoder shapes
    p.kernel = k % 128 == 0 ? 6 : 5;
    const int64_t tiles = ((n + 255) / 256) * ((m + 127) / 128);
    splits = 256 / tiles;
    if (splits > nsteps / 16) splits = nsteps / 16;
  } else {
    // 64 < m <= 128: 128 x 128 tiles with K split to about 512 workgroups
    // (at least 8 steps of 64 per split: 4096 x 4096 at m = 96 takes 8
    // splits, 4096 x 14336 takes 16)
    p.kernel = 1;
    const int64_t tiles = ((n + 127) / 128) * ((m + 127) / 128);
    splits = 512 / tiles;
    if (splits > nsteps / 8) splits = nsteps / 8;
  }
  if (m > 64) {
    int64_t pow2 = 1;  // measured best counts are powers of two
    while (pow2 * 2 <= splits) pow2 *= 2;
    splits = pow2;
  }
  if (splits > cap) splits = cap;
  if (splits > 16) splits = 16;
  if (splits < 1) splits = 1;
  if (forced_splits > 0) splits = forced_splits;
  if (splits > nsteps) splits = nsteps;
  if (splits < 1) splits = 1;
  int64_t per = (nsteps + splits - 1) / splits;
  if (p.kernel == 6) per += per & 1;  // whole 128-k double steps per split
  p.steps_per_split = (int)per;
  p.splits = (int)((nsteps + per - 1) / per);  // no empty split
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  return p;
}

hipError_t launch_tiled(const void* x, const uint8_t* codes, const uint8_t* scales,
                        RowScale rs, void* y, int64_t m, int64_t n, int64_t k,
                        int out_f32, const TiledPlan& plan, void* workspace, int impl,
                        hipStream_t stream) {
  const KScale tensor_scale = kscale(rs);
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  float* ws = reinterpret_cast<float*>(workspace);
  const int M = (int)m, N = (int)n, K = (int)k;
  if (plan.kernel != 0) {
    return impl == kConvHw
               ? launch_lm_plan<kConvHw>(plan, xp, codes, scales, tensor_scale, y, ws, M, N, K, out_f32, stream)
               : launch_lm_plan<kConvPortable>(plan, xp, codes, scales, tensor_scale, y, ws, M, N, K, out_f32, stream);
  }
  const dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
  const bool k32 = (k % 32) == 0;
  if (impl == kConvHw) {
    if (k32) hipLaunchKernelGGL((k_tiled<kConvHw, true>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, M, N, K, out_f32);
    else hipLaunchKernelGGL((k_tiled<kConvHw, false>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, M, N, K, out_f32);
  } else {
    if (k32) hipLaunchKernelGGL((k_tiled<kConvPortable, true>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, M, N, K, out_f32);
    else hipLaunchKernelGGL((k_tiled<kConvPortable, false>), grid, dim3(256), 0, stream, xp, codes, scales, tensor_scale, y, M, N, K, out_f32);
  }
  return hipGetLastError();
}

NVFP4_VARIANT_END
}  // namespace nvfp4
