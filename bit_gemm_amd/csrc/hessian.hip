// GPTQ's damped Hessian from calibration activations on gfx950:
//   H = 2 X^T X + damp * mean(diag(2 X^T X)) * I,   X bf16 [s, k], H fp32 [k, k].
// GPTQ (the published method of Frantar et al., 2022) weighs each column's
// rounding error by the inverse of this matrix; the pages run it inside the
// FourOverSix scales ("SOAR Weekly Champion Notes 07 ...", section "03 How we
// integrated it").
//
// Three launches:
//  * k_xt: X^T into the workspace, [k, sp] bf16 with sp = s rounded up to a
//    multiple of 32 (zero samples past s add nothing), through a padded LDS
//    tile, so that both operands of the product are contiguous along the
//    sample index, the MFMA's reduction axis.
//  * k_hessian: 128 x 128 tiles of H on or above the diagonal, one per
//    workgroup; 4 waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x16_bf16 tiles);
//    32 samples per step, the next step's 16-byte loads in registers while
//    the current one is multiplied out of LDS (two stages, one barrier per
//    step).  bf16 x bf16 products are exact in fp32; the sums are fp32 in a
//    fixed order.  Each tile is stored twice (H_ij and H_ji) off the
//    diagonal, with the factor 2 applied (exact).
//  * k_hessian_damp: one workgroup adds the diagonal in float64 in a fixed
//    order, lambda = fl32(damp * sum / k), and H_ii = fl32(H_ii + lambda).
#include "launchers.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kHT = 128;        // H tile
constexpr int kHS = 32;         // samples per step
constexpr int kHRow = kHS + 8;  // LDS row of one H row / column (bf16): 32 samples + 16-byte pad

__global__ __launch_bounds__(256) void k_xt(const uint16_t* __restrict__ x, int64_t S, int64_t K, int64_t Sp,
                                            uint16_t* __restrict__ xt) {
  __shared__ uint16_t tile[64][66];
  const int64_t c0 = (int64_t)blockIdx.x * 64, s0 = (int64_t)blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;  // r: sample, c: column (consecutive threads: consecutive columns)
    const int64_t s = s0 + r, col = c0 + c;
    tile[r][c] = (s < S && col < K) ? x[s * K + col] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i >> 6, r = i & 63;  // consecutive threads: consecutive samples of one column
    const int64_t s = s0 + r, col = c0 + c;
    if (col < K && s < Sp) xt[col * Sp + s] = tile[r][c];
  }
}

struct HLoads {
  u32x4_t a[2], b[2];  // two 16-byte pieces of the A rows and of the B rows
};

// Tile (I, J), I <= J, of the upper triangle in row order: b -> (I, J).
__device__ __forceinline__ void tile_of(int b, int T, int& I, int& J) {
  int i = 0, rest = b;
  while (rest >= T - i) {
    rest -= T - i;
    ++i;
  }
  I = i;
  J = i + rest;
}

__global__ __launch_bounds__(256) void k_hessian(const uint16_t* __restrict__ xt, int K, int64_t Sp, int T,
                                                 float* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) uint16_t as2[2][kHT * kHRow];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[2][kHT * kHRow];
  int I, J;
  tile_of(blockIdx.x, T, I, J);
  const int i0 = I * kHT, j0 = J * kHT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // loader: thread t -> rows t / 4 and t / 4 + 64 of the tile, 16 bytes at sample offset 8 (t % 4)
  const int lr = threadIdx.x >> 2, lq = threadIdx.x & 3;
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    arow[p] = xt + (int64_t)min(i0 + lr + 64 * p, K - 1) * Sp + 8 * lq;  // rows past k: not stored
    brow[p] = xt + (int64_t)min(j0 + lr + 64 * p, K - 1) * Sp + 8 * lq;
  }
  auto load = [&](HLoads& L, int64_t s) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      L.a[p] = *reinterpret_cast<const u32x4_t*>(arow[p] + s);
      L.b[p] = *reinterpret_cast<const u32x4_t*>(brow[p] + s);
    }
  };
  auto store = [&](const HLoads& L, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      *reinterpret_cast<u32x4_t*>(&as2[st][(lr + 64 * p) * kHRow + 8 * lq]) = L.a[p];
      *reinterpret_cast<u32x4_t*>(&bs2[st][(lr + 64 * p) * kHRow + 8 * lq]) = L.b[p];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // wave tile: H rows 64 (wave / 2) .. +64, columns 64 (wave % 2) .. +64
  const int wm = 64 * (wave >> 1), wn = 64 * (wave & 1);
  const int r32 = lane & 31, hh = lane >> 5;
  const int64_t steps = Sp / kHS;
  HLoads cur;
  if (steps > 0) {
    load(cur, 0);
    store(cur, 0);
    if (steps > 1) load(cur, kHS);
  }
  __syncthreads();
  for (int64_t s = 0; s < steps; ++s) {
    const int st = (int)(s & 1);
    const uint16_t* as = as2[st];
    const uint16_t* bs = bs2[st];
#pragma unroll
    for (int ks = 0; ks < kHS / 16; ++ks) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const bf16x8_t*>(&as[(wm + 32 * a + r32) * kHRow + 16 * ks + 8 * hh]);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bf[b] = *reinterpret_cast<const bf16x8_t*>(&bs[(wn + 32 * b + r32) * kHRow + 16 * ks + 8 * hh]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    // step s + 1 into the other stage (last read in step s - 1, before the
    // barrier that ended it), then step s + 2's loads
    if (s + 1 < steps) store(cur, st ^ 1);
    if (s + 2 < steps) load(cur, (s + 2) * kHS);
    __syncthreads();
  }

  // D of a 32 x 32 tile: lane l, value v -> row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = j0 + wn + 32 * b + r32;
      if (j >= K) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = i0 + wm + 32 * a + 8 * (v / 4) + 4 * hh + (v % 4);
        if (i >= K) continue;
        const float o = 2.0f * acc[a][b][v];
        h[(int64_t)i * K + j] = o;
        if (I != J) h[(int64_t)j * K + i] = o;
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_hessian_damp(float* __restrict__ h, int K, float damp) {
  __shared__ double part[256];
  double t = 0.0;
  for (int i = threadIdx.x; i < K; i += 256) t += (double)h[(int64_t)i * K + i];
  part[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float lambda = (float)((double)damp * (part[0] / (double)K));
  for (int i = threadIdx.x; i < K; i += 256) h[(int64_t)i * K + i] += lambda;
}

}  // namespace

size_t hessian_workspace_bytes(int64_t s, int64_t k) {
  const int64_t sp = (s + kHS - 1) / kHS * kHS;
  return (size_t)k * (size_t)sp * 2;
}

hipError_t launch_hessian(const uint16_t* x, int64_t s, int64_t k, float damp, float* h, void* workspace,
                          hipStream_t stream) {
  const int64_t sp = (s + kHS - 1) / kHS * kHS;
  uint16_t* xt = reinterpret_cast<uint16_t*>(workspace);
  if (sp > 0) {
    hipLaunchKernelGGL(k_xt, dim3((unsigned)((k + 63) / 64), (unsigned)((sp + 63) / 64)), dim3(256), 0, stream, x, s, k,
                       sp, xt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int T = (int)((k + kHT - 1) / kHT);
  hipLaunchKernelGGL(k_hessian, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, stream, xt, (int)k, sp, T, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hessian_damp, dim3(1), dim3(256), 0, stream, h, (int)k, damp);
  return hipGetLastError();
}

}  // namespace nvfp4
