// Input-gradient GEMM of an NVFP4 linear layer on gfx950: dx = dy @ W_hat.
//
// "SOAR 2026 Recap: From Compute Limits to the Open-Source Ecosystem",
// section "3. EAGLE-3 speculative decoding and hybrid architecture
// adaptation", its "Draft training" part: quantization-aware training runs
// the forward GEMM on the FP4 weights and passes gradients straight through
// to the master weights.  The backward pass then needs dx = dy @ W_hat on the
// same packed weights (the weight gradient dy^T x has no FP4 operand).
//
// Here the reduction runs over the weight rows n and the output over the
// weight columns k, so a lane cannot read its MFMA operand straight from the
// row-major packed layout: each 64-row step of the weights is dequantized
// (hardware FP4 decode at unit scale, times sigma: exact in bf16) and stored
// transposed in LDS, [k][n], beside the step's dy tile, [m][n]; both are then
// read as v_mfma_f32_32x32x16_bf16 fragments (8 consecutive n per lane).
// A workgroup covers 128 dy rows x 128 weight columns with 4 waves of 64 x 64
// (2 x 2 MFMA tiles); two LDS stages: while step s's MFMAs read one stage,
// the same waves then fill the other with step s + 1 (already in registers)
// and issue step s + 2's global loads, one barrier per step.  When the tiles
// are few the reduction over n is split over workgroups (fp32 partials, then
// the split reduction).  fp32 accumulation; s_t applied once.
// Where n % 64 == 0 and k % 128 == 0, k_gemm_dx_tr replaces the transposed
// stores with transposing LDS reads and brings dy in by LDS DMA (below).
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {


constexpr int kTM = 128;        // dy rows per workgroup
constexpr int kTK = 128;        // weight columns (outputs) per workgroup
constexpr int kTN = 64;         // weight rows (reduction) per step
constexpr int kRow = kTN + 8;   // LDS row of 64 bf16 + 16 bytes of padding (bank spread, 16-byte aligned)

__device__ __forceinline__ uint32_t bf16_hi_exact(float f) { return __float_as_uint(f) >> 16; }

struct DxLoads {
  u32x4_t dy[4];     // this thread's 4 x 8 bf16 of dy
  uint2 code[2];     // 16 codes of weight rows 2p and 2p+1, one block
  uint32_t sc[2];    // their scale bytes
};

// Epilogue: a wave's 2 x 2 tiles of 32 x 32, rows mw .. +64, columns kw .. +64.
// D of a 32 x 32 tile: lane l, value v -> dy row 8 (v / 4) + 4 (l / 32) + v % 4,
// weight column l % 32.  With a split reduction: raw fp32 partials to plane
// z of the workspace (the reduction kernel applies s_t).
__device__ __forceinline__ void store_dx(const f32x16_t (&acc)[2][2], const float* tensor_scale, void* dx, float* ws,
                                         int M, int K, int mw, int kw, int out_f32) {
  const int lane = threadIdx.x & 63, r32 = lane & 31, h = lane >> 5;
  const bool partial = gridDim.z > 1;
  float* plane = ws + (int64_t)blockIdx.z * M * K;
  const float s_t = partial ? 1.0f : tensor_scale[0];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int k = kw + 32 * b + r32;
      if (k >= K) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mw + 32 * a + 8 * (v / 4) + 4 * h + (v % 4);
        if (m >= M) continue;
        const float o = acc[a][b][v] * s_t;
        const int64_t idx = (int64_t)m * K + k;
        if (partial)
          plane[idx] = o;
        else if (out_f32)
          reinterpret_cast<float*>(dx)[idx] = o;
        else
          reinterpret_cast<uint16_t*>(dx)[idx] = (uint16_t)bf16_rne_bits(o);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_gemm_dx(const uint16_t* __restrict__ dy,
                                                 const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ tensor_scale,
                                                 void* __restrict__ dx, float* __restrict__ ws,
                                                 int M, int N, int K, int steps_per, int out_f32) {
  // two stages of dy[m][n] and W_hat[n][k] stored as [k][n]
  __shared__ __attribute__((aligned(16))) uint16_t as2[2][kTM * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[2][kTK * kRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.x * kTK, m0 = blockIdx.y * kTM;
  // this workgroup's share of the reduction: steps [s_begin, s_end) of 64 rows
  const int s_begin = blockIdx.z * steps_per;
  const int s_end = min((N + kTN - 1) / kTN, s_begin + steps_per);

  // dy: thread -> tile row ar = tid / 2, n half ah = tid % 2 (4 pieces of 8)
  const int ar = tid >> 1, ah = tid & 1;
  const uint16_t* dyrow = dy + (int64_t)min(m0 + ar, M - 1) * N;  // rows past M: not stored
  const bool vec = (N & 7) == 0;  // rows of dy are 16-byte aligned
  // weights: thread -> row pair p = tid % 32 (rows 2p, 2p + 1), block kb = tid / 32
  const int wp = tid & 31, kb = tid >> 5;
  const int kcol = k0 + 16 * kb;  // first weight column of the block
  const bool kin = kcol < K;      // K % 16 == 0: a block is all in or all out

  auto load = [&](DxLoads& L, int s) {
    const int n0 = s * kTN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 32 * ah + 8 * i;
      if (vec && n + 8 <= N) {
        L.dy[i] = *reinterpret_cast<const u32x4_t*>(dyrow + n);
      } else {  // unaligned rows, or the ragged end of a row: zeros past N
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = n + 2 * e < N ? dyrow[n + 2 * e] : 0u;
          const uint32_t hi = n + 2 * e + 1 < N ? dyrow[n + 2 * e + 1] : 0u;
          w[e] = lo | (hi << 16);
        }
        L.dy[i] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int n = n0 + 2 * wp + r;
      if (kin && n < N) {  // rows past N and blocks past K contribute zero
        L.code[r] = *reinterpret_cast<const uint2*>(codes + (int64_t)n * (K / 2) + kcol / 2);
        L.sc[r] = scales[(int64_t)n * (K / 16) + kcol / 16];
      } else {
        L.code[r] = make_uint2(0u, 0u);
        L.sc[r] = 0u;
      }
    }
  };
  auto store = [&](const DxLoads& L, int st) {
    uint16_t* as = as2[st];
    uint16_t* bs = bs2[st];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(&as[ar * kRow + 32 * ah + 8 * i]) = L.dy[i];
    // rows 2p and 2p + 1 of one block: 16 columns, each a bf16 pair (n, n + 1)
    float v0[16], v1[16];
    const float s0 = e4m3_decode(L.sc[0] & 0x7Fu), s1 = e4m3_decode(L.sc[1] & 0x7Fu);
    dequant8_f32<kConvHw>(L.code[0].x, s0, v0);
    dequant8_f32<kConvHw>(L.code[0].y, s0, v0 + 8);
    dequant8_f32<kConvHw>(L.code[1].x, s1, v1);
    dequant8_f32<kConvHw>(L.code[1].y, s1, v1 + 8);
#pragma unroll
    for (int c = 0; c < 16; ++c)
      *reinterpret_cast<uint32_t*>(&bs[(16 * kb + c) * kRow + 2 * wp]) =
          bf16_hi_exact(v0[c]) | (bf16_hi_exact(v1[c]) << 16);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // wave tile: dy rows 64 (wave / 2) .. +64, weight columns 64 (wave % 2) .. +64
  const int wm = 64 * (wave >> 1), wk = 64 * (wave & 1);
  const int r32 = lane & 31, h = lane >> 5;
  DxLoads cur;
  if (s_begin < s_end) {
    load(cur, s_begin);
    store(cur, 0);
    if (s_begin + 1 < s_end) load(cur, s_begin + 1);
  }
  __syncthreads();
  for (int s = s_begin; s < s_end; ++s) {
    const int st = (s - s_begin) & 1;
    const uint16_t* as = as2[st];
    const uint16_t* bs = bs2[st];
#pragma unroll
    for (int ks = 0; ks < kTN / 16; ++ks) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const bf16x8_t*>(&as[(wm + 32 * a + r32) * kRow + 16 * ks + 8 * h]);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bf[b] = *reinterpret_cast<const bf16x8_t*>(&bs[(wk + 32 * b + r32) * kRow + 16 * ks + 8 * h]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    // step s + 1 into the other stage (last read in step s - 1, before the
    // barrier that ended it), then step s + 2's loads
    if (s + 1 < s_end) store(cur, st ^ 1);
    if (s + 2 < s_end) load(cur, s + 2);
    __syncthreads();
  }

  store_dx(acc, tensor_scale, dx, ws, M, K, m0 + wm, k0 + wk, out_f32);
}

// ---------------------------------------------------------------------------
// k_gemm_dx_tr (n % 64 == 0, k % 128 == 0): the same tiles, waves, MFMA order
// and split as k_gemm_dx, but the weights are stored in LDS in their own
// row-major order and transposed by the reads.  Per 64-row step:
//  * thread t dequantizes 32 consecutive columns of weight row t / 4
//    (16 bytes of codes, 2 scale bytes) and stores them as four 16-byte
//    pieces of an LDS row of 128 bf16 (+ 32 bytes of padding);
//  * the dy tile (128 rows x 64 n) arrives by LDS DMA in whole cache lines,
//    16-byte pieces XOR-swizzled by row as in the large-M forward kernel;
//  * a B fragment (8 consecutive n of one weight column per lane) is two
//    ds_read_b64_tr_b16: within each 16-lane group, lane i of the result
//    holds element i % 4 of the 4-element reads of lanes i / 4 + 4 j,
//    j = 0..3, so a lane that reads 4 columns of row 8h + j' gives its
//    neighbours the column values of 4 consecutive rows.
// Against k_gemm_dx: no VGPR round trip for dy, four 16-byte LDS stores
// per thread for the weights instead of sixteen 4-byte ones, and no
// repacking of column pairs.  Loads: dy one step ahead (two stages), weights
// two steps ahead in two register sets, inline asm with counted waits.
constexpr int kWRow = kTK + 16;                 // LDS row of 128 bf16 + 32 bytes
constexpr int kDyStage = kTM * kTN * 2;         // 16 KiB
constexpr int kWStage = kTN * kWRow * 2;        // 18 KiB
constexpr int kTrStage = kDyStage + kWStage;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256, 2) void k_gemm_dx_tr(const uint16_t* __restrict__ dy,
                                                    const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    const float* __restrict__ tensor_scale,
                                                    void* __restrict__ dx, float* __restrict__ ws,
                                                    int M, int N, int K, int steps_per, int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.x * kTK, m0 = blockIdx.y * kTM;
  const int s_begin = blockIdx.z * steps_per;
  const int nst = min(N / kTN - s_begin, steps_per);  // >= 1: n > 0 and the plan has no empty split
  // dy copies: instruction c of wave w takes dy rows 8 (w + 4 c) .. +8 (rows
  // past M read row M - 1, not stored), lane l the 16-byte piece
  // (l % 8) ^ ((row / 2) % 8) of row 8 (w + 4 c) + l / 8
  const uint16_t* dp[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int rho = 8 * (wave + 4 * c) + (lane >> 3);
    dp[c] = dy + (int64_t)min(m0 + rho, M - 1) * N + (int64_t)s_begin * kTN + 8 * ((lane & 7) ^ ((rho >> 1) & 7));
  }
  // weights: thread -> row wr of the step, columns 32 wq .. +32 of the tile
  const int wr = tid >> 2, wq = tid & 3;
  const uint8_t* cp = codes + (int64_t)(s_begin * kTN + wr) * (K / 2) + k0 / 2 + 16 * wq;
  const uint8_t* sp = scales + (int64_t)(s_begin * kTN + wr) * (K / 16) + k0 / 16 + 2 * wq;
  struct WRegs {
    u32x4_t c;   // 32 codes
    uint32_t s;  // 2 scale bytes
  };
  auto issue_w = [&](WRegs& R, int s) {
    s = min(s, nst - 1);  // past the last step: the last step again (not used)
    load_b128_async<0>(R.c, cp + (int64_t)s * kTN * (K / 2));
    load_u16_async<0>(R.s, sp + (int64_t)s * kTN * (K / 16));
  };
  auto issue_dy = [&](int s) {
    const int st = s & 1;
    s = min(s, nst - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) copy16_to_lds(dp[c] + (int64_t)s * kTN, lds + st * kTrStage + 1024 * (wave + 4 * c));
    asm volatile("" ::: "memory");
  };
  auto store_w = [&](const WRegs& R, int st) {
    uint16_t* wl = reinterpret_cast<uint16_t*>(lds + st * kTrStage + kDyStage);
    const float sg0 = scale_at<kConvHw, 0>(R.s), sg1 = scale_at<kConvHw, 1>(R.s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(wl + wr * kWRow + 32 * wq + 8 * i) = dequant8_bf16<kConvHw>(R.c[i], i < 2 ? sg0 : sg1);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // wave tile: dy rows 64 (wave / 2) .. +64, weight columns 64 (wave % 2) .. +64
  const int wm = 64 * (wave >> 1), wk = 64 * (wave & 1);
  const int r32 = lane & 31, h = lane >> 5;
  // transposing reads: lane i of group g (h = g / 2, column half g % 2) reads
  // 4 columns of row 8 h + i / 4 (+ 16 ks, + 4 for the second read)
  const int sl = lane & 15, grp = lane >> 4;
  const int trow = 8 * (grp >> 1) + (sl >> 2);
  const int tcol = wk + 16 * (grp & 1) + 4 * (sl & 3);

  // One step: wait until its weights (set R) and dy copies have landed (only
  // the next step's weights may be in flight), store the weights, barrier
  // (every wave's stores and copies are in LDS, every wave is done with the
  // other stage), issue step s + 1's copies and step s + 2's weights (into
  // R), multiply.
  auto step = [&](int s, WRegs& R) {
    asm volatile("s_waitcnt vmcnt(2)" : "+v"(R.c), "+v"(R.s) : : "memory");
    const int st = s & 1;
    store_w(R, st);
    __syncthreads();
    issue_dy(s + 1);
    issue_w(R, s + 2);
    const uint8_t* dyl = lds + st * kTrStage;
    const uint16_t* wl = reinterpret_cast<const uint16_t*>(lds + st * kTrStage + kDyStage);
#pragma unroll
    for (int ks = 0; ks < kTN / 16; ++ks) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int rho = wm + 32 * a + r32;
        af[a] = *reinterpret_cast<const bf16x8_t*>(dyl + 128 * rho + 16 * ((2 * ks + h) ^ ((rho >> 1) & 7)));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint16_t* p = wl + (16 * ks + trow) * kWRow + tcol + 32 * b;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p);
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p + 4 * kWRow));
        bf[b] = __builtin_bit_cast(bf16x8_t, v8i16_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  };

  WRegs R0, R1;
  issue_dy(0);
  issue_w(R0, 0);
  issue_w(R1, 1);
  for (int s = 0; s < nst; s += 2) {
    step(s, R0);
    if (s + 1 < nst) step(s + 1, R1);
  }
  wait_vm_all();  // the tail's clamped loads land before the workgroup's LDS is released
  store_dx(acc, tensor_scale, dx, ws, M, K, m0 + wm, k0 + wk, out_f32);
}

}  // namespace

DxPlan plan_gemm_dx(int64_t m, int64_t n, int64_t k) {
  DxPlan p{1, 0, 0};
  const int64_t steps = (n + kTN - 1) / kTN;
  const int64_t tiles = ((k + kTK - 1) / kTK) * ((m + kTM - 1) / kTM);
  int splits = 1;
  // split the reduction over workgroups until about 512 of them run, while
  // each keeps at least 4 steps of 64 weight rows
  while (tiles * splits * 2 <= 512 && steps / (splits * 2) >= 4) splits *= 2;
  p.steps_per = (int)((steps + splits - 1) / splits);
  p.splits = p.steps_per > 0 ? (int)((steps + p.steps_per - 1) / p.steps_per) : 1;
  if (p.splits < 1) p.splits = 1;
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)k * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemm_dx(const uint16_t* dy, const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, void* dx, int64_t m, int64_t n, int64_t k,
                          int out_f32, const DxPlan& p, void* workspace, hipStream_t stream) {
  const dim3 grid((unsigned)((k + kTK - 1) / kTK), (unsigned)((m + kTM - 1) / kTM), (unsigned)p.splits);
  float* ws = reinterpret_cast<float*>(workspace);
  if (n > 0 && n % kTN == 0 && k % kTK == 0) {  // n == 0 (zeros) stays with k_gemm_dx, which loads nothing then
    constexpr size_t lds = 2 * (size_t)kTrStage;
    hipError_t e = set_lds_limit<k_gemm_dx_tr>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gemm_dx_tr, grid, dim3(256), lds, stream, dy, codes, scales, tensor_scale, dx, ws, (int)m,
                       (int)n, (int)k, p.steps_per, out_f32);
  } else {
    hipLaunchKernelGGL(k_gemm_dx, grid, dim3(256), 0, stream, dy, codes, scales, tensor_scale, dx, ws,
                       (int)m, (int)n, (int)k, p.steps_per, out_f32);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_split_reduce(ws, RowScale::one(tensor_scale), dx, m * k, k, p.splits, out_f32, stream);
}

}  // namespace nvfp4
