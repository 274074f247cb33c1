// W4A16 GEMM for decode-sized token counts (m <= 64) on gfx950.
//
// y[m, n] = s_t * sum_k x[m, k] * (val(code[n, k]) * sigma[n, k/16]).
// The pages run a W4A16 kernel for small token counts ("SOAR 2026 Recap ...",
// section "1. Quantization and GEMM dispatch"); decode is bound by reading
// the weights from HBM ("SOAR Weekly Champion Notes 08 ...", section "01").
//
// Kernels:
//  * k_skinny_pk (4 < m <= 16, k % 512 == 0, k <= 4096): a persistent form
//    of the full-K layout below; a workgroup per CU walks its 16-row tiles
//    with the activations in LDS once and the next two tiles' weights in
//    flight.  No workspace, one launch.
//  * k_skinny_fx (16 < m <= 64, k <= 4096, at most 256 workgroups of one
//    to four 16-row tiles): a workgroup per group of tiles over the whole
//    K, each wave streaming its K slice and the activations of each step
//    through a private LDS double buffer.  No workspace, one launch.
//  * k_skinny_fk (2 < m <= 16, except 8 < m <= 16 on large matrices: more
//    than 4096 rows or 2^25 weights, K % 512 == 0, and 4 < m <= 8 there
//    with K > 4096, which take the streaming kernel below): a workgroup owns 16 weight rows over the whole K and its
//    waves split K; no workspace, one launch.  Loads of a group of K steps
//    are in flight together and the next group is prefetched while the
//    current one is consumed.
//  * k_skinny_dot (m <= 2): the same layout with VALU dot products.
//  * k_skinny_str + k_reduce (K % 512 == 0: 16 < m <= 64, and 4 < m <= 16
//    on large matrices): one x chunk of 1024 (or 512) staged per workgroup,
//    then hundreds of weight rows streamed through it 16 at a time (x read
//    from L2 once per row group).  (A single launch in which the last
//    workgroup of a tile adds the partials was measured slower here: the
//    device-coherent stores and loads it needs cost more than the second
//    launch.)
//  * k_skinny_pipe + k_reduce (a split count forced by the caller, K % 128
//    == 0): 64 rows x one K chunk of 4 to 16 steps of 128 per workgroup, x
//    staged in LDS by DMA (shared by the 4 waves), fp32 partials in the
//    workspace, then a second kernel adds them in chunk order; k_skinny
//    (16 < m <= 64 with K % 512 != 0, and forced splits the pipelined
//    kernel cannot take) the same without the step pipelining.
// In both, val * sigma (<= 6 significant bits) is exact in bf16, products are
// accumulated in fp32 by v_mfma_f32_16x16x32_bf16 (weights = A operand, 16
// rows; tokens = B operand), and s_t is applied once to the fp32 sum.
// Partial sums are always added in a fixed order: results are reproducible.
#include "launchers.h"
#include "nvfp4_device.h"

#include <type_traits>

namespace nvfp4 {
NVFP4_VARIANT_BEGIN
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWg = 16 * kWaves;
constexpr int kStepK = 128;     // K per step (4 MFMAs of K=32)
constexpr int kMaxSteps = 16;   // K steps per chunk held in registers
constexpr int kLdsBudget = 131072;
constexpr int kFxMaxTiles = 256;  // the single-launch 16 < m <= 64 kernel: at most one workgroup per CU

template <int IMPL>
__device__ __forceinline__ bf16x8_t dequant8(uint32_t d, float sigma) {
  return __builtin_bit_cast(bf16x8_t, dequant8_bf16<IMPL>(d, sigma));
}

__device__ __forceinline__ void store_out(void* y, int64_t idx, float v, int out_f32) {
  if (out_f32)
    reinterpret_cast<float*>(y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)bf16_rne_bits(v);
}

// Full-K kernel (default for m <= 16).  A workgroup of W <= 8 waves owns 16
// weight rows over the whole K.  K is cut into rounds of W * 512: in a round
// wave w covers [round + 512 w, +512), and inside that slice lane group g
// streams its own contiguous quarter (128 codes = 64 bytes of one row, plus
// the 8 scale bytes of those 8 blocks, one load).  The MFMA k order inside a
// wave is therefore (quarter, step, 8-code piece); the activations are
// staged in the same order: each wave copies x[0:m, slice] to its own LDS
// region with one 16-byte load per lane per token row and reads the B
// fragments from there.  Loads of round r+1 are issued before round r is
// consumed (two register buffers), and inside a round the issue order is
// scales, activations, codes (the asm barriers keep the compiler from
// merging or reordering them), so step s only waits for its own code load.
// The W partial sums are added in wave order through LDS: results do not
// depend on timing.
constexpr int kSpw = 4;                 // K steps per wave per round
constexpr int kWaveK = kSpw * kStepK;   // 512
constexpr int kQuarter = kWaveK / 4;    // 128 codes per lane group

template <int MR>
struct Round {
  u32x4_t cw[kSpw];   // codes: 4 x 16 bytes (32 codes each), raw loads
  uint32_t sw[2];     // 8 scale bytes: step s uses bytes 2s, 2s+1
  u32x4_t xv[MR];     // activation pieces of this lane (row m, 8 bf16), raw
  uint32_t ok;        // validity bits: codes 0-3 (+4-7 upper halves), x 8, scales 9
};

__device__ __forceinline__ void mem_barrier() {
  asm volatile("" ::: "memory");      // no merging of loads across this point
  __builtin_amdgcn_sched_barrier(0);  // no scheduling across it either
}

__device__ __forceinline__ u32x4_t zero_unless(bool keep, u32x4_t v) {
  return keep ? v : u32x4_t{0u, 0u, 0u, 0u};
}

// Loads of one round, branch free: every address is clamped into the
// buffers and validity is recorded in R.ok; data outside the buffers is
// replaced by zeros where it is used, not here, so that no load has to be
// waited for before the next one is issued.
template <int MR, bool K32, bool K128>
__device__ __forceinline__ void load_round(Round<MR>& R, const uint8_t* crow, const uint8_t* srow,
                                           bool row_ok, const uint16_t* x, int M, int K, int kw0,
                                           int kq0, int lane) {
  uint32_t ok = 0u;
  // 1. scales of this lane's quarter (needed by the first step)
  if constexpr (K128) {
    const uint2 t = *reinterpret_cast<const uint2*>(srow + min(kq0, K - 128) / 16);
    R.sw[0] = t.x;
    R.sw[1] = t.y;
    ok |= (row_ok && kq0 < K) ? (1u << 9) : 0u;
  } else {
    R.sw[0] = 0u;
    R.sw[1] = 0u;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int kb = kq0 + 16 * b;
      const uint32_t v = srow[min(kb, K - 16) / 16];
      R.sw[b >> 2] |= ((row_ok && kb < K) ? v : 0u) << (8 * (b & 3));
    }
    ok |= 1u << 9;
  }
  mem_barrier();
  // 2. activations: lane holds x[m][kw0 + 8 lane .. +8]
  {
    const int k = kw0 + 8 * lane;
    const int kc = min(k, K - 8);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int mc = min(m, M - 1);
      R.xv[m] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)mc * K + kc);
    }
    ok |= (k < K) ? (1u << 8) : 0u;
  }
  mem_barrier();
  // 3. codes, one 16-byte load per step, in step order
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    const int kk = kq0 + 32 * s;
    if constexpr (K32) {
      R.cw[s] = *reinterpret_cast<const u32x4_t*>(crow + min(kk, K - 32) / 2);
      ok |= (row_ok && kk < K) ? (0x11u << s) : 0u;
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(crow + min(kk, K - 16) / 2);
      const uint2 b = *reinterpret_cast<const uint2*>(crow + min(kk + 16, K - 16) / 2);
      R.cw[s] = u32x4_t{a.x, a.y, b.x, b.y};
      ok |= (row_ok && kk < K) ? (1u << s) : 0u;
      ok |= (row_ok && kk + 16 < K) ? (0x10u << s) : 0u;
    }
    mem_barrier();
  }
  R.ok = ok;
}

template <int MR, int IMPL>
__device__ __forceinline__ void compute_round(const Round<MR>& R, uint16_t* xs, int M, int g,
                                              int r16, int lane, f32x4_t& acc) {
  // stage this round's activations (row stride kWaveK + 8 bf16: 16-byte pad)
  const bool xok = (R.ok >> 8) & 1u;
#pragma unroll
  for (int m = 0; m < MR; ++m)
    *reinterpret_cast<u32x4_t*>(xs + m * (kWaveK + 8) + 8 * lane) = zero_unless(xok && m < M, R.xv[m]);
  const bool sok = (R.ok >> 9) & 1u;
  const int rb = min(r16, MR - 1);
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    const uint32_t s2 = sok ? (R.sw[s >> 1] >> (16 * (s & 1))) & 0xFFFFu : 0u;
    const float sg0 = scale_at<IMPL, 0>(s2), sg1 = scale_at<IMPL, 1>(s2);
    const bool lo = (R.ok >> s) & 1u, hi = (R.ok >> (4 + s)) & 1u;
    bf16x8_t a[4];
    a[0] = dequant8<IMPL>(lo ? R.cw[s][0] : 0u, sg0);
    a[1] = dequant8<IMPL>(lo ? R.cw[s][1] : 0u, sg0);
    a[2] = dequant8<IMPL>(hi ? R.cw[s][2] : 0u, sg1);
    a[3] = dequant8<IMPL>(hi ? R.cw[s][3] : 0u, sg1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t b = zero_unless(
          r16 < M, *reinterpret_cast<const u32x4_t*>(xs + rb * (kWaveK + 8) + g * kQuarter + 32 * s + 8 * j));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
  }
}

// MR = token rows staged per wave (M <= MR <= 16).  ONE: K fits in one
// round (no second register buffer: fewer VGPRs, more workgroups per CU).
template <int MR, int IMPL, bool K32, bool K128, bool ONE>
__global__ __launch_bounds__(512) void k_skinny_fk(const uint16_t* __restrict__ x,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   const KScale tensor_scale,
                                                   void* __restrict__ y, int M, int N, int K,
                                                   int rounds, int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  // LDS: [W][64] f32x4 partial sums, then [W][MR][kWaveK + 8] bf16 activations
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + nwaves * 64 * sizeof(f32x4_t)) +
                 wave * MR * (kWaveK + 8);

  const int row = blockIdx.x * 16 + r16;
  const bool row_ok = row < N;
  const int rowc = min(row, N - 1);
  const uint8_t* crow = codes + (int64_t)rowc * (K / 2);
  const uint8_t* srow = scales + (int64_t)rowc * (K / 16);
  const int round_k = nwaves * kWaveK;
  const int kw = wave * kWaveK;

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (ONE) {
    Round<MR> RA;
    load_round<MR, K32, K128>(RA, crow, srow, row_ok, x, M, K, kw, kw + g * kQuarter, lane);
    compute_round<MR, IMPL>(RA, xs, M, g, r16, lane, acc);
  } else {
    Round<MR> RA, RB;
    load_round<MR, K32, K128>(RA, crow, srow, row_ok, x, M, K, kw, kw + g * kQuarter, lane);
    for (int r = 0; r < rounds; r += 2) {
      const int k1 = (r + 1) * round_k + kw;
      if (r + 1 < rounds) load_round<MR, K32, K128>(RB, crow, srow, row_ok, x, M, K, k1, k1 + g * kQuarter, lane);
      compute_round<MR, IMPL>(RA, xs, M, g, r16, lane, acc);
      if (r + 1 >= rounds) break;
      const int k2 = (r + 2) * round_k + kw;
      if (r + 2 < rounds) load_round<MR, K32, K128>(RA, crow, srow, row_ok, x, M, K, k2, k2 + g * kQuarter, lane);
      compute_round<MR, IMPL>(RB, xs, M, g, r16, lane, acc);
    }
  }

  // cross-wave sum in wave order; lane holds D[n = 4g + i][m = r16]
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  const float s_t = first_scale(tensor_scale);
  f32x4_t t = red[lane];
  for (int w = 1; w < nwaves; ++w) {
    const f32x4_t u = red[w * 64 + lane];
    t[0] += u[0];
    t[1] += u[1];
    t[2] += u[2];
    t[3] += u[3];
  }
  if (r16 >= M) return;
  const int nbase = blockIdx.x * 16 + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (nbase + i < N) store_out(y, (int64_t)r16 * N + nbase + i, t[i] * col_scale(tensor_scale, nbase + i, s_t), out_f32);
}

// Full-K kernel for one or two tokens: VALU dot products instead of MFMAs
// (an MFMA would use 1/16 or 2/16 of its B columns here).  Same workgroup
// layout, loads and rounds as k_skinny_fk.  Each byte of codes becomes a
// bf16 pair (exact E2M1 values; unit-scale hardware decode, or the portable
// decode), v_dot2_f32_bf16 accumulates the products of one 16-weight block
// in fp32, and the block sum is scaled by sigma once.  The four lane groups
// of a row are added with two xor shuffles, the waves in wave order.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <int IMPL, int B>
__device__ __forceinline__ bf16x2_t decode_pair_at(uint32_t d) {
  if constexpr (IMPL == kConvHw) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, B);
  } else {
    const uint32_t lo = __float_as_uint(e2m1_val_portable((d >> (8 * B)) & 0xFu));
    const uint32_t hi = __float_as_uint(e2m1_val_portable((d >> (8 * B + 4)) & 0xFu));
    return __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(hi, lo, 0x07060302u));
  }
}

// sum over the 8 codes of dword d (k = 8 consecutive) times the 8 bf16 of xq.
// (Each element is copied to a scalar before the bit cast: clang's
// __builtin_bit_cast of a vector-element expression reads element 0.)
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

template <int IMPL>
__device__ __forceinline__ float dot8(uint32_t d, u32x4_t xq, float acc) {
  const uint32_t q0 = xq[0], q1 = xq[1], q2 = xq[2], q3 = xq[3];
  acc = __builtin_amdgcn_fdot2_f32_bf16(decode_pair_at<IMPL, 0>(d), as_bf16x2(q0), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(decode_pair_at<IMPL, 1>(d), as_bf16x2(q1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(decode_pair_at<IMPL, 2>(d), as_bf16x2(q2), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(decode_pair_at<IMPL, 3>(d), as_bf16x2(q3), acc, false);
  return acc;
}

template <int MR, int IMPL>
__device__ __forceinline__ void compute_round_dot(const Round<MR>& R, uint16_t* xs, int M, int g,
                                                  int lane, float (&acc)[MR]) {
  const bool xok = (R.ok >> 8) & 1u;
#pragma unroll
  for (int m = 0; m < MR; ++m)
    *reinterpret_cast<u32x4_t*>(xs + m * (kWaveK + 8) + 8 * lane) = zero_unless(xok && m < M, R.xv[m]);
  const bool sok = (R.ok >> 9) & 1u;
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    const uint32_t s2 = sok ? (R.sw[s >> 1] >> (16 * (s & 1))) & 0xFFFFu : 0u;
    const float sg0 = scale_at<IMPL, 0>(s2), sg1 = scale_at<IMPL, 1>(s2);
    const bool lo = (R.ok >> s) & 1u, hi = (R.ok >> (4 + s)) & 1u;
    const uint32_t d0 = lo ? R.cw[s][0] : 0u, d1 = lo ? R.cw[s][1] : 0u;
    const uint32_t d2 = hi ? R.cw[s][2] : 0u, d3 = hi ? R.cw[s][3] : 0u;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint16_t* xb = xs + m * (kWaveK + 8) + g * kQuarter + 32 * s;
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xb);
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(xb + 8);
      const u32x4_t x2 = *reinterpret_cast<const u32x4_t*>(xb + 16);
      const u32x4_t x3 = *reinterpret_cast<const u32x4_t*>(xb + 24);
      const float b0 = dot8<IMPL>(d1, x1, dot8<IMPL>(d0, x0, 0.0f));  // block 2s of the quarter
      const float b1 = dot8<IMPL>(d3, x3, dot8<IMPL>(d2, x2, 0.0f));  // block 2s + 1
      acc[m] += sg0 * b0;
      acc[m] += sg1 * b1;
    }
  }
}

// ONE: K fits in one round (no second register buffer: fewer VGPRs, more
// workgroups per CU).
template <int MR, int IMPL, bool K32, bool K128, bool ONE>
__global__ __launch_bounds__(512) void k_skinny_dot(const uint16_t* __restrict__ x,
                                                    const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    const KScale tensor_scale,
                                                    void* __restrict__ y, int M, int N, int K,
                                                    int rounds, int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  // LDS: [W][MR][16] f32 partial sums, then [W][MR][kWaveK + 8] bf16 activations
  float* red = reinterpret_cast<float*>(lds);
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + nwaves * 64 * sizeof(f32x4_t)) +
                 wave * MR * (kWaveK + 8);

  const int row = blockIdx.x * 16 + r16;
  const bool row_ok = row < N;
  const int rowc = min(row, N - 1);
  const uint8_t* crow = codes + (int64_t)rowc * (K / 2);
  const uint8_t* srow = scales + (int64_t)rowc * (K / 16);
  const int round_k = nwaves * kWaveK;
  const int kw = wave * kWaveK;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  if constexpr (ONE) {
    Round<MR> RA;
    load_round<MR, K32, K128>(RA, crow, srow, row_ok, x, M, K, kw, kw + g * kQuarter, lane);
    compute_round_dot<MR, IMPL>(RA, xs, M, g, lane, acc);
  } else {
    Round<MR> RA, RB;
    load_round<MR, K32, K128>(RA, crow, srow, row_ok, x, M, K, kw, kw + g * kQuarter, lane);
    for (int r = 0; r < rounds; r += 2) {
      const int k1 = (r + 1) * round_k + kw;
      if (r + 1 < rounds) load_round<MR, K32, K128>(RB, crow, srow, row_ok, x, M, K, k1, k1 + g * kQuarter, lane);
      compute_round_dot<MR, IMPL>(RA, xs, M, g, lane, acc);
      if (r + 1 >= rounds) break;
      const int k2 = (r + 2) * round_k + kw;
      if (r + 2 < rounds) load_round<MR, K32, K128>(RA, crow, srow, row_ok, x, M, K, k2, k2 + g * kQuarter, lane);
      compute_round_dot<MR, IMPL>(RB, xs, M, g, lane, acc);
    }
  }
  // lane groups g = 0..3 of a row: ((g0 + g1) + (g2 + g3)) in every lane
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    acc[m] += __shfl_xor(acc[m], 16, 64);
    acc[m] += __shfl_xor(acc[m], 32, 64);
  }
  if (g == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) red[(wave * MR + m) * 16 + r16] = acc[m];
  }
  __syncthreads();
  if (wave != 0 || g != 0 || !row_ok) return;
  const float s_t = first_scale(tensor_scale);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) continue;
    float t = red[m * 16 + r16];
    for (int w = 1; w < nwaves; ++w) t += red[(w * MR + m) * 16 + r16];
    store_out(y, (int64_t)m * N + row, t * col_scale(tensor_scale, row, s_t), out_f32);
  }
}

// Row-per-wave dot-product kernel for one token, k = 2048 NCH (it takes NCH
// <= 2; longer rows and partial chunks take the LDS DMA form below):
// each wave owns two whole weight rows and its 64 lanes run along K, so a
// code load instruction reads 1 KiB of one row (lane l: bytes 1024 c + 16 l
// of chunk c, codes k = 2048 c + 32 l .. +32) and a scale load 128
// contiguous bytes; every row of the workgroup's 8 (4 waves) reads the
// token's activations from LDS, staged once per workgroup (the
// copies are issued before the weight loads, so they land first and the
// multiplies of chunk 0 can start while the later chunks stream in).  Per
// chunk and row a lane forms the two 16-code block sums with v_dot2 on the
// unit-scale decode, scales each by its sigma, and the 64 lane sums of a
// row are added with xor shuffles in a fixed order.  Against the full-K dot
// kernel (rows across lanes, K slices across waves, a cross-wave sum in
// LDS), measured at m = 1 with the first version of this kernel, which then
// served every k = 2048 c up to 16384 (per call, 32 back-to-back calls on
// rotating copies): 4096 x 4096 4.25 against 4.52 us, 14336 x 4096 7.9
// against 8.6, 12288 x 4096 7.2 against 8.8, 28672 x 4096 13.1-14.1
// against 16.2, 4096 x 14336 9.3 against 10.9 us.  Eight rows per
// workgroup measured best over 4 / 8 / 16 waves of 1, 2 or 4 rows (16 rows:
// 4096 x 14336 10.2 us, 4096 x 4096 4.5 us).
constexpr int kRdWaves = 4, kRdRows = 2;  // waves per workgroup, rows per wave
template <int NCH>
__global__ __launch_bounds__(64 * kRdWaves) void k_skinny_rdot(const uint16_t* __restrict__ x,
                                                             const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             const KScale tensor_scale,
                                                             void* __restrict__ y, int N, int out_f32) {
  constexpr int K = 2048 * NCH;
  constexpr int XPT = K / 8 / (64 * kRdWaves);  // 16-byte pieces of x per thread
  static_assert(XPT * 8 * 64 * kRdWaves == K, "every thread copies the same number of x pieces");
  __shared__ __attribute__((aligned(16))) uint16_t xs[K];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * kRdWaves + wave) * kRdRows;
  // Every piece is in range, so no load is conditional: a guarded load would
  // make the compiler wait for the activations before issuing any weight load.
  u32x4_t xv[XPT];
#pragma unroll
  for (int t = 0; t < XPT; ++t) xv[t] = *reinterpret_cast<const u32x4_t*>(x + 8 * (threadIdx.x + 64 * kRdWaves * t));
  const uint8_t* crow[kRdRows];
  const uint8_t* srow[kRdRows];
#pragma unroll
  for (int j = 0; j < kRdRows; ++j) {
    const int row = min(row0 + j, N - 1);  // rows past N read row N - 1, not stored
    crow[j] = codes + (int64_t)row * (K / 2);
    srow[j] = scales + (int64_t)row * (K / 16);
  }
  // chunk-major: chunk c of every row lands before chunk c + 1, so the dot
  // products below start while later chunks are still in flight
  u32x4_t cw[kRdRows][NCH];
  uint32_t sw[kRdRows][NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int j = 0; j < kRdRows; ++j) {
      cw[j][c] = *reinterpret_cast<const u32x4_t*>(crow[j] + 1024 * c + 16 * lane);
      sw[j][c] = *reinterpret_cast<const uint16_t*>(srow[j] + 128 * c + 2 * lane);
    }
  }
#pragma unroll
  for (int t = 0; t < XPT; ++t) *reinterpret_cast<u32x4_t*>(xs + 8 * (threadIdx.x + 64 * kRdWaves * t)) = xv[t];
  __syncthreads();
  float acc[kRdRows] = {};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    u32x4_t xq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xq[q] = *reinterpret_cast<const u32x4_t*>(xs + 2048 * c + 32 * lane + 8 * q);
#pragma unroll
    for (int j = 0; j < kRdRows; ++j) {
      const uint32_t s2 = sw[j][c];
      const float sg0 = scale_at<kConvHw, 0>(s2), sg1 = scale_at<kConvHw, 1>(s2);
      const float b0 = dot8<kConvHw>(cw[j][c][1], xq[1], dot8<kConvHw>(cw[j][c][0], xq[0], 0.0f));
      const float b1 = dot8<kConvHw>(cw[j][c][3], xq[3], dot8<kConvHw>(cw[j][c][2], xq[2], 0.0f));
      acc[j] += sg0 * b0;
      acc[j] += sg1 * b1;
    }
  }
  const float s_t = first_scale(tensor_scale);
#pragma unroll
  for (int j = 0; j < kRdRows; ++j) {
    float v = acc[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int row = row0 + j;
    if (lane == 0 && row < N) store_out(y, row, v * col_scale(tensor_scale, row, s_t), out_f32);
  }
}

// The same dot products with the activations copied into LDS by the LDS
// DMA, issued before the weight loads, and k = 2048 (NCH - 1) + kl for any
// 0 < kl <= 2048 with kl % 32 == 0 and NCH <= 16 (64 KiB of activations): in a partial last chunk only lanes
// < kl / 32 hold codes; the others load piece 0 of that chunk (a valid
// address) and their sums are discarded by a select (the activations they
// read from LDS past k are never written).  The weight loads are inline asm
// in chunk order, so one counted wait (only the weight loads may stay
// outstanding) and a bare barrier make every wave's copies visible, and
// chunk c waits only for its own loads (the compiler's own wait for the
// copies would be vmcnt(0), i.e. for every weight load too).  RW rows per
// wave: one for long rows (16 rows per workgroup halve the x copies per
// weight byte but leave too few waves to overlap the chunks' sums with the
// loads), two for a partial second chunk on tall matrices.  Measured at m = 1
// (per call, 32 calls on rotating copies), whole chunks against the two-row
// kernel above: 4096 x 8192 5.66 against 5.89 us, 4096 x 12288 7.45 against
// 7.87, 4096 x 14336 8.45 against 8.70, 4096 x 16384 9.08 against 9.98,
// 11008 x 6144 8.92 against 9.26; 4096 x 6144 even (4.89 / 4.88); at
// NCH <= 2 slower (14336 x 4096 8.89 against 7.61 us), so whole chunks
// there keep the two-row kernel.  k not a multiple of 2048, against the
// full-K dot kernel that took them before: 5120 x 13824 9.2 against 16.0 us,
// 13824 x 5120 9.3 against 14.5, 4096 x 11008 7.1 against 9.1, 18944 x 3584
// 8.9 (two rows per wave; one row 9.5) against 11.1, 1003 x 2816 2.6
// against 3.4, 3584 x 3584 3.84 against 3.90 us; rows of 9-16 chunks:
// 8192 x 28672 28.1 against 30.7 us, 4096 x 22016 12.2 against 16.3,
// 1024 x 32768 6.8 against 15.2 us.
template <int NCH, int RW, int C>
__device__ __forceinline__ void rdot_dma_chunk(u32x4_t (&cw)[RW][NCH], uint32_t (&sw)[RW][NCH], const uint16_t* xs,
                                               int lane, bool on_last, float (&acc)[RW]) {
#pragma unroll
  for (int j = 0; j < RW; ++j) wait_vm<2 * RW * (NCH - 1 - C)>(cw[j][C], sw[j][C]);
  u32x4_t xq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xq[q] = *reinterpret_cast<const u32x4_t*>(xs + 2048 * C + 32 * lane + 8 * q);
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    const uint32_t s2 = sw[j][C];
    const float sg0 = scale_at<kConvHw, 0>(s2), sg1 = scale_at<kConvHw, 1>(s2);
    const float b0 = dot8<kConvHw>(cw[j][C][1], xq[1], dot8<kConvHw>(cw[j][C][0], xq[0], 0.0f));
    const float b1 = dot8<kConvHw>(cw[j][C][3], xq[3], dot8<kConvHw>(cw[j][C][2], xq[2], 0.0f));
    if constexpr (C == NCH - 1) {
      acc[j] += on_last ? sg0 * b0 : 0.0f;
      acc[j] += on_last ? sg1 * b1 : 0.0f;
    } else {
      acc[j] += sg0 * b0;
      acc[j] += sg1 * b1;
    }
  }
  if constexpr (C + 1 < NCH) rdot_dma_chunk<NCH, RW, C + 1>(cw, sw, xs, lane, on_last, acc);
}

template <int NCH, int RW>
__global__ __launch_bounds__(64 * kRdWaves) void k_skinny_rdot_dma(const uint16_t* __restrict__ x,
                                                                 const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 const KScale tensor_scale,
                                                                 void* __restrict__ y, int N, int K, int out_f32) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2048 * NCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xp = K / 8;  // 16-byte pieces of x (a multiple of 4)
#pragma unroll
  for (int t = 0; t < NCH; ++t) {  // piece i = threadIdx.x + 256 t lands at byte 16 i of xs
    const int i = (int)threadIdx.x + 64 * kRdWaves * t;
    if (i < xp) copy16_to_lds(x + 8 * i, reinterpret_cast<uint8_t*>(xs) + 16 * (64 * kRdWaves * t + 64 * wave));
  }
  const bool on_last = lane < (K - 2048 * (NCH - 1)) / 32;  // this lane holds codes in the last chunk
  const int lane_last = on_last ? lane : 0;
  const int row0 = (blockIdx.x * kRdWaves + wave) * RW;
  const uint8_t* crow[RW];
  const uint8_t* srow[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    const int rr = min(row0 + j, N - 1);  // a row past N reads row N - 1, not stored
    crow[j] = codes + (int64_t)rr * (K / 2);
    srow[j] = scales + (int64_t)rr * (K / 16);
  }
  u32x4_t cw[RW][NCH];
  uint32_t sw[RW][NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int l = c == NCH - 1 ? lane_last : lane;
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      load_b128_async<0>(cw[j][c], crow[j] + 1024 * c + 16 * l);
      load_u16_async<0>(sw[j][c], srow[j] + 128 * c + 2 * l);
    }
  }
  wait_vm_count<2 * RW * NCH>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS read moves above the barrier
  float acc[RW] = {};
  rdot_dma_chunk<NCH, RW, 0>(cw, sw, xs, lane, on_last, acc);
  const float s_t = first_scale(tensor_scale);
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    float v = acc[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int row = row0 + j;
    if (lane == 0 && row < N) store_out(y, row, v * col_scale(tensor_scale, row, s_t), out_f32);
  }
}

template <int NCH>
hipError_t launch_rdot_n(hipStream_t stream, const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                         KScale ts, void* y, int N, int K, int out_f32) {
  if constexpr (NCH == 1) {  // k = 2048 (the planner takes k >= 2048)
    const dim3 grid((unsigned)((N + kRdWaves * kRdRows - 1) / (kRdWaves * kRdRows)));
    hipLaunchKernelGGL((k_skinny_rdot<1>), grid, dim3(64 * kRdWaves), 0, stream, x, codes, scales, ts, y, N, out_f32);
    return hipGetLastError();
  } else {
    if constexpr (NCH == 2) {
      if (K == 2048 * NCH) {  // whole chunks: the two-row kernel staging x through registers
        const dim3 grid((unsigned)((N + kRdWaves * kRdRows - 1) / (kRdWaves * kRdRows)));
        hipLaunchKernelGGL((k_skinny_rdot<NCH>), grid, dim3(64 * kRdWaves), 0, stream, x, codes, scales, ts, y, N,
                           out_f32);
        return hipGetLastError();
      }
      if (N > 8192) {  // a partial second chunk on a tall matrix: two rows per wave
        const dim3 grid((unsigned)((N + 2 * kRdWaves - 1) / (2 * kRdWaves)));
        hipLaunchKernelGGL((k_skinny_rdot_dma<NCH, 2>), grid, dim3(64 * kRdWaves), 0, stream, x, codes, scales, ts,
                           y, N, K, out_f32);
        return hipGetLastError();
      }
    }
    const dim3 grid((unsigned)((N + kRdWaves - 1) / kRdWaves));
    hipLaunchKernelGGL((k_skinny_rdot_dma<NCH, 1>), grid, dim3(64 * kRdWaves), 0, stream, x, codes, scales, ts, y, N,
                       K, out_f32);
    return hipGetLastError();
  }
}

hipError_t launch_rdot(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                       const uint8_t* scales, KScale ts, void* y, int N, int K, int out_f32) {
  switch (p.rdot_chunks) {
    case 1: return launch_rdot_n<1>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 2: return launch_rdot_n<2>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 3: return launch_rdot_n<3>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 4: return launch_rdot_n<4>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 5: return launch_rdot_n<5>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 6: return launch_rdot_n<6>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 7: return launch_rdot_n<7>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 8: return launch_rdot_n<8>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 9: return launch_rdot_n<9>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 10: return launch_rdot_n<10>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 11: return launch_rdot_n<11>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 12: return launch_rdot_n<12>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 13: return launch_rdot_n<13>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 14: return launch_rdot_n<14>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 15: return launch_rdot_n<15>(stream, x, codes, scales, ts, y, N, K, out_f32);
    case 16: return launch_rdot_n<16>(stream, x, codes, scales, ts, y, N, K, out_f32);
    default: return hipErrorInvalidValue;
  }
}

// Persistent full-K kernel (m <= 16, k = W * ROUNDS * 512 for W <= 8 waves
// and ROUNDS in {1, 2, 4}): the full-K layout above, but a workgroup walks
// several 16-row tiles (tiles blockIdx.x, + gridDim.x, ...) and keeps the
// activations in LDS for all of them.  Wave w owns the K slices r W + w
// (r < ROUNDS) of every tile; at the start it copies x[0:MR, its slices]
// into its own LDS region with the LDS DMA (one instruction per token row
// and slice: 512 contiguous bf16, whole cache lines; token rows >= m repeat
// row m - 1, whose outputs are not stored), so the activations cross L2 ->
// CU once per workgroup instead of once per tile.  (Requesting the first
// tile's weights before the copies measured slower: 4096 x 4096 at m = 8,
// 6.3 against 5.9 us.)  Per tile a lane loads, per slice, the 8
// scale bytes and four 16-byte code pieces of its quarter (the full-K
// kernel's layout); the next two tiles' loads are in flight while a tile is
// consumed, and step s waits only until its own loads have landed
// (inline-asm loads with counted waits; loads return in issue order).  The
// W partial tiles are added in wave order through LDS (two buffers by tile
// parity) after a bare barrier (a workgroup fence would also wait for the
// next tile's loads); one wave per tile, in turn, adds and stores.  MR <= 2
// uses VALU dot products, larger MR the 16x16x32 MFMA.
// VALU dot products for one or two tokens with the hardware FP4 decode; the
// portable decode's dot form needs more registers than the in-flight loads
// leave, so it takes the MFMA form (token rows >= m repeat row m - 1).
constexpr bool pk_dot_path(int mr, int impl) { return mr <= 2 && impl == kConvHw; }

template <int ROUNDS>
struct PkTile {
  u32x4_t cw[ROUNDS][kSpw];  // codes: slice r, step s (32 codes of row r16 at k = 128 g + 32 s)
  u32x2_t sw[ROUNDS];        // the 8 scale bytes of the lane's quarter of slice r
};

constexpr int kPkLoadsPerSlice = 1 + kSpw;  // scales, then the four code pieces
constexpr int kPkAhead = 2;                  // tiles whose loads are in flight while one is consumed
constexpr int kPkRow = kWaveK + 8;          // LDS row of one token and slice (bf16), 16-byte pad

template <int R, int ROUNDS>
__device__ __forceinline__ void pk_issue(PkTile<ROUNDS>& T, const uint8_t* const* cp, const uint8_t* const* sp) {
  load_b64_async<0>(T.sw[R], sp[R]);
  load_b128_async<0>(T.cw[R][0], cp[R]);
  load_b128_async<16>(T.cw[R][1], cp[R]);
  load_b128_async<32>(T.cw[R][2], cp[R]);
  load_b128_async<48>(T.cw[R][3], cp[R]);
  if constexpr (R + 1 < ROUNDS) pk_issue<R + 1, ROUNDS>(T, cp, sp);
}

// Slice R, step S of a tile (MFMA), then the following steps.  AFTER = loads
// issued after this tile's (the next tile's).
template <int R, int S, int MR, int IMPL, int ROUNDS, int AFTER>
__device__ __forceinline__ void pk_mfma(PkTile<ROUNDS>& T, const uint16_t* xw, int g, int rb, f32x4_t& acc) {
  wait_vm_b64<(kSpw - 1 - S) + kPkLoadsPerSlice * (ROUNDS - 1 - R) + AFTER>(T.cw[R][S], T.sw[R]);
  const uint32_t s2 = (T.sw[R][S >> 1] >> (16 * (S & 1))) & 0xFFFFu;
  const float sg0 = scale_at<IMPL, 0>(s2), sg1 = scale_at<IMPL, 1>(s2);
  bf16x8_t a[4];
  a[0] = dequant8<IMPL>(T.cw[R][S][0], sg0);
  a[1] = dequant8<IMPL>(T.cw[R][S][1], sg0);
  a[2] = dequant8<IMPL>(T.cw[R][S][2], sg1);
  a[3] = dequant8<IMPL>(T.cw[R][S][3], sg1);
  const uint16_t* xb = xw + (R * MR + rb) * kPkRow + g * kQuarter + 32 * S;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(xb + 8 * j);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  if constexpr (S + 1 < kSpw)
    pk_mfma<R, S + 1, MR, IMPL, ROUNDS, AFTER>(T, xw, g, rb, acc);
  else if constexpr (R + 1 < ROUNDS)
    pk_mfma<R + 1, 0, MR, IMPL, ROUNDS, AFTER>(T, xw, g, rb, acc);
}

// The same for the dot kernel: per token, the two 16-code blocks of the
// step summed in fp32 and scaled by their sigma.
template <int R, int S, int MR, int IMPL, int ROUNDS, int AFTER>
__device__ __forceinline__ void pk_dot(PkTile<ROUNDS>& T, const uint16_t* xw, int g, float (&acc)[MR]) {
  wait_vm_b64<(kSpw - 1 - S) + kPkLoadsPerSlice * (ROUNDS - 1 - R) + AFTER>(T.cw[R][S], T.sw[R]);
  const uint32_t s2 = (T.sw[R][S >> 1] >> (16 * (S & 1))) & 0xFFFFu;
  const float sg0 = scale_at<IMPL, 0>(s2), sg1 = scale_at<IMPL, 1>(s2);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const uint16_t* xb = xw + (R * MR + m) * kPkRow + g * kQuarter + 32 * S;
    const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xb);
    const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(xb + 8);
    const u32x4_t x2 = *reinterpret_cast<const u32x4_t*>(xb + 16);
    const u32x4_t x3 = *reinterpret_cast<const u32x4_t*>(xb + 24);
    const float b0 = dot8<IMPL>(T.cw[R][S][1], x1, dot8<IMPL>(T.cw[R][S][0], x0, 0.0f));
    const float b1 = dot8<IMPL>(T.cw[R][S][3], x3, dot8<IMPL>(T.cw[R][S][2], x2, 0.0f));
    acc[m] += sg0 * b0;
    acc[m] += sg1 * b1;
  }
  if constexpr (S + 1 < kSpw)
    pk_dot<R, S + 1, MR, IMPL, ROUNDS, AFTER>(T, xw, g, acc);
  else if constexpr (R + 1 < ROUNDS)
    pk_dot<R + 1, 0, MR, IMPL, ROUNDS, AFTER>(T, xw, g, acc);
}

template <int MR, int IMPL, int ROUNDS>
__global__ __launch_bounds__(512) void k_skinny_pk(const uint16_t* __restrict__ x,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   const KScale tensor_scale,
                                                   void* __restrict__ y, int M, int N, int K, int out_f32) {
  constexpr bool kDot = pk_dot_path(MR, IMPL);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  uint16_t* xw = reinterpret_cast<uint16_t*>(lds) + wave * (ROUNDS * MR * kPkRow);
  uint8_t* red = lds + (size_t)W * ROUNDS * MR * kPkRow * 2;  // [2][W] partial tiles
  const float s_t = first_scale(tensor_scale);

  // activations of this wave's slices, once (LDS DMA: lane l -> bf16 8l .. 8l + 7)
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m)
      copy16_to_lds(x + (int64_t)min(m, M - 1) * K + (r * W + wave) * kWaveK + 8 * lane,
                    reinterpret_cast<uint8_t*>(xw + (r * MR + m) * kPkRow));

  const int ntiles = (N + 15) / 16;
  const int cnt = (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;  // tiles of this workgroup
  int64_t slice_c[ROUNDS], slice_s[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    slice_c[r] = (int64_t)(r * W + wave) * (kWaveK / 2) + 16 * (kSpw * g);
    slice_s[r] = (int64_t)(r * W + wave) * (kWaveK / 16) + 8 * g;
  }
  // loads of this workgroup's tile i; past the last tile every lane reads
  // the first bytes of the buffers instead (in bounds, one cache line per
  // instruction, never used), so the count of loads in flight stays fixed
  auto issue = [&](PkTile<ROUNDS>& T, int i) __attribute__((always_inline)) {
    const bool real = i < cnt;
    const int t = (int)blockIdx.x + i * (int)gridDim.x;
    const int64_t row = real ? min(16 * t + r16, N - 1) : 0;
    const uint8_t* cp[ROUNDS];
    const uint8_t* sp[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      cp[r] = real ? codes + row * (K / 2) + slice_c[r] : codes;
      sp[r] = real ? scales + row * (K / 16) + slice_s[r] : scales;
    }
    pk_issue<0, ROUNDS>(T, cp, sp);
  };
  auto finish = [&](int i, auto& acc) __attribute__((always_inline)) {  // add the W partial tiles of tile i and store it
    const int par = i & 1;
    const int t = (int)blockIdx.x + i * (int)gridDim.x;
    if constexpr (kDot) {
      float* rf = reinterpret_cast<float*>(red) + (size_t)par * W * MR * 16;
#pragma unroll
      for (int m = 0; m < MR; ++m) {  // lane groups g = 0..3 of a row: ((g0 + g1) + (g2 + g3))
        acc[m] += __shfl_xor(acc[m], 16, 64);
        acc[m] += __shfl_xor(acc[m], 32, 64);
      }
      if (g == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m) rf[(wave * MR + m) * 16 + r16] = acc[m];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (wave == i % W && lane < MR * 16) {
        const int m = lane >> 4, row = 16 * t + (lane & 15);
        float v = rf[lane];
        for (int w = 1; w < W; ++w) v += rf[w * MR * 16 + lane];
        if (m < M && row < N) store_out(y, (int64_t)m * N + row, v * col_scale(tensor_scale, row, s_t), out_f32);
      }
    } else {
      f32x4_t* rf = reinterpret_cast<f32x4_t*>(red) + (size_t)par * W * 64;
      rf[wave * 64 + lane] = acc;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (wave == i % W) {  // lane holds D[n = 4 g + e][m = r16]
        f32x4_t v = rf[lane];
        for (int w = 1; w < W; ++w) {
          const f32x4_t u = rf[w * 64 + lane];
          v[0] += u[0];
          v[1] += u[1];
          v[2] += u[2];
          v[3] += u[3];
        }
        const int nb = 16 * t + 4 * g;
        if (r16 < M) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nb + e < N) store_out(y, (int64_t)r16 * N + nb + e, v[e] * col_scale(tensor_scale, nb + e, s_t), out_f32);
        }
      }
    }
  };
  auto consume = [&](PkTile<ROUNDS>& T, int i, auto after) __attribute__((always_inline)) {
    constexpr int kAfter = decltype(after)::value;  // loads issued after this tile's
    if constexpr (kDot) {
      float acc[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
      pk_dot<0, 0, MR, IMPL, ROUNDS, kAfter>(T, xw, g, acc);
      finish(i, acc);
    } else {
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pk_mfma<0, 0, MR, IMPL, ROUNDS, kAfter>(T, xw, g, min(r16, MR - 1), acc);
      finish(i, acc);
    }
  };
  using Ahead = std::integral_constant<int, kPkAhead * kPkLoadsPerSlice * ROUNDS>;
  // One tile per workgroup (no more tiles than CUs): no look-ahead loads
  // (they would only fill the memory queue), the tile's steps waited for one
  // by one.  (The branch comes before the tile's loads: a register whose load
  // is in flight must not be live across it.)
  if (cnt == 1) {
    PkTile<ROUNDS> T;
    issue(T, 0);
    consume(T, 0, std::integral_constant<int, 0>{});
    return;
  }
  // three register sets: while tile i is consumed the loads of tiles i + 1
  // and i + 2 are in flight
  PkTile<ROUNDS> A, B, C;
  issue(A, 0);
  issue(B, 1);
  for (int i = 0; i < cnt; i += 3) {
    issue(C, i + 2);
    consume(A, i, Ahead{});
    if (i + 1 >= cnt) break;
    issue(A, i + 3);
    consume(B, i + 1, Ahead{});
    if (i + 2 >= cnt) break;
    issue(B, i + 4);
    consume(C, i + 2, Ahead{});
  }
  wait_vm_all();  // the last (unused) loads land before the wave ends
}

// Single-launch full-K kernel for 16 < m <= 64 on matrices of up to 1024
// 16-row tiles (k = W * NSTEP * 128): a workgroup owns T (1 .. 4) tiles of
// 16 weight rows over the whole K, so no fp32 partial planes and no second
// launch; its W waves split K into slices of NSTEP steps of 128, and each
// activation fragment a wave reads feeds all T tiles.  The
// activations (up to 64 x k) do not fit in LDS, so each wave streams its
// slice: per step a lane's row has 32 codes at k = 128 s + 32 g (the four
// lanes of a row read 64 contiguous bytes) and their two scale bytes, and
// the wave copies the step's activations (16 MT token rows x 256 bytes,
// whole cache lines; piece q of row r at slot q ^ (r % 16), so the B
// fragment reads of 16 rows hit 16 bank groups) into one of its two private
// LDS buffers with the LDS DMA.
// Issue order: the activations of steps 0 and 1, then the codes and scales
// of every step (a wave's whole weight slice is in flight at once, so the
// weights cross HBM while the activations stream from L2), then step s + 2's
// activations once step s has read its buffer.  Loads complete in issue
// order, so step s waits (counted, inline-asm loads) for what it needs and
// no more: for s < 2 its weights, after that its activations (measured on
// 4096 x 4096, m = 32 / 48: 8.3 / 9.8 -> 7.8 / 9.0 us against the order
// step by step).  Token rows >= m repeat row m - 1 (outputs not stored).
// No barrier until the W partial tiles are added in wave order through LDS.
template <int MT>
__device__ __forceinline__ void fx_issue_x(const uint16_t* const* xsrc, uint8_t* buf, int s) {
#pragma unroll
  for (int c = 0; c < 4 * MT; ++c) copy16_to_lds(xsrc[c] + kStepK * s, buf + 1024 * c);
  asm volatile("" ::: "memory");
}

// Loads still allowed in flight when step S starts.  Issue order: the
// activation copies of steps 0 and 1 (kx loads each), the weights of steps
// 0 .. P - 1 (kw loads each: codes and scales of T tiles); after step j,
// the copies of step j + 2 and the weights of step j + P.  Step S needs its
// copies and its weights; loads complete in issue order.
template <int NSTEP, int MT, int T, int P>
constexpr int fx_wait_count(int S) {
  const int kx = 4 * MT, kw = 2 * T;
  int end_x[64] = {}, end_w[64] = {};
  int pos = 0;
  for (int t = 0; t < 2 && t < NSTEP; ++t) end_x[t] = (pos += kx);
  for (int t = 0; t < P && t < NSTEP; ++t) end_w[t] = (pos += kw);
  for (int j = 0; j < S; ++j) {
    if (j + 2 < NSTEP) end_x[j + 2] = (pos += kx);
    if (j + P < NSTEP) end_w[j + P] = (pos += kw);
  }
  return pos - (end_x[S] > end_w[S] ? end_x[S] : end_w[S]);
}

template <int T>
__device__ __forceinline__ void fx_issue_w(u32x4_t (&cw)[T], uint32_t (&sb)[T], const uint8_t* const* cp,
                                           const uint8_t* const* sp, int s) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
    load_b128_async<0>(cw[t], cp[t] + 64 * s);
    load_u16_async<0>(sb[t], sp[t] + 8 * s);
  }
  asm volatile("" ::: "memory");
}

// Step S of NSTEP (LDS buffer S % 2, weight registers S % P), then the
// rest: each B fragment read from LDS feeds the MFMAs of all T row tiles.
template <int S, int NSTEP, int MT, int IMPL, int T, int P>
__device__ __forceinline__ void fx_steps(u32x4_t (&cw)[P][T], uint32_t (&sb)[P][T], const uint8_t* const* cp,
                                         const uint8_t* const* sp, const uint16_t* const* xsrc, uint8_t* xbuf, int g,
                                         int c16, f32x4_t (&acc)[T][MT]) {
  constexpr int cur = S & 1, slot = S % P;
  wait_vm<fx_wait_count<NSTEP, MT, T, P>(S)>(cw[slot][0], sb[slot][0]);
#pragma unroll
  for (int t = 1; t < T; ++t) bind_loaded(cw[slot][t], sb[slot][t]);  // landed with the wait above
  bf16x8_t a[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float sg0 = scale_at<IMPL, 0>(sb[slot][t]), sg1 = scale_at<IMPL, 1>(sb[slot][t]);
    a[t][0] = dequant8<IMPL>(cw[slot][t][0], sg0);
    a[t][1] = dequant8<IMPL>(cw[slot][t][1], sg0);
    a[t][2] = dequant8<IMPL>(cw[slot][t][2], sg1);
    a[t][3] = dequant8<IMPL>(cw[slot][t][3], sg1);
  }
  const uint8_t* buf = xbuf + cur * (4096 * MT);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4_t b = *reinterpret_cast<const u32x4_t*>(buf + 256 * (16 * mt + c16) + 16 * ((4 * g + j) ^ c16));
#pragma unroll
      for (int t = 0; t < T; ++t)
        acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t][j], __builtin_bit_cast(bf16x8_t, b), acc[t][mt], 0, 0, 0);
    }
  if constexpr (S + 2 < NSTEP) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this buffer's reads are done before it is refilled
    fx_issue_x<MT>(xsrc, xbuf + cur * (4096 * MT), S + 2);
  }
  if constexpr (S + P < NSTEP) fx_issue_w<T>(cw[slot], sb[slot], cp, sp, S + P);
  if constexpr (S + 1 < NSTEP) fx_steps<S + 1, NSTEP, MT, IMPL, T, P>(cw, sb, cp, sp, xsrc, xbuf, g, c16, acc);
}

// Weight steps in flight: all of a wave's slice for one tile per
// workgroup; fewer with more tiles, so the loaded words stay in registers.
constexpr int fx_weight_ahead(int nstep, int t) { return t == 1 ? nstep : (16 / t < nstep ? 16 / t : nstep); }

template <int MT, int IMPL, int NSTEP, int T>
__global__ __launch_bounds__(T == 1 ? 512 : 256) void k_skinny_fx(const uint16_t* __restrict__ x,
                                                                  const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const KScale tensor_scale,
                                                                  void* __restrict__ y, int M, int N, int K,
                                                                  int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  uint8_t* xbuf = lds + (size_t)wave * 2 * 4096 * MT;            // [2][16 MT rows][256 bytes]
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + (size_t)W * 2 * 4096 * MT);  // [W][T][MT][64]
  const float s_t = first_scale(tensor_scale);
  const int n0 = blockIdx.x * 16 * T;
  const int k0 = wave * NSTEP * kStepK;
  const uint8_t* cp[T];
  const uint8_t* sp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int row = min(n0 + 16 * t + c16, N - 1);  // rows past n read row n - 1 (real data); outputs dropped
    cp[t] = codes + (int64_t)row * (K / 2) + k0 / 2 + 16 * g;
    sp[t] = scales + (int64_t)row * (K / 16) + k0 / 16 + 2 * g;
  }
  // DMA instruction c of a step: token rows 4c .. 4c + 3, lane l -> row
  // 4c + l / 16, piece (l % 16) ^ (row % 16)
  const uint16_t* xsrc[4 * MT];
#pragma unroll
  for (int c = 0; c < 4 * MT; ++c) {
    const int rr = 4 * c + (lane >> 4);
    xsrc[c] = x + (int64_t)min(rr, M - 1) * K + k0 + 8 * ((lane & 15) ^ (rr & 15));
  }
  static_assert(NSTEP >= 2, "two activation buffers per wave");
  constexpr int P = fx_weight_ahead(NSTEP, T);
  fx_issue_x<MT>(xsrc, xbuf, 0);
  fx_issue_x<MT>(xsrc, xbuf + 4096 * MT, 1);
  u32x4_t cw[P][T];
  uint32_t sb[P][T];
#pragma unroll
  for (int s = 0; s < P; ++s) fx_issue_w<T>(cw[s], sb[s], cp, sp, s);
  f32x4_t acc[T][MT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  fx_steps<0, NSTEP, MT, IMPL, T, P>(cw, sb, cp, sp, xsrc, xbuf, g, c16, acc);

  // the W partial tiles, added in wave order; lane holds D[n = 4 g + e][m = 16 mt + c16]
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((wave * T + t) * MT + mt) * 64 + lane] = acc[t][mt];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  for (int i = threadIdx.x; i < T * MT * 64; i += blockDim.x) {
    f32x4_t v = red[i];
    for (int w = 1; w < W; ++w) {
      const f32x4_t u = red[w * T * MT * 64 + i];
      v[0] += u[0];
      v[1] += u[1];
      v[2] += u[2];
      v[3] += u[3];
    }
    const int t = i / (MT * 64), mt = (i >> 6) % MT, l = i & 63;
    const int m = 16 * mt + (l & 15), nb = n0 + 16 * t + 4 * (l >> 4);
    if (m >= M) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (nb + e < N) store_out(y, (int64_t)m * N + nb + e, v[e] * col_scale(tensor_scale, nb + e, s_t), out_f32);
  }
}

// Split-K kernel: 64 rows x one K chunk per workgroup, fp32 partials to the
// workspace when there is more than one chunk (then k_reduce).
template <int MT, int IMPL, bool K32>
__global__ __launch_bounds__(256) void k_skinny(const uint16_t* __restrict__ x,
                                                const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales,
                                                const KScale tensor_scale,
                                                void* __restrict__ y, float* __restrict__ ws,
                                                int M, int N, int K, int kchunk, int splits,
                                                int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;

  const int k0 = blockIdx.y * kchunk;
  const int kend = min(k0 + kchunk, K);
  const int nks = (kend - k0 + kStepK - 1) / kStepK;  // <= kMaxSteps

  const int row = blockIdx.x * kRowsPerWg + wave * 16 + r16;
  const bool row_ok = row < N;
  const uint8_t* crow = codes + (int64_t)row * (K / 2);
  const uint8_t* srow = scales + (int64_t)row * (K / 16);

  u32x4_t cw[kMaxSteps];
  uint32_t sb[kMaxSteps];
#pragma unroll
  for (int ks = 0; ks < kMaxSteps; ++ks) {
    cw[ks] = u32x4_t{0u, 0u, 0u, 0u};
    sb[ks] = 0u;
    if (ks < nks) {
      const int kk = k0 + ks * kStepK + 32 * g;
      if constexpr (K32) {
        if (row_ok && kk < kend) {
          cw[ks] = *reinterpret_cast<const u32x4_t*>(crow + kk / 2);
          sb[ks] = *reinterpret_cast<const uint16_t*>(srow + kk / 16);
        }
      } else {
        if (row_ok && kk < kend) {
          const uint2 a = *reinterpret_cast<const uint2*>(crow + kk / 2);
          cw[ks][0] = a.x;
          cw[ks][1] = a.y;
          sb[ks] = srow[kk / 16];
        }
        if (row_ok && kk + 16 < kend) {
          const uint2 b = *reinterpret_cast<const uint2*>(crow + kk / 2 + 8);
          cw[ks][2] = b.x;
          cw[ks][3] = b.y;
          sb[ks] |= (uint32_t)srow[kk / 16 + 1] << 8;
        }
      }
    }
  }

  // stage x[0:M, k0:kend) in LDS; piece (ks, j, mt, g, mm) = 8 bf16 of
  // x[16 mt + mm][k0 + 128 ks + 32 g + 8 j ..].
  if (kend - k0 == nks * kStepK) {
    // whole K steps: direct global -> LDS copies (no registers): 1 KiB
    // chunk c = (ks, j, mt) holds the pieces of all 64 lanes (g, mm) in lane
    // order, so lane l's 16 bytes land at slot 64 c + l.  Token rows >= M
    // repeat row M-1 (never read: those B operands are zeroed).
    const int nchunk = nks * 4 * MT;
    for (int c = wave; c < nchunk; c += kWaves) {
      const int mt = c % MT, rj = c / MT, j = rj & 3, ks = rj >> 2;
      const int m = min(mt * 16 + r16, M - 1);
      const uint16_t* src = x + (int64_t)m * K + k0 + ks * kStepK + 32 * g + 8 * j;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + 1024 * c),
                                       16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the copies (and everything else) have landed
    asm volatile("" ::: "memory");
  } else {
    // ragged last chunk: eight 16-byte loads per thread in flight, then
    // their LDS stores (zeros beyond kend)
    constexpr int kBatch = 8;
    const int pieces_per_row = nks * 16;
    const int total = M * pieces_per_row;
    for (int p0 = threadIdx.x; p0 < total; p0 += kBatch * blockDim.x) {
      uint4 v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = p0 + i * blockDim.x;
        const int pc = min(p, total - 1);
        const int m = pc / pieces_per_row;
        const int k = k0 + 8 * (pc - m * pieces_per_row);
        v[i] = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + min(k, K - 8));
        if (!(p < total && k < kend)) v[i] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = p0 + i * blockDim.x;
        if (p >= total) break;
        const int m = p / pieces_per_row;
        const int k8 = p - m * pieces_per_row;
        const int ks = k8 >> 4, rem = k8 & 15;
        const int off = ((((ks * 4 + (rem & 3)) * MT + (m >> 4)) * 4 + (rem >> 2)) * 16 + (m & 15)) * 16;
        *reinterpret_cast<uint4*>(lds + off) = v[i];
      }
    }
  }
  __syncthreads();

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool mrow_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) mrow_ok[mt] = (mt * 16 + r16) < M;
#pragma unroll
  for (int ks = 0; ks < kMaxSteps; ++ks) {
    if (ks < nks) {
      const float sg0 = scale_at<IMPL, 0>(sb[ks]), sg1 = scale_at<IMPL, 1>(sb[ks]);
      bf16x8_t a[4];
      a[0] = dequant8<IMPL>(cw[ks][0], sg0);
      a[1] = dequant8<IMPL>(cw[ks][1], sg0);
      a[2] = dequant8<IMPL>(cw[ks][2], sg1);
      a[3] = dequant8<IMPL>(cw[ks][3], sg1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int off = ((((ks * 4 + j) * MT + mt) * 4 + g) * 16 + r16) * 16;
          u32x4_t bv = *reinterpret_cast<const u32x4_t*>(lds + off);
          if (!mrow_ok[mt]) bv = u32x4_t{0u, 0u, 0u, 0u};
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8_t, bv),
                                                            acc[mt], 0, 0, 0);
        }
      }
    }
  }

  const float s_t = first_scale(tensor_scale);
  const int nbase = blockIdx.x * kRowsPerWg + wave * 16 + 4 * g;
  if (splits == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nbase + i < N) store_out(y, (int64_t)m * N + nbase + i, acc[mt][i] * col_scale(tensor_scale, nbase + i, s_t), out_f32);
    }
    return;
  }
  // Several K chunks: fp32 partial sums to the workspace; k_reduce adds them.
  const int64_t mn = (int64_t)M * N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    if (m >= M) continue;
    float* dst = ws + blockIdx.y * mn + (int64_t)m * N + nbase;
    if ((N & 3) == 0 && nbase + 3 < N) {  // 16-byte aligned: nbase and N are multiples of 4
      *reinterpret_cast<float4*>(dst) = float4{acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]};
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nbase + i < N) dst[i] = acc[mt][i];
  }
}

// Per-lane state of k_skinny_pipe, shared by its compile-time step loops.
template <int MT, int NKS>
struct PipeState {
  u32x4_t cw[NKS];           // codes of step s: 32 codes of row r16 at k = 32 g
  uint32_t sb[NKS];          // the two scale bytes of those codes
  const uint8_t* crow;       // codes of this lane's row and quarter, chunk start
  const uint8_t* srow;       // scales, same
  const uint16_t* xsrc[MT];  // x pieces this lane copies, chunk start
  f32x4_t acc[MT];
};

constexpr int pipe_ops_per_step(int mt) { return 2 + mt; }  // codes, scales, MT x copies

// Issue the loads of steps S .. NKS-1, in step order.
template <int S, int MT, int NKS>
__device__ __forceinline__ void pipe_issue(PipeState<MT, NKS>& P, uint8_t* lds, int wave) {
  load_b128_async<S * (kStepK / 2)>(P.cw[S], P.crow);
  load_u16_async<S * (kStepK / 16)>(P.sb[S], P.srow);
#pragma unroll
  for (int i = 0; i < MT; ++i) copy16_to_lds(P.xsrc[i] + S * kStepK, lds + 1024 * (S * 4 * MT + wave + 4 * i));
  asm volatile("" ::: "memory");
  if constexpr (S + 1 < NKS) pipe_issue<S + 1, MT, NKS>(P, lds, wave);
}

// Compute steps S .. NKS-1, each once its own loads have landed.
template <int S, int MT, int IMPL, int NKS>
__device__ __forceinline__ void pipe_compute(PipeState<MT, NKS>& P, const uint8_t* lds, int g,
                                             int r16) {
  wait_vm<(NKS - 1 - S) * pipe_ops_per_step(MT)>(P.cw[S], P.sb[S]);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS read moves above the barrier
  const float sg0 = scale_at<IMPL, 0>(P.sb[S]), sg1 = scale_at<IMPL, 1>(P.sb[S]);
  bf16x8_t a[4];
  a[0] = dequant8<IMPL>(P.cw[S][0], sg0);
  a[1] = dequant8<IMPL>(P.cw[S][1], sg0);
  a[2] = dequant8<IMPL>(P.cw[S][2], sg1);
  a[3] = dequant8<IMPL>(P.cw[S][3], sg1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // token row 16 mt + r16, 16-byte piece 4 g + j, swizzled by r16
      const int off = S * 4096 * MT + 256 * (16 * mt + r16) + 16 * ((4 * g + j) ^ r16);
      const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(lds + off);
      P.acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8_t, bv),
                                                          P.acc[mt], 0, 0, 0);
    }
  }
  if constexpr (S + 1 < NKS) pipe_compute<S + 1, MT, IMPL, NKS>(P, lds, g, r16);
}

// Pipelined split-K kernel (16 < m <= 64, K a multiple of 128): the tile of
// k_skinny (64 weight rows x one K chunk; x staged in LDS in B-operand
// order by the LDS DMA and shared by the 4 waves), but each K step's loads
// (codes, scales, then the step's x pieces) are issued together in step
// order, and step s is computed as soon as its own loads have landed: a
// vmcnt wait that allows exactly the loads issued after step s to be
// outstanding (loads return in issue order), then a bare s_barrier (no
// fence: a workgroup fence would wait for every LDS DMA in flight) so that
// the x pieces copied by the other waves are there too.  The loop over the
// NKS steps is unrolled at compile time and every chunk is exactly NKS
// steps (K a multiple of NKS * 128): no step is conditional, so the
// compiler cannot sink a step's loads into its compute.
template <int MT, int IMPL, int NKS>
__global__ __launch_bounds__(256) void k_skinny_pipe(const uint16_t* __restrict__ x,
                                                     const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     const KScale tensor_scale,
                                                     void* __restrict__ y, float* __restrict__ ws,
                                                     int M, int N, int K, int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;

  const int k0 = blockIdx.y * (NKS * kStepK);

  PipeState<MT, NKS> P;
  // rows past N read row N-1 (real data, finite); their outputs are dropped
  const int row = blockIdx.x * kRowsPerWg + wave * 16 + r16;
  const int rowc = min(row, N - 1);
  P.crow = codes + (int64_t)rowc * (K / 2) + k0 / 2 + 16 * g;
  P.srow = scales + (int64_t)rowc * (K / 16) + k0 / 16 + 2 * g;
  // x of one step: 16 MT token rows x 256 bytes, copied by 4 MT LDS DMA
  // instructions (wave w issues c = w + 4 i), each reading whole cache
  // lines: 4 rows x 256 contiguous bytes, lane l -> row 4 c + l / 16 and
  // 16-byte piece q = (l % 16) ^ (row % 16).  The step lands row-major
  // (256-byte rows) with piece q of row r at slot q ^ (r % 16), so the B
  // fragment reads (16 rows, the same piece) hit 16 different bank groups.
  // Rows >= M repeat row M-1 (finite data): a B column only feeds the
  // output column of its own token, and those outputs are not stored.
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int rr = 4 * (wave + 4 * i) + (lane >> 4);
    const int m = min(rr, M - 1);
    P.xsrc[i] = x + (int64_t)m * K + k0 + 8 * ((lane & 15) ^ (rr & 15));
  }
  pipe_issue<0, MT, NKS>(P, lds, wave);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) P.acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  pipe_compute<0, MT, IMPL, NKS>(P, lds, g, r16);
  const f32x4_t* acc = P.acc;

  const int nbase = blockIdx.x * kRowsPerWg + wave * 16 + 4 * g;
  if (gridDim.y == 1) {
    const float s_t = first_scale(tensor_scale);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nbase + i < N) store_out(y, (int64_t)m * N + nbase + i, acc[mt][i] * col_scale(tensor_scale, nbase + i, s_t), out_f32);
    }
    return;
  }
  const int64_t mn = (int64_t)M * N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    if (m >= M) continue;
    float* dst = ws + blockIdx.y * mn + (int64_t)m * N + nbase;
    if ((N & 3) == 0 && nbase + 3 < N) {
      *reinterpret_cast<float4*>(dst) = float4{acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]};
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nbase + i < N) dst[i] = acc[mt][i];
  }
}

// Streaming split-K kernel (K % 512 == 0: 16 < m <= 64, and 4 < m <= 16
// on large matrices): a workgroup stages x[0:m, K chunk] in LDS once (LDS
// DMA, the pipelined kernel's swizzled layout) and its 4 waves then stream
// `rows` weight rows through it, 16 rows (one MFMA A tile) at a time, the
// next tile's codes and scales in registers while the current one is
// multiplied.  With many rows per workgroup the activations are read from
// L2 once per row group instead of once per 64 rows.
template <int NST>
struct StrTile {
  u32x4_t cw[NST];   // codes of step s: 32 codes of row r16 at k = 32 g
  uint32_t sb[NST];  // their two scale bytes
};

// Issue the loads of steps S .. NST-1 (inline asm: counted by str_step's waits).
template <int S, int NST>
__device__ __forceinline__ void str_load(StrTile<NST>& T, const uint8_t* crow, const uint8_t* srow) {
  load_b128_async<S * (kStepK / 2)>(T.cw[S], crow);
  load_u16_async<S * (kStepK / 16)>(T.sb[S], srow);
  if constexpr (S + 1 < NST) str_load<S + 1, NST>(T, crow, srow);
}

// B fragments of one K step: token tile mt, k piece j (4 g + j of the
// step's 16), this lane's token row 16 mt + r16.
template <int MT>
struct StrB {
  u32x4_t v[4][MT];
};

template <int S, int MT>
__device__ __forceinline__ void str_read_b(StrB<MT>& B, const uint8_t* lds, int g, int r16) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      B.v[j][mt] = *reinterpret_cast<const u32x4_t*>(lds + S * 4096 * MT + 256 * (16 * mt + r16) +
                                                    16 * ((4 * g + j) ^ r16));
}

// Steps S .. NST-1 of one tile.  AFTER = loads issued after this tile's (the
// next tile's 2 NST); stores issued in between only make the waits stricter.
// Step S + 1's B fragments are read from LDS into Bn before step S's MFMAs
// (which use Bc), so the LDS latency is hidden behind them.  Except with 64
// tokens and the portable conversion: there the second set of fragments
// would not fit the architectural registers (the compiler would then copy
// loaded registers before their wait), so each step reads its own.
template <int S, int MT, int IMPL, int NST, int AFTER>
__device__ __forceinline__ void str_step(StrTile<NST>& T, const uint8_t* lds, int g, int r16, f32x4_t* acc,
                                         StrB<MT>& Bc, StrB<MT>& Bn) {
  constexpr bool kPf = !(MT >= 4 && IMPL == kConvPortable);
  if constexpr (S == 0 && kPf) str_read_b<0, MT>(Bc, lds, g, r16);
  if constexpr (kPf && S + 1 < NST) str_read_b<S + 1, MT>(Bn, lds, g, r16);
  if constexpr (!kPf) str_read_b<S, MT>(Bc, lds, g, r16);
  wait_vm<2 * (NST - 1 - S) + AFTER>(T.cw[S], T.sb[S]);
  const float sg0 = scale_at<IMPL, 0>(T.sb[S]), sg1 = scale_at<IMPL, 1>(T.sb[S]);
  bf16x8_t a[4];
  a[0] = dequant8<IMPL>(T.cw[S][0], sg0);
  a[1] = dequant8<IMPL>(T.cw[S][1], sg0);
  a[2] = dequant8<IMPL>(T.cw[S][2], sg1);
  a[3] = dequant8<IMPL>(T.cw[S][3], sg1);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8_t, Bc.v[j][mt]), acc[mt], 0, 0, 0);
  if constexpr (S + 1 < NST) str_step<S + 1, MT, IMPL, NST, AFTER>(T, lds, g, r16, acc, Bn, Bc);
}

template <int MT, int IMPL, int NST>
__global__ __launch_bounds__(256) void k_skinny_str(const uint16_t* __restrict__ x,
                                                    const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    const KScale tensor_scale,
                                                    void* __restrict__ y, float* __restrict__ ws, int M,
                                                    int N, int K, int rows, int out_f32) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int g = lane >> 4, r16 = lane & 15;
  const int k0 = blockIdx.y * (NST * kStepK);
  const int rg0 = blockIdx.x * rows;
  const int ntiles = (min(rows, N - rg0) + 15) / 16;
  auto row_ptrs = [&](int t, const uint8_t*& cp, const uint8_t*& sp) {
    const int row = min(rg0 + 16 * t + r16, N - 1);
    cp = codes + (int64_t)row * (K / 2) + k0 / 2 + 16 * g;
    sp = scales + (int64_t)row * (K / 16) + k0 / 16 + 2 * g;
  };
  // x chunk by LDS DMA, the pipelined kernel's layout: step s = 16 MT token
  // rows x 256 bytes, piece q of row r at slot q ^ (r % 16); DMA instruction
  // c (wave w issues c = w + 4 i) reads rows 4c .. 4c + 3 in whole cache
  // lines.  Rows >= M repeat row M - 1 (their outputs are not stored).
#pragma unroll
  for (int s = 0; s < NST; ++s) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int rr = 4 * (wave + 4 * i) + (lane >> 4);
      copy16_to_lds(x + (int64_t)min(rr, M - 1) * K + k0 + kStepK * s + 8 * ((lane & 15) ^ (rr & 15)),
                    lds + s * 4096 * MT + 1024 * (wave + 4 * i));
    }
  }
  // then the first tile's weights (every wave issues them, clamped, so the
  // count below is the same in every wave); waiting until only those are
  // outstanding means this wave's copies have landed, and after the barrier
  // every wave's have: the x latency overlaps the weights', and the first
  // tile is still consumed step by step as its loads land
  StrTile<NST> A, B;
  const uint8_t *cp, *sp;
  row_ptrs(min(wave, ntiles - 1), cp, sp);
  str_load<0, NST>(A, cp, sp);
  wait_vm<2 * NST>(A.cw[0], A.sb[0]);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS read moves above the barrier
  const float s_t = first_scale(tensor_scale);
  const int64_t mn = (int64_t)M * N;
  auto finish = [&](int t, const f32x4_t* acc) {
    const int nbase = rg0 + 16 * t + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      if (m >= M) continue;
      if (gridDim.y == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nbase + i < N) store_out(y, (int64_t)m * N + nbase + i, acc[mt][i] * col_scale(tensor_scale, nbase + i, s_t), out_f32);
      } else {
        float* dst = ws + blockIdx.y * mn + (int64_t)m * N + nbase;
        if ((N & 3) == 0 && nbase + 3 < N) {
          *reinterpret_cast<float4*>(dst) = float4{acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nbase + i < N) dst[i] = acc[mt][i];
        }
      }
    }
  };
  // Every tile's loads are issued unconditionally (past the last tile the
  // index is clamped: a redundant load of real data), so the code is
  // straight-line between the loop's uniform branches and the waits the
  // compiler counts let the next tile's loads stay in flight.
  for (int t = wave; t < ntiles; t += 8) {
    row_ptrs(min(t + 4, ntiles - 1), cp, sp);
    str_load<0, NST>(B, cp, sp);
    {
      f32x4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      StrB<MT> b0, b1;
      str_step<0, MT, IMPL, NST, 2 * NST>(A, lds, g, r16, acc, b0, b1);
      finish(t, acc);
    }
    if (t + 4 >= ntiles) {
      wait_vm_all();  // the redundant loads of B land before the wave ends
      break;
    }
    row_ptrs(min(t + 8, ntiles - 1), cp, sp);
    str_load<0, NST>(A, cp, sp);
    {
      f32x4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      StrB<MT> b0, b1;
      str_step<0, MT, IMPL, NST, 2 * NST>(B, lds, g, r16, acc, b0, b1);
      finish(t + 4, acc);
    }
  }
  wait_vm_all();
}

template <int MT, int IMPL, int NST>
hipError_t launch_str(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                      const uint8_t* scales, KScale ts, void* y, float* ws, int M, int N, int K,
                      int out_f32) {
  const size_t lds = (size_t)NST * 4096 * MT;
  hipError_t e = set_lds_limit<k_skinny_str<MT, IMPL, NST>>(lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + p.str_rows - 1) / p.str_rows), (unsigned)p.splits);
  hipLaunchKernelGGL((k_skinny_str<MT, IMPL, NST>), grid, dim3(256), lds, stream, x, codes, scales, ts, y, ws,
                     M, N, K, p.str_rows, out_f32);
  e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return split_reduce(ws, ts, y, (int64_t)M * N, N, p.splits, out_f32, stream);
}

// y = s_t * sum over K chunks (in chunk order) of the fp32 partial sums;
// four outputs per thread when m * n is a multiple of 4.  The planes are
// loaded kRedBatch at a time (independent loads in flight together) and
// added in plane order.
constexpr int kRedBatch = 8;

__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ ws, const KScale tensor_scale,
                                                void* __restrict__ y, int64_t mn, int64_t n, int splits,
                                                int out_f32) {
  const float s_t = first_scale(tensor_scale);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if ((mn & 3) == 0) {
    const int64_t mn4 = mn >> 2;
    const float4* p = reinterpret_cast<const float4*>(ws);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn4; i += stride) {
      float4 s = p[i];
      for (int sp = 1; sp < splits; sp += kRedBatch) {
        float4 t[kRedBatch];
#pragma unroll
        for (int b = 0; b < kRedBatch; ++b)
          if (sp + b < splits) t[b] = p[(int64_t)(sp + b) * mn4 + i];
#pragma unroll
        for (int b = 0; b < kRedBatch; ++b) {
          if (sp + b < splits) {
            s.x += t[b].x;
            s.y += t[b].y;
            s.z += t[b].z;
            s.w += t[b].w;
          }
        }
      }
      store_out(y, 4 * i, s.x * col_scale(tensor_scale, (4 * i) % n, s_t), out_f32);
      store_out(y, 4 * i + 1, s.y * col_scale(tensor_scale, (4 * i + 1) % n, s_t), out_f32);
      store_out(y, 4 * i + 2, s.z * col_scale(tensor_scale, (4 * i + 2) % n, s_t), out_f32);
      store_out(y, 4 * i + 3, s.w * col_scale(tensor_scale, (4 * i + 3) % n, s_t), out_f32);
    }
    return;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
    float s = ws[i];
    for (int sp = 1; sp < splits; sp += kRedBatch) {
      float t[kRedBatch];
#pragma unroll
      for (int b = 0; b < kRedBatch; ++b)
        if (sp + b < splits) t[b] = ws[(int64_t)(sp + b) * mn + i];
#pragma unroll
      for (int b = 0; b < kRedBatch; ++b)
        if (sp + b < splits) s += t[b];
    }
    store_out(y, i, s * col_scale(tensor_scale, i % n, s_t), out_f32);
  }
}

// LDS bytes of the persistent full-K kernel: the activation slices of W
// waves plus two buffers of W partial tiles.
size_t pk_lds_bytes(int mr, int w, int rounds, bool dot) {
  const size_t part = dot ? (size_t)mr * 16 * sizeof(float) : 64 * sizeof(f32x4_t);
  return (size_t)w * rounds * mr * kPkRow * 2 + 2 * (size_t)w * part;
}

template <int MR, int IMPL, int ROUNDS>
hipError_t launch_pk(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                     const uint8_t* scales, KScale ts, void* y, int M, int N, int K, int out_f32) {
  const size_t lds = pk_lds_bytes(MR, p.waves, ROUNDS, pk_dot_path(MR, IMPL));
  hipError_t e = set_lds_limit<k_skinny_pk<MR, IMPL, ROUNDS>>(lds);
  if (e != hipSuccess) return e;
  // persistent: at most as many workgroups as can be resident at once
  // (per device, kernel and block shape; a host query, no allocation)
  static std::atomic<int> resident[64][9];
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int per_cu = (dev >= 0 && dev < 64) ? resident[dev][p.waves].load(std::memory_order_relaxed) : 0;
  if (per_cu <= 0) {
    int cus = 0, blocks = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_skinny_pk<MR, IMPL, ROUNDS>, 64 * p.waves, lds);
    if (e != hipSuccess) return e;
    per_cu = cus;  // one workgroup per CU (measured faster than filling every resident slot)
    (void)blocks;
    if (dev >= 0 && dev < 64) resident[dev][p.waves].store(per_cu, std::memory_order_relaxed);
  }
  const int tiles = (N + 15) / 16;
  const dim3 grid((unsigned)(tiles < per_cu ? tiles : per_cu));  // per_cu: workgroups resident at once
  hipLaunchKernelGGL((k_skinny_pk<MR, IMPL, ROUNDS>), grid, dim3(64 * p.waves), lds, stream, x, codes, scales, ts, y,
                     M, N, K, out_f32);
  return hipGetLastError();
}

template <int MR, int IMPL>
hipError_t launch_pk_r(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                       const uint8_t* scales, KScale ts, void* y, int M, int N, int K, int out_f32) {
  if (p.pk_rounds != 1) return hipErrorInvalidValue;  // the planner takes one slice per wave only
  return launch_pk<MR, IMPL, 1>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
}

size_t fx_lds_bytes(int mt, int w, int t) { return (size_t)w * mt * (2 * 4096 + 1024 * t); }

template <int MT, int IMPL, int NSTEP, int T>
hipError_t launch_fx(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                     const uint8_t* scales, KScale ts, void* y, int M, int N, int K, int out_f32) {
  const size_t lds = fx_lds_bytes(MT, p.waves, T);
  hipError_t e = set_lds_limit<k_skinny_fx<MT, IMPL, NSTEP, T>>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_skinny_fx<MT, IMPL, NSTEP, T>), dim3((unsigned)((N + 16 * T - 1) / (16 * T))),
                     dim3(64 * p.waves), lds, stream, x, codes, scales, ts, y, M, N, K, out_f32);
  return hipGetLastError();
}

template <int MT, int IMPL, int T>
hipError_t launch_fx_s(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                       const uint8_t* scales, KScale ts, void* y, int M, int N, int K, int out_f32) {
  switch (p.fx_steps) {
    case 4: return launch_fx<MT, IMPL, 4, T>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    case 8: return launch_fx<MT, IMPL, 8, T>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    default: return hipErrorInvalidValue;
  }
}

template <int MT, int IMPL>
hipError_t launch_fx_n(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x, const uint8_t* codes,
                       const uint8_t* scales, KScale ts, void* y, int M, int N, int K, int out_f32) {
  switch (p.fx_tiles) {
    case 1: return launch_fx_s<MT, IMPL, 1>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    case 2: return launch_fx_s<MT, IMPL, 2>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    case 3: return launch_fx_s<MT, IMPL, 3>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    case 4: return launch_fx_s<MT, IMPL, 4>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    default: return hipErrorInvalidValue;
  }
}

template <auto Kernel>
hipError_t launch_fk_kernel(dim3 grid, int waves, size_t lds, hipStream_t stream,
                            const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                            KScale ts, void* y, int M, int N, int K, int rounds,
                            int out_f32) {
  hipError_t e = set_lds_limit<Kernel>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(Kernel, grid, dim3(64 * waves), lds, stream, x, codes, scales, ts, y, M, N, K,
                     rounds, out_f32);
  return hipGetLastError();
}

template <int MR, int IMPL, bool K32>
hipError_t launch_fk(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x,
                     const uint8_t* codes, const uint8_t* scales, KScale ts, void* y, int M,
                     int N, int K, int out_f32) {
  const dim3 grid((unsigned)((N + 15) / 16));
  const size_t lds = (size_t)p.waves * (64 * sizeof(f32x4_t) + (size_t)MR * (kWaveK + 8) * 2);
  const int rounds = (K + p.waves * kWaveK - 1) / (p.waves * kWaveK);
  // The one-round kernels need fewer VGPRs, so more workgroups fit per CU;
  // that pays when there are more workgroups than MI355X's 256 CUs
  // (measured: 14336 x 4096 at m = 1: 10.8 us against 12.8 us); with one
  // workgroup per CU the two-buffer build is faster (4096 x 4096: 4.8 us
  // against 5.1 us).
  const bool one = rounds == 1 && grid.x > 256;
  if constexpr (MR <= 2) {  // one or two tokens: VALU dot products
    const dim3 block(64 * p.waves);
    if (K % 128 == 0) {
      if (one)
        hipLaunchKernelGGL((k_skinny_dot<MR, IMPL, K32, true, true>), grid, block, lds, stream, x,
                           codes, scales, ts, y, M, N, K, rounds, out_f32);
      else
        hipLaunchKernelGGL((k_skinny_dot<MR, IMPL, K32, true, false>), grid, block, lds, stream, x,
                           codes, scales, ts, y, M, N, K, rounds, out_f32);
    } else {
      if (one)
        hipLaunchKernelGGL((k_skinny_dot<MR, IMPL, K32, false, true>), grid, block, lds, stream, x,
                           codes, scales, ts, y, M, N, K, rounds, out_f32);
      else
        hipLaunchKernelGGL((k_skinny_dot<MR, IMPL, K32, false, false>), grid, block, lds, stream, x,
                           codes, scales, ts, y, M, N, K, rounds, out_f32);
    }
    return hipGetLastError();
  }
  if (K % 128 == 0) {
    if (one) return launch_fk_kernel<k_skinny_fk<MR, IMPL, K32, true, true>>(grid, p.waves, lds, stream, x, codes, scales, ts, y, M, N, K, rounds, out_f32);
    return launch_fk_kernel<k_skinny_fk<MR, IMPL, K32, true, false>>(grid, p.waves, lds, stream, x, codes, scales, ts, y, M, N, K, rounds, out_f32);
  }
  if (one) return launch_fk_kernel<k_skinny_fk<MR, IMPL, K32, false, true>>(grid, p.waves, lds, stream, x, codes, scales, ts, y, M, N, K, rounds, out_f32);
  return launch_fk_kernel<k_skinny_fk<MR, IMPL, K32, false, false>>(grid, p.waves, lds, stream, x, codes, scales, ts, y, M, N, K, rounds, out_f32);
}

template <int MT, int IMPL, int NKS>
hipError_t launch_pipe(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x,
                       const uint8_t* codes, const uint8_t* scales, KScale ts, void* y,
                       float* ws, int M, int N, int K, int out_f32) {
  const size_t lds = (size_t)NKS * 4 * MT * 1024;
  hipError_t e = set_lds_limit<k_skinny_pipe<MT, IMPL, NKS>>(lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + kRowsPerWg - 1) / kRowsPerWg), (unsigned)p.splits);
  hipLaunchKernelGGL((k_skinny_pipe<MT, IMPL, NKS>), grid, dim3(256), lds, stream, x, codes,
                     scales, ts, y, ws, M, N, K, out_f32);
  e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return split_reduce(ws, ts, y, (int64_t)M * N, N, p.splits, out_f32, stream);
}

template <int MT, int IMPL, bool K32>
hipError_t launch_mt(const SkinnyPlan& p, hipStream_t stream, const uint16_t* x,
                     const uint8_t* codes, const uint8_t* scales, KScale ts, void* y,
                     float* ws, int M, int N, int K, int out_f32) {
  if constexpr (MT == 1) {
    if (p.splits == 0 && p.rdot_chunks > 0 && IMPL == kConvHw)  // row-per-wave dot products (m == 1)
      return launch_rdot(p, stream, x, codes, scales, ts, y, N, K, out_f32);
    if (p.splits == 0 && p.pk_rounds > 0) {  // persistent full-K kernel
      if constexpr (K32) {  // the planner takes it for 4 < m <= 16
        if (M <= 8) return launch_pk_r<8, IMPL>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
        return launch_pk_r<16, IMPL>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
      }
      return hipErrorInvalidValue;
    }
    if (p.splits == 0) {  // full-K kernel (one token tile only)
      const int mr = M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 8 : 16)));
      switch (mr) {
        case 1: return launch_fk<1, IMPL, K32>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
        case 2: return launch_fk<2, IMPL, K32>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
        case 4: return launch_fk<4, IMPL, K32>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
        case 8: return launch_fk<8, IMPL, K32>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
        default: return launch_fk<16, IMPL, K32>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
      }
    }
  }
  if (p.fx_steps > 0) {
    if constexpr (K32 && MT >= 2) return launch_fx_n<MT, IMPL>(p, stream, x, codes, scales, ts, y, M, N, K, out_f32);
    return hipErrorInvalidValue;
  }
  if (p.str_rows > 0) {
    if constexpr (K32) {
      if (p.kchunk == 8 * kStepK)
        return launch_str<MT, IMPL, 8>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
      return launch_str<MT, IMPL, 4>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
    }
    return hipErrorInvalidValue;
  }
  if (p.nks > 0) {
    if constexpr (K32) {
      switch (p.nks) {
        case 4: return launch_pipe<MT, IMPL, 4>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
        case 8: return launch_pipe<MT, IMPL, 8>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
        default:
          if constexpr (MT <= 2)
            return launch_pipe<MT, IMPL, 16>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
          return hipErrorInvalidValue;
      }
    }
    return hipErrorInvalidValue;
  }
  auto fn = k_skinny<MT, IMPL, K32>;
  const size_t lds = (size_t)(p.kchunk / kStepK) * 4 * MT * 4 * 16 * 16;
  hipError_t ea = set_lds_limit<k_skinny<MT, IMPL, K32>>(lds);
  if (ea != hipSuccess) return ea;
  const dim3 grid((unsigned)((N + kRowsPerWg - 1) / kRowsPerWg), (unsigned)p.splits);
  hipLaunchKernelGGL(fn, grid, dim3(256), lds, stream, x, codes, scales, ts, y, ws, M, N, K,
                     p.kchunk, p.splits, out_f32);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return split_reduce(ws, ts, y, (int64_t)M * N, N, p.splits, out_f32, stream);
}

template <int IMPL, bool K32>
hipError_t launch_impl(int mt, const SkinnyPlan& p, hipStream_t stream, const uint16_t* x,
                       const uint8_t* codes, const uint8_t* scales, KScale ts, void* y,
                       float* ws, int M, int N, int K, int out_f32) {
  switch (mt) {
    case 1: return launch_mt<1, IMPL, K32>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
    case 2: return launch_mt<2, IMPL, K32>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
    case 3: return launch_mt<3, IMPL, K32>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
    default: return launch_mt<4, IMPL, K32>(p, stream, x, codes, scales, ts, y, ws, M, N, K, out_f32);
  }
}

// Largest split-K chunk (in K steps) for MT token tiles: registers hold 16
// steps and the x chunk (16*MT rows, B-operand order) must fit the LDS budget.
int max_steps(int mt) {
  const int lds_steps = kLdsBudget / (16 * mt * kStepK * 2);
  return lds_steps < kMaxSteps ? lds_steps : kMaxSteps;
}

}  // namespace

hipError_t launch_split_reduce(const float* ws, RowScale rs, void* y, int64_t mn, int64_t n,
                               int splits, int out_f32, hipStream_t stream) {
  return split_reduce(ws, kscale(rs), y, mn, n, splits, out_f32, stream);
}

hipError_t split_reduce(const float* ws, KScale tensor_scale, void* y, int64_t mn, int64_t n, int splits,
                        int out_f32, hipStream_t stream) {
  const int64_t work = (mn & 3) == 0 ? mn / 4 : mn;  // outputs per thread: 4 or 1
  int64_t blocks = (work + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)blocks), dim3(256), 0, stream, ws, tensor_scale, y,
                     mn, n > 0 ? n : 1, splits, out_f32);
  return hipGetLastError();
}

namespace {
// The persistent full-K kernel's shape for (m, k): W waves x `rounds` K
// slices of 512 covering k exactly (W <= 8, rounds in {1, 2, 4}, fewest
// rounds first), with the activations and partial tiles within the LDS
// budget.  False when there is none.
bool pk_shape(int64_t m, int64_t k, int* waves, int* rounds) {
  // measured against the full-K and streaming kernels on 4096 x 4096 and
  // 14336 x 4096 (one 512-wide K slice per wave): faster for 4 < m <= 16
  // (14336 x 4096 at m = 8 / 16: 12.3 / 13.2 against 13.6 / 14.6 us;
  // 4096 x 4096: 5.75 / 6.53 against 5.97 / 6.75 us), even or slower for
  // m <= 4; with several slices per wave (k > 4096: 4096 x 14336) slower
  if (m <= 4 || m > 16 || k < kWaveK || k % kWaveK != 0) return false;
  const int64_t slices = k / kWaveK;
  if (slices > 8) return false;
  const int mr = m <= 8 ? 8 : 16;
  if (pk_lds_bytes(mr, (int)slices, 1, false) > (size_t)159 * 1024) return false;
  *waves = (int)slices;
  *rounds = 1;
  return true;
}
}  // namespace

namespace {
// The single-launch full-K kernel's shape for 16 < m <= 64: W waves (8
// down to 4) x NSTEP in {4, 8} steps of 128 covering k exactly, within
// the LDS budget.  Taken where it measured faster than the streaming
// split-K kernel and its reduction: at most one 16-row tile per CU (a
// second round of workgroups re-streams the activations: 4100 x 4096 at
// m = 32 12.6 against 10.9 us), k <= 4096 (4096 x 8192 at m = 32: 13.6
// against 12.9 us), and m <= 48 unless k <= 2048 (4096 x 4096 at m = 64:
// 12.1 against 11.9 us).  Measured gains: 4096 x 4096 at m = 17 / 32 / 48
// 9.06 / 9.40 / 10.61 -> 7.76 / 8.35 / 9.79 us; 4096 x 2048 at m = 17 / 48
// / 64 8.0 / 9.0 / 9.9 -> 5.4 / 6.4 / 7.7 us.
bool fx_shape(int64_t m, int64_t n, int64_t k, int* waves, int* nsteps, int* tiles) {
  if (m <= 16 || m > 64 || k < kStepK || k % kStepK != 0 || k > 4096) return false;
  if (m > 48 && k > 2048) return false;
  const int mt = (int)((m + 15) / 16);
  const int64_t steps = k / kStepK;
  const int64_t ntiles = (n + 15) / 16;
  if (ntiles > kFxMaxTiles) {
    // T = 2 .. 4 row tiles per workgroup, so that at most 256 workgroups
    // share the activation stream (4 waves of 512-wide K slices).  Measured
    // against the streaming split-K kernel at m = 17 / 32 / 48: 8192 x 4096
    // 12.2 / 13.2 / 15.6 -> 10.6 / 10.9 / 12.6 us (T = 2); 12288 x 4096
    // 14.8 / 15.2 / 18.0 -> 13.9 / 14.7 / 16.8 us (T = 3); 14336 x 2048
    // 11.8 / 12.7 / 14.9 -> 9.9 / 10.3 / 12.2 us (T = 4); with T = 4 and
    // k = 4096 (14336 x 4096) even or slower (16.5 / 17.6 / 20.0 against
    // 17.0 / 17.0 / 20.1 us), so not taken there.
    const int64_t t = (ntiles + kFxMaxTiles - 1) / kFxMaxTiles;
    if (t > 4 || (t == 4 && k > 2048)) return false;
    if ((ntiles + t - 1) / t < 192) return false;  // keep at least 3/4 of the CUs busy
    const int64_t ns = steps / 4;
    if (steps % 4 != 0 || (ns != 4 && ns != 8)) return false;
    if (fx_lds_bytes(mt, 4, (int)t) > (size_t)159 * 1024) return false;
    *waves = 4;
    *nsteps = (int)ns;
    *tiles = (int)t;
    return true;
  }
  for (int w = 8; w >= 4; --w) {
    if (steps % w != 0) continue;
    const int64_t ns = steps / w;
    if (ns != 4 && ns != 8) continue;
    if (fx_lds_bytes(mt, w, 1) > (size_t)159 * 1024) continue;
    *waves = w;
    *nsteps = (int)ns;
    *tiles = 1;
    return true;
  }
  return false;
}
}  // namespace

SkinnyPlan plan_skinny_base(int64_t m, int64_t n, int64_t k, int forced_splits);

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int forced_splits) {
  int w = 0, r = 0, t = 0;
  // one token, 2048 <= k <= 32768 with k % 32 == 0: the row-per-wave
  // dot-product kernel over ceil(k / 2048) chunks of 2048 (the portable
  // decode takes the full-K kernel with the same plan's waves).  Below one
  // whole chunk most lanes would hold no codes, and the full-K kernel is
  // faster (8192 x 512 2.99 against 3.64 us, 32768 x 768 5.31 against 7.64,
  // 16384 x 1024 4.62 against 4.95 us)
  if (forced_splits <= 0 && m == 1 && k >= 2048 && k % 32 == 0 && k <= 32768) {
    SkinnyPlan p = plan_skinny_base(m, n, k, forced_splits);
    if (p.splits == 0) {
      p.rdot_chunks = (int)((k + 2047) / 2048);
      return p;
    }
  }
  if (forced_splits <= 0 && fx_shape(m, n, k, &w, &r, &t)) {
    SkinnyPlan p{};
    p.splits = 1;
    p.waves = w;
    p.fx_steps = r;
    p.fx_tiles = t;
    return p;
  }
  if (forced_splits <= 0 && pk_shape(m, k, &w, &r)) {
    SkinnyPlan p{};
    p.splits = 0;
    p.waves = w;
    p.pk_rounds = r;
    p.steps_per_wave = kSpw;
    return p;
  }
  return plan_skinny_base(m, n, k, forced_splits);
}

SkinnyPlan plan_skinny_base(int64_t m, int64_t n, int64_t k, int forced_splits) {
  SkinnyPlan p{};
  const int mt = (int)((m + 15) / 16);
  const int64_t ksteps = (k + kStepK - 1) / kStepK;
  // 8 < m <= 16 on large matrices (more 16-row workgroups than CUs, or more
  // than 2^25 weights), and 4 < m <= 8 there when K needs more than one
  // round of the full-K kernel (k > 4096): the full-K kernel's 16-token
  // build needs ~141 KiB of LDS per workgroup (one per CU), so its
  // workgroups run in several serial rounds or few of them stream long rows;
  // the split-K kernels are faster there (14336 x 4096 at m = 16: streaming
  // 15.3, pipelined 17.4, full-K 20.6 us; 4096 x 14336 at m = 16: streaming
  // 16.6, full-K 20.0 us; 13824 x 5120 at m = 8: 16.1 against 28.9 us;
  // 8192 x 28672 at m = 8: 39.6 against 47.4 us).  With one round (k <=
  // 4096) the full-K kernel stays faster up to 8 tokens (14336 x 4096 at
  // m = 5: 13.0 against 14.1 us); at 3-4 tokens the two are about even.
  const bool pipe_small = forced_splits <= 0 && (m > 8 || (m > 4 && k > 4096)) &&
                          ((n + 15) / 16 > 256 || n * k > ((int64_t)1 << 25)) && k % 512 == 0;
  if (forced_splits <= 0 && mt == 1 && k > 0 && !pipe_small) {
    // full K per workgroup: one 512-wide slice per wave and round, up to 8
    // waves (longer K loops over rounds)
    int64_t waves = (k + kWaveK - 1) / kWaveK;
    if (waves < 1) waves = 1;
    if (waves > 8) waves = 8;
    // one or two tokens on more than 1024 row tiles (e.g. gate and up
    // stacked, 28672 x 4096): four waves of two rounds, the second round's
    // loads in flight while the first is multiplied - 32 back-to-back calls
    // at m = 1 / 2: 519 / 568 against 549 / 592 us; on 768 tiles (q, k, v
    // stacked) it was even or slower (296 / 334 against 294 / 319 us)
    if (m <= 2 && (n + 15) / 16 > 1024 && k <= 4096 && waves > 4) waves = 4;
    // at most one workgroup per CU (n <= 4096): as few waves as keep the
    // number of rounds, so none idles in the last one (4096 x 14336 at m =
    // 2 / 3: 7 waves 12.06 / 13.26 against 8 waves 12.45 / 13.82 us; 4096 x
    // 6144 at m = 2 / 4: 6 waves 7.60 / 7.99 against 7.95 / 8.44 us); with
    // more workgroups than CUs it measured even or slower (13824 x 5120 at
    // m = 2: 17.61 against 17.45 us)
    if ((n + 15) / 16 <= 256) {
      const int64_t slices = (k + kWaveK - 1) / kWaveK;
      const int64_t rounds = (slices + waves - 1) / waves;
      waves = (slices + rounds - 1) / rounds;
    }
    p.splits = 0;
    p.waves = (int)waves;
    p.steps_per_wave = kSpw;
    return p;
  }
  const int64_t tiles = (n + kRowsPerWg - 1) / kRowsPerWg;
  if (forced_splits <= 0 && (mt >= 2 || pipe_small) && k % (4 * kStepK) == 0) {
    // 16 < m <= 64 (and the large-matrix 8 < m <= 16 above): the streaming
    // kernel, K chunks of 1024 (512 when k % 1024 != 0: against the
    // pipelined kernel, 14336 x 4608 at m = 32 / 48: 20.1 / 24.0 against
    // 24.6 / 30.3 us) and row groups sized so that about 256 workgroups
    // run (one per CU).  Measured against the pipelined kernel:
    // 14336 x 4096 / 4096 x 14336 / 4096 x 4096 at m = 32: 17.5 / 19.3 /
    // 10.0 us against 21.6 / 23.4 / 10.7 us; at m = 48: 21.0 / 22.3 / 11.4
    // against 26.8 / 28.1 / 12.8 us (4096 x 4096 at m = 17: 9.6 against
    // 9.4 us, the one case where it is not faster).
    const int64_t nst = k % (8 * kStepK) == 0 ? 8 : 4;
    const int64_t splits = k / (nst * kStepK);
    int64_t groups = 256 / splits;
    if (groups < 1) groups = 1;
    const int64_t t16 = (n + 15) / 16;
    const int64_t per = (t16 + groups - 1) / groups;
    p.str_rows = (int)(16 * per);
    p.kchunk = (int)(nst * kStepK);
    p.splits = (int)splits;
    p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
    return p;
  }
  if (k > 0 && k % kStepK == 0) {
    // pipelined kernel: chunks of exactly NKS in {4, 8, 16} steps (NKS
    // dividing the K steps), the x chunk (NKS * MT KiB) within the LDS budget
    const int64_t lds_steps = kLdsBudget / (4 * mt * 1024);
    int64_t nks = 0;
    if (forced_splits > 0) {
      const int64_t sp = forced_splits > ksteps ? ksteps : forced_splits;
      const int64_t want = (ksteps + sp - 1) / sp;
      if ((want == 4 || want == 8 || want == 16) && want <= lds_steps && ksteps % want == 0)
        nks = want;
    } else if (ksteps % 4 == 0) {
      // 4-step chunks: the most workgroups and the smallest LDS footprint
      // (up to 3 workgroups per CU); measured fastest on 4096 x 4096,
      // 14336 x 4096 and 4096 x 14336 for m = 17 .. 64 (longer chunks keep
      // fewer, longer-lived workgroups per CU and hide less latency)
      nks = 4;
    }
    if (nks > 0) {
      p.nks = (int)nks;
      p.kchunk = (int)(nks * kStepK);
      p.splits = (int)(ksteps / nks);
      p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
      return p;
    }
  }
  int64_t splits = forced_splits;
  if (splits <= 0) splits = (256 + tiles / 2) / tiles;  // about one workgroup per CU
  if (splits < 1) splits = 1;
  if (splits > 64) splits = 64;
  if (splits > ksteps) splits = ksteps < 1 ? 1 : ksteps;
  int64_t steps_per = (ksteps + splits - 1) / splits;
  if (steps_per < 1) steps_per = 1;
  const int64_t cap = max_steps(mt);
  if (steps_per > cap) steps_per = cap;
  p.kchunk = (int)(steps_per * kStepK);
  p.splits = (int)((ksteps + steps_per - 1) / steps_per);
  if (p.splits < 1) p.splits = 1;
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  return p;
}

hipError_t launch_skinny(const void* x, const uint8_t* codes, const uint8_t* scales,
                         RowScale rs, void* y, int64_t m, int64_t n, int64_t k,
                         int out_f32, const SkinnyPlan& plan, void* workspace, int impl,
                         hipStream_t stream) {
  const KScale tensor_scale = kscale(rs);
  const int mt = (int)((m + 15) / 16);
  const bool k32 = (k % 32) == 0;
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  float* ws = reinterpret_cast<float*>(workspace);
  const int M = (int)m, N = (int)n, K = (int)k;
  if (impl == kConvHw)
    return k32 ? launch_impl<kConvHw, true>(mt, plan, stream, xp, codes, scales, tensor_scale, y, ws, M, N, K, out_f32)
               : launch_impl<kConvHw, false>(mt, plan, stream, xp, codes, scales, tensor_scale, y, ws, M, N, K, out_f32);
  return k32 ? launch_impl<kConvPortable, true>(mt, plan, stream, xp, codes, scales, tensor_scale, y, ws, M, N, K, out_f32)
             : launch_impl<kConvPortable, false>(mt, plan, stream, xp, codes, scales, tensor_scale, y, ws, M, N, K, out_f32);
}

NVFP4_VARIANT_END
}  // namespace nvfp4
