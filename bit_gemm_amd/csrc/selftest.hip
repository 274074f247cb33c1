// Validation of the gfx950 scaled FP4 and the FP8 (E4M3) conversion
// instructions against the library's portable ALU rounding and decoding
// (nvfp4_device.h).  The
// hardware path (NVFP4_IMPL_HWCVT) is only the default when every counter
// here is zero on the device.
#include "launchers.h"
#include "nvfp4_device.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ void count(uint32_t* counter, uint32_t c) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0 && c != 0u) atomicAdd(counter, c);
}

__device__ __forceinline__ uint32_t sw_code(float v) {
  return e2m1_rne_portable(fabsf(v)) | ((__float_as_uint(v) >> 28) & 8u);
}

// [0]: every non-NaN fp32 bit pattern i (both signs), paired with pattern
// i ^ 0x00400000, through all four byte selectors of the packing conversion
// (operand order alternating, so the nibble order is checked too).
__global__ __launch_bounds__(256) void k_round(uint32_t* counters) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t bad = 0u, tested = 0u;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
    const uint32_t ba = (uint32_t)i, bb = ba ^ 0x00400000u;
    const float a = __uint_as_float(ba), b = __uint_as_float(bb);
    if (a != a || b != b) continue;  // NaN
    const uint32_t hw = e2m1_pack8_hw(a, b, b, a, a, b, b, a);
    const uint32_t ab = sw_code(a) | (sw_code(b) << 4), ba2 = sw_code(b) | (sw_code(a) << 4);
    const uint32_t sw = ab | (ba2 << 8) | (ab << 16) | (ba2 << 24);
    bad += (hw != sw) ? 1u : 0u;
    tested += 1u;
  }
  count(&counters[0], bad);
  count(&counters[4], tested);
}

// [1] decode of all 256 bytes, [2] scaled fp32 decode, [3] scaled bf16
// decode, for sigma over all 127 non-negative finite E4M3 values.
__global__ __launch_bounds__(256) void k_decode(uint32_t* counters) {
  const uint32_t byte = threadIdx.x;  // 0..255
  const uint32_t scode = blockIdx.x;  // 0..126
  const float sigma = e4m3_decode(scode);
  const uint32_t word = byte * 0x01010101u;
  const float lo = e2m1_val_portable(byte & 0xFu), hi = e2m1_val_portable(byte >> 4);
  uint32_t bad1 = 0u, bad2 = 0u, bad3 = 0u;
  if (scode == 0) {
    // the byte under test at each selector position, other bytes different
    const uint32_t other = (byte ^ 0x5Au) * 0x01010101u;
#define DEC_AT(J)                                                                        \
  {                                                                                      \
    const uint32_t wj = (other & ~(0xFFu << (8 * J))) | (byte << (8 * J));              \
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wj, 1.0f, J);                \
    bad1 += (__float_as_uint(v[0]) != __float_as_uint(lo) ||                             \
             __float_as_uint(v[1]) != __float_as_uint(hi)) ? 1u : 0u;                    \
  }
    DEC_AT(0) DEC_AT(1) DEC_AT(2) DEC_AT(3)
#undef DEC_AT
  }
  {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, sigma, 1);
    const float el = lo * sigma, eh = hi * sigma;
    bad2 = (__float_as_uint(v[0]) != __float_as_uint(el) || __float_as_uint(v[1]) != __float_as_uint(eh)) ? 1u : 0u;
    const bf16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sigma, 2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    bad3 = (hb != pack_bf16_exact(el, eh)) ? 1u : 0u;
  }
  count(&counters[1], bad1);
  count(&counters[2], bad2);
  count(&counters[3], bad3);
  // [5] unit-scale decode straight to bf16 pairs from each byte position
  uint32_t bad5 = 0u;
  if (scode == 0) {
    const uint32_t other = (byte ^ 0xA5u) * 0x01010101u;
    const uint32_t want = pack_bf16_exact(lo, hi);
#define DEC16_AT(J)                                                                       \
  {                                                                                       \
    const uint32_t wj = (other & ~(0xFFu << (8 * J))) | (byte << (8 * J));               \
    const bf16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wj, 1.0f, J);            \
    bad5 += (__builtin_bit_cast(uint32_t, h) != want) ? 1u : 0u;                          \
  }
    DEC16_AT(0) DEC16_AT(1) DEC16_AT(2) DEC16_AT(3)
#undef DEC16_AT
  }
  count(&counters[5], bad5);
  // [6] E4M3 scale decode by the fp8 conversion, each byte position: the
  // signed bit decode for every byte, NaN for the two NaN patterns
  uint32_t bad6 = 0u;
  if (scode == 0) {
    const uint32_t other = (byte ^ 0x3Cu) * 0x01010101u;
    const float mag = e4m3_decode(byte & 0x7Fu);
    const float want = (byte & 0x80u) ? -mag : mag;
    const bool nan_pattern = (byte & 0x7Fu) == 0x7Fu;
#define E4M3_AT(J)                                                                        \
  {                                                                                       \
    const uint32_t wj = (other & ~(0xFFu << (8 * J))) | (byte << (8 * J));               \
    const float v = scale_at<kConvHw, J>(wj);                                             \
    bad6 += (nan_pattern ? (v == v) : (__float_as_uint(v) != __float_as_uint(want))) ? 1u : 0u; \
  }
    E4M3_AT(0) E4M3_AT(1) E4M3_AT(2) E4M3_AT(3)
#undef E4M3_AT
  }
  count(&counters[6], bad6);
}

__global__ void k_zero8(uint32_t* c) {
  if (threadIdx.x < 8) c[threadIdx.x] = 0u;
}

}  // namespace

hipError_t launch_selftest_cvt(uint32_t* counters, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero8, dim3(1), dim3(64), 0, stream, counters);
  hipLaunchKernelGGL(k_round, dim3(8192), dim3(256), 0, stream, counters);
  hipLaunchKernelGGL(k_decode, dim3(127), dim3(256), 0, stream, counters);
  return hipGetLastError();
}

}  // namespace nvfp4
