// Device helpers shared by the gfx950 kernels of libnvfp4: E4M3 scale
// rounding, E2M1 (FP4) rounding and decoding, bf16 packing, MFMA operand
// types, and the host-side LDS opt-in.  Compiled only for gfx950 (CDNA4,
// wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launchers.h"

#include <atomic>

namespace nvfp4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA A/B operand
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(16))) float f32x16_t;  // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr float kFltMax = 3.40282346638528859811704183484516925e+38f;

// E4M3 (bias 7, 3 mantissa bits, max 448, S.1111.111 = NaN) round to nearest
// even of u >= 0.  Returns the rounded value and writes the bit pattern to
// *code; a result above 448 is an overflow: *code = 0x7F and NaN is returned.
__device__ __forceinline__ float e4m3_rne(float u, uint32_t* code) {
  if (u < 0x1p-6f) {
    // Subnormal range: the quantum is 2^-9.  u * 512 is exact, rintf rounds
    // to nearest even; 8 becomes the smallest normal (pattern 0x08).
    float m = __builtin_rintf(u * 512.0f);
    *code = (uint32_t)m;
    return m * 0x1p-9f;
  }
  uint32_t b = __float_as_uint(u);
  // keep 3 mantissa bits: add just under half an ulp of the kept bits plus
  // the kept LSB (ties to even), then clear the 20 dropped bits
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  uint32_t e = (r >> 23);  // biased fp32 exponent, >= 121 here
  uint32_t c = ((e - 120u) << 3) | ((r >> 20) & 7u);  // E4M3 exponent = e - 127 + 7
  if (c > 0x7Eu) {
    *code = 0x7Fu;
    return __builtin_nanf("");
  }
  *code = c;
  return __uint_as_float(r);
}

// Value of an E4M3 bit pattern with the sign bit clear (0x00..0x7E).
// Branch free (both forms, then a select): the GEMM kernels decode two
// scales per K step and lane.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * 0x1p-9f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// Signed value of the E4M3 block scale in byte J of `word`.  kConvHw:
// gfx950's OCP E4M3 -> fp32 conversion with a byte selector (exact: every
// E4M3 value is an fp32; checked over all 256 bytes at each byte position by
// nvfp4_selftest_cvt), one instruction.  Otherwise the bit decode above.
// The NaN patterns 0x7F / 0xFF are never written by the quantizer.
template <int IMPL, int J>
__device__ __forceinline__ float scale_at(uint32_t word) {
  static_assert(J >= 0 && J < 4, "byte selector");
  if constexpr (IMPL == kConvHw) {
    return __builtin_amdgcn_cvt_f32_fp8((int)word, J);
  } else {
    const uint32_t b = (word >> (8 * J)) & 0xFFu;
    const float v = e4m3_decode(b & 0x7Fu);
    return (b & 0x80u) ? -v : v;
  }
}

// E2M1 magnitude index (0..7 <-> 0, .5, 1, 1.5, 2, 3, 4, 6) of v >= 0, round
// to nearest with ties to the even index, saturating; NaN -> 0, +inf -> 7.
// The index is the number of grid midpoints below v: ">" at a midpoint whose
// upper neighbour has an odd index, ">=" where it is even.
__device__ __forceinline__ uint32_t e2m1_rne_portable(float v) {
  return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) +
         (uint32_t)(v >= 1.75f) + (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) +
         (uint32_t)(v > 5.0f);
}

// Magnitude of an E2M1 magnitude index.  Indices 2..7 are normal numbers
// 2^(e-1) * (1 + m/2) with index = 2e + m, whose fp32 bit pattern is
// (index + 252) << 22; 0 and 1 are the subnormals 0 and 0.5.
__device__ __forceinline__ float e2m1_mag_portable(uint32_t idx) {
  return idx < 2u ? 0.5f * (float)idx : __uint_as_float((idx + 252u) << 22);
}

// Signed value of a 4-bit code (bit 3 = sign).
__device__ __forceinline__ float e2m1_val_portable(uint32_t code) {
  return __uint_as_float(__float_as_uint(e2m1_mag_portable(code & 7u)) | ((code & 8u) << 28));
}

// gfx950 scaled conversions, used with a unit scale.  Each conversion turns
// two fp32 into two FP4 codes (first operand in the low nibble) and writes
// them to the byte of the destination that its selector names, keeping the
// other bytes; so eight values become one word, element i at bits 4i..4i+3.
__device__ __forceinline__ uint32_t e2m1_pack8_hw(float v0, float v1, float v2, float v3,
                                                  float v4, float v5, float v6, float v7) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v2, v3, 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v4, v5, 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v6, v7, 1.0f, 3);
}

// Round an fp32 to bf16, nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Two fp32 values that are exact in bf16 -> packed bf16x2 (lo in bits 0-15).
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 codes of `d` (code i in bits 4i..4i+3, the packed row order) times the
// block scale sigma, as 8 fp32 values v[0..7] in k order.  The product has at
// most 6 significant bits (2 of the E2M1 value, 4 of the E4M3 scale), so it
// is exact in fp32 and in bf16.  kConvHw decodes each byte with gfx950's
// FP4 -> fp32 conversion at unit scale (exact; checked on every code byte by
// nvfp4_selftest_cvt), the portable form from the bit patterns.
template <int IMPL>
__device__ __forceinline__ void dequant8_f32(uint32_t d, float sigma, float* v) {
  if constexpr (IMPL == kConvHw) {
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    v[0] = v0[0] * sigma;
    v[1] = v0[1] * sigma;
    v[2] = v1[0] * sigma;
    v[3] = v1[1] * sigma;
    v[4] = v2[0] * sigma;
    v[5] = v2[1] * sigma;
    v[6] = v3[0] * sigma;
    v[7] = v3[1] * sigma;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = e2m1_val_portable((d >> (4 * i)) & 0xFu) * sigma;
  }
}

// The same 8 values as bf16 in k order (an MFMA operand of 8 k): exact, so
// packing keeps the high half of each fp32.
template <int IMPL>
__device__ __forceinline__ u32x4_t dequant8_bf16(uint32_t d, float sigma) {
  float v[8];
  dequant8_f32<IMPL>(d, sigma, v);
  return u32x4_t{pack_bf16_exact(v[0], v[1]), pack_bf16_exact(v[2], v[3]), pack_bf16_exact(v[4], v[5]),
                 pack_bf16_exact(v[6], v[7])};
}

// Streaming (non-temporal) accesses for data that one kernel reads or writes
// exactly once: the weight matrix in the amax and quantization passes, the
// dequantized output.  The hint lets the caches evict these lines first;
// measured 3-5 % faster on those kernels.
__device__ __forceinline__ float4 load_f4_stream(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store_u4_stream(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(u32x4_t{a, b, c, d}, reinterpret_cast<u32x4_t*>(p));
}

// Host side: above 64 KiB a kernel must opt in to more dynamic LDS (gfx950
// has 160 KiB per CU; 1 KiB is left for the kernels' static LDS).  Done once per kernel:
// Loads whose completion the kernel waits for itself.  The compiler's own
// wait insertion counts LDS DMA copies as a different kind of vector-memory
// event from plain loads, and with both kinds in flight it can only wait for
// everything (vmcnt(0)); loads written as inline asm are invisible to it, and
// wait_vm below (which takes the loaded registers as operands, so nothing
// that reads them can move above it) waits for exactly as many as needed.
// (The asm bodies are compiled for the device only: the host pass of a HIP
// source also reads device functions and has no VGPR constraint.)
template <int OFF>
__device__ __forceinline__ void load_b128_async(u32x4_t& d, const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(d) : "v"(p), "i"(OFF) : "memory");
#endif
}
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
template <int OFF>
__device__ __forceinline__ void load_b64_async(u32x2_t& d, const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_dwordx2 %0, %1, off offset:%2" : "=v"(d) : "v"(p), "i"(OFF) : "memory");
#endif
}
template <int OFF>
__device__ __forceinline__ void load_u16_async(uint32_t& d, const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_ushort %0, %1, off offset:%2" : "=v"(d) : "v"(p), "i"(OFF) : "memory");
#endif
}
// Wait until at most V vector-memory operations of this wave are
// outstanding (loads return in issue order); V is capped at 63, the
// counter's limit, which only waits longer.
template <int V>
__device__ __forceinline__ void wait_vm(u32x4_t& c, uint32_t& sbv) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(c), "+v"(sbv) : "n"(V > 63 ? 63 : V) : "memory");
#endif
}

// LDS DMA of 16 bytes per lane: lane l's bytes land at dst + 16 l (dst is
// wave-uniform).
__device__ __forceinline__ void copy16_to_lds(const uint16_t* src, uint8_t* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
#endif
}

// Wait until at most V vector-memory operations of this wave are
// outstanding, binding two 16-byte and two 4-byte loaded values (see wait_vm).
template <int V>
__device__ __forceinline__ void wait_vm4(u32x4_t& a, u32x4_t& b, uint32_t& c, uint32_t& e) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(e) : "n"(V > 63 ? 63 : V) : "memory");
#endif
}

// Same, binding a 16-byte and an 8-byte loaded value.
template <int V>
__device__ __forceinline__ void wait_vm_b64(u32x4_t& a, u32x2_t& b) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(a), "+v"(b) : "n"(V > 63 ? 63 : V) : "memory");
#endif
}

// After a counted wait that also covers them: marks a 16-byte and a 4-byte
// loaded value as written here, so no use moves above it.
__device__ __forceinline__ void bind_loaded(u32x4_t& c, uint32_t& s) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(c), "+v"(s));
#endif
}

// Wait until at most V vector-memory operations of this wave are
// outstanding, binding no register: for LDS DMA copies issued before V
// loads (their data is read from LDS after a barrier, not from registers).
template <int V>
__device__ __forceinline__ void wait_vm_count() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V > 63 ? 63 : V) : "memory");
#endif
}

// Wait until every vector-memory operation of this wave has completed.
__device__ __forceinline__ void wait_vm_all() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// the flag is per template argument, i.e. per kernel instantiation.
template <auto Kernel>
hipError_t set_lds_limit(size_t lds) {
  static std::atomic<bool> done{false};
  if (lds <= 65536 || done.load(std::memory_order_relaxed)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 159 * 1024);
  if (e == hipSuccess) done.store(true, std::memory_order_relaxed);
  return e;
}

}  // namespace nvfp4
