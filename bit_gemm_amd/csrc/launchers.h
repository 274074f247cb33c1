// Internal host-side launchers of the gfx950 kernels (called by api.cpp
// after argument validation).  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// The fp32 tensor scale of every output column (weight row) of a GEMM: one
// scale, or one per group of stacked weight matrices (rows [0, b1), [b1, b2),
// [b2, b3), [b3, n); a boundary of INT32_MAX is absent).  Boundaries are
// multiples of 16.  The GEMM sources are compiled twice: once for one scale
// per call (the kernels read ts[0] as always), once with NVFP4_GROUPED set
// into namespace nvfp4::grouped, whose epilogues read each column's scale.
struct RowScale {
  const float* ts;
  int b1, b2, b3;
  __host__ __device__ static RowScale one(const float* t) { return RowScale{t, INT32_MAX, INT32_MAX, INT32_MAX}; }
};

#ifndef NVFP4_GROUPED
#define NVFP4_GROUPED 0
#endif
#if NVFP4_GROUPED
#define NVFP4_VARIANT_BEGIN namespace grouped {
#define NVFP4_VARIANT_END }
#else
#define NVFP4_VARIANT_BEGIN
#define NVFP4_VARIANT_END
#endif

NVFP4_VARIANT_BEGIN
// What the kernels take: the plain build the tensor scale pointer (exactly
// as before groups existed), the grouped build the whole RowScale.
#if NVFP4_GROUPED
typedef RowScale KScale;
inline KScale kscale(const RowScale& r) { return r; }
__device__ __forceinline__ float first_scale(const RowScale& r) { return r.ts[0]; }
// The scale of output column col.
__device__ __forceinline__ float col_scale(const RowScale& rs, int64_t col, float) {
  return rs.ts[(col >= rs.b1) + (col >= rs.b2) + (col >= rs.b3)];
}
#else
typedef const float* __restrict__ KScale;
inline const float* kscale(const RowScale& r) { return r.ts; }
__device__ __forceinline__ float first_scale(const float* t) { return t[0]; }
__device__ __forceinline__ float col_scale(const float*, int64_t, float s0) { return s0; }
#endif
// The split-K reduction as the GEMM launchers call it (launch_split_reduce
// for callers outside them).
hipError_t split_reduce(const float* ws, KScale ts, void* y, int64_t mn, int64_t n, int splits, int out_f32,
                        hipStream_t stream);
NVFP4_VARIANT_END

// Conversion implementations (see NVFP4_IMPL_* in nvfp4.h).
enum ConvImpl { kConvPortable = 1, kConvHw = 2 };

hipError_t launch_quantize_fos(const float* w, int64_t n, int64_t k, const float* amax_in,
                               float* amax_out, float* tensor_scale, uint8_t* codes,
                               uint8_t* scales, uint8_t* m4_mask, int impl, hipStream_t stream);

hipError_t launch_tensor_amax(const float* w, int64_t count, float* amax_out, hipStream_t stream);

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                          void* out, int64_t n, int64_t k, int out_f32, hipStream_t stream);

// Skinny (m <= 64) path.  splits == 0: full-K kernel with `waves` waves per
// workgroup.  splits >= 1: split-K kernel over `kchunk`-wide K chunks, plus a
// reduction kernel when splits > 1 (fp32 partials [splits, m, n] in the
// workspace); nks > 0 selects the pipelined split-K kernel with nks K steps
// unrolled (K a multiple of 128), nks == 0 the general one.
struct SkinnyPlan {
  int splits;
  int kchunk;
  int waves;
  int steps_per_wave;
  int nks;
  size_t ws_bytes;
  int str_rows;   // > 0: streaming kernel with row groups of str_rows rows
  int pk_rounds;  // > 0 (with splits == 0): persistent full-K kernel, `waves` waves x pk_rounds K slices of 512
  int fx_steps;   // > 0: single-launch full-K kernel, `waves` waves x fx_steps K steps of 128 (16 < m <= 64)
  int fx_tiles;   // with fx_steps: 16-row weight tiles per workgroup (1 .. 4)
  int rdot_chunks;  // > 0 (with splits == 0, m == 1): row-per-wave dot-product kernel over rdot_chunks chunks of 2048 k (the last may be partial)
};
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int forced_splits);
hipError_t launch_skinny(const void* x, const uint8_t* codes, const uint8_t* scales,
                         RowScale tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                         int out_f32, const SkinnyPlan& plan, void* workspace, int impl,
                         hipStream_t stream);

// y = s_t * (sum of `splits` fp32 planes [splits, mn] in plane order),
// rounded to the output type; n = columns of y (for per-column scales).
hipError_t launch_split_reduce(const float* ws, RowScale tensor_scale, void* y, int64_t mn, int64_t n,
                               int splits, int out_f32, hipStream_t stream);

// Tiled bf16-MFMA path (any m).  kernel: 0 = 128 x 128 single-stage kernel
// (any K); kernels for K a multiple of 64, weight rows x tokens per
// workgroup: 1 = 128 x 128, 3 = 128 x 64, 4 = 256 x 64 (weights and
// activations staged in LDS), 5 = 256 x 128 with the weights in registers;
// they may split K over `splits` workgroups of `steps_per_split` 64-wide
// steps (fp32 partials [splits, m, n] in the workspace, then the reduction).
struct TiledPlan {
  int kernel;
  int splits;
  int steps_per_split;
  size_t ws_bytes;
};
TiledPlan plan_tiled(int64_t m, int64_t n, int64_t k, int forced_splits);
hipError_t launch_tiled(const void* x, const uint8_t* codes, const uint8_t* scales,
                        RowScale tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                        int out_f32, const TiledPlan& plan, void* workspace, int impl,
                        hipStream_t stream);

// The same three entry points for stacked matrices with one scale per group
// (the sources compiled with NVFP4_GROUPED).
namespace grouped {
hipError_t launch_skinny(const void* x, const uint8_t* codes, const uint8_t* scales, RowScale tensor_scale, void* y,
                         int64_t m, int64_t n, int64_t k, int out_f32, const SkinnyPlan& plan, void* workspace,
                         int impl, hipStream_t stream);
hipError_t launch_split_reduce(const float* ws, RowScale tensor_scale, void* y, int64_t mn, int64_t n, int splits,
                               int out_f32, hipStream_t stream);
hipError_t launch_tiled(const void* x, const uint8_t* codes, const uint8_t* scales, RowScale tensor_scale, void* y,
                        int64_t m, int64_t n, int64_t k, int out_f32, const TiledPlan& plan, void* workspace,
                        int impl, hipStream_t stream);
}  // namespace grouped

// dx[m, k] = s_t * sum_n dy[m, n] * (val * sigma)[n, k] (bf16 dy, packed W):
// 128 x 128 output tiles, the reduction split over `splits` workgroups of
// `steps_per` 64-row steps when tiles are few (fp32 partials [splits, m, k]
// in the workspace, then the split reduction).
struct DxPlan {
  int splits;
  int steps_per;
  size_t ws_bytes;
};
DxPlan plan_gemm_dx(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_dx(const uint16_t* dy, const uint8_t* codes, const uint8_t* scales,
                          const float* tensor_scale, void* dx, int64_t m, int64_t n, int64_t k,
                          int out_f32, const DxPlan& p, void* workspace, hipStream_t stream);
// Activations (bf16 [m, k]) to NVFP4 with the standard block scale; xs
// (optional) receives val * sigma as bf16; with comb_scale, also writes
// s_t * w_scale[0] there.
hipError_t launch_quantize_act(const uint16_t* x, int64_t m, int64_t k, const float* amax_in,
                               float* amax_out, float* tensor_scale, uint8_t* codes,
                               uint8_t* scales, uint16_t* xs, const float* w_scale,
                               float* comb_scale, hipStream_t stream);
// GPTQ inside FourOverSix scales (k % 64 == 0): workspace of
// gptq_workspace_bytes(n, k) (working copy of w, two panels of errors).
size_t gptq_workspace_bytes(int64_t n, int64_t k);
hipError_t launch_gptq(const float* w, int64_t n, int64_t k, const float* hinv_u,
                       const float* amax_in, float* amax_out, float* tensor_scale,
                       uint8_t* codes, uint8_t* scales, uint8_t* m4_mask, void* workspace,
                       int impl, hipStream_t stream);

// GPTQ's damped Hessian H = 2 X^T X + damp * mean(diag) * I (bf16 X [s, k],
// fp32 H [k, k]); workspace: X^T as bf16 [k, s rounded up to 32].
size_t hessian_workspace_bytes(int64_t s, int64_t k);
hipError_t launch_hessian(const uint16_t* x, int64_t s, int64_t k, float damp, float* h, void* workspace,
                          hipStream_t stream);

// Thread-local error text and status codes of the C ABI (api.cpp), for
// entry points defined in other sources.
void clear_error();
int set_error(int status, const char* msg);
int set_hip_error(hipError_t e, const char* where);
int device_ok();  // NVFP4_OK if the current device is gfx950, else the error status

hipError_t launch_selftest_cvt(uint32_t* counters, hipStream_t stream);

// Read-only stream over `bytes` (a multiple of 16) of device memory:
// `grid` workgroups of 256 threads, `loads_in_flight` (2, 4, 8 or 16)
// 16-byte loads per thread in flight, non-temporal loads if `nontemporal`;
// sink: 64 device words, written only for one data-dependent value.
hipError_t launch_stream_read(const void* buf, int64_t bytes, int grid, int loads_in_flight, int nontemporal,
                              uint32_t* sink, hipStream_t stream);

}  // namespace nvfp4
