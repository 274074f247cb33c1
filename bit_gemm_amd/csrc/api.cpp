// C ABI of libnvfp4 (declared in include/nvfp4.h): argument validation,
// device check, dispatch to the gfx950 kernels, status and error strings.
// Validation runs on the host before any HIP call, so invalid calls return
// an error without touching the GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/nvfp4.h"
#include "launchers.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(NVFP4_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // each dimension < 2^31
constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int64_t kMaxHessianK = 65536;  // H is k x k fp32: 16 GiB at the limit

// Per-device cache of the gfx950 check: 0 unknown, 1 ok, 2 unsupported.
std::atomic<int> g_dev_ok[64];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(NVFP4_ERR_UNSUPPORTED_DEVICE, "device index %d", dev);
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(NVFP4_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return NVFP4_OK;
}

// Conversion implementation used by NVFP4_IMPL_DEFAULT: the gfx950
// instructions with a unit scale, validated bit-exact against the portable
// code on the device by nvfp4_selftest_cvt (counters [0] and [1] zero: every
// fp32 -> FP4 rounding and every FP4 decode).  The scaled decode forms
// (counters [2], [3]) are not exact for non-power-of-two scales and are not
// used.
constexpr int kDefaultImpl = nvfp4::kConvHw;

int resolve_impl(int impl, int* out) {
  if (impl == NVFP4_IMPL_DEFAULT) {
    *out = kDefaultImpl;
  } else if (impl == NVFP4_IMPL_PORTABLE) {
    *out = nvfp4::kConvPortable;
  } else if (impl == NVFP4_IMPL_HWCVT) {
    *out = nvfp4::kConvHw;
  } else {
    return fail(NVFP4_ERR_INVALID_VALUE, "impl %d is not a NVFP4_IMPL_* value", impl);
  }
  return NVFP4_OK;
}

int check_nk(int64_t n, int64_t k) {
  if (n < 0 || k < 0) return fail(NVFP4_ERR_INVALID_VALUE, "negative dimension (n=%lld, k=%lld)", (long long)n, (long long)k);
  if (k % 16 != 0) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k=%lld is not a multiple of 16", (long long)k);
  if (n >= kMaxDim || k >= kMaxDim || (n > 0 && k > kMaxElems / n))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "matrix too large (n=%lld, k=%lld)", (long long)n, (long long)k);
  return NVFP4_OK;
}

// Path selection: the lower-latency kernel for the shape ([Recap] section 1
// picks between its two GEMMs the same way), from latencies measured on
// MI355X (4096 x 4096, 14336 x 4096 and 4096 x 14336 weights, m = 1..256,
// and shapes with other k): the skinny kernels win up to m = 64 on all
// three decoder shapes, the tiled kernels above.  Shapes the streaming
// skinny kernel does not take (k % 512 != 0) keep the tiled path for
// 16 < m <= 64 on large matrices; with k % 64 != 0 the tiled path has only
// its single-stage kernel, so the skinny path keeps m <= 64 there.
int choose_path(int64_t m, int64_t n, int64_t k, int path) {
  if (path != NVFP4_PATH_AUTO) return path;
  if (n >= ((int64_t)1 << 27)) return NVFP4_PATH_TILED;  // beyond the skinny kernels' grid
  if (m <= 16) {
    // 8 < m <= 16 on more than 4096 rows when no split-K skinny kernel
    // applies (k % 512 != 0): the full-K kernel's 16-token workgroups (one
    // per CU) run in serial rounds, and the tiled kernel is faster
    // (5120 x 13888 at m = 16: 34.6 against 44.2 us; 14336 x 4224 at m = 9:
    // 25.7 against 31.7 us; 11008 x 4224 at m = 12: 23.4 against 24.4 us)
    if (m > 8 && n > 4096 && k % 512 != 0 && k % 64 == 0 && n * k > ((int64_t)1 << 25))
      return NVFP4_PATH_TILED;
    return NVFP4_PATH_SKINNY;
  }
  if (m > 64) return NVFP4_PATH_TILED;
  // 16 < m <= 64 with k % 512 == 0: the streaming skinny kernel is faster
  // than the tiled kernel on every decoder shape (14336 x 4096 at m = 64:
  // 23.9 against 31.4 us; 4096 x 14336: 26.0 against 31.8 us) and with
  // 512-wide K chunks (14336 x 4608: 27.1 against 34.1 us)
  if (k % 512 == 0) return NVFP4_PATH_SKINNY;
  // other k: the unpipelined split-K kernel only on small matrices; on large
  // ones the tiled kernel is faster from m = 17 (4096 x 11008 at m = 24 / 48:
  // 22.9 / 25.3 against 30.7 / 35.9 us; 14336 x 4224 at m = 48: 32.4
  // against 43.1 us; 4096 x 4224 keeps the skinny path: 15.4 against 19.3 us)
  if (k % 64 != 0 || n * k <= (int64_t(1) << 25)) return NVFP4_PATH_SKINNY;
  return NVFP4_PATH_TILED;
}

}  // namespace

namespace nvfp4 {
// Error reporting and the device check for entry points defined in other
// sources (the no-allocation GEMM in noalloc.hip).
void clear_error() { g_last_error.clear(); }
int set_error(int status, const char* msg) { return fail(status, "%s", msg); }
int set_hip_error(hipError_t e, const char* where) { return hip_fail(e, where); }
int device_ok() { return check_device(); }
}  // namespace nvfp4

extern "C" {

NVFP4_API int nvfp4_version(void) { return 100; }  // 0.1.0

NVFP4_API const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_INVALID_VALUE: return "NVFP4_ERR_INVALID_VALUE";
    case NVFP4_ERR_UNSUPPORTED_SHAPE: return "NVFP4_ERR_UNSUPPORTED_SHAPE";
    case NVFP4_ERR_MISALIGNED: return "NVFP4_ERR_MISALIGNED";
    case NVFP4_ERR_WORKSPACE_TOO_SMALL: return "NVFP4_ERR_WORKSPACE_TOO_SMALL";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP";
    case NVFP4_ERR_UNSUPPORTED_DEVICE: return "NVFP4_ERR_UNSUPPORTED_DEVICE";
    default: return "NVFP4_ERR_UNKNOWN";
  }
}

NVFP4_API const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

NVFP4_API int nvfp4_quantize_fos_ex(const float* w, int64_t n, int64_t k, const float* amax_in,
                                    float* amax_out, float* tensor_scale, uint8_t* codes,
                                    uint8_t* scales, uint8_t* m4_mask, int impl, void* stream) {
  g_last_error.clear();
  int st = check_nk(n, k);
  if (st) return st;
  const bool empty = (n == 0 || k == 0);
  if (!amax_out || !tensor_scale) return fail(NVFP4_ERR_INVALID_VALUE, "amax_out and tensor_scale are required");
  if (!empty && (!w || !codes || !scales)) return fail(NVFP4_ERR_INVALID_VALUE, "w, codes and scales are required");
  if (!aligned(amax_out, 4) || !aligned(tensor_scale, 4) || (amax_in && !aligned(amax_in, 4)))
    return fail(NVFP4_ERR_MISALIGNED, "scalar arguments must be 4-byte aligned");
  if (!empty && (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 16) || (m4_mask && !aligned(m4_mask, 16))))
    return fail(NVFP4_ERR_MISALIGNED, "w, codes, scales and m4_mask must be 16-byte aligned");
  int ci = 0;
  if ((st = resolve_impl(impl, &ci))) return st;
  if ((st = check_device())) return st;
  hipError_t e = nvfp4::launch_quantize_fos(w, n, k, amax_in, amax_out, tensor_scale, codes, scales,
                                            m4_mask, ci, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return NVFP4_OK;
}

NVFP4_API size_t nvfp4_quantize_fos_gptq_workspace_size(int64_t n, int64_t k) {
  if (n < 0 || k < 0 || n >= kMaxDim || k >= kMaxDim || (n > 0 && k > kMaxElems / n)) return 0;
  return nvfp4::gptq_workspace_bytes(n, k);
}

NVFP4_API int nvfp4_quantize_fos_gptq(const float* w, int64_t n, int64_t k, const float* hinv_u,
                                      const float* amax_in, float* amax_out, float* tensor_scale,
                                      uint8_t* codes, uint8_t* scales, uint8_t* m4_mask,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_nk(n, k);
  if (st) return st;
  if (k % 64 != 0) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k=%lld: GPTQ needs k %% 64 == 0", (long long)k);
  // the largest launch (first trailing update) must stay below 2^32 work-items
  if ((k / 64) * ((n + 63) / 64) + (n + 15) / 16 >= ((int64_t)1 << 24))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "n=%lld, k=%lld: too large for one GPTQ launch", (long long)n, (long long)k);
  const bool empty = (n == 0 || k == 0);
  if (!amax_out || !tensor_scale) return fail(NVFP4_ERR_INVALID_VALUE, "amax_out and tensor_scale are required");
  if (!empty && (!w || !codes || !scales || !hinv_u))
    return fail(NVFP4_ERR_INVALID_VALUE, "w, hinv_u, codes and scales are required");
  if (!aligned(amax_out, 4) || !aligned(tensor_scale, 4) || (amax_in && !aligned(amax_in, 4)))
    return fail(NVFP4_ERR_MISALIGNED, "scalar arguments must be 4-byte aligned");
  if (!empty && (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 16) || !aligned(hinv_u, 16) ||
                 (m4_mask && !aligned(m4_mask, 16))))
    return fail(NVFP4_ERR_MISALIGNED, "w, hinv_u, codes, scales and m4_mask must be 16-byte aligned");
  const size_t need = empty ? 0 : nvfp4::gptq_workspace_bytes(n, k);
  if (need > 0) {
    if (workspace_bytes < need)
      return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!workspace) return fail(NVFP4_ERR_INVALID_VALUE, "workspace is NULL");
    if (!aligned(workspace, 16)) return fail(NVFP4_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  }
  int ci = 0;
  if ((st = resolve_impl(NVFP4_IMPL_DEFAULT, &ci))) return st;
  if ((st = check_device())) return st;
  hipError_t e = nvfp4::launch_gptq(w, n, k, hinv_u, amax_in, amax_out, tensor_scale, codes, scales,
                                    m4_mask, workspace, ci, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq launch");
  return NVFP4_OK;
}

NVFP4_API size_t nvfp4_gptq_hessian_workspace_size(int64_t s, int64_t k) {
  if (s < 0 || k < 0 || k > kMaxHessianK || s >= kMaxDim || (k > 0 && s > kMaxElems / k)) return 0;
  return nvfp4::hessian_workspace_bytes(s, k);
}

NVFP4_API int nvfp4_gptq_hessian(const void* x, int64_t s, int64_t k, float damp, float* h, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (s < 0 || k < 0) return fail(NVFP4_ERR_INVALID_VALUE, "negative dimension (s=%lld, k=%lld)", (long long)s, (long long)k);
  if (k > kMaxHessianK || s >= kMaxDim || (k > 0 && s > kMaxElems / k))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "s=%lld, k=%lld: too large (k <= %lld)", (long long)s, (long long)k,
                (long long)kMaxHessianK);
  if (!(damp >= 0.0f) || !std::isfinite(damp)) return fail(NVFP4_ERR_INVALID_VALUE, "damp must be finite and >= 0");
  if (k == 0) return NVFP4_OK;
  if (!h || (s > 0 && !x)) return fail(NVFP4_ERR_INVALID_VALUE, "x and h are required");
  if (!aligned(h, 4) || (x && !aligned(x, 2))) return fail(NVFP4_ERR_MISALIGNED, "x must be 2-byte and h 4-byte aligned");
  const size_t need = nvfp4::hessian_workspace_bytes(s, k);
  if (need > 0) {
    if (workspace_bytes < need)
      return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!workspace) return fail(NVFP4_ERR_INVALID_VALUE, "workspace is NULL");
    if (!aligned(workspace, 16)) return fail(NVFP4_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  }
  int st = check_device();
  if (st) return st;
  hipError_t e = nvfp4::launch_hessian(reinterpret_cast<const uint16_t*>(x), s, k, damp, h, workspace,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hessian launch");
  return NVFP4_OK;
}

NVFP4_API int nvfp4_tensor_amax(const float* w, int64_t n, int64_t k, float* amax_out, void* stream) {
  g_last_error.clear();
  if (n < 0 || k < 0) return fail(NVFP4_ERR_INVALID_VALUE, "negative dimension");
  if (n >= kMaxDim || k >= kMaxDim || (n > 0 && k > kMaxElems / n))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "matrix too large");
  if ((n * k) % 4 != 0) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "n * k must be a multiple of 4");
  if (!amax_out) return fail(NVFP4_ERR_INVALID_VALUE, "amax_out is required");
  if (n * k > 0 && !w) return fail(NVFP4_ERR_INVALID_VALUE, "w is required");
  if (!aligned(amax_out, 4) || (n * k > 0 && !aligned(w, 16)))
    return fail(NVFP4_ERR_MISALIGNED, "w must be 16-byte and amax_out 4-byte aligned");
  int st = check_device();
  if (st) return st;
  hipError_t e = nvfp4::launch_tensor_amax(w, n * k, amax_out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "amax launch");
  return NVFP4_OK;
}

NVFP4_API int nvfp4_quantize_fos(const float* w, int64_t n, int64_t k, const float* amax_in,
                                 float* amax_out, float* tensor_scale, uint8_t* codes,
                                 uint8_t* scales, uint8_t* m4_mask, void* stream) {
  return nvfp4_quantize_fos_ex(w, n, k, amax_in, amax_out, tensor_scale, codes, scales, m4_mask,
                               NVFP4_IMPL_DEFAULT, stream);
}

NVFP4_API int nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                            void* w_out, int64_t n, int64_t k, int out_dtype, void* stream) {
  g_last_error.clear();
  int st = check_nk(n, k);
  if (st) return st;
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_F32)
    return fail(NVFP4_ERR_INVALID_VALUE, "out_dtype %d", out_dtype);
  if (n == 0 || k == 0) return NVFP4_OK;
  if (!codes || !scales || !tensor_scale || !w_out) return fail(NVFP4_ERR_INVALID_VALUE, "null pointer argument");
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(w_out, 16) || !aligned(tensor_scale, 4))
    return fail(NVFP4_ERR_MISALIGNED, "codes, scales, w_out must be 16-byte aligned");
  if ((st = check_device())) return st;
  hipError_t e = nvfp4::launch_dequant(codes, scales, tensor_scale, w_out, n, k, out_dtype == NVFP4_F32,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return NVFP4_OK;
}

NVFP4_API int nvfp4_w4a16_gemm_path(int64_t m, int64_t n, int64_t k) {
  return choose_path(m, n, k, NVFP4_PATH_AUTO);
}

NVFP4_API size_t nvfp4_w4a16_gemm_workspace_size_ex(int64_t m, int64_t n, int64_t k, int path,
                                                    int split_k) {
  if (m <= 0 || n <= 0 || k <= 0 || split_k < 0) return 0;
  const int p = choose_path(m, n, k, path);
  if (p == NVFP4_PATH_SKINNY) return m > 64 ? 0 : nvfp4::plan_skinny(m, n, k, split_k).ws_bytes;
  if (p == NVFP4_PATH_TILED) return nvfp4::plan_tiled(m, n, k, split_k).ws_bytes;
  return 0;
}

NVFP4_API size_t nvfp4_w4a16_gemm_workspace_size(int64_t m, int64_t n, int64_t k) {
  return nvfp4_w4a16_gemm_workspace_size_ex(m, n, k, NVFP4_PATH_AUTO, 0);
}

namespace {
// The W4A16 GEMM with one tensor scale per output column group (see RowScale).
int gemm_common(const void* x, const uint8_t* codes, const uint8_t* scales, nvfp4::RowScale rs, void* y,
                int64_t m, int64_t n, int64_t k, int out_dtype, void* workspace, size_t workspace_bytes,
                int path, int split_k, int impl, void* stream) {
  const float* tensor_scale = rs.ts;
  int st = check_nk(n, k);
  if (st) return st;
  if (m < 0) return fail(NVFP4_ERR_INVALID_VALUE, "negative m=%lld", (long long)m);
  if (m >= kMaxDim || (m > 0 && n > 0 && m > kMaxElems / n) || (m > 0 && k > 0 && m > kMaxElems / k))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "m=%lld too large", (long long)m);
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_F32)
    return fail(NVFP4_ERR_INVALID_VALUE, "out_dtype %d", out_dtype);
  if (path != NVFP4_PATH_AUTO && path != NVFP4_PATH_SKINNY && path != NVFP4_PATH_TILED)
    return fail(NVFP4_ERR_INVALID_VALUE, "path %d", path);
  if (split_k < 0) return fail(NVFP4_ERR_INVALID_VALUE, "split_k %d", split_k);
  int ci = 0;
  if ((st = resolve_impl(impl, &ci))) return st;
  const int p = choose_path(m, n, k, path);
  if (p == NVFP4_PATH_SKINNY && m > 64)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "the skinny path takes m <= 64 (m=%lld)", (long long)m);
  // a launch grid stays below 2^32 work-items: the skinny kernels run up to
  // 512 threads per 16 weight rows
  if (p == NVFP4_PATH_SKINNY && n >= ((int64_t)1 << 27))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "the skinny path takes n < 2^27 (n=%lld)", (long long)n);
  if (m == 0 || n == 0) return NVFP4_OK;
  if (!y || !tensor_scale) return fail(NVFP4_ERR_INVALID_VALUE, "y and tensor_scale are required");
  if (k > 0 && (!x || !codes || !scales)) return fail(NVFP4_ERR_INVALID_VALUE, "x, codes and scales are required");
  if (!aligned(y, 16) || !aligned(tensor_scale, 4) || (k > 0 && (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 16))))
    return fail(NVFP4_ERR_MISALIGNED, "x, codes, scales, y must be 16-byte aligned");
  nvfp4::SkinnyPlan plan{};
  nvfp4::TiledPlan tplan{};
  size_t need = 0;
  if (p == NVFP4_PATH_SKINNY) {
    plan = nvfp4::plan_skinny(m, n, k, split_k);
    need = plan.ws_bytes;
  } else {
    tplan = nvfp4::plan_tiled(m, n, k, split_k);
    need = tplan.ws_bytes;
  }
  if (need > 0) {
    if (workspace_bytes < need)
      return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (!workspace) return fail(NVFP4_ERR_INVALID_VALUE, "workspace is NULL");
    if (!aligned(workspace, 16)) return fail(NVFP4_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  }
  if ((st = check_device())) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  const bool grouped = rs.b1 != INT32_MAX;
  const int f32 = out_dtype == NVFP4_F32;
  if (p == NVFP4_PATH_SKINNY)
    e = grouped ? nvfp4::grouped::launch_skinny(x, codes, scales, rs, y, m, n, k, f32, plan, workspace, ci, s)
                : nvfp4::launch_skinny(x, codes, scales, rs, y, m, n, k, f32, plan, workspace, ci, s);
  else
    e = grouped ? nvfp4::grouped::launch_tiled(x, codes, scales, rs, y, m, n, k, f32, tplan, workspace, ci, s)
                : nvfp4::launch_tiled(x, codes, scales, rs, y, m, n, k, f32, tplan, workspace, ci, s);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return NVFP4_OK;
}
}  // namespace

NVFP4_API int nvfp4_w4a16_gemm_ex(const void* x, const uint8_t* codes, const uint8_t* scales,
                                  const float* tensor_scale, void* y, int64_t m, int64_t n,
                                  int64_t k, int out_dtype, void* workspace,
                                  size_t workspace_bytes, int path, int split_k, int impl,
                                  void* stream) {
  g_last_error.clear();
  return gemm_common(x, codes, scales, nvfp4::RowScale::one(tensor_scale), y, m, n, k, out_dtype, workspace,
                     workspace_bytes, path, split_k, impl, stream);
}

NVFP4_API int nvfp4_w4a16_gemm_grouped(const void* x, const uint8_t* codes, const uint8_t* scales,
                                       const float* tensor_scales, const int64_t* group_rows, int groups,
                                       void* y, int64_t m, int64_t k, int out_dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (groups < 1 || groups > 4) return fail(NVFP4_ERR_INVALID_VALUE, "groups=%d: 1 to 4", groups);
  if (!group_rows) return fail(NVFP4_ERR_INVALID_VALUE, "group_rows is required");
  int64_t n = 0;
  int b[3] = {INT32_MAX, INT32_MAX, INT32_MAX};
  for (int g = 0; g < groups; ++g) {
    if (group_rows[g] <= 0 || group_rows[g] % 16 != 0)
      return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "group %d has %lld rows: a positive multiple of 16", g,
                  (long long)group_rows[g]);
    if (g > 0) b[g - 1] = (int)n;
    n += group_rows[g];
    if (n >= ((int64_t)1 << 27)) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "too many rows (%lld)", (long long)n);
  }
  return gemm_common(x, codes, scales, nvfp4::RowScale{tensor_scales, b[0], b[1], b[2]}, y, m, n, k, out_dtype,
                     workspace, workspace_bytes, NVFP4_PATH_AUTO, 0, NVFP4_IMPL_DEFAULT, stream);
}

NVFP4_API int nvfp4_w4a16_gemm(const void* x, const uint8_t* codes, const uint8_t* scales,
                               const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                               int out_dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return nvfp4_w4a16_gemm_ex(x, codes, scales, tensor_scale, y, m, n, k, out_dtype, workspace,
                             workspace_bytes, NVFP4_PATH_AUTO, 0, NVFP4_IMPL_DEFAULT, stream);
}

NVFP4_API size_t nvfp4_w4a16_gemm_dx_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim ||
      m > kMaxElems / k || n > kMaxElems / k)
    return 0;
  return nvfp4::plan_gemm_dx(m, n, k).ws_bytes;
}

NVFP4_API int nvfp4_w4a16_gemm_dx(const void* dy, const uint8_t* codes, const uint8_t* scales,
                                  const float* tensor_scale, void* dx, int64_t m, int64_t n, int64_t k,
                                  int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_nk(n, k);
  if (st) return st;
  if (m < 0) return fail(NVFP4_ERR_INVALID_VALUE, "negative m=%lld", (long long)m);
  if (m >= kMaxDim || (m > 0 && n > 0 && m > kMaxElems / n) || (m > 0 && k > 0 && m > kMaxElems / k))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "m=%lld too large", (long long)m);
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_F32)
    return fail(NVFP4_ERR_INVALID_VALUE, "out_dtype %d", out_dtype);
  if (m == 0 || k == 0) return NVFP4_OK;
  if (!dx || !tensor_scale) return fail(NVFP4_ERR_INVALID_VALUE, "dx and tensor_scale are required");
  if (n > 0 && (!dy || !codes || !scales)) return fail(NVFP4_ERR_INVALID_VALUE, "dy, codes and scales are required");
  if (!aligned(dx, 16) || !aligned(tensor_scale, 4) || (n > 0 && (!aligned(dy, 16) || !aligned(codes, 16) || !aligned(scales, 16))))
    return fail(NVFP4_ERR_MISALIGNED, "dy, codes, scales, dx must be 16-byte aligned");
  const nvfp4::DxPlan plan = nvfp4::plan_gemm_dx(m, n, k);
  if (plan.ws_bytes > 0) {
    if (workspace_bytes < plan.ws_bytes)
      return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, plan.ws_bytes);
    if (!workspace) return fail(NVFP4_ERR_INVALID_VALUE, "workspace is NULL");
    if (!aligned(workspace, 16)) return fail(NVFP4_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  }
  if ((st = check_device())) return st;
  hipError_t e = nvfp4::launch_gemm_dx(static_cast<const uint16_t*>(dy), codes, scales, tensor_scale, dx, m, n, k,
                                       out_dtype == NVFP4_F32, plan, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm_dx launch");
  return NVFP4_OK;
}

NVFP4_API int nvfp4_quantize_act(const void* x, int64_t m, int64_t k, const float* amax_in,
                                 float* amax_out, float* tensor_scale, uint8_t* codes,
                                 uint8_t* scales, void* x_blockscaled, void* stream) {
  g_last_error.clear();
  int st = check_nk(m, k);
  if (st) return st;
  const bool empty = (m == 0 || k == 0);
  if (!amax_out || !tensor_scale) return fail(NVFP4_ERR_INVALID_VALUE, "amax_out and tensor_scale are required");
  if (!empty && (!x || !codes || !scales)) return fail(NVFP4_ERR_INVALID_VALUE, "x, codes and scales are required");
  if (!aligned(amax_out, 4) || !aligned(tensor_scale, 4) || (amax_in && !aligned(amax_in, 4)))
    return fail(NVFP4_ERR_MISALIGNED, "scalar arguments must be 4-byte aligned");
  if (!empty && (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 16) ||
                 (x_blockscaled && !aligned(x_blockscaled, 16))))
    return fail(NVFP4_ERR_MISALIGNED, "x, codes, scales and x_blockscaled must be 16-byte aligned");
  if ((st = check_device())) return st;
  hipError_t e = nvfp4::launch_quantize_act(static_cast<const uint16_t*>(x), m, k, amax_in, amax_out,
                                            tensor_scale, codes, scales, static_cast<uint16_t*>(x_blockscaled),
                                            nullptr, nullptr, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize_act launch");
  return NVFP4_OK;
}

// W4A4 workspace: 256 bytes of scalars (amax, activation tensor scale, the
// product of both tensor scales), the block-scaled bf16 activations, their
// codes and scales, then the GEMM's own workspace; each piece 256-aligned
// from the first 256-byte boundary of the caller's (16-byte aligned)
// buffer, whose size includes the 240 bytes that rounding may skip.
static size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }
static size_t w4a4_act_bytes(int64_t m, int64_t k) {
  const size_t e = (size_t)m * (size_t)k;
  return 256 + round256(2 * e) + round256(e / 2) + round256(e / 16);
}
constexpr size_t kW4a4Slack = 240;

NVFP4_API size_t nvfp4_w4a4_gemm_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim ||
      m > kMaxElems / k || m > kMaxElems / n)
    return 0;
  return kW4a4Slack + w4a4_act_bytes(m, k) + nvfp4_w4a16_gemm_workspace_size(m, n, k);
}

NVFP4_API int nvfp4_w4a4_gemm(const void* x, const uint8_t* codes, const uint8_t* scales,
                              const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                              int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_nk(n, k);
  if (st) return st;
  if (m < 0) return fail(NVFP4_ERR_INVALID_VALUE, "negative m=%lld", (long long)m);
  if (m >= kMaxDim || (m > 0 && n > 0 && m > kMaxElems / n) || (m > 0 && k > 0 && m > kMaxElems / k))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "m=%lld too large", (long long)m);
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_F32)
    return fail(NVFP4_ERR_INVALID_VALUE, "out_dtype %d", out_dtype);
  if (m == 0 || n == 0) return NVFP4_OK;
  if (!y || !tensor_scale) return fail(NVFP4_ERR_INVALID_VALUE, "y and tensor_scale are required");
  if (k > 0 && (!x || !codes || !scales)) return fail(NVFP4_ERR_INVALID_VALUE, "x, codes and scales are required");
  if (!aligned(y, 16) || !aligned(tensor_scale, 4) || (k > 0 && (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 16))))
    return fail(NVFP4_ERR_MISALIGNED, "x, codes, scales, y must be 16-byte aligned");
  if (k == 0) return nvfp4_w4a16_gemm(x, codes, scales, tensor_scale, y, m, n, k, out_dtype, nullptr, 0, stream);
  const size_t act = w4a4_act_bytes(m, k);
  const size_t gws = nvfp4_w4a16_gemm_workspace_size(m, n, k);
  if (workspace_bytes < kW4a4Slack + act + gws)
    return fail(NVFP4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes,
                kW4a4Slack + act + gws);
  if (!workspace) return fail(NVFP4_ERR_INVALID_VALUE, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(NVFP4_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if ((st = check_device())) return st;
  const uintptr_t wsa = reinterpret_cast<uintptr_t>(workspace);
  uint8_t* base = static_cast<uint8_t*>(workspace) + (((wsa + 255) & ~(uintptr_t)255) - wsa);
  float* sc = reinterpret_cast<float*>(base);  // [0] amax, [1] s_t of x, [2] product of tensor scales
  const size_t e = (size_t)m * (size_t)k;
  uint16_t* xs = reinterpret_cast<uint16_t*>(base + 256);
  uint8_t* xc = base + 256 + round256(2 * e);
  uint8_t* xsc = xc + round256(e / 2);
  hipError_t he = nvfp4::launch_quantize_act(static_cast<const uint16_t*>(x), m, k, nullptr, sc, sc + 1, xc, xsc,
                                             xs, tensor_scale, sc + 2, reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "quantize_act launch");
  // the bf16 MFMA GEMM of the block-scaled activations, scaled once by the
  // product of both tensor scales
  return nvfp4_w4a16_gemm(xs, codes, scales, sc + 2, y, m, n, k, out_dtype, base + act, gws, stream);
}

NVFP4_API int nvfp4_stream_read(const void* buf, size_t bytes, int grid, int loads_in_flight, int nontemporal,
                                uint32_t* sink, void* stream) {
  g_last_error.clear();
  if (bytes == 0) return NVFP4_OK;
  if (!buf || !sink) return fail(NVFP4_ERR_INVALID_VALUE, "buf and sink are required");
  if (bytes % 16 != 0) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "bytes=%zu is not a multiple of 16", bytes);
  if (bytes >= ((size_t)1 << 40)) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "bytes=%zu too large", bytes);
  if (grid < 1 || grid > 65536) return fail(NVFP4_ERR_INVALID_VALUE, "grid %d (1 .. 65536)", grid);
  if (loads_in_flight != 2 && loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16)
    return fail(NVFP4_ERR_INVALID_VALUE, "loads_in_flight %d (2, 4, 8 or 16)", loads_in_flight);
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(NVFP4_ERR_MISALIGNED, "buf must be 16-byte, sink 4-byte aligned");
  int st = check_device();
  if (st) return st;
  hipError_t e = nvfp4::launch_stream_read(buf, (int64_t)bytes, grid, loads_in_flight, nontemporal != 0, sink,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  return NVFP4_OK;
}

NVFP4_API int nvfp4_selftest_cvt(uint32_t* counters_out, void* stream) {
  g_last_error.clear();
  if (!counters_out) return fail(NVFP4_ERR_INVALID_VALUE, "counters_out is NULL");
  if (!aligned(counters_out, 4)) return fail(NVFP4_ERR_MISALIGNED, "counters_out must be 4-byte aligned");
  int st = check_device();
  if (st) return st;
  hipError_t e = nvfp4::launch_selftest_cvt(counters_out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selftest launch");
  return NVFP4_OK;
}

}  // extern "C"
