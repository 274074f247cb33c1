// W4A16 GEMM for callers that cannot allocate device memory: code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc.
//
// nvfp4_w4a16_gemm needs a caller workspace whenever its plan splits K (fp32
// partial sums [splits, m, n], then the reduction kernel).  This variant
// takes no workspace: the partials go to `scratch`, a fixed array in device
// memory that the loader places on each GPU the library runs on and that
// stays there until the process ends.  Shapes whose plan needs more than
// kScratchBytes are rejected before anything is launched.
//
// In host code `scratch` names a host-side stand-in, not a device address:
// the address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device on the first call made with that device current, and only that
// pointer reaches the kernels.  Every call on one GPU shares its array and
// finds there whatever the last call left: the partial planes are written in
// full before they are read, so nothing needs clearing, but calls that
// overlap on one GPU (concurrent streams or threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>

#include "../../include/nvfp4.h"
#include "launchers.h"

namespace {
constexpr size_t kScratchBytes = (size_t)32 << 20;  // 32 MiB per GPU
std::atomic<void*> g_scratch_ptr[64];                // per device: the address of its `scratch`
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

extern "C" {

NVFP4_API size_t nvfp4_noalloc_scratch_bytes(void) { return kScratchBytes; }

NVFP4_API int nvfp4_w4a16_gemm_noalloc(const void* x, const uint8_t* codes, const uint8_t* scales,
                                       const float* tensor_scale, void* y, int64_t m, int64_t n, int64_t k,
                                       int out_dtype, void* stream) {
  nvfp4::clear_error();
  // 0 for invalid arguments (the GEMM below reports them) and for plans that
  // do not split K
  const size_t need = nvfp4_w4a16_gemm_workspace_size(m, n, k);
  if (need > kScratchBytes) {
    char msg[256];
    std::snprintf(msg, sizeof msg,
                  "m=%lld, n=%lld, k=%lld needs %zu bytes of split-K scratch; the no-allocation entry point "
                  "holds %zu bytes per GPU (use nvfp4_w4a16_gemm with a workspace)",
                  (long long)m, (long long)n, (long long)k, need, kScratchBytes);
    return nvfp4::set_error(NVFP4_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  void* ws = nullptr;
  if (need > 0) {
    int st = nvfp4::device_ok();
    if (st) return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return nvfp4::set_hip_error(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return nvfp4::set_error(NVFP4_ERR_UNSUPPORTED_DEVICE, "device index beyond 63");
    ws = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ws) {
      e = hipGetSymbolAddress(&ws, HIP_SYMBOL(scratch));  // this device's copy (it is current)
      if (e != hipSuccess || !ws) return nvfp4::set_hip_error(e, "hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev].store(ws, std::memory_order_release);
    }
  }
  return nvfp4_w4a16_gemm(x, codes, scales, tensor_scale, y, m, n, k, out_dtype, ws, ws ? kScratchBytes : 0,
                          stream);
}

}  // extern "C"
