// Read-only streaming kernel: the HBM read ceiling of this GPU at a given
// size, the bound the decode GEMMs are held against.  Decode reads every
// weight from HBM once per token, so the W4A16 GEMM at small token counts is
// a read stream ("SOAR Weekly Champion Notes 08 ...", section "01 A Brief
// Recap of Speculative Decoding").
//
// Each thread keeps U independent 16-byte loads in flight over a grid-stride
// loop (the last index is clamped, so every load is in bounds) and folds the
// data into one word; a workgroup writes its word only if it equals a fixed
// value, so the loads cannot be removed and almost nothing is written.
#include "launchers.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

template <int U, bool NT>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = min(i + u * stride, n16 - 1);
      v[u] = NT ? __builtin_nontemporal_load(p + j) : p[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 63] = acc;
}

template <int U>
hipError_t launch_u(const void* buf, int64_t n16, int grid, int nontemporal, uint32_t* sink, hipStream_t s) {
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL((k_stream_read<U, true>), dim3(grid), dim3(256), 0, s, p, n16, sink);
  else
    hipLaunchKernelGGL((k_stream_read<U, false>), dim3(grid), dim3(256), 0, s, p, n16, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, int grid, int loads_in_flight, int nontemporal,
                              uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  switch (loads_in_flight) {
    case 2: return launch_u<2>(buf, n16, grid, nontemporal, sink, stream);
    case 4: return launch_u<4>(buf, n16, grid, nontemporal, sink, stream);
    case 8: return launch_u<8>(buf, n16, grid, nontemporal, sink, stream);
    default: return launch_u<16>(buf, n16, grid, nontemporal, sink, stream);
  }
}

}  // namespace nvfp4
