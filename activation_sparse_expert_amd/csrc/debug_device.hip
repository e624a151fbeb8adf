// Inspection and measurement kernels behind the debug entry points of the ABI:
// the pinned binary32 silu and channel score evaluated on device arrays (the
// same device functions the forward kernels call), and a plain read stream that
// gives the device's measured HBM read ceiling.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace moe_sel {
namespace {

using namespace dev;

__global__ __launch_bounds__(kThreads) void k_silu(const float* z, float* out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) out[i] = silu_pinned(z[i]);
}

__global__ __launch_bounds__(kThreads) void k_score(const int32_t* dg, const int32_t* du, const int32_t* xexp,
                                                    const float4* stats, int kind, float* h, float* score,
                                                    int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float hh, sc;
    pinned_score(dg[i], du[i], xexp[i], stats[i], hh, sc, kind);
    h[i] = hh;
    score[i] = sc;
  }
}

// Every 16-byte piece of the buffer is read once: blocks take consecutive
// 64 KiB spans (each thread 16 loads in flight), XOR what they read, and one
// thread per block folds the result into the sink so the loads cannot be
// dropped. pieces: number of 16-byte pieces.
constexpr int kReadPer = 16;
__global__ __launch_bounds__(kThreads) void k_read(const uint4* buf, int64_t pieces, uint32_t* sink) {
  const int64_t span = (int64_t)kThreads * kReadPer;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * span; base < pieces; base += (int64_t)gridDim.x * span) {
    uint4 v[kReadPer];
#pragma unroll
    for (int u = 0; u < kReadPer; ++u) {
      const int64_t i = base + (int64_t)u * kThreads + threadIdx.x;
      v[u] = i < pieces ? buf[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kReadPer; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  acc = wave_max_u(acc);  // any fold that keeps the loads
  if (threadIdx.x == 0) atomicXor(sink, acc);
}

int grid_for(int64_t n, int64_t per_block, int cap) {
  const int64_t g = (n + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_debug_silu(const float* z, float* out, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_silu, dim3(grid_for(n, kThreads, 65536)), dim3(kThreads), 0, s, z, out, n);
  return hipGetLastError();
}

hipError_t launch_debug_score(const int32_t* dg, const int32_t* du, const int32_t* xexp, const float4* stats,
                              int kind, float* h, float* score, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_score, dim3(grid_for(n, kThreads, 65536)), dim3(kThreads), 0, s, dg, du, xexp, stats, kind,
                     h, score, n);
  return hipGetLastError();
}

hipError_t launch_read_stream(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t pieces = (int64_t)(bytes / 16);
  // a few resident blocks per CU, each looping over 64 KiB spans
  hipLaunchKernelGGL(k_read, dim3(grid_for(pieces, (int64_t)kThreads * kReadPer, 2048)), dim3(kThreads), 0, s,
                     (const uint4*)buf, pieces, sink);
  return hipGetLastError();
}

}  // namespace moe_sel
