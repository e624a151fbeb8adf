// Per-layer glue of a stacked decode step around the routed-MoE block: the
// router logits of a token from its hidden state, and the residual stream
// carried to the next layer with a root-mean-square renormalisation.
//
// The pages measure MoE blocks inside decoding ("KAIST drops calibration from
// MoE decoding, speeds up blocks by up to 2.69x over vLLM", opening paragraph:
// every decoded token reads its routed experts); these two steps are the
// plainest way to chain blocks into a decode step over many layers.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "internal.h"

namespace moe_sel {
namespace {

using namespace dev;

constexpr int kMaxPieces = 8;  // 16-byte pieces per thread: d <= 8 * 8 * 256

// logits[t][e] = sum_i x[t][i] w[e][i]: one wave per (token, expert), fp32 accumulation
__global__ __launch_bounds__(kThreads) void k_router(const uint16_t* x, const uint16_t* w, int d, int n_experts,
                                                     float* logits) {
  const int t = blockIdx.y;
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= n_experts) return;
  const uint16_t* xr = x + (size_t)t * d;
  const uint16_t* wr = w + (size_t)e * d;
  float s = 0.0f;
  for (int i = 8 * lane; i < d; i += 512) {
    const uint4 xv = *(const uint4*)(xr + i), wv = *(const uint4*)(wr + i);
    s += bf16lo(xv.x) * bf16lo(wv.x) + bf16hi(xv.x) * bf16hi(wv.x);
    s += bf16lo(xv.y) * bf16lo(wv.y) + bf16hi(xv.y) * bf16hi(wv.y);
    s += bf16lo(xv.z) * bf16lo(wv.z) + bf16hi(xv.z) * bf16hi(wv.z);
    s += bf16lo(xv.w) * bf16lo(wv.w) + bf16hi(xv.w) * bf16hi(wv.w);
  }
  s = wave_sum(s);
  if (lane == 0) logits[(size_t)t * n_experts + e] = s;
}

// out = bf16(v / sqrt(mean(v^2) + eps)), v = x + y; one block per token
__global__ __launch_bounds__(kThreads) void k_resnorm(const uint16_t* x, const uint16_t* y, int d, float eps,
                                                      uint16_t* out) {
  __shared__ float s_w[kWaves];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int npc = d / 8;
  float v[kMaxPieces][8];
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < kMaxPieces; ++u) {
    const int pc = tid + u * kThreads;
    if (pc < npc) {
      const uint4 xv = *(const uint4*)(x + (size_t)t * d + 8 * pc), yv = *(const uint4*)(y + (size_t)t * d + 8 * pc);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[u][2 * h] = bf16lo(xw[h]) + bf16lo(yw[h]);
        v[u][2 * h + 1] = bf16hi(xw[h]) + bf16hi(yw[h]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += v[u][q] * v[u][q];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) s_w[tid >> 6] = ss;
  __syncthreads();
  const float ms = ((s_w[0] + s_w[1]) + (s_w[2] + s_w[3])) / (float)d;
  const float scale = 1.0f / sqrtf(ms + eps);
#pragma unroll
  for (int u = 0; u < kMaxPieces; ++u) {
    const int pc = tid + u * kThreads;
    if (pc < npc) {
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o[h] = (uint32_t)f32_to_bf16_dev(v[u][2 * h] * scale) |
               ((uint32_t)f32_to_bf16_dev(v[u][2 * h + 1] * scale) << 16);
      *(uint4*)(out + (size_t)t * d + 8 * pc) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* w, int batch, int d, int n_experts, float* logits,
                         hipStream_t stream) {
  hipLaunchKernelGGL(k_router, dim3((n_experts + kWaves - 1) / kWaves, batch), dim3(kThreads), 0, stream, x, w, d,
                     n_experts, logits);
  return hipGetLastError();
}

hipError_t launch_resnorm(const uint16_t* x, const uint16_t* y, int batch, int d, float eps, uint16_t* out,
                          hipStream_t stream) {
  hipLaunchKernelGGL(k_resnorm, dim3(batch), dim3(kThreads), 0, stream, x, y, d, eps, out);
  return hipGetLastError();
}

}  // namespace moe_sel
