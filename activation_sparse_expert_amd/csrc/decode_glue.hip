// Per-layer glue of a stacked decode step around the routed-MoE block: the
// router logits of a token from its hidden state, the residual stream carried
// to the next layer with a root-mean-square renormalisation, and both in one
// launch (the next layer's router reads the renormalised state it forms).
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

// Both steps in one launch: x_out = bf16(v / sqrt(mean(v^2) + eps)), v = x + y,
// and logits[t][e] = sum_i x_out[t][i] w[e][i]. One wave per (token, expert):
// every wave loads the token's x and y and the expert's router row at once
// (16-byte pieces l + 64 i, all in flight: one round trip), forms v and its
// mean square itself (the same lane order in every wave, so every wave gets
// the same scale), then the router dot with the rounded x_out; the expert-0
// wave of the token writes x_out.
constexpr int kGluePieces = 8;  // pieces per lane: d <= 4096

__global__ __launch_bounds__(kThreads) void k_resnorm_router(const uint16_t* x, const uint16_t* y, const uint16_t* w,
                                                             int d, int n_experts, float eps, uint16_t* x_out,
                                                             float* logits) {
  const int t = blockIdx.y;
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= n_experts) return;
  const int npc = d / 8;
  const uint16_t* xr = x + (size_t)t * d;
  const uint16_t* yr = y + (size_t)t * d;
  const uint16_t* wr = w + (size_t)e * d;
  uint4 xv[kGluePieces], yv[kGluePieces], wv[kGluePieces];
#pragma unroll
  for (int u = 0; u < kGluePieces; ++u) {
    const int pc = lane + 64 * u;
    if (pc < npc) {
      xv[u] = *(const uint4*)(xr + 8 * pc);
      yv[u] = *(const uint4*)(yr + 8 * pc);
      wv[u] = *(const uint4*)(wr + 8 * pc);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < kGluePieces; ++u) {
    if (lane + 64 * u < npc) {
      const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w}, yw[4] = {yv[u].x, yv[u].y, yv[u].z, yv[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float v0 = bf16lo(xw[h]) + bf16lo(yw[h]), v1 = bf16hi(xw[h]) + bf16hi(yw[h]);
        ss += v0 * v0;
        ss += v1 * v1;
      }
    }
  }
  const float scale = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
  uint16_t* outr = e == 0 ? x_out + (size_t)t * d : nullptr;
  float s = 0.0f;
#pragma unroll
  for (int u = 0; u < kGluePieces; ++u) {
    const int pc = lane + 64 * u;
    if (pc < npc) {
      const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w}, yw[4] = {yv[u].x, yv[u].y, yv[u].z, yv[u].w};
      const uint32_t ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint16_t n0 = f32_to_bf16_dev((bf16lo(xw[h]) + bf16lo(yw[h])) * scale);
        const uint16_t n1 = f32_to_bf16_dev((bf16hi(xw[h]) + bf16hi(yw[h])) * scale);
        s += bf16f(n0) * bf16lo(ww[h]) + bf16f(n1) * bf16hi(ww[h]);
        o[h] = (uint32_t)n0 | ((uint32_t)n1 << 16);
      }
      if (outr) *(uint4*)(outr + 8 * pc) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  s = wave_sum(s);
  if (lane == 0) logits[(size_t)t * n_experts + e] = s;
}

}  // namespace

hipError_t launch_resnorm_router(const uint16_t* x, const uint16_t* y, const uint16_t* w, int batch, int d,
                                 int n_experts, float eps, uint16_t* x_out, float* logits, hipStream_t stream) {
  hipLaunchKernelGGL(k_resnorm_router, dim3((n_experts + kWaves - 1) / kWaves, batch), dim3(kThreads), 0, stream, x, y,
                     w, d, n_experts, eps, x_out, logits);
  return hipGetLastError();
}

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
