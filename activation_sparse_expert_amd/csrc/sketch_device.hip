// Ternary sketch codes and per-channel statistics built on the device (page
// "KAIST drops calibration from MoE decoding, speeds up blocks by up to 2.69x
// over vLLM", section "A reader built from weights alone": every element of a
// channel's gate and up rows becomes -1, 0 or +1 against a threshold taken
// from the row's mean magnitude, with one scale per row, and the score also
// uses the norm of the channel's down column).
//
// The results are bit-identical to the host preparation: each statistic is
// the exactly rounded value of an exact sum, so no summation order can change
// it. A finite bf16 magnitude is M * 2^(p - 133) with an integer M < 256 and a
// binade p in [0, 253]. One wave handles one channel and first adds the
// integers M (or M^2 for the down column) into 256 per-binade integer bins in
// LDS; these sums are exact (below 2^30 for d <= 16384). The bins are then
// folded into one multi-word integer across the wave and rounded once to
// binary64, ties to even, which is what the host's exact accumulator does.
//
// Per channel j (rows of the [m][3][d] channel-major weights):
//   S = sum |w_i| over the row, mean = S / d (binary64), delta = ratio * mean
//   t_i = sign(w_i) if |w_i| > delta else 0
//   alpha = (float)(sum of |w_i| with t_i != 0 / nnz), 0 when nnz = 0
//   ||down_j|| = (float)sqrt(sum of down_ij^2), the sum exact, the root binary64
// The codes are written in the device layout of the score kernels: t + 1 at
// bits 8ii + 2a of the dword holding elements 64b + 16w + 4a + ii.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "internal.h"

#pragma clang fp contract(off)

namespace moe_sel {
namespace {

constexpr int kSkWaves = 4;  // channels per block, one per wave
constexpr int kBins = 256;   // binades 0..253 and two bins that stay empty

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Exactly rounded binary64 of X * 2^lsb_exp, where the non-negative integer X
// is spread over the wave: lane l holds a piece x_l < 2^61 that sits at 32-bit
// word l / G, i.e. X = sum_l x_l * 2^(32 * (l / G)). ND words hold X after the
// carries. Every lane returns the same value.
template <int G, int ND>
__device__ double exact_round(uint64_t x, int lsb_exp) {
  uint64_t lo = x & 0xFFFFFFFFull, hi = x >> 32;
  for (int o = 1; o < G; o <<= 1) {
    lo += shfl_xor_u64(lo, o);
    hi += shfl_xor_u64(hi, o);
  }
  // word k = low halves of group k + high halves of group k - 1, then carries
  uint32_t w[ND];
  uint64_t carry = 0;
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    uint64_t t = carry;
    if (k * G < 64) t += shfl_u64(lo, k * G);
    if (k >= 1 && (k - 1) * G < 64) t += shfl_u64(hi, (k - 1) * G);
    w[k] = (uint32_t)t;
    carry = t >> 32;
  }
  // top non-zero word and the two below it, plus whether anything lies lower
  int top = -1;
#pragma unroll
  for (int k = 0; k < ND; ++k)
    if (w[k]) top = k;
  if (top < 0) return 0.0;
  uint32_t a = 0, b = 0, c = 0, below = 0;
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    if (k == top) a = w[k];
    if (k == top - 1) b = w[k];
    if (k == top - 2) c = w[k];
    if (k < top - 2) below |= w[k];
  }
  // V = a:b:c (96 bits, value V * 2^(32 * (top - 2))), leading one at bit 64 + ma
  const int ma = 31 - __clz(a);
  const int sh = 12 + ma;  // V >> sh keeps 53 bits
  const uint64_t ab = ((uint64_t)a << 32) | b;
  uint64_t mant;
  int rbit;
  bool sticky;
  if (sh <= 32) {
    mant = (ab << (32 - sh)) | (sh == 32 ? 0u : (uint64_t)(c >> sh));
    rbit = (c >> (sh - 1)) & 1;
    sticky = (c & ((1u << (sh - 1)) - 1u)) != 0u;
  } else {
    const int s2 = sh - 32;  // 1 .. 11
    mant = ab >> s2;
    rbit = (int)((ab >> (s2 - 1)) & 1u);
    sticky = (ab & ((1ull << (s2 - 1)) - 1ull)) != 0ull || c != 0u;
  }
  sticky = sticky || below != 0u;
  int ex = sh + 32 * (top - 2) + lsb_exp;
  if (rbit && (sticky || (mant & 1ull))) {
    ++mant;
    if (mant == (1ull << 53)) {
      mant >>= 1;
      ++ex;
    }
  }
  return ldexp((double)mant, ex);
}

// |w| of a finite bf16 as M * 2^(p - 133)
__device__ __forceinline__ void bf16_binade(uint32_t bits, uint32_t& M, int& p) {
  const int e = (int)((bits >> 7) & 0xFFu);
  const uint32_t f = bits & 0x7Fu;
  M = e ? 128u + f : f;
  p = e ? e - 1 : 0;
}

// Sums of the bins 4l .. 4l+3 of one lane, weighted by 2^(step * i), placed in
// its 32-bit word: step 1 for magnitudes (G = 8 lanes per word), step 2 for
// squares (G = 4).
__device__ __forceinline__ uint64_t lane_piece(const uint32_t* bins, int lane, int step) {
  const uint32_t* q = bins + 4 * lane;
  const uint64_t v = (uint64_t)q[0] + ((uint64_t)q[1] << step) + ((uint64_t)q[2] << (2 * step)) +
                     ((uint64_t)q[3] << (3 * step));
  return step == 1 ? v << (4 * (lane & 7)) : v << (8 * (lane & 3));
}

__global__ __launch_bounds__(kSkWaves * 64) void k_sketch(const uint16_t* __restrict__ wch, int d, int m,
                                                         double ratio, uint32_t* __restrict__ codes,
                                                         float4* __restrict__ stats) {
  __shared__ uint32_t s_bins[kSkWaves][3][kBins];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t ch = (size_t)blockIdx.x * kSkWaves + wv;  // e * m + j; the grid covers E * m exactly
  const int e = (int)(ch / m), j = (int)(ch % m);
  uint32_t* bins = &s_bins[wv][0][0];
  const uint16_t* row = wch + ch * 3 * d;
  const int np = d / 8;                 // 16-byte pieces per row
  const int rounds = (np + 63) / 64;    // uniform over the wave

  for (int i = lane; i < 3 * kBins; i += 64) bins[i] = 0u;
  __syncthreads();
  // pass 1: binade sums of |gate|, |up| and down^2
  for (int r = 0; r < 3; ++r) {
    const uint4* src = (const uint4*)(row + (size_t)r * d);
    uint32_t* br = bins + r * kBins;
    for (int it = 0; it < rounds; ++it) {
      const int p = lane + 64 * it;
      if (p < np) {
        const uint4 v = src[p];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          uint32_t M;
          int pos;
          bf16_binade(wd[h >> 1] >> (16 * (h & 1)), M, pos);
          if (M) atomicAdd(&br[pos], r == 2 ? M * M : M);
        }
      }
    }
  }
  __syncthreads();
  const double sum_g = exact_round<8, 10>(lane_piece(bins, lane, 1), -133);
  const double sum_u = exact_round<8, 10>(lane_piece(bins + kBins, lane, 1), -133);
  const double sum_sq = exact_round<4, 18>(lane_piece(bins + 2 * kBins, lane, 2), -266);
  const double delta_g = ratio * (sum_g / (double)d);
  const double delta_u = ratio * (sum_u / (double)d);
  __syncthreads();
  for (int i = lane; i < 2 * kBins; i += 64) bins[i] = 0u;
  __syncthreads();
  // pass 2: codes, kept sums and counts
  const int g = j / kGroup, cl = j % kGroup;
  uint32_t* ce = codes + (size_t)e * codes_dwords_per_expert(d, m);
  int nnz[2] = {0, 0};
  for (int r = 0; r < 2; ++r) {
    const uint4* src = (const uint4*)(row + (size_t)r * d);
    uint32_t* bk = bins + r * kBins;
    const double delta = r ? delta_u : delta_g;
    for (int it = 0; it < rounds; ++it) {
      const int p = lane + 64 * it;
      const bool live = p < np;  // lanes l and l ^ 1 are live together (np is even)
      uint32_t word = 0;
      if (live) {
        const uint4 v = src[p];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t bits = (wd[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
          uint32_t M;
          int pos;
          bf16_binade(bits, M, pos);
          uint32_t code = 1u;
          if (M && ldexp((double)M, pos - 133) > delta) {
            code = (bits & 0x8000u) ? 0u : 2u;
            atomicAdd(&bk[pos], M);
            ++nnz[r];
          }
          const int o = 8 * (p & 1) + h;  // element within the 16-element dword
          word |= code << (8 * (o & 3) + 2 * (o >> 2));
        }
      }
      word |= (uint32_t)__shfl_xor((int)word, 1, 64);
      if (live && !(p & 1)) ce[codes_dword_index(d, m, g, r, p >> 3, cl, (p & 7) >> 1)] = word;
    }
  }
  int cnt_g = nnz[0], cnt_u = nnz[1];
  for (int o = 32; o > 0; o >>= 1) {
    cnt_g += __shfl_xor(cnt_g, o, 64);
    cnt_u += __shfl_xor(cnt_u, o, 64);
  }
  __syncthreads();
  const double kept_g = exact_round<8, 10>(lane_piece(bins, lane, 1), -133);
  const double kept_u = exact_round<8, 10>(lane_piece(bins + kBins, lane, 1), -133);
  if (lane == 0) {
    float4 st;
    st.x = cnt_g ? (float)(kept_g / (double)cnt_g) : 0.0f;
    st.y = cnt_u ? (float)(kept_u / (double)cnt_u) : 0.0f;
    st.z = (float)sqrt(sum_sq);
    st.w = 0.0f;
    stats[ch] = st;
  }
}

}  // namespace

std::string sketch_stats_device(const uint16_t* wch_dev, int n_experts, int d, int m, double ratio,
                                uint32_t* codes_dev, float* stats_dev, void* stream) {
  if (n_experts <= 0) return std::string();
  if (d % kBlock || m % kGroup || d > 16384) return "device sketch: unsupported shape";
  const size_t channels = (size_t)n_experts * m;  // a multiple of kSkWaves since m % 64 == 0
  hipLaunchKernelGGL(k_sketch, dim3((unsigned)(channels / kSkWaves)), dim3(kSkWaves * 64), 0, (hipStream_t)stream,
                     wch_dev, d, m, ratio, codes_dev, (float4*)stats_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return std::string("device sketch: ") + hipGetErrorString(e);
  return std::string();
}

}  // namespace moe_sel
