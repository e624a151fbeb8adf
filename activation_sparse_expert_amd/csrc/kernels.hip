// Device kernels of the routed-MoE block with sketch-based top-k channel
// selection, written for gfx950 (CDNA4, 64-wide wavefronts).
//
// Phases of one forward call, in order (pages cited by title and section):
//   route+quantise  top_e experts per token, gate weights, int8 activations
//                   ("KAIST drops calibration from MoE decoding...", opening
//                   paragraph: each token reads its routed experts);
//   score           ternary-sketch GEMV over packed 2-bit codes, pinned binary32
//                   channel scores (same page, "A reader built from weights alone");
//   select          per (token, expert) top-k by radix passes over the score bits,
//                   lowest index on ties, output ascending (same page, "Top-k
//                   instead of a threshold"); also the compensation coordinates
//                   z = Q^T h_hat over the skipped channels;
//   gate/up         SwiGLU activations of the selected channels only, from the
//                   channel-major bf16 layout (fp32 accumulation);
//   down            per output slice, sum of h_j * down_j over the selected
//                   channels plus the low-rank term P z;
//   combine         gate-weighted sum over a token's experts, bf16 output.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "internal.h"
#include "kernels.h"

namespace moe_sel {
namespace {

using namespace dev;

// ===========================================================================
// Phase 1: routing and activation quantisation, one block per token.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_route_quant(FwdArgs a) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ int s_sel[64];
  __shared__ float s_selv[64];
  __shared__ uint32_t s_amax[kWaves];

  // --- top_e experts: repeated block arg-max, larger logit first, lower index on ties
  const float* L = a.logits + (size_t)t * a.n_experts;
  constexpr int kMaxPer = 4;  // n_experts <= 1024
  float v[kMaxPer];
  bool live[kMaxPer];
  for (int u = 0; u < kMaxPer; ++u) {
    const int idx = tid + u * kThreads;
    live[u] = idx < a.n_experts;
    v[u] = live[u] ? L[idx] : 0.0f;
  }
  for (int s = 0; s < a.top_e; ++s) {
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
    for (int u = 0; u < kMaxPer; ++u) {
      const int idx = tid + u * kThreads;
      if (live[u] && (bi == 0x7FFFFFFF || v[u] > bv)) {
        bv = v[u];
        bi = idx;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      const bool take = (oi != 0x7FFFFFFF) && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
      if (take) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_v[wave] = bv;
      s_i[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float fv = s_v[0];
      int fi = s_i[0];
      for (int w = 1; w < kWaves; ++w) {
        const int oi = s_i[w];
        const float ov = s_v[w];
        if (oi != 0x7FFFFFFF && (fi == 0x7FFFFFFF || ov > fv || (ov == fv && oi < fi))) {
          fv = ov;
          fi = oi;
        }
      }
      s_sel[s] = fi;
      s_selv[s] = fv;
    }
    __syncthreads();
    const int chosen = s_sel[s];
    for (int u = 0; u < kMaxPer; ++u)
      if (tid + u * kThreads == chosen) live[u] = false;
  }
  if (tid < a.top_e) {
    const float top = s_selv[0];
    float denom = 0.0f;
    for (int s = 0; s < a.top_e; ++s) denom += __expf(s_selv[s] - top);
    const int p = t * a.top_e + tid;
    a.pair_expert[p] = s_sel[tid];
    a.pair_w[p] = __expf(s_selv[tid] - top) / denom;
  }

  // --- int8 activations with a power-of-two scale
  const uint16_t* x = a.x + (size_t)t * a.d;
  uint32_t amax = 0;
  for (int i = tid; i < a.d; i += kThreads) amax = max(amax, (uint32_t)(x[i] & 0x7FFFu));
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, 64));
  if (lane == 0) s_amax[wave] = amax;
  __syncthreads();
  amax = s_amax[0];
  for (int w = 1; w < kWaves; ++w) amax = max(amax, s_amax[w]);
  int e = 0;
  if (amax != 0) {
    const float av = __uint_as_float(amax << 16);
    int ex;
    (void)__builtin_frexpf(av, &ex);  // av = f * 2^ex, f in [0.5, 1)
    e = ex - 7;
    if (__builtin_ldexpf(av, -e) > 127.0f) e += 1;
  }
  if (tid == 0) a.xexp[t] = e;
  int8_t* q = a.xq + (size_t)t * a.d;
  for (int i = tid; i < a.d; i += kThreads) {
    const float xv = __uint_as_float((uint32_t)x[i] << 16);
    q[i] = amax ? (int8_t)(int)__builtin_rintf(__builtin_ldexpf(xv, -e)) : (int8_t)0;
  }
}

// ===========================================================================
// Phase 2: sketch scores. One block per (pair, 64-channel group): wave w scores
// matrix w/2 (gate, up) over half w%2 of the hidden dimension; lane = channel.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_score(FwdArgs a) {
  extern __shared__ int4 s_xq4[];  // d bytes of int8 activations
  __shared__ int s_part[kWaves][64];
  const int groups = a.m / kGroup;
  const int p = blockIdx.x / groups, g = blockIdx.x % groups;
  const int t = p / a.top_e;
  const int e = a.pair_expert[p];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int4* xsrc = (const int4*)(a.xq + (size_t)t * a.d);
  for (int i = tid; i < a.d / 16; i += kThreads) s_xq4[i] = xsrc[i];
  __syncthreads();
  const int mat = wave >> 1, half = wave & 1;
  const int nb = a.d / kBlock;
  const int b0 = half ? nb / 2 : 0, b1 = half ? nb : nb / 2;
  const uint4* cp = (const uint4*)(a.codes + (size_t)e * codes_dwords_per_expert(a.d, a.m) +
                                   codes_dword_index(a.d, a.m, g, mat, 0, lane, 0));
  int acc = 0, qs = 0;
  for (int b = b0; b < b1; ++b) {
    const uint4 c = cp[(size_t)b * 64];
    const int4* xb = s_xq4 + b * 4;
    const int4 x0 = xb[0], x1 = xb[1], x2 = xb[2], x3 = xb[3];
    acc = dot_codes16(c.x, x0, acc);
    acc = dot_codes16(c.y, x1, acc);
    acc = dot_codes16(c.z, x2, acc);
    acc = dot_codes16(c.w, x3, acc);
    qs = byte_sum4(x0, qs);
    qs = byte_sum4(x1, qs);
    qs = byte_sum4(x2, qs);
    qs = byte_sum4(x3, qs);
  }
  s_part[wave][lane] = acc - qs;  // sum (code - 1) * q = sum t * q
  __syncthreads();
  if (wave == 0) {
    const int dg = s_part[0][lane] + s_part[1][lane];
    const int du = s_part[2][lane] + s_part[3][lane];
    const int j = g * kGroup + lane;
    const float4 st = a.stats[(size_t)e * a.m + j];
    float h, sc;
    pinned_score(dg, du, a.xexp[t], st, h, sc);
    a.hhat[(size_t)p * a.m + j] = h;
    a.score[(size_t)p * a.m + j] = sc;
  }
}

// ===========================================================================
// Phase 3: top-k per pair by four 8-bit radix passes over the score bits
// (non-negative binary32 scores order like their bit patterns), then an
// index-order compaction with wave ballots. One block per pair.
// Also z = sum over skipped channels of h_hat_j * Q[j, :].
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_select(FwdArgs a) {
  extern __shared__ uint32_t s_dyn[];  // keys [m], then selection bits [m/32]
  __shared__ int s_hist[256];
  __shared__ int s_tmp[kWaves + 1];
  __shared__ int s_digit, s_gt;
  __shared__ float s_z[kWaves][128];
  const int p = blockIdx.x;
  const int m = a.m, k = a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* s_keys = s_dyn;
  uint32_t* s_bits = s_dyn + m;
  const float* sc = a.score + (size_t)p * m;
  for (int j = tid; j < m; j += kThreads) s_keys[j] = __float_as_uint(sc[j]);
  for (int w = tid; w < m / 32; w += kThreads) s_bits[w] = 0u;
  __syncthreads();
  int* idx_out = a.sel_idx + (size_t)p * m;
  int count = 0;
  if (k >= m) {
    for (int j = tid; j < m; j += kThreads) idx_out[j] = j;
    for (int w = tid; w < m / 32; w += kThreads) s_bits[w] = 0xFFFFFFFFu;
    count = m;
  } else if (k > 0) {
    uint32_t prefix = 0, pmask = 0;
    int krem = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      s_hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < m; j += kThreads) {
        const uint32_t key = s_keys[j];
        if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // thread tid owns bin 255 - tid: an inclusive scan over threads is a suffix scan over bins
      const int c = s_hist[255 - tid];
      int incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (lane == 63) s_tmp[wave] = incl;
      __syncthreads();
      for (int w = 0; w < wave; ++w) incl += s_tmp[w];
      if (incl - c < krem && krem <= incl) {
        s_digit = 255 - tid;
        s_gt = incl - c;
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      pmask |= 255u << shift;
      krem -= s_gt;
      __syncthreads();
    }
    // prefix is the k-th largest key; take every larger key and the krem lowest-index equal keys
    int run_eq = 0, run_sel = 0;
    for (int base = 0; base < m; base += kThreads) {
      const int j = base + tid;
      const uint32_t key = j < m ? s_keys[j] : 0u;
      const bool gt = j < m && key > prefix;
      const bool eq = j < m && key == prefix;
      int eq_tot, sel_tot;
      const int eq_before = block_excl_count(eq, s_tmp, &eq_tot);
      const bool take = gt || (eq && run_eq + eq_before < krem);
      const int sel_before = block_excl_count(take, s_tmp, &sel_tot);
      if (take) {
        idx_out[run_sel + sel_before] = j;
        atomicOr(&s_bits[j >> 5], 1u << (j & 31));
      }
      run_eq += eq_tot;
      run_sel += sel_tot;
    }
    count = run_sel;
  }
  __syncthreads();
  if (tid == 0) a.sel_count[p] = count;
  // compensation coordinates over the skipped channels
  const int r = a.r;
  if (r > 0) {
    const int e = a.pair_expert[p];
    const uint16_t* Q = a.qmat + (size_t)e * m * r;
    const float* hh = a.hhat + (size_t)p * m;
    float z0 = 0.0f, z1 = 0.0f;
    for (int j = wave; j < m; j += kWaves) {
      if ((s_bits[j >> 5] >> (j & 31)) & 1u) continue;
      const float hj = hh[j];
      const uint16_t* row = Q + (size_t)j * r;
      if (lane < r) z0 += hj * __uint_as_float((uint32_t)row[lane] << 16);
      if (lane + 64 < r) z1 += hj * __uint_as_float((uint32_t)row[lane + 64] << 16);
    }
    s_z[wave][lane] = z0;
    s_z[wave][lane + 64] = z1;
    __syncthreads();
    if (tid < r) {
      float z = 0.0f;
      for (int w = 0; w < kWaves; ++w) z += s_z[w][tid];
      a.zvec[(size_t)p * r + tid] = z;
    }
  }
}

// ===========================================================================
// Phase 4: SwiGLU activations of the selected channels (or all, dense).
// One block per (pair, chunk of kChunk channels); thread t owns 16-byte slots
// t, t+256, ... of the hidden dimension.
// ===========================================================================
constexpr int kChunk = 4;
constexpr int kMaxSlots = 8;  // d <= 16384

__global__ __launch_bounds__(kThreads) void k_gate_up(FwdArgs a, int dense) {
  __shared__ float s_red[kWaves][2 * kChunk];
  const int m = a.m, d = a.d;
  const int count = dense ? m : a.k;
  const int chunks = (count + kChunk - 1) / kChunk;
  const int p = blockIdx.x / chunks, ch = blockIdx.x % chunks;
  const int t = p / a.top_e;
  const int e = a.pair_expert[p];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nslots = d / 8;
  const uint16_t* xrow = a.x + (size_t)t * d;
  float xv[kMaxSlots][8];
  for (int u = 0; u < kMaxSlots; ++u) {
    const int s = tid + u * kThreads;
    if (s < nslots) {
      const uint4 w = *(const uint4*)(xrow + 8 * s);
      xv[u][0] = bf16lo(w.x); xv[u][1] = bf16hi(w.x);
      xv[u][2] = bf16lo(w.y); xv[u][3] = bf16hi(w.y);
      xv[u][4] = bf16lo(w.z); xv[u][5] = bf16hi(w.z);
      xv[u][6] = bf16lo(w.w); xv[u][7] = bf16hi(w.w);
    }
  }
  const int* idx = a.sel_idx + (size_t)p * m;
  float gs[kChunk], us[kChunk];
  for (int c = 0; c < kChunk; ++c) {
    gs[c] = 0.0f;
    us[c] = 0.0f;
    const int i = ch * kChunk + c;
    if (i >= count) continue;
    const int j = dense ? i : idx[i];
    const uint16_t* base = a.wch + ((size_t)e * m + j) * 3 * d;
    for (int u = 0; u < kMaxSlots; ++u) {
      const int s = tid + u * kThreads;
      if (s < nslots) {
        gs[c] += dot8_bf16(*(const uint4*)(base + 8 * s), xv[u]);
        us[c] += dot8_bf16(*(const uint4*)(base + d + 8 * s), xv[u]);
      }
    }
  }
  for (int c = 0; c < kChunk; ++c) {
    const float g = wave_sum(gs[c]);
    const float u = wave_sum(us[c]);
    if (lane == 0) {
      s_red[wave][2 * c] = g;
      s_red[wave][2 * c + 1] = u;
    }
  }
  __syncthreads();
  if (tid < kChunk) {
    const int i = ch * kChunk + tid;
    if (i < count) {
      float g = 0.0f, u = 0.0f;
      for (int w = 0; w < kWaves; ++w) {
        g += s_red[w][2 * tid];
        u += s_red[w][2 * tid + 1];
      }
      a.hsel[(size_t)p * m + i] = silu_f32(g) * u;
    }
  }
}

// ===========================================================================
// Phase 5: one block per (pair, 64-element output slice): sum over the pair's
// selected channels of h_i * down_j[slice] (128-byte pieces), plus P z.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_down(FwdArgs a, int dense) {
  __shared__ float s_red[32][65];
  const int m = a.m, d = a.d;
  const int slices = d / 64;
  const int p = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int e = a.pair_expert[p];
  const int count = dense ? m : a.sel_count[p];
  const int tid = threadIdx.x;
  const int part = tid & 7, row = tid >> 3;  // 32 rows x 8 parts of 16 bytes
  const int* idx = a.sel_idx + (size_t)p * m;
  const float* hs = a.hsel + (size_t)p * m;
  float acc[8];
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  for (int i = row; i < count; i += 32) {
    const int j = dense ? i : idx[i];
    const uint4 w = *(const uint4*)(a.wch + (((size_t)e * m + j) * 3 + 2) * d + 64 * sl + 8 * part);
    const float h = hs[i];
    acc[0] += h * bf16lo(w.x); acc[1] += h * bf16hi(w.x);
    acc[2] += h * bf16lo(w.y); acc[3] += h * bf16hi(w.y);
    acc[4] += h * bf16lo(w.z); acc[5] += h * bf16hi(w.z);
    acc[6] += h * bf16lo(w.w); acc[7] += h * bf16hi(w.w);
  }
  for (int q = 0; q < 8; ++q) s_red[row][part * 8 + q] = acc[q];
  __syncthreads();
  if (tid < 64) {
    float y = 0.0f;
    for (int rr = 0; rr < 32; ++rr) y += s_red[rr][tid];
    const int r = a.r;
    if (!dense && r > 0) {
      const uint16_t* P = a.pmat + (size_t)e * r * d;
      const float* z = a.zvec + (size_t)p * r;
      for (int c = 0; c < r; ++c) y += z[c] * __uint_as_float((uint32_t)P[(size_t)c * d + 64 * sl + tid] << 16);
    }
    a.ypart[(size_t)p * d + 64 * sl + tid] = y;
  }
}

// ===========================================================================
// Phase 6: gate-weighted sum over a token's experts, bf16 output.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_combine(FwdArgs a) {
  const int per_tok = (a.d + kThreads - 1) / kThreads;
  const int t = blockIdx.x / per_tok, blk = blockIdx.x % per_tok;
  const int i = blk * kThreads + threadIdx.x;
  if (i >= a.d) return;
  float y = 0.0f;
  for (int s = 0; s < a.top_e; ++s) {
    const int p = t * a.top_e + s;
    y += a.pair_w[p] * a.ypart[(size_t)p * a.d + i];
  }
  a.out[(size_t)t * a.d + i] = f32_to_bf16_dev(y);
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, bool dense, hipStream_t stream) {
  const int pairs = a.batch * a.top_e;
  hipLaunchKernelGGL(k_route_quant, dim3(a.batch), dim3(kThreads), 0, stream, a);
  if (!dense) {
    hipLaunchKernelGGL(k_score, dim3(pairs * (a.m / kGroup)), dim3(kThreads), (size_t)a.d, stream, a);
    hipLaunchKernelGGL(k_select, dim3(pairs), dim3(kThreads), (size_t)(a.m + a.m / 32) * 4, stream, a);
  }
  const int count = dense ? a.m : a.k;
  if (count > 0) {
    const int chunks = (count + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(k_gate_up, dim3(pairs * chunks), dim3(kThreads), 0, stream, a, dense ? 1 : 0);
  }
  hipLaunchKernelGGL(k_down, dim3(pairs * (a.d / 64)), dim3(kThreads), 0, stream, a, dense ? 1 : 0);
  const int per_tok = (a.d + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_combine, dim3(a.batch * per_tok), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe_sel
