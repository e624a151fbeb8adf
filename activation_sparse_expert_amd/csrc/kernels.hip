// Expert-grouped multi-kernel forward of the routed-MoE block with sketch-based
// top-k channel selection, for gfx950 (CDNA4, 64-wide wavefronts, MFMA).
//
// Used for batches above the single-launch limit and for shapes the single
// launch does not cover (large m). The (token, expert) pairs of a call are
// grouped by expert into tiles of up to 32 tokens, so every weight byte an
// expert needs is read once per tile, not once per token: the sketch codes once
// per tile, and each channel row once per tile when at least one of the tile's
// tokens selected it (the union of the tokens' selections). Each token still
// uses only its own k channels: the others are masked out of its activations.
//
// Phases (pages cited by title and section):
//   route+quantise  per token: top_e experts, gate weights, int8 activations
//                   ("KAIST drops calibration from MoE decoding...", opening
//                   paragraph: every token reads its routed experts' weights);
//   plan            pairs sorted by (expert, token), cut into expert tiles;
//   score           per (tile, 64-channel group): ternary-sketch scores of every
//                   channel for every token of the tile, an int8 MFMA contraction
//                   of the 2-bit codes with the activations, then the pinned
//                   binary32 score (same page, "A reader built from weights
//                   alone"); also the group's share of Q^T h_hat;
//   select          per pair: the k largest scores, lower index on ties (same
//                   page, "Top-k instead of a threshold");
//   union           per tile: union of the tokens' selections, with per-channel
//                   token masks;
//   gate/up         per (tile, 16 union channels): bf16 MFMA of the channel rows
//                   with the tile's activations, SwiGLU, masked per token; the
//                   tile's last block finishes the compensation coordinates
//                   z = Q^T h_hat over each token's skipped channels;
//   down            per (tile, 64 outputs): bf16 MFMA of the activations with the
//                   down columns of the union channels and, as r extra columns,
//                   the low-rank map P applied to z;
//   combine         per token: gate-weighted sum over its experts, bf16 output.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "kernels.h"

namespace moe_sel {
namespace {

using namespace dev;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kT = kTileTokens;  // tokens per tile
constexpr int kMSub = kT / 16;   // MFMA subtiles of 16 tokens
constexpr int kCh = 16;          // union channels per gate/up block
constexpr int kPlanThreads = 1024;

// Phase marks of the one-pair-tile kernels: ROW_MARK(kern, ev) compiles to
// nothing unless the library is built with MOE_SEL_TIMELINE, which records the
// wall clock of thread 0 of each of the first 512 blocks (kern: 0 score, 1
// gate/up, 2 down, 3 combine; the events are listed at each kernel).
#ifdef MOE_SEL_TIMELINE
__device__ unsigned long long g_row_marks[4 * 512 * 8];
#define ROW_MARK(kern, ev)                                                                       \
  do {                                                                                           \
    if (threadIdx.x == 0 && blockIdx.x < 512) g_row_marks[((kern) * 512 + blockIdx.x) * 8 + (ev)] = wall_clock64(); \
  } while (0)
#else
#define ROW_MARK(kern, ev) ((void)0)
#endif

// Phase marks of the expert-tile gate/up (kern 0) and down (kern 1) kernels,
// the same way: thread 0 of each of the first 8192 blocks; events 0 entry, 1
// tile known, 2 weights consumed, 3 end (a block with no work: 0 and 3 only).
#ifdef MOE_SEL_TIMELINE
__device__ unsigned long long g_tile_marks[2 * 8192 * 4];
#define TILE_MARK_AT(kern, idx, ev)                                                          \
  do {                                                                                       \
    if (threadIdx.x == 0 && (idx) < 8192) g_tile_marks[((kern) * 8192 + (idx)) * 4 + (ev)] = wall_clock64(); \
  } while (0)
#else
#define TILE_MARK_AT(kern, idx, ev) ((void)0)
#endif
#define TILE_MARK(kern, ev) TILE_MARK_AT(kern, blockIdx.x, ev)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// four byte-wide codes (t + 1) per dword, in hidden-element order (see the code layout)
__device__ __forceinline__ i32x4 expand_codes(uint32_t w) {
  return i32x4{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
               (int)((w >> 6) & 0x03030303u)};
}

// ===========================================================================
// Routing and activation quantisation, one block per token.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_route_quant(FwdArgs a, int pair_tiles) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ int s_sel[64];
  __shared__ float s_selv[64];
  __shared__ uint32_t s_amax[kWaves];
  __shared__ int s_qs[kWaves];

  // the token's activations, 16-byte pieces in registers (d <= 16384), in flight
  // while the experts are chosen
  constexpr int kXP = 8;
  const int npc = a.d / 8;
  const uint16_t* x = a.x + (size_t)t * a.d;
  uint4 xv[kXP];
#pragma unroll
  for (int u = 0; u < kXP; ++u) {
    const int pc = tid + u * kThreads;
    xv[u] = pc < npc ? *(const uint4*)(x + 8 * pc) : make_uint4(0, 0, 0, 0);
  }

  // top_e experts, larger logit first, lower index on ties (-0 equal to +0): one
  // wave's DPP rounds for few experts and picks, else repeated block arg-max
  const float* L = a.logits + (size_t)t * a.n_experts;
  if (a.top_e <= 16 && a.n_experts <= 256) {
    if (wave == 0) {
      if (a.n_experts <= 64) wave_topk_route<1>(L, a.n_experts, a.top_e, s_sel, s_selv);
      else if (a.n_experts <= 128) wave_topk_route<2>(L, a.n_experts, a.top_e, s_sel, s_selv);
      else wave_topk_route<4>(L, a.n_experts, a.top_e, s_sel, s_selv);
    }
    __syncthreads();
  } else {
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
  }
  if (tid < a.top_e) {
    const float top = s_selv[0];
    float denom = 0.0f;
    for (int s = 0; s < a.top_e; ++s) denom += __expf(s_selv[s] - top);
    const int p = t * a.top_e + tid;
    a.pair_expert[p] = s_sel[tid];
    a.pair_w[p] = __expf(s_selv[tid] - top) / denom;
    if (pair_tiles) {
      // the plan is one single-token tile per pair, in pair order
      a.tile_expert[p] = s_sel[tid];
      a.tile_first[p] = p;
      a.tile_n[p] = 1;
      a.tpair[p] = p;
      if (p == 0) *a.n_tiles = a.batch * a.top_e;
    }
  }

  // int8 activations with a power-of-two scale, and their sum
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < kXP; ++u) {
    const uint32_t w4[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) amax = max(amax, max(w4[h] & 0x7FFFu, (w4[h] >> 16) & 0x7FFFu));
  }
  amax = wave_max_u(amax);
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
  int qs = 0;
#pragma unroll
  for (int u = 0; u < kXP; ++u) {
    const int pc = tid + u * kThreads;
    if (pc < npc) {
      const uint32_t w4[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t bits = (w4[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
        const float xf = __uint_as_float(bits << 16);
        const int qi = amax ? (int)__builtin_rintf(__builtin_ldexpf(xf, -e)) : 0;
        qs += qi;
        packed[h >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (h & 3));
      }
      *(uint2*)(q + 8 * pc) = make_uint2(packed[0], packed[1]);
    }
  }
  qs = wave_sum_i(qs);
  if (lane == 0) s_qs[wave] = qs;
  __syncthreads();
  if (tid == 0) a.xqsum[t] = s_qs[0] + s_qs[1] + s_qs[2] + s_qs[3];
}

// ===========================================================================
// Gate/up work items a tile of n tokens is given, one per chunk of kCh union
// channels: as many as its largest union can fill (n k channels, all m for
// dense and threshold calls), at least one (a k = 0 call still writes its
// compensation share). The plan lays them out tile by tile; the union kernel
// fills them; the gate/up kernel runs one block per item, so its live blocks
// come first in the grid instead of interleaved with chunks past the unions.
__device__ __forceinline__ int gu_chunk_bound(const FwdArgs& a, int n, int dense) {
  const int maxch = a.m / kCh;
  if (dense || a.thr_mode) return maxch;
  const long u = min((long)a.m, (long)n * a.k);
  return max(1, (int)((u + kCh - 1) / kCh));
}

// Plan: pairs sorted by (expert, token) and cut into tiles of up to kT tokens.
// One block. Pairs of a token have distinct experts, so within an expert the
// order by token is the order by pair index, and a token's rank among an
// expert's tokens is a popcount over per-expert token bitmaps of a chunk.
// ===========================================================================
__global__ __launch_bounds__(kPlanThreads) void k_plan(FwdArgs a, int dense) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_run[1024];
  __shared__ uint32_t s_bm[1024 * 4];  // per expert: bitmap of the chunk's tokens (<= 128)
  __shared__ int s_wc[16], s_wt[16], s_wk[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.n_experts, P = a.batch * a.top_e;
  if (tid < E) {
    s_cnt[tid] = 0;
    s_run[tid] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) atomicAdd(&s_cnt[a.pair_expert[p]], 1);
  __syncthreads();
  // exclusive scans over experts of the pair counts and of the tile counts
  const int c = tid < E ? s_cnt[tid] : 0;
  const int nt = (c + kT - 1) / kT;
  int nk = 0;  // gate/up work items of this expert's tiles
  for (int i = 0; i < nt; ++i) nk += gu_chunk_bound(a, min(kT, c - i * kT), dense);
  const int ic = wave_incl_scan(c), it = wave_incl_scan(nt), ik = wave_incl_scan(nk);
  if (lane == 63) {
    s_wc[wave] = ic;
    s_wt[wave] = it;
    s_wk[wave] = ik;
  }
  __syncthreads();
  int bc = 0, bt = 0, bk = 0, tot_t = 0, tot_k = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    bc += w < wave ? s_wc[w] : 0;
    bt += w < wave ? s_wt[w] : 0;
    bk += w < wave ? s_wk[w] : 0;
    tot_t += s_wt[w];
    tot_k += s_wk[w];
  }
  const int off = bc + ic - c, toff = bt + it - nt;
  if (tid < E) {
    s_off[tid] = off;
    int ko = bk + ik - nk;
    for (int i = 0; i < nt; ++i) {
      const int tn = min(kT, c - i * kT);
      a.tile_expert[toff + i] = tid;
      a.tile_first[toff + i] = off + i * kT;
      a.tile_n[toff + i] = tn;
      a.tile_choff[toff + i] = ko;
      ko += gu_chunk_bound(a, tn, dense);
    }
  }
  if (tid == 0) {
    *a.n_tiles = tot_t;
    *a.n_items = tot_k;
  }
  // stable placement, chunks of ct tokens (ct * top_e <= 1024 pairs, ct <= 128)
  const int ct = max(1, min(128, kPlanThreads / a.top_e));
  for (int t0 = 0; t0 < a.batch; t0 += ct) {
    for (int i = tid; i < E * 4; i += kPlanThreads) s_bm[i] = 0u;
    __syncthreads();
    const int tl = tid / a.top_e;
    const int t = t0 + tl;
    const bool live = tl < ct && t < a.batch;
    const int p = t * a.top_e + tid % a.top_e;
    const int e = live ? a.pair_expert[p] : 0;
    if (live) atomicOr(&s_bm[e * 4 + (tl >> 5)], 1u << (tl & 31));
    __syncthreads();
    if (live) {
      int rank = s_run[e];
      for (int w = 0; w < (tl >> 5); ++w) rank += __popc(s_bm[e * 4 + w]);
      rank += __popc(s_bm[e * 4 + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
      a.tpair[s_off[e] + rank] = p;
    }
    __syncthreads();
    if (tid < E)
      s_run[tid] += __popc(s_bm[tid * 4]) + __popc(s_bm[tid * 4 + 1]) + __popc(s_bm[tid * 4 + 2]) +
                    __popc(s_bm[tid * 4 + 3]);
    __syncthreads();
  }
}

// ===========================================================================
// Sketch scores of one tile for one 64-channel group: int8 MFMA 16x16x64.
// Wave w owns channels 16w..16w+15 of the group for both matrices; N = tokens
// in subtiles of 16. C = sum (code) * q = D + sum q, so D = C - sum q.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_score_g(FwdArgs a) {
  extern __shared__ float s_dyn_score[];  // h [kT][64], then Q rows [64][r]
  const int d = a.d, m = a.m, r = a.r;
  const int groups = m / kGroup;
  const int tile = blockIdx.x / groups, grp = blockIdx.x % groups;
  // tile entries are read with the tile count (tile < max_tiles keeps them in
  // bounds) and used only for live tiles
  const int ntl = *a.n_tiles;
  const int e = a.tile_expert[tile], first = a.tile_first[tile], n = a.tile_n[tile];
  if (tile >= ntl) return;
  const int nsub = (n + 15) >> 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  float* s_h = s_dyn_score;
  float* s_q = s_dyn_score + kT * 64;

  const int8_t* xr[kMSub];
#pragma unroll
  for (int ns = 0; ns < kMSub; ++ns) {
    const int j = 16 * ns + li;
    const int pp = a.tpair[first + (j < n ? j : 0)];
    xr[ns] = a.xq + (size_t)(pp / a.top_e) * d + 16 * lg;
  }
  const size_t ebase = (size_t)e * codes_dwords_per_expert(d, m);
  const uint32_t* cg = a.codes + ebase + codes_dword_index(d, m, grp, 0, 0, 16 * wave + li, lg);
  const uint32_t* cu = a.codes + ebase + codes_dword_index(d, m, grp, 1, 0, 16 * wave + li, lg);
  // lane holds C[channel 4 lg + v][token li] of each subtile
  const int ch0 = 64 * grp + 16 * wave + 4 * lg;
  float4 st[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) st[v] = a.stats[(size_t)e * m + ch0 + v];
  const int nb = d / kBlock;
  // Main loop over groups of 4 code blocks: lane (i + 16 g) loads channel i's
  // 16-byte piece of block b + g and feeds its dword q to MFMA q, whose B operand
  // is the matching 16 activations; the contraction order over the hidden
  // dimension is permuted, which leaves the exact integer sums unchanged.
  const size_t blk4 = (size_t)64;  // u32x4 per (group, matrix, block)
  const u32x4* cg4 = (const u32x4*)(a.codes + ebase + codes_dword_index(d, m, grp, 0, lg, 16 * wave + li, 0));
  const u32x4* cu4 = (const u32x4*)(a.codes + ebase + codes_dword_index(d, m, grp, 1, lg, 16 * wave + li, 0));
  // scores and h_hat of token subtile ns from its exact integer sums
  auto finish = [&](int ns, const i32x4& accg, const i32x4& accu) {
    const int j = 16 * ns + li;
    if (j < n) {
      const int pp = a.tpair[first + j];
      const int t = pp / a.top_e;
      const int xe = a.xexp[t], qs = a.xqsum[t];
      float h[4], sc[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) pinned_score(accg[v] - qs, accu[v] - qs, xe, st[v], h[v], sc[v], a.score_kind);
      *(float4*)(a.hhat + (size_t)pp * m + ch0) = make_float4(h[0], h[1], h[2], h[3]);
      *(float4*)(a.score + (size_t)pp * m + ch0) = make_float4(sc[0], sc[1], sc[2], sc[3]);
      if (r > 0)
#pragma unroll
        for (int v = 0; v < 4; ++v) s_h[j * 64 + 16 * wave + 4 * lg + v] = h[v];
    }
  };
  // Every code load feeds all NS token subtiles of the tile, so a tile of more
  // than 16 tokens streams its codes once instead of once per subtile.
  static_assert(kMSub == 2, "one or two token subtiles per tile");
  auto run = [&](auto ns_count) {
    constexpr int NS = decltype(ns_count)::value;
    constexpr int SB = NS == 1 ? 2 : 1;  // groups of four code blocks per iteration
    i32x4 accg[NS], accu[NS];
    const int8_t* x4[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      accg[ns] = accu[ns] = i32x4{0, 0, 0, 0};
      x4[ns] = xr[ns] - 16 * lg + 64 * lg;  // token row + block offset lg
    }
    int b = 0;
    for (; b + 4 * SB <= nb; b += 4 * SB) {
      u32x4 wg[SB], wu[SB];
      i32x4 xv[SB][4][NS];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        wg[u] = cg4[(size_t)(b + 4 * u) * blk4];
        wu[u] = cu4[(size_t)(b + 4 * u) * blk4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) xv[u][q][ns] = *(const i32x4*)(x4[ns] + 64 * (b + 4 * u) + 16 * q);
      }
      // every load of the batch issued before the first product
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < SB; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x4 eg = expand_codes(wg[u][q]), eu = expand_codes(wu[u][q]);
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            accg[ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(eg, xv[u][q][ns], accg[ns], 0, 0, 0);
            accu[ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(eu, xv[u][q][ns], accu[ns], 0, 0, 0);
          }
        }
    }
    for (; b + 4 <= nb; b += 4) {
      const u32x4 wg = cg4[(size_t)b * blk4], wu = cu4[(size_t)b * blk4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x4 eg = expand_codes(wg[q]), eu = expand_codes(wu[q]);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const i32x4 xv = *(const i32x4*)(x4[ns] + 64 * b + 16 * q);
          accg[ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(eg, xv, accg[ns], 0, 0, 0);
          accu[ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(eu, xv, accu[ns], 0, 0, 0);
        }
      }
    }
    // remaining blocks one at a time: lane (i + 16 g) takes dword g of block b
    for (; b < nb; ++b) {
      const i32x4 eg = expand_codes(cg[(size_t)b * 256]), eu = expand_codes(cu[(size_t)b * 256]);
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const i32x4 xv = *(const i32x4*)(xr[ns] + 64 * b);
        accg[ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(eg, xv, accg[ns], 0, 0, 0);
        accu[ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(eu, xv, accu[ns], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) finish(ns, accg[ns], accu[ns]);
  };
  if (nsub > 1)
    run(std::integral_constant<int, 2>{});
  else
    run(std::integral_constant<int, 1>{});
  if (r == 0) return;
  // Q rows of the group (64 r bf16, r <= 128) into registers, all in flight
  // with the codes; written to LDS after the main loop
  constexpr int kQg = 64 * 128 / 8 / kThreads;
  const int qpieces = 8 * r;
  const uint4* qsrc = (const uint4*)(a.qmat + ((size_t)e * m + 64 * grp) * r);
  uint4 qv[kQg];
#pragma unroll
  for (int u = 0; u < kQg; ++u) {
    const int i = tid + u * kThreads;
    qv[u] = i < qpieces ? qsrc[i] : make_uint4(0, 0, 0, 0);
  }

#pragma unroll
  for (int u = 0; u < kQg; ++u) {
    const int i = tid + u * kThreads;
    if (i < qpieces) {
      const uint32_t w4[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        s_q[8 * i + 2 * h] = bf16lo(w4[h]);
        s_q[8 * i + 2 * h + 1] = bf16hi(w4[h]);
      }
    }
  }
  __syncthreads();
  // this group's share of Q^T h_hat for every token of the tile
  const int groups_r = groups * r;
  for (int i = tid; i < n * r; i += kThreads) {
    const int j = i / r, c = i % r;
    float z = 0.0f;
#pragma unroll 8
    for (int ch = 0; ch < 64; ++ch) z += s_h[j * 64 + ch] * s_q[ch * r + c];
    a.gzpart[(size_t)(first + j) * groups_r + grp * r + c] = z;  // by tile slot
  }
}

// ===========================================================================
// Sketch scores for one-pair tiles (batch 1 and small sparse batches), one
// block per (pair, 64-channel group) with 8 waves, each an eighth of the
// hidden dimension for both matrices. Lane l is channel l of the group and
// reads its 16-byte code piece of each 64-element block, so one load
// instruction reads a block's 1 KiB of the group at once; the token's x_q sits
// in LDS, and each read of it serves the gate and the up codes (the LDS
// broadcast, not the dot products, limits this loop). The exact integer dots
// of the eighths are added in LDS, then scores and h_hat as above, and the
// group's share of Q^T h_hat.
// ===========================================================================
// kernels for one-pair tiles (batch 1, small sparse batches): 8 waves per block
constexpr int kB1Threads = 512, kB1Waves = kB1Threads / 64;
constexpr int kB1Pieces = 8;  // 16-byte pieces per lane and row: d <= 4096
constexpr int kSB1Blk = 16;  // code blocks per wave in flight

// Routing of one token by a 512-thread block (n_experts <= 256), the same
// order as the routing kernel: the rank of a logit
// is the count of larger order keys (larger logit first, lower index first),
// two threads per expert; gate weights are the softmax over the chosen logits.
__device__ __forceinline__ void route_b1(const float* logits, int n_experts, int top_e, int* s_ids, float* s_w,
                                         uint64_t* s_key, float* s_val) {
  const int tid = threadIdx.x;
  if (tid < n_experts) {
    const float v = logits[tid];
    s_key[tid] = order_key(logit_order_bits(v), tid);
    s_val[tid] = v;
  }
  __syncthreads();
  const int i = tid >> 1, half = tid & 1;
  int rank = 0;
  if (i < n_experts) {
    const uint64_t ki = s_key[i];
    for (int j = half; j < n_experts; j += 2) rank += s_key[j] > ki;
  }
  rank += __shfl_xor(rank, 1, 64);
  if (i < n_experts && half == 0 && rank < top_e) {
    s_ids[rank] = i;
    s_w[rank] = s_val[i];
  }
  __syncthreads();
  route_softmax(s_w, top_e);
  __syncthreads();
}

// self_route (one pair per tile, no routing kernel launched): every block
// routes its token and quantises its x itself, as the routing kernel would, and
// the blocks of group 0 write their pair's routing and one-token tile for the
// later kernels.
// X16: int16 activations (the score ablation; self-routing calls only), an
// instance of its own so that its registers do not cost the int8 one occupancy
template <bool X16>
__global__ __launch_bounds__(kB1Threads) void k_score_b1(FwdArgs a, int self_route) {
  extern __shared__ float s_dyn_sb1[];  // x_q [2d] bytes (int8, or int16 high then low bytes), then Q rows [64][r]
  __shared__ int s_part[kB1Waves][64], s_part2[kB1Waves][64];
  __shared__ float s_h[64];
  __shared__ uint64_t s_rkey[256];
  __shared__ float s_rval[256];
  __shared__ int s_ids[64];
  __shared__ float s_w[64];
  __shared__ int s_red[2][kB1Waves];
  const int d = a.d, m = a.m, r = a.r, groups = m / kGroup;
  const int tile = blockIdx.x / groups, grp = blockIdx.x % groups;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npc = d / 8;
  int8_t* s_xq = (int8_t*)s_dyn_sb1;
  float* s_q = s_dyn_sb1 + d / 2;
  constexpr bool x16 = X16;
  int e, pp;
  uint4 xv = make_uint4(0, 0, 0, 0);
  ROW_MARK(0, 0);  // marks: 0 entry, 1 routed, 2 x_q and Q rows in LDS, 3 dots summed, 4 end
  if (self_route) {
    if (tile >= a.batch * a.top_e) return;  // one single-token tile per routed pair
    const int tt = tile / a.top_e;
    if (tid < npc) xv = *(const uint4*)(a.x + (size_t)tt * d + 8 * tid);
    route_b1(a.logits + (size_t)tt * a.n_experts, a.n_experts, a.top_e, s_ids, s_w, s_rkey, s_rval);
    pp = tile;
    e = s_ids[tile % a.top_e];
    ROW_MARK(0, 1);
  } else {
    const int ntl = *a.n_tiles;
    e = a.tile_expert[tile];
    const int first = a.tile_first[tile];
    if (tile >= ntl) return;
    pp = a.tpair[first];
  }
  const int t = pp / a.top_e;
  // wave w takes the code blocks [b0, b1) of both matrices (an eighth of the
  // hidden dimension; d >= 512 gives every wave a block), so each x_q read
  // from LDS feeds the gate and the up dot
  const int nb = d / kBlock;
  const int b0 = nb * wave / kB1Waves, b1 = nb * (wave + 1) / kB1Waves;
  const uint4* cpg = (const uint4*)(a.codes + (size_t)e * codes_dwords_per_expert(d, m) +
                                    codes_dword_index(d, m, grp, 0, 0, lane, 0));
  const uint4* cpu = (const uint4*)(a.codes + (size_t)e * codes_dwords_per_expert(d, m) +
                                    codes_dword_index(d, m, grp, 1, 0, lane, 0));
  // every global load first: codes, Q rows, statistics, and x_q when it comes from the routing kernel
  constexpr int kSB1Pair = kSB1Blk / 2;  // blocks of both matrices in flight
  uint4 cbg[kSB1Pair], cbu[kSB1Pair];
#pragma unroll
  for (int i = 0; i < kSB1Pair; ++i) {
    cbg[i] = cpg[(size_t)min(b0 + i, b1 - 1) * 64];
    cbu[i] = cpu[(size_t)min(b0 + i, b1 - 1) * 64];
  }
  constexpr int kQv = 64 * 128 * 2 / 16 / kB1Threads;  // 16-byte Q pieces per thread, r <= 128
  const int qpieces = 8 * r;
  const uint4* qsrc = (const uint4*)(a.qmat + ((size_t)e * m + 64 * grp) * r);
  uint4 qv[kQv];
#pragma unroll
  for (int u = 0; u < kQv; ++u) {
    const int i = tid + u * kB1Threads;
    qv[u] = i < qpieces ? qsrc[i] : make_uint4(0, 0, 0, 0);
  }
  const float4 st = a.stats[(size_t)e * m + 64 * grp + lane];
  int4 xqv = make_int4(0, 0, 0, 0);
  if (!self_route && tid < d / 16) xqv = ((const int4*)(a.xq + (size_t)t * d))[tid];
  int xe, qs;
  if (self_route) {
    // int8 activations with a power-of-two scale, and their sum
    uint32_t amax = 0;
    const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) amax = max(amax, max(w4[h] & 0x7FFFu, (w4[h] >> 16) & 0x7FFFu));
    amax = wave_max_u(amax);
    if (lane == 0) s_red[0][wave] = (int)amax;
    __syncthreads();
    amax = (uint32_t)s_red[0][0];
#pragma unroll
    for (int w = 1; w < kB1Waves; ++w) amax = max(amax, (uint32_t)s_red[0][w]);
    xe = amax ? score_exponent(amax, x16) : 0;
    int qsum = 0;
    if (tid < npc) {
      uint32_t packed[2] = {0u, 0u}, low[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t bits = (w4[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
        const int qi = amax ? (int)__builtin_rintf(__builtin_ldexpf(__uint_as_float(bits << 16), -xe)) : 0;
        qsum += qi;
        packed[h >> 2] |= ((uint32_t)(x16 ? qi >> 8 : qi) & 0xFFu) << (8 * (h & 3));
        low[h >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (h & 3));
      }
      *(uint2*)(s_xq + 8 * tid) = make_uint2(packed[0], packed[1]);
      if (x16) *(uint2*)(s_xq + d + 8 * tid) = make_uint2(low[0], low[1]);
    }
    qsum = wave_sum_i(qsum);
    if (lane == 0) s_red[1][wave] = qsum;
    if (grp == 0 && tid == 0) {
      a.pair_expert[pp] = e;
      a.pair_w[pp] = s_w[pp % a.top_e];
      a.tile_expert[pp] = e;
      a.tile_first[pp] = pp;
      a.tile_n[pp] = 1;
      a.tpair[pp] = pp;
      if (pp == 0) *a.n_tiles = a.batch * a.top_e;
    }
    __syncthreads();
    qs = 0;
#pragma unroll
    for (int w = 0; w < kB1Waves; ++w) qs += s_red[1][w];
  } else {
    xe = a.xexp[t];
    qs = a.xqsum[t];
    if (tid < d / 16) ((int4*)s_xq)[tid] = xqv;
  }
#pragma unroll
  for (int u = 0; u < kQv; ++u) {
    const int i = tid + u * kB1Threads;
    if (i < qpieces) {
      const uint4 q4 = qv[u];
      const uint32_t w4[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        s_q[8 * i + 2 * h] = bf16lo(w4[h]);
        s_q[8 * i + 2 * h + 1] = bf16hi(w4[h]);
      }
    }
  }
  __syncthreads();  // x_q and the Q rows in LDS
  ROW_MARK(0, 2);
  CodeAcc accg, accu, accg_lo, accu_lo;  // *_lo: the low bytes of int16 activations
  for (int c0 = b0; c0 < b1; c0 += kSB1Pair) {
    if (c0 != b0) {
#pragma unroll
      for (int i = 0; i < kSB1Pair; ++i) {
        cbg[i] = cpg[(size_t)min(c0 + i, b1 - 1) * 64];
        cbu[i] = cpu[(size_t)min(c0 + i, b1 - 1) * 64];
      }
    }
#pragma unroll
    for (int i = 0; i < kSB1Pair; ++i) {
      if (c0 + i < b1) {
        const int4* xb = (const int4*)(s_xq + 64 * (c0 + i));
        const int4 x0 = xb[0], x1 = xb[1], x2 = xb[2], x3 = xb[3];
        dot_codes16(cbg[i].x, x0, accg);
        dot_codes16(cbg[i].y, x1, accg);
        dot_codes16(cbg[i].z, x2, accg);
        dot_codes16(cbg[i].w, x3, accg);
        dot_codes16(cbu[i].x, x0, accu);
        dot_codes16(cbu[i].y, x1, accu);
        dot_codes16(cbu[i].z, x2, accu);
        dot_codes16(cbu[i].w, x3, accu);
        if (x16) {
          const int4* xl = (const int4*)(s_xq + d + 64 * (c0 + i));
          const int4 l0 = xl[0], l1 = xl[1], l2 = xl[2], l3 = xl[3];
          dot_codes16_u(cbg[i].x, l0, accg_lo);
          dot_codes16_u(cbg[i].y, l1, accg_lo);
          dot_codes16_u(cbg[i].z, l2, accg_lo);
          dot_codes16_u(cbg[i].w, l3, accg_lo);
          dot_codes16_u(cbu[i].x, l0, accu_lo);
          dot_codes16_u(cbu[i].y, l1, accu_lo);
          dot_codes16_u(cbu[i].z, l2, accu_lo);
          dot_codes16_u(cbu[i].w, l3, accu_lo);
        }
      }
    }
  }
  // sums of (t + 1) x_q over the wave's blocks, gate then up
  s_part[wave][lane] = x16 ? 256 * code_acc_total(accg) + code_acc_total(accg_lo) : code_acc_total(accg);
  s_part2[wave][lane] = x16 ? 256 * code_acc_total(accu) + code_acc_total(accu_lo) : code_acc_total(accu);
  __syncthreads();
  ROW_MARK(0, 3);
  if (wave == 0) {
    int dg = 0, du = 0;
#pragma unroll
    for (int w = 0; w < kB1Waves; ++w) {
      dg += s_part[w][lane];
      du += s_part2[w][lane];
    }
    float h, sc;
    pinned_score(dg - qs, du - qs, xe, st, h, sc, a.score_kind);
    const int j = 64 * grp + lane;
    a.hhat[(size_t)pp * m + j] = h;
    a.score[(size_t)pp * m + j] = sc;
    s_h[lane] = h;
  }
  if (r == 0) return;
  __syncthreads();
  if (tid < r) {
    float z = 0.0f;
#pragma unroll 8
    for (int ch = 0; ch < 64; ++ch) z += s_h[ch] * s_q[ch * r + tid];
    a.gzpart[((size_t)pp * groups + grp) * r + tid] = z;
  }
  ROW_MARK(0, 4);
}

// ===========================================================================
// Top-k per pair, one block of 16 waves per pair, each thread holding its keys
// in registers. Non-negative binary32 scores order like their bit patterns,
// whose bit 31 is clear. A histogram of the bits 30..19 (4096 bins, a
// sixteenth of an octave each) finds the bin holding the k-th largest key;
// keys in higher bins are taken, and when that bin holds at most kSelCand keys
// they are ranked exactly by (score desc, index asc), four threads per
// candidate. Otherwise (ties, clusters) radix passes over the bits 31..20,
// 19..9 and 8..0 narrow the boundary bin down the same way; if all three run,
// the k-th key itself is known and equal keys are taken lowest index first.
// Selections are gathered in a bitmap, which then yields the ascending index
// list by a word-level scan.
// ===========================================================================
constexpr int kSelCand = 256;
constexpr int kSelMaxWords = 512;  // m <= 16384
constexpr int kSelThreads = 1024, kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 4096;     // first pass: bits 30..19

// Phase marks of the select blocks: SEL_MARK(ev) compiles to nothing unless
// the library is built with MOE_SEL_TIMELINE, which records the wall clock of
// thread 0 of each of the first 64 blocks (events: 0 entry, 1 histogram
// built, 2 boundary bin found, 3 candidates placed, 4 candidates ranked, 5
// bitmap complete, 6 index list written).
#ifdef MOE_SEL_TIMELINE
__device__ unsigned long long g_sel_marks[64 * 8];
#define SEL_MARK(ev)                                                                       \
  do {                                                                                     \
    if (threadIdx.x == 0 && blockIdx.x < 64) g_sel_marks[blockIdx.x * 8 + (ev)] = wall_clock64(); \
  } while (0)
#else
#define SEL_MARK(ev) ((void)0)
#endif

// exclusive scan over the 1024 threads of a select block; s_w: kSelWaves ints
__device__ __forceinline__ int sel_excl_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = s_w[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Boundary bin of the kr-th largest key in a histogram of BPT * 1024 bins
// (thread t owns bins BPT t .. BPT t + BPT - 1); writes s_sc[0..2] = (bin,
// keys in higher bins, keys in the bin). Barriers inside.
template <int BPT>
__device__ __forceinline__ void sel_find_bin(const int* s_hist, int kr, int* s_tmp, int* s_sc) {
  __syncthreads();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int h[BPT], c = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = s_hist[BPT * tid + i];
    c += h[i];
  }
  // keys in bins above this thread's: those of the later waves, then of the
  // later lanes of this wave (s_tmp is not written again before the barrier
  // that ends this call)
  const int incl = wave_incl_scan(c);
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int above = __builtin_amdgcn_readlane(incl, 63) - incl;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) above += w > wave ? s_tmp[w] : 0;
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (above < kr && kr <= above + h[i]) {
      s_sc[0] = BPT * tid + i;
      s_sc[1] = above;
      s_sc[2] = h[i];
    }
    above += h[i];
  }
  __syncthreads();
}

// A wave's predicate ORed into the bitmap: the wave's lanes hold the 64
// indices j0 .. j0 + 63 (j0 a multiple of 64), so the two words are this
// wave's alone in a pass. All lanes of the wave call.
__device__ __forceinline__ void mark_wave(uint32_t* bits, int j0, bool pred) {
  const uint64_t b = __ballot(pred);
  const int lane = threadIdx.x & 63;
  if (lane == 0 && (uint32_t)b) bits[j0 >> 5] |= (uint32_t)b;
  if (lane == 32 && (uint32_t)(b >> 32)) bits[(j0 >> 5) + 1] |= (uint32_t)(b >> 32);
}

// Key slot u of a thread is j = tid + 1024 u. As m is a multiple of 64, a
// wave's slot is valid in all lanes or none: the guard compares the wave's
// first index (a scalar) with m, a scalar branch with no per-key exec masks.
#define SEL_FOR_KEYS(BODY)                                     \
  _Pragma("unroll") for (int u = 0; u < KPT; ++u) {            \
    [[maybe_unused]] const int j = tid + u * kSelThreads;      \
    if (jw0 + u * kSelThreads < m) { BODY }                    \
  }

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void k_select(FwdArgs a, int pair_tiles) {
  static_assert(KPT <= 64, "lane u keeps key slot u's ballot");
  __shared__ __align__(16) int s_hist[kSelBins];  // histograms, then candidates
  __shared__ __align__(8) uint32_t s_bits[kSelMaxWords];
  __shared__ __align__(16) int s_tmp[kSelWaves + 2];
  __shared__ int s_sc[4];
  const int p = blockIdx.x;
  const int m = a.m, k = a.k, words = m / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int jw0 = __builtin_amdgcn_readfirstlane(tid - lane);  // the wave's first key index
  const bool topk = k > 0 && k < m;
  const uint32_t* keys = (const uint32_t*)(a.score + (size_t)p * m);
  SEL_MARK(0);
  // every key slot loads unconditionally (slots past m read key m - 1 and are
  // never used), so all of a thread's loads are in flight at once; under the
  // slots' guards each load waited for the one before
  uint32_t key[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) key[u] = keys[min(tid + u * kSelThreads, m - 1)];
  if (tid < words) s_bits[tid] = k >= m ? 0xFFFFFFFFu : 0u;
  if (topk) *(int4*)(s_hist + 4 * tid) = make_int4(0, 0, 0, 0);
  if (tid == 0) s_sc[3] = 0;  // candidate slots taken in the first pass
  __syncthreads();
  if (topk) {
    SEL_FOR_KEYS(atomicAdd(&s_hist[key[u] >> 19], 1);)
    SEL_MARK(1);
    sel_find_bin<kSelBins / kSelThreads>(s_hist, k, s_tmp, s_sc);
    SEL_MARK(2);
    // candidates: keys with (key >> cshift) == cval
    uint32_t cval = (uint32_t)s_sc[0];
    int cshift = 19;
    int krem = k - s_sc[1], ncand = s_sc[2];
    bool exact_key = false;
    bool placed = false;  // candidates already in s_hist (first pass)
    int nc = 0;           // this thread's candidates
    uint64_t* ck = (uint64_t*)s_hist;  // kSelCand order keys (the histogram is consumed)
    int* cidx = s_hist + 2 * kSelCand;
    if (ncand <= kSelCand) {
      // keys above the boundary bin into the bitmap: lane u of a wave keeps
      // the wave's slot-u ballot (two words, whole: no other wave writes them)
      // and all slots are stored at once after the pass; the bin's keys take
      // slots one by one (there are few) instead of from a block scan
      uint32_t above_lo = 0, above_hi = 0;
      SEL_FOR_KEYS(const uint32_t dg = key[u] >> 19; const uint64_t ab = __ballot(dg > cval);
                   above_lo = lane == u ? (uint32_t)ab : above_lo;
                   above_hi = lane == u ? (uint32_t)(ab >> 32) : above_hi; if (dg == cval) {
                     const int slot = atomicAdd(&s_sc[3], 1);
                     ck[slot] = order_key(key[u], j);
                     cidx[slot] = j;
                   })
      if (lane < KPT && jw0 + lane * kSelThreads < m)
        *(uint64_t*)(s_bits + ((jw0 + lane * kSelThreads) >> 5)) = ((uint64_t)above_hi << 32) | above_lo;
      placed = true;
    } else {
      // ties or clusters: radix passes over the bits 31..20, 19..9 and 8..0 of the
      // key; after each pass keys in higher bins are taken and only the boundary
      // bin stays
      constexpr int kShift[3] = {20, 9, 0};
      constexpr int kBins[3] = {2048, 2048, 512};
      uint32_t prefix = 0;  // boundary bits above the current pass
      krem = k;
      int level = 0;
      for (; level < 3; ++level) {
        const int sh = kShift[level], hi = level == 0 ? 32 : kShift[level - 1];
        const uint32_t dmask = (uint32_t)kBins[level] - 1u;
        __syncthreads();
        s_hist[2 * tid] = 0;
        s_hist[2 * tid + 1] = 0;
        __syncthreads();
        SEL_FOR_KEYS(if (level == 0 || (key[u] >> hi) == prefix) atomicAdd(&s_hist[(key[u] >> sh) & dmask], 1);)
        sel_find_bin<2>(s_hist, krem, s_tmp, s_sc);
        const uint32_t dsel = (uint32_t)s_sc[0];
        SEL_FOR_KEYS(mark_wave(s_bits, j - lane,
                               (level == 0 || (key[u] >> hi) == prefix) && ((key[u] >> sh) & dmask) > dsel);)
        krem -= s_sc[1];
        ncand = s_sc[2];
        prefix = (prefix << (hi - sh)) | dsel;
        if (ncand <= kSelCand) {
          ++level;
          break;
        }
      }
      cshift = kShift[level - 1];
      cval = prefix;
      exact_key = ncand > kSelCand;  // all three passes ran: prefix is the k-th key itself
      if (!exact_key) {
        SEL_FOR_KEYS(nc += (key[u] >> cshift) == cval;)
      }
    }
    if (!exact_key) {
      // the boundary bin's keys (after the radix passes: at scan positions),
      // ranked exactly, four threads per candidate
      if (!placed) {
        int ctot;
        int slot = sel_excl_scan(nc, s_tmp, &ctot);
        SEL_FOR_KEYS(if ((key[u] >> cshift) == cval) {
          ck[slot] = order_key(key[u], j);
          cidx[slot] = j;
          ++slot;
        })
      }
      __syncthreads();
      SEL_MARK(3);
      const int c = tid >> 2, part = tid & 3;
      const bool live = c < ncand;
      const uint64_t kc = live ? ck[c] : 0ull;
      int rank = 0;
      if (live)
#pragma unroll 4
        for (int o = part; o < ncand; o += 4) rank += ck[o] > kc;
      rank += __shfl_xor(rank, 1, 64);
      rank += __shfl_xor(rank, 2, 64);
      if (live && part == 0 && rank < krem) {
        const int ic = cidx[c];
        atomicOr(&s_bits[ic >> 5], 1u << (ic & 31));
      }
      SEL_MARK(4);
    } else {
      // the krem lowest-index copies of the k-th key, one word per thread
      __syncthreads();
      uint32_t eq = 0;
      if (tid < words)
#pragma unroll 8
        for (int b = 0; b < 32; ++b) eq |= (uint32_t)(keys[32 * tid + b] == cval) << b;
      int eq_tot;
      const int eq_before = sel_excl_scan(__popc(eq), s_tmp, &eq_tot);
      int want = max(0, min(__popc(eq), krem - eq_before));
      uint32_t takeq = 0, rest = eq;
      while (want-- > 0) {
        const uint32_t low = rest & (0u - rest);
        takeq |= low;
        rest ^= low;
      }
      if (tid < words) s_bits[tid] |= takeq;
    }
  }
  if (a.thr_mode) {
    // threshold selector: every channel whose score exceeds the threshold
    __syncthreads();
    SEL_FOR_KEYS(mark_wave(s_bits, j - lane, key[u] > a.thr_bits);)
  }
  __syncthreads();
  SEL_MARK(5);
  // Ascending index list from the bitmap: wave 0 turns the words' bit counts
  // into exclusive prefix sums (8 words per lane; the histogram's LDS is free
  // by now), then each wave places its own key slots: the 64 channels of a
  // wave's slot are two bitmap words, so a selected lane's rank is the prefix
  // before them plus the selected lanes below it, and the wave's stores cover
  // consecutive list entries.
  int* s_pre = s_hist;  // [kSelMaxWords + 1]
  if (tid < 64) {
    constexpr int kWpl = kSelMaxWords / 64;
    int c[kWpl], sum = 0;
#pragma unroll
    for (int i = 0; i < kWpl; ++i) {
      const int q = kWpl * lane + i;
      c[i] = q < words ? __popc(s_bits[q]) : 0;
      sum += c[i];
    }
    const int incl = wave_incl_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < kWpl; ++i) {
      s_pre[kWpl * lane + i] = run;
      run += c[i];
    }
    if (lane == 63) s_pre[kSelMaxWords] = incl;
  }
  __syncthreads();
  int* idx_out = a.sel_idx + (size_t)p * m;
  // one pair per tile: tile p is pair p alone, and its union is the selection
  // itself (the row kernels that read it need no token masks)
  int* ul = pair_tiles ? a.ulist + (size_t)p * m : nullptr;
  // every slot's two words and prefix are read first (clamped inside the
  // arrays; slots past m are not used), so the reads wait once, not per slot
  uint64_t wbits[KPT];
  int pre[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int q = min((jw0 + u * kSelThreads) >> 5, kSelMaxWords - 2);
    wbits[u] = *(const uint64_t*)(s_bits + q);
    pre[u] = s_pre[q];
  }
  SEL_FOR_KEYS(if ((wbits[u] >> lane) & 1u) {
    const int pos = pre[u] + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(wbits[u] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)wbits[u], 0u));
    idx_out[pos] = j;
    if (ul) ul[pos] = j;
  })
  if (tid < words) a.selbits[(size_t)p * words + tid] = s_bits[tid];
  if (tid == 0) {
    const int tot = s_pre[kSelMaxWords];
    a.sel_count[p] = tot;
    if (ul) a.ucount[p] = tot;
  }
  SEL_MARK(6);
}
#undef SEL_FOR_KEYS

// 32 x 32 bit-matrix transpose in registers (Hacker's Delight, "Transposing a
// bit matrix"): five rounds of masked swaps of 16-, 8-, 4-, 2- and 1-bit blocks.
// Afterwards bit i of A[b] is what bit b of A[i] was.
__device__ __forceinline__ void transpose32(uint32_t (&A)[32]) {
  constexpr uint32_t kMask[5] = {0x55555555u, 0x33333333u, 0x0F0F0F0Fu, 0x00FF00FFu, 0x0000FFFFu};
#pragma unroll
  for (int lj = 4; lj >= 0; --lj) {
    const int j = 1 << lj;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int k = ((q >> lj) << (lj + 1)) | (q & (j - 1));  // rows with bit lj clear
      const uint32_t t = ((A[k] >> j) ^ A[k | j]) & kMask[lj];
      A[k] ^= t << j;
      A[k | j] ^= t;
    }
  }
}

// ===========================================================================
// Union of a tile's selections: ascending channel list and, per listed
// channel, the mask of the tile's tokens that selected it. One block per tile.
// ===========================================================================
__global__ __launch_bounds__(kThreads) void k_union(FwdArgs a, int dense) {
  __shared__ int s_tmp[kWaves];
  const int tile = blockIdx.x;
  const int ntl = *a.n_tiles, first = a.tile_first[tile], n = a.tile_n[tile];
  const int e = a.tile_expert[tile], choff = a.tile_choff[tile];
  if (tile >= ntl) return;
  const int m = a.m, words = m / 32;
  const int tid = threadIdx.x;
  int* ul = a.ulist + (size_t)tile * m;
  uint64_t* um = a.umask + (size_t)tile * m;
  // the tile's gate/up work items: channel of union position pos, and (once the
  // union's size is known) the headers and the positions past the union
  const int nb = gu_chunk_bound(a, n, dense);
  int* items = a.gu_items + (size_t)choff * kGuItemInts;
  auto item_ch = [&](int pos, int ch) { items[(pos / kCh) * kGuItemInts + 8 + pos % kCh] = ch; };
  auto finish_items = [&](int uc) {
    for (int pos = uc + tid; pos < nb * kCh; pos += kThreads) item_ch(pos, 0);
    if (tid < nb) {
      int* h = items + tid * kGuItemInts;
      h[0] = tile;
      h[1] = tid;
      h[2] = e;
      h[3] = first;
      h[4] = n;
      h[5] = uc;
    }
  };
  if (dense) {  // (dense gate/up blocks map themselves to every chunk: no items)
    const uint64_t all = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    for (int j = tid; j < m; j += kThreads) {
      ul[j] = j;
      um[j] = all;
    }
    if (tid == 0) a.ucount[tile] = m;
    if (tid < n) a.slot_ucount[first + tid] = m;
    return;
  }
  if (n == 1) {
    const int pp = a.tpair[first];
    const int cnt = a.sel_count[pp];
    for (int j = tid; j < cnt; j += kThreads) {
      const int ch = a.sel_idx[(size_t)pp * m + j];
      ul[j] = ch;
      um[j] = 1ull;
      item_ch(j, ch);
    }
    if (tid == 0) a.ucount[tile] = cnt;
    if (tid == 0) a.slot_ucount[first] = cnt;
    finish_items(cnt);
    return;
  }
  // one thread per bitmap word: the tokens' words, their union, then the listed
  // channels of the word with their token masks at exclusive-scan positions
  __shared__ int s_p[kT];
  if (tid < n) s_p[tid] = a.tpair[first + tid];
  __syncthreads();
  int run = 0;
  for (int base = 0; base < words; base += kThreads) {
    const int w = base + tid;
    uint32_t v[kT];
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      v[i] = (i < n && w < words) ? a.selbits[(size_t)s_p[i] * words + w] : 0u;
      u |= v[i];
    }
    int tot;
    int pos = run + block_excl_scan(__popc(u), s_tmp, &tot);
    // token masks of the word's 32 channels at once: v[bit] bit i = token i selected it
    static_assert(kT == 32, "the union masks transpose a 32 x 32 bit matrix");
    transpose32(v);
#pragma unroll
    for (int bit = 0; bit < 32; ++bit) {
      if ((u >> bit) & 1u) {
        ul[pos] = 32 * w + bit;
        um[pos] = (uint64_t)v[bit];
        item_ch(pos, 32 * w + bit);
        ++pos;
      }
    }
    run += tot;
  }
  if (tid == 0) a.ucount[tile] = run;
  if (tid < n) a.slot_ucount[first + tid] = run;  // for k_zfin, which runs per slot
  finish_items(run);
}

// ===========================================================================
// SwiGLU of 16 union channels for every token of a tile: bf16 MFMA 16x16x32
// (M = channels, N = tokens, K = hidden), the hidden dimension split over the
// four waves. Activations of tokens that did not select a channel are zero.
// Expert-tile activations (here, k_zfin, k_down_g) sit in the activation
// buffer's row of the token's tile slot (tile_first + token), so the down
// kernel addresses them without the slot's pair index.
// Blocks of a sparse call also leave their channels' share of Q^T h_hat per
// token, from which k_zfin finishes the compensation coordinates.
//
// ===========================================================================
struct GateUpSmem {
  f32x4 acc[kWaves][2][64];  // 8 KiB
  float hz[kCh][kT];
  float qr[kCh * 128];
};

// uc, e, first, n: the tile's union size, expert, first slot and tokens; ja:
// the block's union channel for lane li (read with them, clamped into the
// expert: positions past the union are masked where they are used)
__device__ __forceinline__ void gate_up_item(const FwdArgs& a, int dense, int tile, int chunk, int item,
                                             GateUpSmem& sm, int uc, int e, int first, int n, int ja) {
  auto& s_acc = sm.acc;
  auto& s_hz = sm.hz;
  float* s_qr = sm.qr;
  const int d = a.d, m = a.m;
  const int maxch = m / kCh;
  TILE_MARK_AT(0, item, 1);
  const int nsub = (n + 15) >> 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int r = dense ? 0 : a.r;
  const int* ul = a.ulist + (size_t)tile * m;
  const uint64_t* um = a.umask + (size_t)tile * m;

  // A rows: union channel 16 chunk + li; B columns: token 16 ns + li (clamped)
  const uint16_t* grow = a.wch + ((size_t)e * m + ja) * 3 * d + 8 * lg;
  const uint16_t* urow = grow + d;
  const uint16_t* xr[kMSub];
#pragma unroll
  for (int ns = 0; ns < kMSub; ++ns) {
    const int j = 16 * ns + li;
    const int pp = a.tpair[first + (j < n ? j : 0)];
    xr[ns] = a.x + (size_t)(pp / a.top_e) * d + 8 * lg;
  }
  // the compensation share's inputs, in flight with the weights (sparse): the
  // Q rows of the block's channels (r <= 128 bf16 each: at most one 16-byte
  // piece a thread), and h_hat of each (channel, token) the token selected
  // (kCh x kT values: two a thread), zero elsewhere. Lane c < kCh of every
  // wave holds the block's channel c (the A rows), so the channel indices come
  // from a lane shuffle, not a load; the token masks and pairs load with the
  // channel indices, and every load is unconditional at a clamped address and
  // masked afterwards, so none of them waits on a branch or adds a round trip
  // before the weights.
  // (the raw values are masked where the tail uses them: a select here would
  // wait for its load).
  const int qpr = (r & 7) == 0 ? r / 8 : 0;  // 16-byte pieces of a Q row (rows not 16-byte aligned: later)
  constexpr int kHz = kCh * kT / kThreads;
  uint4 qp = make_uint4(0, 0, 0, 0);
  float hzv[kHz];
  uint64_t umv[kHz];
  if (r > 0) {
    int tpv[kHz];
#pragma unroll
    for (int u = 0; u < kHz; ++u) {
      const int i = tid + u * kThreads, hc = i / kT, j = i % kT;
      umv[u] = um[min(kCh * chunk + hc, max(uc - 1, 0))];
      tpv[u] = a.tpair[first + min(j, n - 1)];
    }
    if (qpr) qp = *(const uint4*)(a.qmat + ((size_t)e * m + __shfl(ja, min(tid / qpr, kCh - 1), 64)) * r + 8 * (tid % qpr));
#pragma unroll
    for (int u = 0; u < kHz; ++u) hzv[u] = a.hhat[(size_t)tpv[u] * m + __shfl(ja, (tid + u * kThreads) / kT, 64)];
  }
  const int nsteps = d / 32;
  const int kpad = a.kpad;
  // wave 0 finishes token subtile ns from the four waves' sums: lane holds
  // channels 4 lg + v, token 16 ns + li
  auto finish = [&](int ns, const f32x4& accg, const f32x4& accu) {
    s_acc[wave][0][lane] = accg;
    s_acc[wave][1][lane] = accu;
    TILE_MARK_AT(0, item, 2);
    __syncthreads();
    if (wave == 0) {
      const int j = 16 * ns + li;
      f32x4 g = s_acc[0][0][lane], u = s_acc[0][1][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        g += s_acc[w][0][lane];
        u += s_acc[w][1][lane];
      }
      uint16_t hb[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pos = kCh * chunk + 4 * lg + v;
        const bool member = pos < uc && j < n && ((um[pos] >> j) & 1ull);
        const float h = member ? silu_f32(g[v]) * u[v] : 0.0f;
        hb[v] = f32_to_bf16_dev(h);
      }
      if (j < n) {
        uint2 w2;
        w2.x = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
        w2.y = (uint32_t)hb[2] | ((uint32_t)hb[3] << 16);
        *(uint2*)(a.hbuf + (size_t)(first + j) * kpad + kCh * chunk + 4 * lg) = w2;
      }
    }
    __syncthreads();
  };
  // Wave w takes the contiguous quarter [s_beg, s_end) of the hidden
  // dimension's 32-element steps, so a batch of U steps reads U x 64
  // consecutive bytes of each of the 16 rows (quarters interleaved step by
  // step left each batch's pieces 256 bytes apart). Every weight load feeds
  // all NS token subtiles of the tile, so a tile of more than 16 tokens reads
  // its rows once instead of once per subtile.
  const int s_beg = nsteps * wave / kWaves, s_end = nsteps * (wave + 1) / kWaves;
  static_assert(kMSub == 2, "one or two token subtiles per tile");
  auto run = [&](auto ns_count) {
    constexpr int NS = decltype(ns_count)::value;
    constexpr int U = 4;
    f32x4 accg[NS], accu[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) accg[ns] = accu[ns] = f32x4{0.f, 0.f, 0.f, 0.f};
    int s = s_beg;
    for (; s + U <= s_end; s += U) {
      u32x4 gv[U], uv[U], xv[U][NS];
      // the weights first: the first batch's are issued while the token rows'
      // pair indices are still on their way
#pragma unroll
      for (int u = 0; u < U; ++u) {
        gv[u] = *(const u32x4*)(grow + 32 * (s + u));
        uv[u] = *(const u32x4*)(urow + 32 * (s + u));
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) xv[u][ns] = *(const u32x4*)(xr[ns] + 32 * (s + u));
      // every load of the batch issued before the first product (the scheduler
      // would otherwise interleave them with the MFMAs and keep few in flight)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          accg[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(gv[u]), as_bf16x8(xv[u][ns]), accg[ns], 0, 0, 0);
          accu[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(uv[u]), as_bf16x8(xv[u][ns]), accu[ns], 0, 0, 0);
        }
    }
    for (; s < s_end; ++s) {
      const int k0 = 32 * s;
      const u32x4 gv = *(const u32x4*)(grow + k0), uv = *(const u32x4*)(urow + k0);
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const u32x4 xv = *(const u32x4*)(xr[ns] + k0);
        accg[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(gv), as_bf16x8(xv), accg[ns], 0, 0, 0);
        accu[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(uv), as_bf16x8(xv), accu[ns], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) finish(ns, accg[ns], accu[ns]);
  };
  if (nsub > 1)
    run(std::integral_constant<int, 2>{});
  else
    run(std::integral_constant<int, 1>{});
  if (r == 0) {
    TILE_MARK_AT(0, item, 3);
    return;
  }
  // Q^T h_hat over this block's selected channels, per token
  if (qpr) {
    if (tid < kCh * qpr) {
      const bool live = kCh * chunk + tid / qpr < uc;
      const uint32_t w4[4] = {live ? qp.x : 0u, live ? qp.y : 0u, live ? qp.z : 0u, live ? qp.w : 0u};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        s_qr[8 * tid + 2 * h] = bf16lo(w4[h]);
        s_qr[8 * tid + 2 * h + 1] = bf16hi(w4[h]);
      }
    }
  } else {
    for (int i = tid; i < kCh * r; i += kThreads) {
      const int ci = i / r, c = i % r;
      const int pos = kCh * chunk + ci;
      s_qr[i] = pos < uc ? __uint_as_float((uint32_t)a.qmat[((size_t)e * m + ul[pos]) * r + c] << 16) : 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kHz; ++u) {
    const int i = tid + u * kThreads, hc = i / kT, j = i % kT;
    s_hz[hc][j] = j < n && kCh * chunk + hc < uc && ((umv[u] >> j) & 1ull) ? hzv[u] : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < n * r; i += kThreads) {
    const int j = i / r, c = i % r;
    float z = 0.0f;
#pragma unroll
    for (int ci = 0; ci < kCh; ++ci) z += s_hz[ci][j] * s_qr[ci * r + c];
    a.zsel[((size_t)(first + j) * maxch + chunk) * r + c] = z;  // by tile slot
  }
  TILE_MARK_AT(0, item, 3);
}

__global__ __launch_bounds__(kThreads) void k_gate_up_g(FwdArgs a, int dense) {
  __shared__ GateUpSmem sm;
  TILE_MARK(0, 0);
  const int li = threadIdx.x & 15;
  int tile, chunk, e, first, n, uc, ch;
  bool live;
  if (dense) {
    // every chunk of every tile: union position p is channel p
    const int maxch = a.m / kCh;
    tile = blockIdx.x / maxch;
    chunk = blockIdx.x % maxch;
    const int ntl = *a.n_tiles;
    e = a.tile_expert[tile];
    first = a.tile_first[tile];
    n = a.tile_n[tile];
    uc = a.m;
    ch = kCh * chunk + li;
    live = tile < ntl;
  } else {
    // block b runs work item b of the call (items of a tile are consecutive;
    // the blocks past the last item exit): the item's tile entries and its 16
    // channels come in one round trip. An item past its tile's union (the
    // items are laid out for the largest union) exits too.
    const int* item = a.gu_items + (size_t)blockIdx.x * kGuItemInts;
    const int nit = *a.n_items;
    tile = item[0];
    chunk = item[1];
    e = item[2];
    first = item[3];
    n = item[4];
    uc = item[5];
    ch = item[8 + li];
    live = (int)blockIdx.x < nit && chunk < max(1, (uc + kCh - 1) / kCh);
  }
  if (!live) {
    TILE_MARK(0, 3);
    return;
  }
  gate_up_item(a, dense, tile, chunk, blockIdx.x, sm, uc, e, first, n, min(max(ch, 0), a.m - 1));
}

// sum of p[q * stride] for q < count in index order, N loads in flight at a time
// (the last batch masked, so no tail runs one load per round trip)
template <int N>
__device__ __forceinline__ float sum_strided(const float* p, size_t stride, int count) {
  float s = 0.0f;
  for (int q = 0; q < count; q += N) {
    float part[N];
#pragma unroll
    for (int u = 0; u < N; ++u) part[u] = q + u < count ? p[(size_t)(q + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < N; ++u)
      if (q + u < count) s += part[u];
  }
  return s;
}

// ===========================================================================
// Gate/up for one-pair tiles (one token each): the same 16-channel blocks as above,
// computed as row dot products, since a single token leaves an MFMA's other
// 15 columns empty. Wave w takes channels 2w and 2w + 1 of the block; lane l
// holds the 16-byte pieces l + 64 i of x and of both rows, so each load
// instruction reads 1 KiB of a row in one run. fp32 products summed per lane,
// then over the wave. Sparse blocks also leave a part of z = Q^T h_hat over
// the skipped channels: the score blocks' shares of an even slice of the
// groups minus the block's own channels' share, so that z is the sum of the
// pair's gate/up blocks' parts.
// ===========================================================================

// nchg: chunks per tile in the grid, enough for the largest union of the call
static_assert(2 * kB1Waves == kCh, "each wave of the batch-1 gate/up block takes two channels");
__global__ __launch_bounds__(kB1Threads) void k_gate_up_b1(FwdArgs a, int dense, int nchg) {
  __shared__ float s_hz[kCh];
  __shared__ float s_qr[kCh * 128];
  const int d = a.d, m = a.m;
  const int maxch = m / kCh;
  const int tile = blockIdx.x / nchg, chunk = blockIdx.x % nchg;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // this wave's two channel indices, read with the tile's entries before the union size is known
  const int pos0 = kCh * chunk + 2 * wave;
  ROW_MARK(1, 0);  // marks: 0 entry, 1 tile known, 2 rows in and dotted, 3 activations written, 4 end
  const int* ul = a.ulist + (size_t)tile * m;
  const int ul0 = ul[min(pos0, m - 1)], ul1 = ul[min(pos0 + 1, m - 1)];
  const int ntl = *a.n_tiles, uc = a.ucount[tile];
  const int e = a.tile_expert[tile], first = a.tile_first[tile];
  if (tile >= ntl) return;
  const int nch = max(1, (uc + kCh - 1) / kCh);
  if (chunk >= nch) return;
  ROW_MARK(1, 1);
  const int r = dense ? 0 : a.r;
  const int pp = a.tpair[first];
  const int npc = d / 8;
  const uint16_t* xr = a.x + (size_t)(pp / a.top_e) * d;
  const uint16_t* rows[2];
  bool live[2];
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    live[ci] = pos0 + ci < uc;
    rows[ci] = a.wch + ((size_t)e * m + min(max(ci ? ul1 : ul0, 0), m - 1)) * 3 * d;
  }
  uint4 xv[kB1Pieces], gv[2][kB1Pieces], uv[2][kB1Pieces];
#pragma unroll
  for (int i = 0; i < kB1Pieces; ++i) {
    const int pc = lane + 64 * i;
    xv[i] = pc < npc ? *(const uint4*)(xr + 8 * pc) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int ci = 0; ci < 2; ++ci) {
      const bool ld = pc < npc && live[ci];
      gv[ci][i] = ld ? *(const uint4*)(rows[ci] + 8 * pc) : make_uint4(0, 0, 0, 0);
      uv[ci][i] = ld ? *(const uint4*)(rows[ci] + d + 8 * pc) : make_uint4(0, 0, 0, 0);
    }
  }
  // the compensation share's inputs (sparse), addressed with this wave's own
  // channel indices and issued after its rows (no wait before the rows): lane
  // l < 2 r / 8 loads 16-byte piece l % (r / 8) of channel l / (r / 8)'s Q row,
  // lanes 0 and 1 h_hat of the two channels; zero for channels past the union.
  // Ranks that are not a multiple of 8 read Q at the end instead.
  const int qpr = (r & 7) == 0 ? r / 8 : 0;
  uint4 qp = make_uint4(0, 0, 0, 0);
  float hzv = 0.0f;
  // The block also adds up groups [g0, g1) of the score blocks' per-group
  // shares of Q^T h_hat (the groups spread evenly over the pair's nch blocks),
  // so that the down kernel sums one vector per gate/up block. Thread t < r
  // takes column t; the first two groups load with the rows (every thread,
  // clamped, so no load waits on a branch), any further ones at the end.
  const int groups = m / kGroup;
  const int g0 = groups * chunk / nch, g1 = groups * (chunk + 1) / nch;
  const float* gzc = a.gzpart + (size_t)pp * groups * r + min(tid, max(r - 1, 0));
  float gzv[2] = {0.0f, 0.0f};
  if (r > 0) {
    const int qc = lane / max(qpr, 1);
    if (lane < 2 * qpr && live[qc & 1])
      qp = *(const uint4*)(a.qmat + ((size_t)e * m + ((qc & 1) ? ul1 : ul0)) * r + 8 * (lane % qpr));
    if (lane < 2 && live[lane]) hzv = a.hhat[(size_t)pp * m + (lane ? ul1 : ul0)];
#pragma unroll
    for (int u = 0; u < 2; ++u) gzv[u] = gzc[(size_t)min(g0 + u, groups - 1) * r];
  }
  float sg[2] = {0.0f, 0.0f}, su[2] = {0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kB1Pieces; ++i) {
    if (lane + 64 * i < npc) {
#pragma unroll
      for (int ci = 0; ci < 2; ++ci) {
        sg[ci] = dot8_bf16_packed(gv[ci][i], xv[i], sg[ci]);
        su[ci] = dot8_bf16_packed(uv[ci][i], xv[i], su[ci]);
      }
    }
  }
  ROW_MARK(1, 2);
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    const float g = wave_sum(sg[ci]), u = wave_sum(su[ci]);
    if (lane == 0 && pos0 + ci < uc) a.hbuf[(size_t)pp * a.kpad + pos0 + ci] = f32_to_bf16_dev(silu_f32(g) * u);
  }
  ROW_MARK(1, 3);
  if (r == 0) return;
  // this wave's two channels' Q rows and h_hat into the block's arrays
  if (qpr) {
    if (lane < 2 * qpr) {
      const uint32_t w4[4] = {qp.x, qp.y, qp.z, qp.w};
      float* dst = s_qr + (2 * wave + lane / qpr) * r + 8 * (lane % qpr);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        dst[2 * h] = bf16lo(w4[h]);
        dst[2 * h + 1] = bf16hi(w4[h]);
      }
    }
  } else {
    for (int i = lane; i < 2 * r; i += 64) {
      const int ci = i / r, c = i % r;
      s_qr[(2 * wave + ci) * r + c] =
          live[ci] ? __uint_as_float((uint32_t)a.qmat[((size_t)e * m + (ci ? ul1 : ul0)) * r + c] << 16) : 0.0f;
    }
  }
  if (lane < 2) s_hz[2 * wave + lane] = hzv;
  __syncthreads();
  if (tid < r) {
    float z = 0.0f;
#pragma unroll
    for (int ci = 0; ci < kCh; ++ci) z += s_hz[ci] * s_qr[ci * r + tid];
    // this block's groups (in order) minus its selected channels' share
    float gs = g0 < g1 ? gzv[0] : 0.0f;
    if (g0 + 1 < g1) gs += gzv[1];
    for (int g = g0 + 2; g < g1; ++g) gs += gzc[(size_t)g * r];
    a.zsel[((size_t)pp * maxch + chunk) * r + tid] = gs - z;
  }
  ROW_MARK(1, 4);
}

// ===========================================================================
// Down projection for one-pair tiles (one token each): y = sum_k h_k B_k over the
// tile's K rows (union channels' down columns, then the rows of P^T), as row
// axpys. A block takes a slice of SW outputs and one of kc row ranges; in each
// round wave w takes 8 rows, lane l the pieces l + 64 i of the slice, so each
// load reads 1 KiB of a row in one run. Wave sums meet in LDS in a fixed
// order; every block writes its partial, zero when its range is empty. A block
// whose range reaches the P^T rows first finishes their activations z = Q^T
// h_hat over the skipped channels, in fp32: the sum of the gate/up blocks'
// parts, loaded before the block's first rows so that it is ready while
// they stream in.
// ===========================================================================
constexpr int kB1Rows = 8;  // rows per wave per round

template <int NP>
__global__ __launch_bounds__(kB1Threads) void k_down_b1(FwdArgs a, int dense, int kc, int rpb) {
  constexpr int SW = 512 * NP;
  constexpr int kRound = kB1Waves * kB1Rows;
  __shared__ float s_red[kB1Waves][SW];
  __shared__ float s_zp[kB1Waves][64];
  __shared__ float s_z[128];
  const int d = a.d, m = a.m;
  const int slices = d / SW;
  const int per_tile = slices * kc;
  const int tile = blockIdx.x / per_tile, rem = blockIdx.x % per_tile;
  const int sl = rem % slices, kci = rem / slices;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // rows [kb, kb + rpb) of the K range (rpb from the launch: kc rpb covers the
  // largest K); the first round's channel indices are read with the tile's
  // entries, before the union size is known
  const int kb = kci * rpb;
  ROW_MARK(2, 0);  // marks: 0 entry, 1 tile known, 2 z ready, 3 rows summed, 4 end
  const int* ul = a.ulist + (size_t)tile * m;
  int ulv[kB1Rows];
#pragma unroll
  for (int i = 0; i < kB1Rows; ++i) ulv[i] = ul[min(kb + kB1Rows * wave + i, m - 1)];
  const int ntl = *a.n_tiles, uc = a.ucount[tile];
  const int e = a.tile_expert[tile], first = a.tile_first[tile];
  if (tile >= ntl) return;
  ROW_MARK(2, 1);
  const int r = dense ? 0 : a.r;
  const int K = uc + r;
  const int ke = min(K, kb + rpb);
  const int pp = a.tpair[first];
  const uint16_t* hr = a.hbuf + (size_t)pp * a.kpad;
  const size_t col = (size_t)SW * sl;
  uint4 wv[kB1Rows][NP];
  uint32_t hv[kB1Rows];  // the rows' activations (bf16 bits; rows past the union take z below)
  // loads of the rows k0 .. k0 + 7 (channel indices from ulv in the first round)
  // and of their activations, which every lane reads unconditionally (clamped
  // inside the row) so that the round waits for them once, with the rows
  auto load_round = [&](int k0, bool first_round) {
#pragma unroll
    for (int i = 0; i < kB1Rows; ++i) hv[i] = hr[min(k0 + i, a.kpad - 1)];
#pragma unroll
    for (int i = 0; i < kB1Rows; ++i) {
      const int k = k0 + i;
      if (k < ke) {
        const int ch = first_round ? ulv[i] : (k < uc ? ul[k] : 0);
        const uint16_t* row = k < uc ? a.wch + (((size_t)e * m + min(max(ch, 0), m - 1)) * 3 + 2) * d
                                     : a.pmat + ((size_t)e * a.r + (k - uc)) * d;
#pragma unroll
        for (int q = 0; q < NP; ++q) wv[i][q] = *(const uint4*)(row + col + 8 * (lane + 64 * q));
      }
    }
  };
  int k0 = kb + kB1Rows * wave;
  // this block's rows reach P^T: z = Q^T h_hat over the skipped channels, the
  // sum of the nch gate/up blocks' parts (wave w adds parts c0 .. c1 - 1 of
  // columns lane + 64 i); the first kZv parts of the first 64 columns load
  // before the rows, clamped, the rest after them
  constexpr int kZv = 16;
  const bool zblock = r > 0 && ke > max(uc, kb);
  const int maxch = m / kCh;
  const int nch = max(1, (uc + kCh - 1) / kCh);
  const int c0 = nch * wave / kB1Waves, c1 = nch * (wave + 1) / kB1Waves;
  const float* zs = a.zsel + (size_t)pp * maxch * r;
  float zv[kZv];
  if (zblock) {
    const float* zc = zs + min(lane, r - 1);
#pragma unroll
    for (int u = 0; u < kZv; ++u) zv[u] = zc[(size_t)min(c0 + u, maxch - 1) * r];
  }
  if (k0 < ke) load_round(k0, true);
  if (zblock) {
    const bool all_kept = a.k >= m;
    for (int cb = 0; cb < r; cb += 64) {
      const int c = cb + lane;
      float z = 0.0f;
      if (c < r && !all_kept) {
        if (cb == 0) {
#pragma unroll
          for (int u = 0; u < kZv; ++u)
            if (c0 + u < c1) z += zv[u];
          z += sum_strided<16>(zs + (size_t)(c0 + kZv) * r + c, r, c1 - c0 - kZv);
        } else {
          z = sum_strided<16>(zs + (size_t)c0 * r + c, r, c1 - c0);
        }
      }
      s_zp[wave][lane] = z;
      __syncthreads();
      if (wave == 0 && c < r) {
        float zt[kB1Waves];
#pragma unroll
        for (int w = 0; w < kB1Waves; ++w) zt[w] = s_zp[w][lane];
#pragma unroll
        for (int h = kB1Waves / 2; h > 0; h >>= 1)
#pragma unroll
          for (int w = 0; w < h; ++w) zt[w] += zt[w + h];
        s_z[c] = zt[0];
      }
      __syncthreads();
    }
  }
  ROW_MARK(2, 2);
  float acc[NP][8];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int o = 0; o < 8; ++o) acc[q][o] = 0.0f;
  for (; k0 < ke; k0 += kRound) {
#pragma unroll
    for (int i = 0; i < kB1Rows; ++i) {
      const int k = k0 + i;
      if (k < ke) {
        const float h = k < uc ? __uint_as_float(hv[i] << 16) : s_z[k - uc];
#pragma unroll
        for (int q = 0; q < NP; ++q) axpy8_bf16(h, wv[i][q], acc[q]);
      }
    }
    if (k0 + kRound < ke) load_round(k0 + kRound, false);
  }
  ROW_MARK(2, 3);
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int o = 0; o < 8; ++o) s_red[wave][8 * (lane + 64 * q) + o] = acc[q][o];
  __syncthreads();
  float* yp = a.ypart + ((size_t)kci * a.batch * a.top_e + pp) * d + col;
  for (int o = tid; o < SW; o += kB1Threads) {
    float y = 0.0f;
#pragma unroll
    for (int w = 0; w < kB1Waves; ++w) y += s_red[w][o];
    yp[o] = y;
  }
  ROW_MARK(2, 4);
}

// ===========================================================================
// After gate/up, one block per tile slot (a token of a tile): z = Q^T h_hat
// over the token's skipped channels, i.e. the score blocks' per-group shares
// (all channels) minus the gate/up blocks' selected-channel shares, each
// summed in block order, written to the activation columns after the union;
// then zeros up to the next multiple of 32 columns. The grid is the call's
// pairs (every slot holds one), and the slot's union size is its only entry,
// so no block waits for tile entries or exits without work.
// ===========================================================================

constexpr int kZThreads = 256, kZWaves = kZThreads / 64;

__global__ __launch_bounds__(kZThreads) void k_zfin(FwdArgs a) {
  __shared__ float s_part[kZWaves][64];
  const int slot = blockIdx.x;  // the shares and the activations are kept by tile slot
  const int uc = a.slot_ucount[slot];
  const int m = a.m, r = a.r, maxch = m / kCh, kpad = a.kpad, groups = m / kGroup;
  const int nch = max(1, (uc + kCh - 1) / kCh);
  const int kend = (uc + r + 31) / 32 * 32;
  const bool all_kept = a.k >= m;
  // wave q sums its quarter of the groups and of the gate/up blocks
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g0 = groups * q / kZWaves, g1 = groups * (q + 1) / kZWaves;
  const int c0 = nch * q / kZWaves, c1 = nch * (q + 1) / kZWaves;
  const float* gz = a.gzpart + (size_t)slot * groups * r;
  const float* zs = a.zsel + (size_t)slot * maxch * r;
  for (int cb = 0; cb < kend - uc; cb += 64) {
    const int c = cb + lane;
    float z = 0.0f;
    if (c < r && !all_kept)
      z = sum_strided<8>(gz + (size_t)g0 * r + c, r, g1 - g0) - sum_strided<8>(zs + (size_t)c0 * r + c, r, c1 - c0);
    s_part[q][lane] = z;
    __syncthreads();
    if (q == 0 && c < kend - uc) {
      float zt[kZWaves];
#pragma unroll
      for (int w = 0; w < kZWaves; ++w) zt[w] = s_part[w][lane];
      // pairwise, in a fixed order
#pragma unroll
      for (int h = kZWaves / 2; h > 0; h >>= 1)
#pragma unroll
        for (int w = 0; w < h; ++w) zt[w] += zt[w + h];
      a.hbuf[(size_t)slot * kpad + uc + c] = f32_to_bf16_dev(zt[0]);
    }
    __syncthreads();
  }
}

// ===========================================================================
// Down projection of a tile for SW = 64 NW outputs: bf16 MFMA 16x16x32 with
// M = tokens, N = outputs (16 NW per wave), K = the union channels' down columns
// followed by the r rows of P^T (whose activations are z). Each stage stages
// KS channels x SW outputs through LDS: a thread loads 4 channel rows x 8
// outputs (16 bytes each, so a row is read in SW * 2-byte runs), transposes the
// 4 x 8 block in registers and writes one 8-byte LDS row piece per output.
// With few tiles the K range is split over kc blocks, each writing its own
// partial output, which the combine adds in a fixed order.
// ===========================================================================
constexpr int kDownChCap = 1024;

template <int NW>
__global__ __launch_bounds__(kThreads) void k_down_g(FwdArgs a, int dense, int kc) {
  constexpr int SW = 64 * NW;      // outputs per block
  constexpr int OG = SW / 8;       // 8-output groups
  constexpr int CG = kThreads / OG;
  constexpr int RPT = 4;           // channel rows per thread per stage
  constexpr int KS = RPT * CG;     // channels per stage
  constexpr int PITCH = KS + 8;    // halfwords per LDS row (one output)
  __shared__ __align__(16) uint16_t s_b[SW * PITCH];
  __shared__ int s_ch[kDownChCap];  // the block's K-range rows: channel, or -1 - (row of P^T)
  const int d = a.d, m = a.m;
  const int slices = d / SW;
  const int per_tile = slices * kc;
  const int tile = blockIdx.x / per_tile, rem = blockIdx.x % per_tile;
  const int sl = rem % slices, kci = rem / slices;
  TILE_MARK(1, 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int* ul = a.ulist + (size_t)tile * m;
  // The block takes the tile's stages kci, kci + kc, kci + 2 kc, ... (KS rows
  // each), so which union positions it reads does not depend on the union's
  // size: their channel indices load here, with the tile's entries, in one
  // round trip (thread t: stage t / KS of the block, row t % KS; clamped into
  // the tile's list, and positions past the union are not used as indices).
  constexpr int kIdxPer = kDownChCap / kThreads;
  int uidx[kIdxPer];
#pragma unroll
  for (int q = 0; q < kIdxPer; ++q) {
    const int t = tid + q * kThreads;
    uidx[q] = ul[min(KS * (kci + kc * (t / KS)) + t % KS, m - 1)];
  }
  const int ntl = *a.n_tiles, uc = a.ucount[tile];
  const int e = a.tile_expert[tile], first = a.tile_first[tile], n = a.tile_n[tile];
  if (tile >= ntl) {
    TILE_MARK(1, 3);
    return;
  }
  const int r = dense ? 0 : a.r;
  const int K = uc + r;
  const int nst = (K + KS - 1) / KS;
  const int spc = nst > kci ? (nst - kci + kc - 1) / kc : 0;  // this block's stages
  const int msub = (n + 15) >> 4;
  const int kpad = a.kpad;
  const int og = tid % OG, cg = tid / OG;
  const size_t col = (size_t)SW * sl + 8 * og;
  // the block's rows, read from LDS on each stage's load path: a union
  // position's channel, or -1 - (row of P^T); rows past K (the last stage's
  // tail, whose activations are zero) take any channel of the expert. The
  // split keeps spc KS <= kDownChCap (checked at launch).
#pragma unroll
  for (int q = 0; q < kIdxPer; ++q) {
    const int t = tid + q * kThreads;
    const int k = KS * (kci + kc * (t / KS)) + t % KS;
    if (t < spc * KS) s_ch[t] = k < uc || k >= K ? min(max(uidx[q], 0), m - 1) : -1 - (k - uc);
  }
  // the output rows' pairs, in flight with the weights
  int prow[kMSub][4];
#pragma unroll
  for (int ms = 0; ms < kMSub; ++ms)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * ms + 4 * lg + v;
      prow[ms][v] = a.tpair[first + (j < n ? j : 0)];
    }
  __syncthreads();
  // row `row` of the block's stage i
  auto brow = [&](int i, int row) -> const uint16_t* {
    const int c = s_ch[KS * i + row];
    if (c >= 0) return a.wch + (((size_t)e * m + c) * 3 + 2) * d + col;
    return a.pmat + ((size_t)e * a.r + (-1 - c)) * d + col;
  };
  const uint16_t* hrow[kMSub];
#pragma unroll
  for (int ms = 0; ms < kMSub; ++ms) {
    const int j = 16 * ms + li;
    hrow[ms] = a.hbuf + (size_t)(first + (j < n ? j : 0)) * kpad + 8 * lg;
  }
  f32x4 acc[kMSub][NW];
#pragma unroll
  for (int ms = 0; ms < kMSub; ++ms)
#pragma unroll
    for (int nw = 0; nw < NW; ++nw) acc[ms][nw] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one stage: the activations and rows of the stage after it go into the
  // other buffers first (activations clamped inside the row), then this
  // stage's, issued one stage earlier, are waited for, which leaves the next
  // stage's loads in flight; two buffer sets alternate (the loop is unrolled by
  // two), so no register copy waits for a load
  typedef u32x4 ActBuf[KS / 32][kMSub];
  auto load_act = [&](int st, ActBuf& va) {
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks)
#pragma unroll
      for (int ms = 0; ms < kMSub; ++ms) va[ks][ms] = *(const u32x4*)(hrow[ms] + min(KS * st + 32 * ks, kpad - 32));
  };
  // stage i of the block is the tile's stage kci + kc i
  auto stage = [&](int i, const u32x4 (&cur)[RPT], const ActBuf& va, u32x4 (&nxt)[RPT], ActBuf& nva) {
    // (the last stage loads its own rows again: a branch here would leave the
    // waits below unable to count the loads in flight)
    const int in = i + 1 < spc ? i + 1 : i;
    const int st = kci + kc * i;
    load_act(kci + kc * in, nva);
#pragma unroll
    for (int q = 0; q < RPT; ++q) nxt[q] = *(const u32x4*)brow(in, RPT * cg + q);
    // 4 x 8 transpose: output o gets channels RPT cg .. RPT cg + 3
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      uint2 w;
      const uint32_t x0 = cur[0][o >> 1], y0 = cur[1][o >> 1], x1 = cur[2][o >> 1], y1 = cur[3][o >> 1];
      w.x = (o & 1) ? ((x0 >> 16) | (y0 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (y0 << 16));
      w.y = (o & 1) ? ((x1 >> 16) | (y1 & 0xFFFF0000u)) : ((x1 & 0xFFFFu) | (y1 << 16));
      *(uint2*)(s_b + (8 * og + o) * PITCH + RPT * cg) = w;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks) {
      const int k0 = KS * st + 32 * ks;
      if (k0 < K) {
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) {
          const u32x4 bv = *(const u32x4*)(s_b + (16 * NW * wave + 16 * nw + li) * PITCH + 32 * ks + 8 * lg);
#pragma unroll
          for (int ms = 0; ms < kMSub; ++ms)
            if (ms < msub)
              acc[ms][nw] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[ks][ms]), as_bf16x8(bv), acc[ms][nw], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  };
  u32x4 buf0[RPT], buf1[RPT];
  ActBuf va0, va1;
  if (spc > 0) {
    load_act(kci, va0);
#pragma unroll
    for (int q = 0; q < RPT; ++q) buf0[q] = *(const u32x4*)brow(0, RPT * cg + q);
  }
  TILE_MARK(1, 1);
  for (int i = 0; i < spc; i += 2) {
    stage(i, buf0, va0, buf1, va1);
    if (i + 1 < spc) stage(i + 1, buf1, va1, buf0, va0);
  }
  TILE_MARK(1, 2);
  // lane holds C[token 16 ms + 4 lg + v][output 16 NW wave + 16 nw + li]
  float* yp = a.ypart + (size_t)kci * a.batch * a.top_e * d;
#pragma unroll
  for (int ms = 0; ms < kMSub; ++ms)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * ms + 4 * lg + v;
      if (ms < msub && j < n) {
        float* yrow = yp + (size_t)prow[ms][v] * d + (size_t)SW * sl + 16 * NW * wave + li;
#pragma unroll
        for (int nw = 0; nw < NW; ++nw) yrow[16 * nw] = acc[ms][nw][v];
      }
    }
  TILE_MARK(1, 3);
}

// Per token and 64 outputs (one block): the four waves take contiguous quarters
// of the token's (pair, split) partials, each thread loading its quarter's
// values of one output, up to N in flight, and adding them gate-weighted; the
// quarters are then added in wave order and the sum is written as bf16. Spread
// over d / 64 blocks per token, the partials stream through many CUs at once.
__global__ __launch_bounds__(kThreads) void k_combine(FwdArgs a, int kc) {
  constexpr int N = 16;  // partial values in flight per thread
  __shared__ float s_y[kWaves][64];
  __shared__ float s_pw[64];  // the token's gate weights (top_e <= 64)
  const int per_tok = a.d / 64;
  const int t = blockIdx.x / per_tok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = (blockIdx.x % per_tok) * 64 + lane;
  const size_t kstride = (size_t)a.batch * a.top_e * a.d;
  const float* base = a.ypart + (size_t)t * a.top_e * a.d + i;
  const float* w = a.pair_w + (size_t)t * a.top_e;
  const int total = a.top_e * kc;
  const int v_lo = total * wave / kWaves, v_hi = total * (wave + 1) / kWaves;
  ROW_MARK(3, 0);  // marks: 0 entry, 1 partials summed, 2 end
  // the gate weights, read once into LDS (one round trip, instead of one per
  // partial added)
  if (threadIdx.x < a.top_e) s_pw[threadIdx.x] = w[threadIdx.x];
  __syncthreads();
  float y = 0.0f;
  for (int v0 = v_lo; v0 < v_hi; v0 += N) {
    float part[N];
    int ls = v0 / kc, lq = v0 % kc;  // pair and split of value v0
#pragma unroll
    for (int u = 0; u < N; ++u) {
      part[u] = v0 + u < v_hi ? base[(size_t)lq * kstride + (size_t)ls * a.d] : 0.0f;
      if (++lq == kc) {
        lq = 0;
        ++ls;
      }
    }
    ls = v0 / kc;
    lq = v0 % kc;
#pragma unroll
    for (int u = 0; u < N; ++u) {
      if (v0 + u < v_hi) y += s_pw[ls] * part[u];
      if (++lq == kc) {
        lq = 0;
        ++ls;
      }
    }
  }
  s_y[wave][lane] = y;
  __syncthreads();
  ROW_MARK(3, 1);
  if (wave == 0) {
    float o = 0.0f;
#pragma unroll
    for (int g = 0; g < kWaves; ++g) o += s_y[g][lane];
    a.out[(size_t)t * a.d + i] = f32_to_bf16_dev(o);
  }
  ROW_MARK(3, 2);
}

}  // namespace

// k_select keeps the selection bitmap (m/32 words) in LDS
bool grouped_supported(int d, int m) { return d >= 64 && m / 32 <= kSelMaxWords; }

int grouped_down_width(int d) { return d % 256 == 0 ? 256 : 64; }

bool grouped_b1_supported(int d) { return d % 512 == 0 && d <= 64 * 8 * kB1Pieces; }

int grouped_down_split_b1(int kmax, int r) {
  const int rounds = (kmax + r + kB1Waves * kB1Rows - 1) / (kB1Waves * kB1Rows);
  return std::max(1, std::min(kMaxDownSplit, rounds));
}

int grouped_down_split(int max_tiles, int d, int kmax, int r) {
  const int sw = grouped_down_width(d);
  const int blocks = max_tiles * (d / sw);
  int kc = (kDownTargetBlocks + blocks - 1) / blocks;
  // no block takes more than kDownMaxStages stages of the longest tile
  const int ks = sw == 256 ? 32 : 128;
  const int nst_max = (kmax + r + ks - 1) / ks;
  kc = std::max(kc, (nst_max + kDownMaxStages - 1) / kDownMaxStages);
  return kc < 1 ? 1 : (kc > kMaxDownSplit ? kMaxDownSplit : kc);
}

#ifdef MOE_SEL_TIMELINE
// copies the select blocks' phase marks (64 blocks x 8 wall-clock values) to host
extern "C" int moe_sel_timeline_select(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_sel_marks), sizeof(g_sel_marks));
}
// copies the one-pair-tile kernels' phase marks (4 kernels x 512 blocks x 8 values) to host
extern "C" int moe_sel_timeline_rows(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_row_marks), sizeof(g_row_marks));
}
// copies the expert-tile kernels' phase marks (2 kernels x 8192 blocks x 4 values) to host
extern "C" int moe_sel_timeline_tiles(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_tile_marks), sizeof(g_tile_marks));
}
#endif

hipError_t launch_forward(const FwdArgs& a, bool dense, hipStream_t stream) {
  const int pairs = a.batch * a.top_e;
  // One pair per tile (row kernels, no plan, no union) or pairs grouped by
  // expert into tiles of up to kT tokens; max_tiles >= pairs in the first case.
  const bool pair_tiles = grouped_b1_supported(a.d) && grouped_pair_tiles(a.batch, a.top_e, a.n_experts, dense);
  const bool b1 = pair_tiles;
  // the score blocks route and quantise their tokens themselves
  const bool self_route = pair_tiles && !dense && a.n_experts <= 256;
  // int16 score activations exist only where the score blocks quantise x themselves
  if (!dense && a.score_kind == 3 && !self_route) return hipErrorNotSupported;
  const int groups = a.m / kGroup;
  if (!self_route)
    hipLaunchKernelGGL(k_route_quant, dim3(a.batch), dim3(kThreads), 0, stream, a, pair_tiles ? 1 : 0);
  if (!pair_tiles) hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, stream, a, dense ? 1 : 0);
  if (!dense) {
    if (b1 && a.score_kind == 3)
      hipLaunchKernelGGL(k_score_b1<true>, dim3(a.max_tiles * groups), dim3(kB1Threads),
                         2 * (size_t)a.d + 256 * (size_t)a.r, stream, a, self_route ? 1 : 0);
    else if (b1)
      hipLaunchKernelGGL(k_score_b1<false>, dim3(a.max_tiles * groups), dim3(kB1Threads),
                         2 * (size_t)a.d + 256 * (size_t)a.r, stream, a, self_route ? 1 : 0);
    else
      hipLaunchKernelGGL(k_score_g, dim3(a.max_tiles * groups), dim3(kThreads),
                         ((size_t)kT * 64 + (size_t)64 * a.r) * 4, stream, a);
    const int pt = pair_tiles ? 1 : 0;
    if (a.m <= kSelThreads)
      hipLaunchKernelGGL(k_select<1>, dim3(pairs), dim3(kSelThreads), 0, stream, a, pt);
    else if (a.m <= 4 * kSelThreads)
      hipLaunchKernelGGL(k_select<4>, dim3(pairs), dim3(kSelThreads), 0, stream, a, pt);
    else
      hipLaunchKernelGGL(k_select<16>, dim3(pairs), dim3(kSelThreads), 0, stream, a, pt);
  }
  // with one pair per tile the select kernel writes the unions itself
  if (dense || !pair_tiles)
    hipLaunchKernelGGL(k_union, dim3(a.max_tiles), dim3(kThreads), 0, stream, a, dense ? 1 : 0);
  // the largest union a tile can have: k channels per token of the tile, at most m
  const int tile_tokens = pair_tiles ? 1 : std::min(a.batch, kT);
  const int kmax = (dense || a.thr_mode) ? a.m : (int)std::min<long>(a.m, (long)a.k * tile_tokens);
  if (b1) {
    const int nchg = std::max(1, (kmax + kCh - 1) / kCh);
    hipLaunchKernelGGL(k_gate_up_b1, dim3(a.max_tiles * nchg), dim3(kB1Threads), 0, stream, a, dense ? 1 : 0, nchg);
  } else {
    hipLaunchKernelGGL(k_gate_up_g, dim3(a.max_tiles * (a.m / kCh)), dim3(kThreads), 0, stream, a, dense ? 1 : 0);
  }
  // the row down kernel finishes the compensation coordinates itself
  if (!dense && !b1) hipLaunchKernelGGL(k_zfin, dim3(a.batch * a.top_e), dim3(kZThreads), 0, stream, a);
  const int sw = grouped_down_width(a.d);
  if (b1) {
    const int kc1 = grouped_down_split_b1(kmax, dense ? 0 : a.r);
    // rows per block: a multiple of one round with kc1 blocks covering the largest K
    constexpr int kRound = kB1Waves * kB1Rows;
    const int kall = kmax + (dense ? 0 : a.r);
    const int rpb = ((kall + kc1 - 1) / kc1 + kRound - 1) / kRound * kRound;
    if (a.d % 1024 == 0)
      hipLaunchKernelGGL(k_down_b1<2>, dim3(a.max_tiles * (a.d / 1024) * kc1), dim3(kB1Threads), 0, stream, a,
                         dense ? 1 : 0, kc1, rpb);
    else
      hipLaunchKernelGGL(k_down_b1<1>, dim3(a.max_tiles * (a.d / 512) * kc1), dim3(kB1Threads), 0, stream, a,
                         dense ? 1 : 0, kc1, rpb);
    hipLaunchKernelGGL(k_combine, dim3(a.batch * (a.d / 64)), dim3(kThreads), 0, stream, a, kc1);
    return hipGetLastError();
  }
  const int kc = grouped_down_split(a.max_tiles, a.d, kmax, dense ? 0 : a.r);
  {
    // every block's rows fit its LDS index list (the split guarantees it)
    const int ks = sw == 256 ? 32 : 128;
    const int nst_max = (kmax + (dense ? 0 : a.r) + ks - 1) / ks;
    if ((nst_max + kc - 1) / kc * ks > kDownChCap) return hipErrorInvalidValue;
  }
  if (sw == 256)
    hipLaunchKernelGGL(k_down_g<4>, dim3(a.max_tiles * (a.d / 256) * kc), dim3(kThreads), 0, stream, a, dense ? 1 : 0, kc);
  else
    hipLaunchKernelGGL(k_down_g<1>, dim3(a.max_tiles * (a.d / 64) * kc), dim3(kThreads), 0, stream, a, dense ? 1 : 0, kc);
  hipLaunchKernelGGL(k_combine, dim3(a.batch * (a.d / 64)), dim3(kThreads), 0, stream, a, kc);
  return hipGetLastError();
}

}  // namespace moe_sel
