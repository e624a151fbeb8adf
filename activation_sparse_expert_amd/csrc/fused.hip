// Fused single-launch forward for small batches on gfx950.
//
// One kernel runs the whole block; its workgroups take one of three roles by
// block index, producers always below their consumers:
//
//   [0, n_score)            score    one (token, expert) pair x 32 (or 64) channels:
//                                    route + quantise (redundant per block), the
//                                    2-bit sketch GEMV, pinned channel scores,
//                                    h_hat, and this group's share of Q^T h_hat;
//   [.., + n_gather)        gather   one pair x C selected channels: repeats the
//                                    pair's top-k selection on the m published
//                                    scores, reads its C channels' bf16 gate/up/
//                                    down vectors (one 12*d-byte run each), SwiGLU
//                                    and the gate-weighted down partial over all
//                                    of d; chunk 0 also forms z = Q^T h_hat over
//                                    the skipped channels;
//   [.., + n_combine)       combine  one token x 64 output elements: prefetches
//                                    its slice of P for the routed experts, sums
//                                    the token's partials and P z, writes bf16.
//
// "Top-k instead of a threshold" and "A reader built from weights alone" (page
// "KAIST drops calibration from MoE decoding, speeds up blocks by up to 2.69x
// over vLLM") give the selection and the compensation; the dense variant reads
// every channel and has no score blocks.
//
// Hand-off: every value that crosses workgroups has exactly one consumer and a
// slot of its own, holding the sentinel 0xFFFFFFFF when empty (a NaN pattern
// that no arithmetic here produces). Producers write their slots with
// device-coherent stores and move on; consumers poll the data itself with
// device-coherent loads until no sentinel is left, then write the sentinel back,
// so every call starts from empty slots and HIP-graph replays stay valid. Waits
// are bounded; on time-out an error bit is set and the block proceeds.
//
// Decode-time work is latency bound, so every role issues all of its global
// loads before consuming any (fixed unrolled counts, clamped addresses, masked
// contributions).
//
// The launch requires every block to be resident at once (checked on the host
// with the occupancy API).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "device_common.h"
#include "internal.h"
#include "kernels.h"

namespace moe_sel {
namespace {

using namespace dev;

constexpr int kMaxChunkSparse = 8;   // channels per gather block, all loaded at once
constexpr int kMaxChunkDense = 12;   // (158 VGPRs for d <= 2048: three blocks per CU)
constexpr int kMaxKeysPer = 16;      // m <= 16 * 256
constexpr int kDirectRank = 64;      // boundary-bin keys ranked by their owners (more: radix passes)
static_assert(kWaves == 4, "the select reads its four wave totals as one int4");
constexpr int kScoreBlk = 16;        // sketch blocks in flight per lane group pair (d = 2048 in one batch)
constexpr int kZPass = 4;            // compensation row passes loaded together
constexpr int kZWarm = 16;           // Q pieces per thread in flight while the z block warms L2
constexpr int kMaxZPart = 4;         // zpart values per thread ((m / 32) * r <= 1024)
constexpr int kMaxP = 4;             // 16-byte P pieces per combine thread (top_e * r <= 256)
constexpr int kCombPer = 8;          // producers whose partials a combine thread polls per batch
constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr uint64_t kEmpty64 = 0xFFFFFFFFFFFFFFFFull;

struct Smem {
  int ids[64];
  float w[64];
  union {
    int hist[2048];                // radix select
    uint64_t route[3 * kThreads];  // routing scratch
  };
  alignas(16) int cand[2 * kThreads];  // boundary-bin candidates of the select (order keys)
  int tmp[kWaves + 2];
  alignas(16) int sel_ws[kWaves];  // wave totals of the select's first scan
  alignas(16) int sel_ws2[kWaves]; // and of its second
  alignas(16) int sel_b[4];        // boundary bin, keys above it, keys in it, candidates placed
  uint64_t sel_t;                  // order key of the last boundary-bin key taken
  float red[kWaves][2 * kMaxChunkDense];
  uint32_t amax[kWaves];
  int qsum[kWaves][4];             // per wave: sum of x_q over each quarter of d (the score role's split)
};

__device__ __forceinline__ bool empty(float v) { return __float_as_uint(v) == kEmpty; }

__device__ __forceinline__ uint64_t ld_coh64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_coh(float* p) { st_coh(p, __uint_as_float(kEmpty)); }

// Bounded waits: a wait loop calls spent() before each poll round and gives up
// once `limit` rounds have been polled (at once for limit 0). The decision is
// uniform over the threads that wait together. gave_up() records it: lane 0 of
// every wave that gave up sets the error bit.
__device__ __forceinline__ bool spent(int& spins, int limit) {
  if (spins >= limit) return true;
  if (spins++ > 0) __builtin_amdgcn_s_sleep(2);
  return false;
}
__device__ __forceinline__ void gave_up(int* err, int bit) {
  if ((threadIdx.x & 63) == 0) atomicOr(err, bit);
}
constexpr float kPoison = __builtin_nanf("");

// Phase marks for measuring the kernel's timeline: MARK(ev) compiles to nothing
// unless the library is built with MOE_SEL_TIMELINE, which records the wall
// clock of thread 0 of each block at each mark (events 0..7 per block; their
// meaning by role: 0 entry, 1 routed, 2 first wait over / dots done, 3 select
// done / second wait over, 4 SwiGLU done, 5 end; gather only: 6 gate and up
// rows in, 7 down rows in).
#ifdef MOE_SEL_TIMELINE
constexpr int kMarkEvents = 8, kMarkBlocks = 8192;
__device__ unsigned long long g_marks[kMarkBlocks * kMarkEvents];
#define MARK(ev)                                                                        \
  do {                                                                                  \
    if (threadIdx.x == 0 && blockIdx.x < kMarkBlocks) g_marks[blockIdx.x * kMarkEvents + (ev)] = wall_clock64(); \
  } while (0)
// where each block runs: XCC_ID (hardware register 20) above HW_ID (register 4:
// CU, shader array and engine in bits 8..15)
__device__ unsigned long long g_place[kMarkBlocks];
#define PLACE()                                                                             \
  do {                                                                                      \
    if (threadIdx.x == 0 && blockIdx.x < kMarkBlocks)                                       \
      g_place[blockIdx.x] = ((unsigned long long)__builtin_amdgcn_s_getreg((3 << 11) | 20) << 32) | \
                            (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 4);              \
  } while (0)
#else
#define MARK(ev) ((void)0)
#define PLACE() ((void)0)
#endif

template <int SLOTS>
__device__ __forceinline__ void load_x(const uint16_t* x, int d, uint4 (&xv)[SLOTS]) {
  const int nslots = d / 8;
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int s = threadIdx.x + u * kThreads;
    xv[u] = s < nslots ? *(const uint4*)(x + 8 * s) : make_uint4(0, 0, 0, 0);
  }
}

// int8 activations with a power-of-two scale into LDS (xq[0, d)); returns the
// exponent. With x16 the activations are int16, stored as their high bytes in
// xq[0, d) and their low bytes in xq[d, 2d). Each wave's sums of the
// activations over the four quarters of d (64-element blocks
// [nb q / 4, nb (q + 1) / 4)) go to sm.qsum (read them after the next barrier).
template <int SLOTS>
__device__ __forceinline__ int quantise_to_lds(const uint4 (&xv)[SLOTS], int d, int8_t* xq, Smem& sm, bool x16) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nslots = d / 8;
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const uint32_t w4[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) amax = max(amax, max(w4[q] & 0x7FFFu, (w4[q] >> 16) & 0x7FFFu));
  }
  amax = wave_max_u(amax);
  if (lane == 0) sm.amax[wave] = amax;
  __syncthreads();
  amax = sm.amax[0];
  for (int w = 1; w < kWaves; ++w) amax = max(amax, sm.amax[w]);
  const int e_t = amax ? score_exponent(amax, x16) : 0;
  int qs[4] = {0, 0, 0, 0};
  const int nb = nslots >> 3;
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int s = tid + u * kThreads;
    if (s < nslots) {
      float f[8];
      unpack8(xv[u], f);
      uint32_t lo = 0, hi = 0, lo2 = 0, hi2 = 0;  // bytes 0..3 and 4..7: high (or only) bytes, then low bytes
      int sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = (int)__builtin_rintf(__builtin_ldexpf(f[q], -e_t));
        const int b = (int)__builtin_rintf(__builtin_ldexpf(f[q + 4], -e_t));
        lo |= ((uint32_t)(x16 ? a >> 8 : a) & 0xFFu) << (8 * q);
        hi |= ((uint32_t)(x16 ? b >> 8 : b) & 0xFFu) << (8 * q);
        lo2 |= ((uint32_t)a & 0xFFu) << (8 * q);
        hi2 |= ((uint32_t)b & 0xFFu) << (8 * q);
        sum += a + b;
      }
      *(uint2*)(xq + 8 * s) = make_uint2(lo, hi);
      if (x16) *(uint2*)(xq + d + 8 * s) = make_uint2(lo2, hi2);
      const int b = s >> 3;
      const int q = (b >= nb / 4) + (b >= nb * 2 / 4) + (b >= nb * 3 / 4);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k == q) qs[k] += sum;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    qs[k] = wave_sum_i(qs[k]);
    if (lane == 0) sm.qsum[wave][k] = qs[k];
  }
  return e_t;
}

__device__ __forceinline__ void route(const FusedArgs& a, int t, Smem& sm, bool with_weights = true) {
  block_route(a.logits + (size_t)t * a.n_experts, a.n_experts, a.top_e, sm.ids, sm.w, sm.route, with_weights);
}

// ---------------------------------------------------------------------------
// score role: one (token, expert) pair x SC = a.score_ch channels (32 or 64),
// so that a pair's sketch bytes spread over m / SC blocks
// ---------------------------------------------------------------------------
template <int SLOTS, int SC>
__device__ __forceinline__ void score_role(const FusedArgs& a, int bid, Smem& sm, unsigned char* dyn) {
  constexpr int lps = 64 / SC;  // lane groups per wave: 2 (SC = 32) or 1
  const int zg = a.m / SC;
  const int p = bid / zg, sb = bid % zg;
  const int t = p / a.top_e, slot = p % a.top_e;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  const bool x16 = a.score_kind == 3;                        // int16 activations (score ablation)
  int8_t* s_xq = (int8_t*)dyn;                               // 2d bytes: x_q (int8), or high then low bytes
  uint16_t* s_q = (uint16_t*)(dyn + 2 * a.d);                // SC x r bf16
  float* s_h = (float*)(dyn + 2 * a.d + 64 * r * 2);         // SC
  float* s_sc = s_h + 64;                                    // SC
  int* s_part = (int*)(s_sc + 64);                           // kWaves x 64

  uint4 xv[SLOTS];
  load_x<SLOTS>(a.x + (size_t)t * a.d, a.d, xv);  // in flight during the routing
  route(a, t, sm, false);                          // the expert only: no gate weights here
  MARK(1);
  const int e = sm.ids[slot];
  // every global load of this block: the sketch codes, the SC Q rows, the statistics.
  // Lane = (lane group, channel c); wave = (matrix, half of the d parts). The d
  // range splits into 2 * lps parts of whole 64-element blocks (quarters for
  // SC = 32, halves for 64); a load instruction reads lps runs of 64 * 16 / lps
  // bytes of one code block row each.
  const int c = lane & (SC - 1), mat = wave >> 1;
  constexpr int nparts = 2 * lps;
  const int part = (wave & 1) * lps + lane / SC;
  const int j0 = sb * SC;  // first channel of the block
  const int nb = a.d / kBlock;
  const int b0 = nb * part / nparts, b1 = nb * (part + 1) / nparts;  // empty when nb is small
  // code block b of this lane's channel and matrix sits 1 KiB * b past the row
  // start; loads are addressed as a block-uniform base plus a 32-bit lane offset,
  // every lane issuing all of them (clamped to its part's last block, or block 0
  // for an empty part), so none is masked
  constexpr int kSB = kScoreBlk / lps;  // blocks per load batch: a part of d = 2048
  const char* cbase = (const char*)(a.codes + (size_t)e * codes_dwords_per_expert(a.d, a.m) +
                                    codes_dword_index(a.d, a.m, j0 / kGroup, 0, 0, 0, 0));
  const uint32_t row_off = (uint32_t)codes_dword_index(a.d, a.m, 0, mat, 0, j0 % kGroup + c, 0) * 4u;
  const int nblk = b1 - b0, blast = max(b1 - 1, 0);
  uint4 cb[kSB];
#pragma unroll
  for (int i = 0; i < kSB; ++i)
    cb[i] = *(const uint4*)(cbase + (row_off + (uint32_t)min(b0 + i, blast) * 1024u));
  const uint4* qsrc = (const uint4*)(a.qmat + ((size_t)e * a.m + (size_t)j0) * r);
  const int qpieces = SC * r / 8;
  constexpr int kQv = SC * 128 / 8 / kThreads;  // pieces per thread for r <= 128
  uint4 qv[kQv];
#pragma unroll
  for (int u = 0; u < kQv; ++u)
    qv[u] = tid + u * kThreads < qpieces ? qsrc[tid + u * kThreads] : make_uint4(0, 0, 0, 0);
  const float4 st = a.stats[(size_t)e * a.m + j0 + c];
  const int e_t = quantise_to_lds<SLOTS>(xv, a.d, s_xq, sm, x16);
  __syncthreads();  // x_q in LDS
  // sum of x_q over this thread's part of d: quarters sum directly, halves are two quarters
  const int q0 = part * 4 / nparts, q1 = (part + 1) * 4 / nparts;
  int qs = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q >= q0 && q < q1) qs += sm.qsum[w][q];
  CodeAcc acc, acc_lo;  // acc_lo: the low bytes of int16 activations
  for (int c0 = 0; c0 < nblk; c0 += kSB) {
    if (c0 != 0) {
#pragma unroll
      for (int i = 0; i < kSB; ++i)
        cb[i] = *(const uint4*)(cbase + (row_off + (uint32_t)min(b0 + c0 + i, blast) * 1024u));
    }
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      if (c0 + i < nblk) {
        const int4* xb = (const int4*)(s_xq + 64 * (b0 + c0 + i));
        dot_codes16(cb[i].x, xb[0], acc);
        dot_codes16(cb[i].y, xb[1], acc);
        dot_codes16(cb[i].z, xb[2], acc);
        dot_codes16(cb[i].w, xb[3], acc);
        if (x16) {
          const int4* xl = (const int4*)(s_xq + a.d + 64 * (b0 + c0 + i));
          dot_codes16_u(cb[i].x, xl[0], acc_lo);
          dot_codes16_u(cb[i].y, xl[1], acc_lo);
          dot_codes16_u(cb[i].z, xl[2], acc_lo);
          dot_codes16_u(cb[i].w, xl[3], acc_lo);
        }
      }
    }
  }
  MARK(2);
  const int cx = x16 ? 256 * code_acc_total(acc) + code_acc_total(acc_lo) : code_acc_total(acc);
  s_part[wave * 64 + lane] = cx - qs;  // sum (code - 1) * q = sum t * q
#pragma unroll
  for (int u = 0; u < kQv; ++u) {
    const int i = tid + u * kThreads;
    if (i < qpieces) ((uint4*)s_q)[i] = qv[u];
  }
  __syncthreads();
  if (tid < SC) {  // every part of each matrix: waves 0, 1 (gate) and 2, 3 (up), all lane groups
    int dg = 0, du = 0;
    for (int k = 0; k < 64; k += SC) {
      dg += s_part[k + c] + s_part[64 + k + c];
      du += s_part[128 + k + c] + s_part[192 + k + c];
    }
    float h, sc;
    pinned_score(dg, du, e_t, st, h, sc, a.score_kind);
    s_h[c] = h;
    s_sc[c] = sc;
  }
  __syncthreads();
  if (wave == 0) {
    // publish (score, h_hat) of the block's channels once, for every reader of the pair
    if (lane < SC) {
      const uint64_t v = (uint64_t)__float_as_uint(s_sc[lane]) | ((uint64_t)__float_as_uint(s_h[lane]) << 32);
      st_coh64(&a.xscore[(size_t)p * a.m + j0 + lane], v);
      st_coh(&a.hhat[(size_t)p * a.m + j0 + lane], s_h[lane]);  // for inspection only
      st_coh(&a.score[(size_t)p * a.m + j0 + lane], s_sc[lane]);
    }
  } else if (wave == kWaves - 1) {
    // this block's share of Q^T h_hat over its channels, for the z block
    for (int col = lane; col < r; col += 64) {
      float z = 0.0f;
#pragma unroll 16
      for (int j = 0; j < SC; ++j) z += s_h[j] * bf16f(s_q[j * r + col]);
      st_coh(&a.zpart[((size_t)p * zg + sb) * r + col], z);
    }
  }
  MARK(3);
  MARK(5);
}

// ---------------------------------------------------------------------------
// gather role
// ---------------------------------------------------------------------------
// Top-k (1 <= k < m) of the m keys of a pair (binary32 bits of non-negative
// scores, so their unsigned order is the scores' order) held consecutively, R
// per thread (thread t: channels t R .. t R + R - 1): writes the selected
// channels in ascending order to s_sel[0..k). Larger scores first, equal scores
// to the lower channel index ("Top-k instead of a threshold").
//   1. a 2048-bin histogram of key bits 30..20 (an eighth of an octave a bin);
//   2. the bin D holding the k-th largest key, by one scan of the bin counts;
//   3. the keys in bin D ranked exactly (larger first, lower index first) by one
//      wave, which publishes the order key of the last one taken (a bin of more
//      than kDirectRank keys, from ties or clusters, goes to three radix passes
//      that give the k-th key T, equal keys taken lowest index first);
//   4. the ascending positions of the taken keys, by one more scan.
// sm.hist and sm.sel_b[3] must be zero, with a barrier passed since. Barriers
// inside (all threads call).
template <int MK>
__device__ __forceinline__ void select_consecutive(const uint32_t (&key)[MK], int R, int m, int k, Smem& sm,
                                                   int* s_sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = tid * R;
#pragma unroll
  for (int u = 0; u < MK; ++u)
    if (u < R && j0 + u < m) atomicAdd(&sm.hist[key[u] >> 20], 1);
  __syncthreads();
  int h[8];
  {
    const int4 lo = *(const int4*)&sm.hist[tid * 8], hi = *(const int4*)&sm.hist[tid * 8 + 4];
    h[0] = lo.x; h[1] = lo.y; h[2] = lo.z; h[3] = lo.w;
    h[4] = hi.x; h[5] = hi.y; h[6] = hi.z; h[7] = hi.w;
  }
  int cnt = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) cnt += h[b];
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) sm.sel_ws[wave] = incl;
  __syncthreads();
  const int4 ws = *(const int4*)sm.sel_ws;
  const int before = incl - cnt + (wave > 0 ? ws.x : 0) + (wave > 1 ? ws.y : 0) + (wave > 2 ? ws.z : 0);
  const int above = ws.x + ws.y + ws.z + ws.w - before - cnt;  // keys in the bins above this thread's eight
  if (above < k && k <= above + cnt) {
    // the one thread whose bins hold the k-th largest key walks them, without
    // branches (the other waves go straight to the barrier)
    int acc = above, bd = 0, ad = 0, nd = 0;
    bool found = false;
#pragma unroll
    for (int b = 7; b >= 0; --b) {
      const bool here = !found && k <= acc + h[b];
      bd = here ? b : bd;
      ad = here ? acc : ad;
      nd = here ? h[b] : nd;
      found = found || here;
      acc += h[b];
    }
    sm.sel_b[0] = tid * 8 + bd;
    sm.sel_b[1] = ad;
    sm.sel_b[2] = nd;
  }
  __syncthreads();
  const int4 sb = *(const int4*)sm.sel_b;
  const uint32_t D = (uint32_t)sb.x;
  const int krem = k - sb.y, ncand = sb.z;
  bool take[MK];
  if (ncand <= kDirectRank) {
    // the boundary bin's keys go to a list: each wave takes its slots with one
    // LDS atomic, its lanes place their keys by ballot offsets
    uint64_t* s_cand = (uint64_t*)sm.cand;
    uint64_t bal[MK];
    int wcount = 0;
#pragma unroll
    for (int u = 0; u < MK; ++u) {
      bal[u] = __ballot(u < R && j0 + u < m && (key[u] >> 20) == D);
      wcount += __popcll(bal[u]);
    }
    if (wcount) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&sm.sel_b[3], wcount);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int u = 0; u < MK; ++u) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u], 0));
        if ((bal[u] >> lane) & 1) s_cand[base + below] = order_key(key[u], j0 + u);
        base += __popcll(bal[u]);
      }
    }
    // zero keys pad the list to a multiple of 8 (an order key of 0 is below
    // every real one, so the padding never counts)
    if (tid < 8) s_cand[ncand + tid] = 0ull;
    __syncthreads();
    // wave 0 ranks the list, one entry per lane (larger first, lower index
    // first; the order keys are distinct), and publishes the order key of
    // rank krem - 1: the bin's keys at or above it are taken
    if (wave == 0) {
      const uint64_t mine = lane < ncand ? s_cand[lane] : 0ull;
      const ulonglong2* c2 = (const ulonglong2*)s_cand;
      int rank = 0;
      for (int i = 0; i < ncand; i += 8) {
        const ulonglong2 a0 = c2[i / 2], a1 = c2[i / 2 + 1], a2 = c2[i / 2 + 2], a3 = c2[i / 2 + 3];
        rank += (a0.x > mine) + (a0.y > mine) + (a1.x > mine) + (a1.y > mine) + (a2.x > mine) + (a2.y > mine) +
                (a3.x > mine) + (a3.y > mine);
      }
      if (lane < ncand && rank == krem - 1) sm.sel_t = mine;
    }
    __syncthreads();
    const uint64_t t_ord = sm.sel_t;
#pragma unroll
    for (int u = 0; u < MK; ++u) {
      const bool valid = u < R && j0 + u < m;
      const uint32_t dg = key[u] >> 20;
      take[u] = valid && (dg > D || (dg == D && order_key(key[u], j0 + u) >= t_ord));
    }
  } else {
    uint32_t T;
    int kr;
    block_topk_radix<MK>(key, R, m, k, sm.hist, sm.tmp, T, kr);
    int n_eq = 0;
#pragma unroll
    for (int u = 0; u < MK; ++u) n_eq += (u < R && j0 + u < m) && key[u] == T;
    int eq_total;
    int eq_before = block_excl_scan(n_eq, sm.tmp, &eq_total);
#pragma unroll
    for (int u = 0; u < MK; ++u) {
      const bool valid = u < R && j0 + u < m;
      const bool eq = valid && key[u] == T;
      take[u] = valid && (key[u] > T || (eq && eq_before < kr));
      eq_before += eq;
    }
  }
  int n = 0;
#pragma unroll
  for (int u = 0; u < MK; ++u) n += take[u];
  const int incl2 = wave_incl_scan(n);
  if (lane == 63) sm.sel_ws2[wave] = incl2;
  __syncthreads();
  const int4 ws2 = *(const int4*)sm.sel_ws2;
  int pos = incl2 - n + (wave > 0 ? ws2.x : 0) + (wave > 1 ? ws2.y : 0) + (wave > 2 ? ws2.z : 0);
#pragma unroll
  for (int u = 0; u < MK; ++u)
    if (take[u]) s_sel[pos++] = j0 + u;
}

// Waits for the pair's m (score, h_hat) values in the pair's slots (and, for the
// z block, the pair's zpart slots), then selects the pair's top-k: the selected
// channels ascending in s_sel[0..k); for the z block also the sketch
// activations in s_hh and the zpart values in s_zp. Chunk 0 also records the
// selection for inspection. Every reader calls empty_pair_slots at its end.
template <int MK>  // key slots per thread: m <= MK * kThreads
__device__ __forceinline__ bool gather_select_mk(const FusedArgs& a, int p, int c, bool with_zpart, Smem& sm,
                                                 float* s_hh, int* s_sel, float* s_zp) {
  const int tid = threadIdx.x, m = a.m, k = a.k, r = a.r;
  const int zg = m / a.score_ch;
  const int R = (m + kThreads - 1) / kThreads;  // consecutive channels per thread
  const uint64_t* slots = a.xscore + (size_t)p * m + (size_t)tid * R;
  const int nzp = with_zpart ? zg * r : 0;
  float* zslots = a.zpart + (size_t)p * zg * r;
  // cleared for the select, ordered before it by the polling barrier
#pragma unroll
  for (int b = 0; b < 8; ++b) sm.hist[tid * 8 + b] = 0;
  if (tid == 0) sm.sel_b[3] = 0;
  uint64_t v[MK];
  float zv[kMaxZPart];
  uint32_t pending = 0;  // bit u: key slot u; bit 16 + u: zpart slot u
#pragma unroll
  for (int u = 0; u < MK; ++u) {
    v[u] = 0ull;
    if (u < R && tid * R + u < m) pending |= 1u << u;
  }
#pragma unroll
  for (int u = 0; u < kMaxZPart; ++u) {
    zv[u] = 0.0f;
    if (tid + u * kThreads < nzp) pending |= 1u << (16 + u);
  }
  int spins = 0;
  bool bad = false;
  while (true) {
    if (spent(spins, a.spin_limit)) {
      bad = true;
      break;
    }
#pragma unroll
    for (int u = 0; u < MK; ++u)
      if ((pending >> u) & 1) v[u] = ld_coh64(slots + u);
#pragma unroll
    for (int u = 0; u < kMaxZPart; ++u)
      if ((pending >> (16 + u)) & 1) zv[u] = ld_coh(zslots + tid + u * kThreads);
#pragma unroll
    for (int u = 0; u < MK; ++u)
      if ((uint32_t)v[u] != kEmpty) pending &= ~(1u << u);
#pragma unroll
    for (int u = 0; u < kMaxZPart; ++u)
      if (!empty(zv[u])) pending &= ~(1u << (16 + u));
    if (__syncthreads_and(pending == 0)) break;
  }
  MARK(2);
  if (bad) {
    // slots still empty after giving up hold no score: rank them as 0 (the
    // sentinel's key bits would index past the select's histogram) with a NaN
    // sketch activation; the caller poisons what it publishes
    gave_up(a.err, 1);
#pragma unroll
    for (int u = 0; u < MK; ++u)
      if ((uint32_t)v[u] == kEmpty) v[u] = (uint64_t)__float_as_uint(kPoison) << 32;
  }
  uint32_t key[MK];
#pragma unroll
  for (int u = 0; u < MK; ++u) key[u] = (u < R && tid * R + u < m) ? (uint32_t)v[u] : 0u;
  if (with_zpart) {
#pragma unroll
    for (int u = 0; u < MK; ++u)
      if (u < R && tid * R + u < m) s_hh[tid * R + u] = __uint_as_float((uint32_t)(v[u] >> 32));
#pragma unroll
    for (int u = 0; u < kMaxZPart; ++u) {
      const int i = tid + u * kThreads;
      if (i < nzp) {
        s_zp[i] = zv[u];
        clear_coh(zslots + i);
      }
    }
  }
  if (k >= m || k <= 0) {
    for (int j = tid; j < k; j += kThreads) s_sel[j] = j;
  } else {
    select_consecutive<MK>(key, R, m, k, sm, s_sel);
  }
  __syncthreads();
  if (c == 0)
    for (int i = tid; i < k; i += kThreads) a.sel_idx[(size_t)p * m + i] = s_sel[i];  // for inspection only
  MARK(3);
  return bad;
}

// The select with as few key slots per thread as m allows (4 covers m <= 1024).
// Returns true when the wait for the scores gave up.
__device__ __forceinline__ bool gather_select(const FusedArgs& a, int p, int c, bool with_zpart, Smem& sm,
                                              float* s_hh, int* s_sel, float* s_zp) {
  if (a.m <= 4 * kThreads) return gather_select_mk<4>(a, p, c, with_zpart, sm, s_hh, s_sel, s_zp);
  return gather_select_mk<kMaxKeysPer>(a, p, c, with_zpart, sm, s_hh, s_sel, s_zp);
}

// Called by every reader of pair p's score slots at its end, when it has read
// them (all threads): each reader counts itself, and the one that completes the
// count of a.ncs readers empties the slots and sets the count back to 0, so that
// the next call starts from empty slots. The count's round trip is waited for
// here, at the end, off the path to the output.
__device__ __forceinline__ void empty_pair_slots(const FusedArgs& a, int p, Smem& sm) {
  if (threadIdx.x == 0) sm.tmp[0] = atomicAdd(&a.readers[p], 1);
  __syncthreads();
  if (sm.tmp[0] != a.ncs - 1) return;
  uint64_t* slots = a.xscore + (size_t)p * a.m;
  for (int j = threadIdx.x; j < a.m; j += kThreads) st_coh64(slots + j, kEmpty64);
  if (threadIdx.x == 0) st_coh(&a.readers[p], 0);
}

template <bool DENSE, int SLOTS>
__device__ __forceinline__ void gather_role(const FusedArgs& a, int bid, Smem& sm, unsigned char* dyn) {
  constexpr int kMaxChunk = DENSE ? kMaxChunkDense : kMaxChunkSparse;
  // sparse chunks are always kMaxChunkSparse channels (checked at launch), so
  // their loads carry no runtime guard and each use waits only for its own load
  const int C = DENSE ? a.chunk : kMaxChunkSparse;
  const int d = a.d, m = a.m;
  const int p = bid / a.nc, c = bid % a.nc;
  const int t = p / a.top_e, slot = p % a.top_e;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nslots = d / 8;  // 16-byte pieces of a hidden vector
  float* s_hh = (float*)dyn;                 // m: sketch activations (the z block's only)
  int* s_sel = (int*)(dyn + 4 * (size_t)m);  // m: the selection, ascending
  float* s_zp = (float*)(dyn + 8 * (size_t)m);  // zpart rows: the z block's only

  uint4 xv[SLOTS];  // eight bf16 of x per slot (zero past d)
  const uint16_t* xrow = a.x + (size_t)t * d;
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int s = tid + u * kThreads;
    xv[u] = s < nslots ? *(const uint4*)(xrow + 8 * s) : make_uint4(0, 0, 0, 0);
  }
  route(a, t, sm);
  MARK(1);
  const int count = DENSE ? m : a.k;
  const int first = c * C;
  int mine = count - first;
  mine = mine < 0 ? 0 : (mine > C ? C : mine);
  const bool bad = DENSE ? false : gather_select(a, p, c, false, sm, s_hh, s_sel, s_zp);
  const int e = sm.ids[slot];
  const float wp = sm.w[slot];
  if (!DENSE && c == 0 && tid == 0) {  // routing and selection of the pair, for inspection
    a.pair_expert[p] = e;
    a.pair_w[p] = wp;
    a.sel_count[p] = count;
  }
  // ---- every load of this block's channels at once (clamped; masked below)
  const uint16_t* wbase = a.wch + (size_t)e * m * 3 * d;
  uint4 gv[kMaxChunk][SLOTS], uv[kMaxChunk][SLOTS], dv[kMaxChunk][SLOTS];
  int jj[kMaxChunk];
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    const int ii = mine > 0 ? min(i, mine - 1) : 0;
    jj[i] = DENSE ? min(first + ii, m - 1) : (mine > 0 ? s_sel[first + ii] : 0);
  }
  // gate and up rows of every channel first, then the down rows: the SwiGLU dots
  // wait only for the former, and run while the down rows are in flight
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    if (i < C) {
      const uint16_t* row = wbase + (size_t)jj[i] * 3 * d;
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        const int s = min(tid + u * kThreads, nslots - 1);
        gv[i][u] = *(const uint4*)(row + 8 * s);
        uv[i][u] = *(const uint4*)(row + d + 8 * s);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    if (i < C) {
      const uint16_t* row = wbase + (size_t)jj[i] * 3 * d;
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        const int s = min(tid + u * kThreads, nslots - 1);
        dv[i][u] = *(const uint4*)(row + 2 * d + 8 * s);
      }
    }
  }
  // ---- SwiGLU of the C channels
  float gs[kMaxChunk], us[kMaxChunk];
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    gs[i] = 0.0f;
    us[i] = 0.0f;
    if (i < C) {
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        gs[i] = dot8_bf16_packed(gv[i][u], xv[u], gs[i]);
        us[i] = dot8_bf16_packed(uv[i][u], xv[u], us[i]);
      }
    }
  }
  MARK(6);
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    if (i < C) {
      const float gw = wave_sum(gs[i]);
      const float uw = wave_sum(us[i]);
      if (lane == 0) {
        sm.red[wave][2 * i] = gw;
        sm.red[wave][2 * i + 1] = uw;
      }
    }
  }
  __syncthreads();
  MARK(4);
  float yacc[SLOTS][8];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u)
#pragma unroll
    for (int q = 0; q < 8; ++q) yacc[u][q] = 0.0f;
  // lane i of every wave finishes channel i's activation (the wave partial sums
  // in wave order); the axpys take it from that lane
  float hl = 0.0f;
  if (lane < C && lane < mine) {
    float g = 0.0f, u = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      g += sm.red[w][2 * lane];
      u += sm.red[w][2 * lane + 1];
    }
    hl = wp * (silu_f32(g) * u);
  }
#pragma unroll
  for (int i = 0; i < kMaxChunk; ++i) {
    if (i < C && i < mine) {
      const float h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl), i));
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) axpy8_bf16(h, dv[i][s], yacc[s]);
    }
  }
  MARK(7);
  if (bad)  // the selection came from incomplete scores: publish NaN
#pragma unroll
    for (int u = 0; u < SLOTS; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) yacc[u][q] = kPoison;
  // ---- result: down partial (slice-major [t][slice][producer][64]); a
  // thread's eight values are 32 contiguous bytes, so a wave's two 16-byte
  // stores write whole lines
  const int slices = d / 64;
  const int qt = a.top_e * a.nc;
  const int q = slot * a.nc + c;
  const __amdgpu_buffer_rsrc_t prs = coh_rsrc(a.partial, (uint32_t)((size_t)a.batch * slices * qt * 256));
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int s = tid + u * kThreads;
    if (s < nslots) {
      const int sl = s >> 3, off = (s & 7) * 8;
      const uint32_t at = (uint32_t)(((((size_t)t * slices + sl) * qt + q) * 64 + off) * 4);
      st_coh128(prs, at, make_uint4(__float_as_uint(yacc[u][0]), __float_as_uint(yacc[u][1]),
                                    __float_as_uint(yacc[u][2]), __float_as_uint(yacc[u][3])));
      st_coh128(prs, at + 16, make_uint4(__float_as_uint(yacc[u][4]), __float_as_uint(yacc[u][5]),
                                         __float_as_uint(yacc[u][6]), __float_as_uint(yacc[u][7])));
    }
  }
  if (!DENSE) empty_pair_slots(a, p, sm);
  MARK(5);
}

// ---------------------------------------------------------------------------
// z role: one block per pair (sparse, r > 0), off the gather blocks' critical
// path: it selects like a gather block, then finishes the compensation
// coordinates z = sum_g zpart[g] - sum_{j selected} h_hat_j Q[j, :] and hands
// z to every combine block of the token.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void z_role(const FusedArgs& a, int p, Smem& sm, unsigned char* dyn) {
  const int d = a.d, m = a.m, r = a.r;
  const int t = p / a.top_e, slot = p % a.top_e;
  const int tid = threadIdx.x;
  const int zg = m / a.score_ch;                        // zpart rows: one per score block
  float* s_hh = (float*)dyn;                    // m
  int* s_sel = (int*)(dyn + 4 * (size_t)m);     // m
  float* s_zp = (float*)(dyn + 8 * (size_t)m);  // zg * r
  float* s_zr = s_zp + zg * r;                          // kThreads x 8, then r
  route(a, t, sm);
  MARK(1);
  const int e = sm.ids[slot];
  {
    // read the expert's whole Q (m x r bf16) once while the scores are still being
    // computed, so that the selected rows read after the select come from this
    // XCD's L2; the values only feed a store that k >= 0 (checked at launch) rules out
    const uint4* qall = (const uint4*)(a.qmat + (size_t)e * m * r);
    const int n16 = m * r / 8;
    uint32_t acc = 0;
    for (int b = 0; b < n16; b += kZWarm * kThreads) {
      uint4 qw[kZWarm];
#pragma unroll
      for (int u = 0; u < kZWarm; ++u) {
        const int i = b + u * kThreads + tid;
        qw[u] = i < n16 ? qall[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kZWarm; ++u) acc ^= qw[u].x ^ qw[u].y ^ qw[u].z ^ qw[u].w;
    }
    if (a.k < 0 && tid == 0) a.err[0] = (int)acc;
  }
  const bool bad = gather_select(a, p, a.nc, true, sm, s_hh, s_sel, s_zp);
  const int count = a.k;
  // thread t owns 8 consecutive columns (group t % (r/8)) of rows t / (r/8) + n * rows_per_pass
  float zacc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) zacc[q] = 0.0f;
  const int cgs = r >> 3, cg = tid % cgs, row = tid / cgs, rows_per_pass = kThreads / cgs;
  const uint16_t* Q = a.qmat + (size_t)e * m * r + 8 * cg;
  for (int i0 = 0; i0 < count || i0 < zg; i0 += rows_per_pass * kZPass) {
    uint4 qv[kZPass];
#pragma unroll
    for (int u = 0; u < kZPass; ++u) {
      const int i = i0 + u * rows_per_pass + row;
      qv[u] = i < count ? *(const uint4*)(Q + (size_t)s_sel[i] * r) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kZPass; ++u) {
      const int i = i0 + u * rows_per_pass + row;
      if (i < count) axpy8_bf16(-s_hh[s_sel[i]], qv[u], zacc);
      if (i < zg)
#pragma unroll
        for (int q = 0; q < 8; ++q) zacc[q] += s_zp[i * r + 8 * cg + q];
    }
  }
#pragma unroll
  for (int qq = 0; qq < 8; ++qq) s_zr[tid * 8 + qq] = zacc[qq];
  __syncthreads();
  // column sums over the threads sharing a column group, then one copy per
  // combine block of the token
  float* s_zc = s_zr + kThreads * 8;  // r
  if (tid < r) {
    float z = 0.0f;
#pragma unroll 8
    for (int th = tid >> 3; th < kThreads; th += cgs) z += s_zr[th * 8 + (tid & 7)];
    s_zc[tid] = bad ? kPoison : z;
  }
  __syncthreads();
  const int slices = d / 64;
  for (int i = tid; i < 2 * slices * r; i += kThreads) {
    const int col = i % r, half_slice = i / r;
    st_coh(&a.zcopy[(((size_t)t * 2 * slices + half_slice) * a.top_e + slot) * r + col], s_zc[col]);
  }
  empty_pair_slots(a, p, sm);
  MARK(5);
}

// ---------------------------------------------------------------------------
// combine role: one token x 32 output elements (half of a 64-wide slice)
// ---------------------------------------------------------------------------
template <bool DENSE>
__device__ __forceinline__ void combine_role(const FusedArgs& a, int bid, Smem& sm, unsigned char* dyn) {
  const int d = a.d;
  const int slices = d / 64;
  const int t = bid / (2 * slices), hs = bid % (2 * slices);  // hs: half-slice index
  const int sl = hs >> 1, hf = hs & 1;
  const int tid = threadIdx.x;
  const int q4 = tid & 7, pg = tid >> 3;  // elements 4 q4 .. 4 q4 + 3, producer group (32)
  const int qt = a.top_e * a.nc;
  const int r = DENSE ? 0 : a.r;
  const int rdiv = r > 0 ? r : 1;
  float* s_red = (float*)dyn;                 // kThreads x 8
  float* s_z = s_red + kThreads * 8;          // top_e x r
  float* s_y = s_z + 256;                     // 32 x 32

  // an earlier wait on this context gave up: its late stores may sit in slots
  // that this call reads, so the output is NaN until the host clears the error
  const bool poisoned = ld_coh(a.err) != 0;
  route(a, t, sm);
  MARK(1);
  // prefetch P[e][c][32 elements] for the token's experts: top_e * r rows of 64 bytes
  const int npieces = a.top_e * r * 4;
  uint4 pv[kMaxP];
#pragma unroll
  for (int u = 0; u < kMaxP; ++u) {
    const int i = min(tid + u * kThreads, max(npieces - 1, 0));
    const int part = i & 3, row = i >> 2;
    const int s = row / rdiv, cc = row % rdiv;
    pv[u] = npieces ? *(const uint4*)(a.pmat + ((size_t)sm.ids[s] * r + cc) * d + 64 * sl + 32 * hf + 8 * part)
                    : make_uint4(0, 0, 0, 0);
  }
  float* zsrc = a.zcopy + ((size_t)t * 2 * slices + hs) * a.top_e * rdiv;
  const bool zthread = r > 0 && tid < a.top_e * r;
  int spins = 0;
  // z first (it usually lands before the last partial), so that P z for these
  // elements is done while the partials are still arriving
  if (r > 0) {
    float z = 0.0f;
    bool zpend = zthread;
    while (true) {
      if (spent(spins, a.spin_limit)) {
        gave_up(a.err, 2);
        z = kPoison;
        break;
      }
      if (zpend) {
        z = ld_coh(zsrc + tid);
        if (!empty(z)) zpend = false;
      }
      if (__all(!zpend)) break;
    }
    if (zthread) {
      s_z[tid] = z;
      clear_coh(zsrc + tid);
    }
  }
  __syncthreads();
  MARK(2);
  // P z for these elements: every thread's pieces share part (tid & 3): elements 8*part..+7
  float pz[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) pz[q] = 0.0f;
#pragma unroll
  for (int u = 0; u < kMaxP; ++u) {
    const int i = tid + u * kThreads;
    if (i < npieces) {
      const int row = i >> 2;
      const int s = row / rdiv, cc = row % rdiv;
      axpy8_bf16(sm.w[s] * s_z[s * r + cc], pv[u], pz);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) s_red[tid * 8 + q] = pz[q];
  __syncthreads();
  // P z of elements 4 q4 .. + 3: element 8 part + qq has pieces from threads
  // th == part (mod 4); this thread takes th = part + 4 (2 pg) and part + 4 (2 pg + 1)
  float yz[4];
  {
    const int part = q4 >> 1, qq = (q4 & 1) * 4;
    const float4 a0 = *(const float4*)&s_red[(part + 8 * pg) * 8 + qq];
    const float4 a1 = *(const float4*)&s_red[(part + 8 * pg + 4) * 8 + qq];
    yz[0] = a0.x + a1.x;
    yz[1] = a0.y + a1.y;
    yz[2] = a0.z + a1.z;
    yz[3] = a0.w + a1.w;
  }
  // every wave polls its own slots with 16-byte loads: elements 4 q4 .. + 3 of
  // the partials of producers pg + 32 u, in batches of 32 * kCombPer; values are
  // summed in producer order
  MARK(4);
  const __amdgpu_buffer_rsrc_t prs = coh_rsrc(a.partial, (uint32_t)((size_t)a.batch * slices * qt * 256));
  const uint32_t row0 = (uint32_t)((((size_t)t * slices + sl) * qt) * 256 + (32 * hf + 4 * q4) * 4);
  float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = 0; base < qt; base += 32 * kCombPer) {
    uint4 v[kCombPer];
    uint32_t pending = 0;
#pragma unroll
    for (int u = 0; u < kCombPer; ++u) {
      v[u] = make_uint4(0, 0, 0, 0);
      if (base + pg + 32 * u < qt) pending |= 1u << u;
    }
    while (true) {
      if (spent(spins, a.spin_limit)) {
        gave_up(a.err, 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = kPoison;
        break;
      }
#pragma unroll
      for (int u = 0; u < kCombPer; ++u)
        if ((pending >> u) & 1) v[u] = ld_coh128(prs, row0 + (uint32_t)(base + pg + 32 * u) * 256);
#pragma unroll
      for (int u = 0; u < kCombPer; ++u)
        if (v[u].x != kEmpty && v[u].y != kEmpty && v[u].z != kEmpty && v[u].w != kEmpty) pending &= ~(1u << u);
      if (__all(pending == 0)) break;
    }
#pragma unroll
    for (int u = 0; u < kCombPer; ++u) {
      if (base + pg + 32 * u < qt) {
        y[0] += __uint_as_float(v[u].x);
        y[1] += __uint_as_float(v[u].y);
        y[2] += __uint_as_float(v[u].z);
        y[3] += __uint_as_float(v[u].w);
        st_coh128(prs, row0 + (uint32_t)(base + pg + 32 * u) * 256, make_uint4(kEmpty, kEmpty, kEmpty, kEmpty));
      }
    }
  }
  *(float4*)&s_y[pg * 32 + 4 * q4] = make_float4(y[0] + yz[0], y[1] + yz[1], y[2] + yz[2], y[3] + yz[3]);
  __syncthreads();
  MARK(3);
  if (tid < 32) {
    float o = 0.0f;
#pragma unroll 8
    for (int g = 0; g < 32; ++g) o += s_y[g * 32 + tid];
    a.out[(size_t)t * d + 64 * sl + 32 * hf + tid] = f32_to_bf16_dev(poisoned ? kPoison : o);
  }
  MARK(5);
}

template <bool DENSE, int SLOTS>
__global__ __launch_bounds__(kThreads) void k_fused(FusedArgs a) {
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ Smem sm;
  MARK(0);
  PLACE();
  // blocks in role order: every score block first (their code streams start
  // first), then the gather, z and combine blocks; producers sit below their
  // consumers
  int bid = blockIdx.x;
  if (!DENSE) {
    if (bid < a.n_score) {
      if (a.score_ch == kFusedScoreChMin) score_role<SLOTS, kFusedScoreChMin>(a, bid, sm, s_dyn);
      else score_role<SLOTS, 2 * kFusedScoreChMin>(a, bid, sm, s_dyn);
      return;
    }
    bid -= a.n_score;
  }
  if (bid < a.n_gather) {
    gather_role<DENSE, SLOTS>(a, bid, sm, s_dyn);
    return;
  }
  bid -= a.n_gather;
  if (!DENSE) {
    if (bid < a.n_z) {
      z_role(a, bid, sm, s_dyn);
      return;
    }
    bid -= a.n_z;
  }
  combine_role<DENSE>(a, bid, sm, s_dyn);
}

}  // namespace

#ifdef MOE_SEL_TIMELINE
// copies the phase marks (kMarkBlocks x kMarkEvents wall-clock values) to host
extern "C" int moe_sel_timeline_read(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_marks), sizeof(g_marks));
}
// copies the blocks' placements (kMarkBlocks values) to host
extern "C" int moe_sel_timeline_place(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_place), sizeof(g_place));
}
#endif

bool fused_supported(int d, int m, int r, int top_e) {
  return d <= 4096 && m <= kMaxKeysPer * kThreads && top_e * r <= 256 && top_e <= 64 &&
         (m / (2 * kFusedScoreChMin)) * r <= kMaxZPart * kThreads && (r == 0 || (kThreads % r == 0 && r % 8 == 0));
}

int fused_max_chunk(bool dense) { return dense ? kMaxChunkDense : kMaxChunkSparse; }

bool fused_narrow_score_ok(int m, int r) { return (m / kFusedScoreChMin) * r <= kMaxZPart * kThreads; }

size_t fused_lds_bytes(int d, int m, int r) {
  const size_t score = 2 * (size_t)d + 128 * (size_t)r + 512 + 1024;
  const size_t gather = 8 * (size_t)m + 4 * (size_t)(m / kFusedScoreChMin) * (size_t)std::max(r, 1) +
                        (size_t)kThreads * 8 * 4 + 4 * (size_t)std::max(r, 1);
  const size_t combine = (size_t)kThreads * 8 * 4 + 256 * 4 + 32 * 32 * 4;
  return std::max(score, std::max(gather, combine));
}

static const void* fused_kernel(bool dense, int d) {
  const int slots = (d / 8 + kThreads - 1) / kThreads;
  if (dense) return slots <= 1 ? (const void*)k_fused<true, 1> : (const void*)k_fused<true, 2>;
  return slots <= 1 ? (const void*)k_fused<false, 1> : (const void*)k_fused<false, 2>;
}

int fused_blocks_per_cu(bool dense, int d, int m, int r) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_kernel(dense, d), kThreads, fused_lds_bytes(d, m, r)) !=
      hipSuccess)
    return 0;
  return n;
}

int fused_grid(const FusedArgs& a, bool dense) {
  return (dense ? 0 : a.n_score + a.n_z) + a.n_gather + a.n_combine;
}

hipError_t launch_fused(const FusedArgs& a, bool dense, hipStream_t stream) {
  if (dense ? (a.chunk != 8 && a.chunk != kMaxChunkDense) : a.chunk != kMaxChunkSparse) return hipErrorInvalidValue;
  void* args[] = {(void*)&a};
  return hipLaunchKernel(fused_kernel(dense, a.d), dim3(fused_grid(a, dense)), dim3(kThreads), args,
                         fused_lds_bytes(a.d, a.m, a.r), stream);
}

}  // namespace moe_sel
