// Device helpers shared by the multi-kernel and the fused forward paths.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe_sel {
namespace dev {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// ---------------------------------------------------------------------------
// binary32 silu with every operation separately rounded (no contraction):
// Cody & Waite reduction with ln 2 split as 2839/4096 plus the binary32 nearest
// to the remainder, degree-7 Taylor series of e^r, then z / (1 + e^-z); the
// argument is cut at |z| > 87 (z itself above, +0 below).
// ---------------------------------------------------------------------------
constexpr float kL2E = 1.44269504088896340736f;
constexpr float kLn2Hi = 2839.0f / 4096.0f;
constexpr float kLn2Lo = (float)(0.693147180559945309417232121458 - 2839.0 / 4096.0);
constexpr float kF2 = (float)(1.0 / 2.0);
constexpr float kF3 = (float)(1.0 / 6.0);
constexpr float kF4 = (float)(1.0 / 24.0);
constexpr float kF5 = (float)(1.0 / 120.0);
constexpr float kF6 = (float)(1.0 / 720.0);
constexpr float kF7 = (float)(1.0 / 5040.0);

__device__ __forceinline__ float silu_pinned(float z) {
#pragma clang fp contract(off)
  if (z > 87.0f) return z;
  if (z < -87.0f) return 0.0f;
  const float t = -z;
  const float n = __builtin_rintf(t * kL2E);
  const float r = (t - n * kLn2Hi) - n * kLn2Lo;
  float p = kF7;
  p = p * r + kF6;
  p = p * r + kF5;
  p = p * r + kF4;
  p = p * r + kF3;
  p = p * r + kF2;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const float et = __builtin_ldexpf(p, (int)n);
  return z / (1.0f + et);
}

// Channel score from the exact integer sketch dots: G = alpha_g * Dg * 2^xexp,
// U = alpha_u * Du * 2^xexp, h = silu_pinned(G) * U, score = |h| * ||down||.
// kind (ablations of the score; h is the same for all): 0 = |h| * ||down||,
// 1 = |silu_pinned(G)| * ||down|| (gate sketch only), 2 = |h| (no down norm).
__device__ __forceinline__ void pinned_score(int dg, int du, int xexp, float4 st, float& h, float& score,
                                             int kind = 0) {
#pragma clang fp contract(off)
  const float g = __builtin_ldexpf(st.x * (float)dg, xexp);
  const float u = __builtin_ldexpf(st.y * (float)du, xexp);
  const float sg = silu_pinned(g);
  h = sg * u;
  // kind 3 (int16 activations) ranks by the full score
  score = kind == 1 ? __builtin_fabsf(sg) * st.z : (kind == 2 ? __builtin_fabsf(h) : __builtin_fabsf(h) * st.z);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ void unpack8(uint4 w, float* x) {
  x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
  x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
  x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
  x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
}

__device__ __forceinline__ float dot8_bf16(uint4 w, const float* x) {
  float s = bf16lo(w.x) * x[0];
  s += bf16hi(w.x) * x[1];
  s += bf16lo(w.y) * x[2];
  s += bf16hi(w.y) * x[3];
  s += bf16lo(w.z) * x[4];
  s += bf16hi(w.z) * x[5];
  s += bf16lo(w.w) * x[6];
  s += bf16hi(w.w) * x[7];
  return s;
}

// The same dot with x also as eight bf16 (packed pairs): four v_dot2_f32_bf16,
// each adding two exact bf16 products to the binary32 accumulator.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_bf16_packed(uint4 w, uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc, false);
  return acc;
}

__device__ __forceinline__ void axpy8_bf16(float a, uint4 w, float* y) {
  y[0] += a * bf16lo(w.x); y[1] += a * bf16hi(w.x);
  y[2] += a * bf16lo(w.y); y[3] += a * bf16hi(w.y);
  y[4] += a * bf16lo(w.z); y[5] += a * bf16hi(w.z);
  y[6] += a * bf16lo(w.w); y[7] += a * bf16hi(w.w);
}

__device__ __forceinline__ uint16_t f32_to_bf16_dev(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // a NaN stays a (quiet) NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Wavefront reductions and scans on DPP row operations (VALU data movement:
// quad permutes, row mirrors and the gfx9 row broadcasts), not LDS shuffles.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF, bool BOUND = false>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, BOUND);
}
template <int CTRL, int ROW_MASK = 0xF, bool BOUND = false>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, BOUND));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

// sum over the 64 lanes, returned to every lane
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kQuadXor1>(v);
  v += dpp_f<kQuadXor2>(v);
  v += dpp_f<kRowHalfMirror>(v);
  v += dpp_f<kRowMirror>(v);
  v += dpp_f<kRowBcast15, 0xA>(v);
  v += dpp_f<kRowBcast31, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kQuadXor1>(v);
  v += dpp_i<kQuadXor2>(v);
  v += dpp_i<kRowHalfMirror>(v);
  v += dpp_i<kRowMirror>(v);
  v += dpp_i<kRowBcast15, 0xA>(v);
  v += dpp_i<kRowBcast31, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kQuadXor1>((int)v));
  v = max(v, (uint32_t)dpp_i<kQuadXor2>((int)v));
  v = max(v, (uint32_t)dpp_i<kRowHalfMirror>((int)v));
  v = max(v, (uint32_t)dpp_i<kRowMirror>((int)v));
  v = max(v, (uint32_t)dpp_i<kRowBcast15, 0xA>((int)v));
  v = max(v, (uint32_t)dpp_i<kRowBcast31, 0xC>((int)v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// inclusive prefix sum over the lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<kRowShr1, 0xF, true>(v);
  v += dpp_i<kRowShr2, 0xF, true>(v);
  v += dpp_i<kRowShr4, 0xF, true>(v);
  v += dpp_i<kRowShr8, 0xF, true>(v);
  v += dpp_i<kRowBcast15, 0xA>(v);
  v += dpp_i<kRowBcast31, 0xC>(v);
  return v;
}

// exclusive prefix sum over the block in thread order; *total = block sum.
// s_tmp[kWaves]; two barriers (all threads call).
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_tmp[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// 2-bit offset-binary codes (t + 1) of 16 hidden elements against 16 int8
// activations: the four byte-aligned 2-bit fields of each shift line up with
// four consecutive activations.
// Sum of code * x_q over the 16 elements of one code dword, accumulated in three
// parts so that the codes need masks but only one shift: the codes of elements
// 4..7 enter multiplied by 4 and those of elements 8..15 by 16 (every byte stays
// within int8: code << 4 <= 32). The exact sum is code_acc_total().
struct CodeAcc {
  int s1 = 0, s4 = 0, s16 = 0;
};

__device__ __forceinline__ void dot_codes16(uint32_t cw, int4 x, CodeAcc& a) {
  a.s1 = __builtin_amdgcn_sdot4((int)(cw & 0x03030303u), x.x, a.s1, false);
  a.s4 = __builtin_amdgcn_sdot4((int)(cw & 0x0C0C0C0Cu), x.y, a.s4, false);
  a.s16 = __builtin_amdgcn_sdot4((int)(cw & 0x30303030u), x.z, a.s16, false);
  a.s16 = __builtin_amdgcn_sdot4((int)((cw >> 2) & 0x30303030u), x.w, a.s16, false);
}

// s4 and s16 are exact multiples of 4 and 16, so the shifts divide exactly
__device__ __forceinline__ int code_acc_total(const CodeAcc& a) { return a.s1 + (a.s4 >> 2) + (a.s16 >> 4); }

// The same with four unsigned activation bytes per dword (the low bytes of
// int16 activations): codes and bytes both unsigned, sums below 2^31.
__device__ __forceinline__ void dot_codes16_u(uint32_t cw, int4 x, CodeAcc& a) {
  a.s1 = (int)__builtin_amdgcn_udot4(cw & 0x03030303u, (uint32_t)x.x, (uint32_t)a.s1, false);
  a.s4 = (int)__builtin_amdgcn_udot4(cw & 0x0C0C0C0Cu, (uint32_t)x.y, (uint32_t)a.s4, false);
  a.s16 = (int)__builtin_amdgcn_udot4(cw & 0x30303030u, (uint32_t)x.z, (uint32_t)a.s16, false);
  a.s16 = (int)__builtin_amdgcn_udot4((cw >> 2) & 0x30303030u, (uint32_t)x.w, (uint32_t)a.s16, false);
}

// Score activations: int8 (the method) or int16 (an ablation of the score),
// q = rint(x * 2^-e) with the smallest e that keeps max|q| <= 2^(bits-1) - 1.
// amax_bits: the largest |x| as bf16 bits (non-zero).
__device__ __forceinline__ int score_exponent(uint32_t amax_bits, bool x16) {
  const float av = __uint_as_float(amax_bits << 16);
  int ex;
  (void)__builtin_frexpf(av, &ex);  // av = f * 2^ex, f in [0.5, 1)
  int e = x16 ? ex - 15 : ex - 7;
  if (__builtin_ldexpf(av, -e) > (x16 ? 32767.0f : 127.0f)) e += 1;
  return e;
}

// exclusive count of `flag` over the block in thread order; *total = block count.
// Uses s_tmp[kWaves]; contains barriers (all threads must call).
__device__ __forceinline__ int block_excl_count(bool flag, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t mask = __ballot(flag);
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  if (lane == 0) s_tmp[wave] = __popcll(mask);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_tmp[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + below;
}

// Writes the selected channel indices (all keys > T, then the krem lowest-index
// keys == T), ascending, to out[0..k). Returns k. All threads call.
__device__ __forceinline__ int block_compact(const uint32_t* s_keys, int m, uint32_t T, int krem, int* out,
                                             int* s_tmp) {
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < m; base += kThreads) {
    const int j = base + threadIdx.x;
    const uint32_t key = j < m ? s_keys[j] : 0u;
    const bool gt = j < m && key > T;
    const bool eq = j < m && key == T;
    int eq_tot, sel_tot;
    const int eq_before = block_excl_count(eq, s_tmp, &eq_tot);
    const bool take = gt || (eq && run_eq + eq_before < krem);
    const int sel_before = block_excl_count(take, s_tmp, &sel_tot);
    if (take) out[run_sel + sel_before] = j;
    run_eq += eq_tot;
    run_sel += sel_tot;
  }
  return run_sel;
}

// ---------------------------------------------------------------------------
// Order keys: a 64-bit integer per (value, index) whose unsigned order is
// "larger value first, lower index first", so a rank is a count of larger keys
// (one compare each, no branches).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int)u >> 31) | 0x80000000u);
}
// Order bits of a logit: -0 and +0 are equal values, so both map to +0's bits
// (ties between them then go to the lower index).
__device__ __forceinline__ uint32_t logit_order_bits(float f) { return float_order_bits(f == 0.0f ? 0.0f : f); }
__device__ __forceinline__ uint64_t order_key(uint32_t ordered_value, int index) {
  return ((uint64_t)ordered_value << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)index);
}

// Gate weights of the routed experts, in place: s_w[0..top_e) holds their
// logits in rank order (largest first) and receives the softmax over them. The
// exponentials are taken in parallel by wave 0 and the denominator is summed in
// rank order. The caller synchronises before and after.
__device__ __forceinline__ void route_softmax(float* s_w, int top_e) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const float v = lane < top_e ? s_w[lane] : 0.0f;
    const float top = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
    const float ex = __expf(v - top);
    float den = 0.0f;
    for (int s = 0; s < top_e; ++s) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), s));
    if (lane < top_e) s_w[lane] = ex / den;
  }
}

// Maximum of v over the 64 lanes, returned to every lane: DPP moves within rows
// of 16 lanes (quad swaps, then rotations by 4 and 8), then the row broadcasts
// of lanes 15 and 31, which leave the total in lane 63. No LDS traffic.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast 15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast 31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Routing by one wave for small top_e: lane l holds the logits of experts
// l + 64 u and keeps the largest order bits it has left (0 once it has none:
// no live key is below 0). Each of top_e rounds takes the wave-wide maximum of
// the lanes' bests; when one lane holds it, that lane takes its lowest u
// holding it (the lower index). When several do, the lowest index is the lowest
// u holding it, then the lowest lane (a ballot per u). The winning lane writes
// s_ids[rank] and the logit in s_w[rank], and recomputes its best.
template <int KPER>
__device__ __forceinline__ void wave_topk_route(const float* logits, int n_experts, int top_e, int* s_ids,
                                                float* s_w) {
  const int lane = threadIdx.x & 63;
  uint32_t ob[KPER];
  float val[KPER];
  uint32_t alive = 0;  // bit u: expert lane + 64 u not yet taken
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int idx = lane + 64 * u;
    if (idx < n_experts) alive |= 1u << u;
    val[u] = idx < n_experts ? logits[idx] : 0.0f;
    ob[u] = logit_order_bits(val[u]);
  }
  uint32_t best = 0;
#pragma unroll
  for (int u = 0; u < KPER; ++u)
    if ((alive >> u) & 1) best = max(best, ob[u]);
  for (int s = 0; s < top_e; ++s) {
    const uint32_t m = wave_max_dpp(best);
    uint64_t wmask = __ballot(alive != 0 && best == m);
    int forced_u = -1;
    if (__popcll(wmask) > 1) {
#pragma unroll
      for (int u = 0; u < KPER; ++u) {
        const uint64_t bm = __ballot(((alive >> u) & 1) && ob[u] == m);
        if (forced_u < 0 && bm) {
          forced_u = u;
          wmask = bm;
        }
      }
    }
    if (lane == __builtin_ctzll(wmask)) {
      int wu = forced_u;
#pragma unroll
      for (int u = KPER - 1; u >= 0; --u)
        if (forced_u < 0 && ((alive >> u) & 1) && ob[u] == m) wu = u;
      alive &= ~(1u << wu);
      s_ids[s] = lane + 64 * wu;
      float w = val[0];
#pragma unroll
      for (int u = 1; u < KPER; ++u)
        if (u == wu) w = val[u];
      s_w[s] = w;
      best = 0;
#pragma unroll
      for (int u = 0; u < KPER; ++u)
        if ((alive >> u) & 1) best = max(best, ob[u]);
    }
  }
}

// Compiler-level ordering of LDS accesses inside one wavefront (a wave's LDS
// operations execute in order, so wave-synchronous code needs no s_barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Routing by rank for n_experts <= 64 * KPER (at most 256): lane l of every wave
// holds the order keys (order bits, then lower index first) of experts l + 64 u,
// and wave w counts, for each of them, the larger keys among the experts
// [w * len, (w + 1) * len), reading that range two keys at a time from a copy the
// wave wrote itself (no barrier). After one block barrier the four counts of
// expert i sum to its rank, and the ranks below top_e are the routed experts.
// Keys past n_experts are 0, below every live key. s_scr: 16 * 64 * KPER bytes.
template <int KPER>
__device__ __forceinline__ void rank_route(const float* logits, int n_experts, int top_e, int* s_ids, float* s_w,
                                           void* s_scr) {
  constexpr int kSpan = 64 * KPER;       // experts covered, padded
  constexpr int kLen = kSpan / kWaves;   // experts each wave compares against (16, 32 or 64)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t* s_key = (uint64_t*)s_scr;                  // wave w's range at w * kLen
  uint32_t* s_cnt = (uint32_t*)(s_key + kSpan);        // per expert: byte w = wave w's count
  float* s_val = (float*)(s_cnt + kSpan);
  uint64_t key[KPER];
  float val[KPER];
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int i = lane + 64 * u;
    val[u] = i < n_experts ? logits[i] : 0.0f;
    key[u] = i < n_experts ? order_key(logit_order_bits(val[u]), i) : 0ull;
  }
  // the wave's comparison range is register u = r0 / 64 of lanes r0 % 64 .. + kLen
  const int r0 = wave * kLen, l0 = r0 % 64;
  if (lane >= l0 && lane < l0 + kLen) {
    uint64_t kk = key[0];
#pragma unroll
    for (int u = 1; u < KPER; ++u)
      if (u == r0 / 64) kk = key[u];
    s_key[r0 + lane - l0] = kk;
  }
  if (wave == 0) {
#pragma unroll
    for (int u = 0; u < KPER; ++u) s_val[lane + 64 * u] = val[u];
  }
  wave_lds_sync();
  int rk[KPER];
#pragma unroll
  for (int u = 0; u < KPER; ++u) rk[u] = 0;
  const ulonglong2* kp = (const ulonglong2*)(s_key + r0);
#pragma unroll 4
  for (int j = 0; j < kLen / 2; ++j) {
    const ulonglong2 kk = kp[j];
#pragma unroll
    for (int u = 0; u < KPER; ++u) rk[u] += (int)(kk.x > key[u]) + (int)(kk.y > key[u]);
  }
  unsigned char* cnt = (unsigned char*)s_cnt;
#pragma unroll
  for (int u = 0; u < KPER; ++u) cnt[4 * (lane + 64 * u) + wave] = (unsigned char)rk[u];
  __syncthreads();
  for (int i = threadIdx.x; i < n_experts; i += kThreads) {
    const int r = (int)__builtin_amdgcn_udot4(s_cnt[i], 0x01010101u, 0u, false);
    if (r < top_e) {
      s_ids[r] = i;
      s_w[r] = s_val[i];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Routing of one token by the whole block (n_experts <= 1024): for n_experts <=
// 256 by rank_route; otherwise the rank of every logit (larger first, lower
// index first) is the count of larger order keys, computed by all threads in
// parallel over parts of the expert range, and ranks below top_e are the routed
// experts. The gate weights are the softmax
// over their logits (skipped when with_weights is false). s_scr: 2 * n_experts
// uint64 + n_experts ints of LDS scratch. Barriers inside; s_ids (and s_w)
// valid when it returns.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void block_route(const float* logits, int n_experts, int top_e, int* s_ids, float* s_w,
                                            void* s_scr, bool with_weights = true) {
  const int tid = threadIdx.x;
  if (n_experts <= 256) {
    if (n_experts <= 64) rank_route<1>(logits, n_experts, top_e, s_ids, s_w, s_scr);
    else if (n_experts <= 128) rank_route<2>(logits, n_experts, top_e, s_ids, s_w, s_scr);
    else rank_route<4>(logits, n_experts, top_e, s_ids, s_w, s_scr);
    if (with_weights) {
      route_softmax(s_w, top_e);
      __syncthreads();
    }
    return;
  }
  uint64_t* s_key = (uint64_t*)s_scr;
  int* s_rank = (int*)(s_key + n_experts);
  float* s_val = (float*)(s_rank + n_experts);
  for (int i = tid; i < n_experts; i += kThreads) {
    const float v = logits[i];
    s_key[i] = order_key(logit_order_bits(v), i);
    s_val[i] = v;
    s_rank[i] = 0;
  }
  __syncthreads();
  // thread -> (expert i, part of the comparison range)
  const int span = n_experts < kThreads ? n_experts : kThreads;
  const int parts = kThreads / span;
  const int len = (n_experts + parts - 1) / parts;
  for (int i0 = 0; i0 < n_experts; i0 += span) {
    const int i = i0 + tid % span, part = tid / span;
    if (i < n_experts && part < parts) {
      const uint64_t ki = s_key[i];
      const int j0 = part * len, j1 = min(n_experts, j0 + len);
      int rank = 0;
#pragma unroll 8
      for (int j = j0; j < j1; ++j) rank += s_key[j] > ki;
      if (parts > 1) atomicAdd(&s_rank[i], rank);
      else s_rank[i] = rank;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_experts; i += kThreads) {
    const int rk = s_rank[i];
    if (rk < top_e) {
      s_ids[rk] = i;
      s_w[rk] = s_val[i];
    }
  }
  __syncthreads();
  if (with_weights) {
    route_softmax(s_w, top_e);
    __syncthreads();
  }
}

__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int incl = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(incl, 63);
  return incl - v;
}

// ---------------------------------------------------------------------------
// Top-k of m <= kThreads * KPT non-negative binary32 scores (bit patterns keep
// their order), k in [1, m): three most-significant-digit radix passes over bits
// 30..20, 19..9 and 8..0, each a 2048-bin LDS histogram and a block suffix scan,
// give the k-th largest key T and krem = how many keys equal to T are taken
// (the lowest-index ones). Thread t owns the consecutive keys [t*KPT, t*KPT+KPT).
// s_hist: 2048 ints; s_tmp: kWaves + 2 ints. Barriers inside (all threads call).
// ---------------------------------------------------------------------------
template <int KPT>
__device__ __forceinline__ void block_topk_radix(const uint32_t (&key)[KPT], int per, int m, int k, int* s_hist,
                                                 int* s_tmp, uint32_t& T, int& krem_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  constexpr int kShift[3] = {20, 9, 0};
  constexpr uint32_t kDigitMask[3] = {0x7FFu, 0x7FFu, 0x1FFu};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass];
    const uint32_t dmask = kDigitMask[pass];
#pragma unroll
    for (int b = 0; b < 8; ++b) s_hist[tid * 8 + b] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int j = tid * per + u;
      if (u < per && j < m && (key[u] & pmask) == prefix) atomicAdd(&s_hist[(key[u] >> shift) & dmask], 1);
    }
    __syncthreads();
    int h[8], c = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      h[b] = s_hist[tid * 8 + b];
      c += h[b];
    }
    int total;
    const int before = block_excl_scan(c, s_tmp, &total);
    int above = total - before - c;  // keys whose digit is above this thread's 8 bins
#pragma unroll
    for (int b = 7; b >= 0; --b) {
      if (above < krem && krem <= above + h[b]) {
        s_tmp[kWaves] = tid * 8 + b;
        s_tmp[kWaves + 1] = above;
      }
      above += h[b];
    }
    __syncthreads();
    prefix |= (uint32_t)s_tmp[kWaves] << shift;
    pmask |= dmask << shift;
    krem -= s_tmp[kWaves + 1];
    __syncthreads();
  }
  T = prefix;
  krem_out = krem;
}

// Top-k selection flags for the keys a thread owns (consecutive [t*KPT, t*KPT+KPT)):
// one radix pass on bits 30..20 finds the 2048-bin bucket holding the k-th
// largest key; keys above it are taken, and the bucket's keys are ranked exactly
// by pairwise comparison in the order (larger key first, lower index first). A
// bucket of more than kThreads keys falls back to the three-pass threshold.
// Returns per-key ascending output ranks in sel[] (-1 if not selected) and the
// count. 1 <= k < m. s_hist: 2048 ints; s_cand: 2 * kThreads ints, 8-byte aligned; s_take: m
// bytes; s_tmp: kWaves + 2 ints. Barriers inside (all threads call).
// Callers that pass PREZEROED have cleared s_hist and s_tmp[kWaves + 1] and
// passed a block barrier since.
__device__ __forceinline__ void block_topk_prezero(int* s_hist, int* s_tmp) {
#pragma unroll
  for (int b = 0; b < 8; ++b) s_hist[threadIdx.x * 8 + b] = 0;
  if (threadIdx.x == 0) s_tmp[kWaves + 1] = 0;
}

template <int KPT, bool PREZEROED = false>
__device__ __forceinline__ int block_topk_select_strided(const uint32_t (&key)[KPT], int per, int m, int k, int* s_hist, int* s_cand,
                                                 unsigned char* s_take, int* s_tmp, int (&sel)[KPT]) {
  const int tid = threadIdx.x;
  if (!PREZEROED) {
    block_topk_prezero(s_hist, s_tmp);
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if ((u < per && tid * per + u < m)) atomicAdd(&s_hist[key[u] >> 20], 1);
  __syncthreads();
  int h[8], c = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    h[b] = s_hist[tid * 8 + b];
    c += h[b];
  }
  int total;
  const int before = block_excl_scan(c, s_tmp, &total);
  int above = total - before - c;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    if (above < k && k <= above + h[b]) {
      s_hist[0] = tid * 8 + b;  // bucket (bin 0's count is no longer needed)
      s_hist[1] = above;
      s_hist[2] = h[b];
    }
    above += h[b];
  }
  __syncthreads();
  const uint32_t D = (uint32_t)s_hist[0];
  const int krem = k - s_hist[1];
  const int ncand = s_hist[2];
  bool take[KPT];
  // the radix fallback clears s_hist; every thread has read the three words
  // above before it passes this barrier (the candidate branch writes no s_hist)
  if (ncand > kThreads) __syncthreads();
  if (ncand <= kThreads) {
    uint64_t* ck = (uint64_t*)s_cand;  // order keys of the bucket's keys
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int j = tid * per + u;
      if (u < per && j < m && (key[u] >> 20) == D) {
        const int slot = atomicAdd(&s_tmp[kWaves + 1], 1);
        ck[slot] = order_key(key[u], j);
      }
    }
    __syncthreads();
    // nt consecutive threads per candidate, each counting larger keys among every
    // nt-th candidate; the index comes back out of the order key
    const int nt = ncand <= kThreads / 4 ? 4 : (ncand <= kThreads / 2 ? 2 : 1);
    const int ci = tid / nt, part = tid % nt;
    if (ci < ncand) {
      const uint64_t kc = ck[ci];
      int rank = 0;
#pragma unroll 8
      for (int o = part; o < ncand; o += nt) rank += ck[o] > kc;
      if (nt >= 2) rank += __shfl_xor(rank, 1, 64);
      if (nt >= 4) rank += __shfl_xor(rank, 2, 64);
      if (part == 0) s_take[0xFFFFFFFFu - (uint32_t)kc] = rank < krem;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int j = tid * per + u;
      const uint32_t dg = key[u] >> 20;
      take[u] = u < per && j < m && (dg > D || (dg == D && s_take[j]));
    }
  } else {
    uint32_t T;
    int kr;
    block_topk_radix<KPT>(key, per, m, k, s_hist, s_tmp, T, kr);
    int n_eq = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) n_eq += ((u < per && tid * per + u < m) && key[u] == T);
    int eq_total;
    int eq_before = block_excl_scan(n_eq, s_tmp, &eq_total);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool valid = (u < per && tid * per + u < m);
      const bool eq = valid && key[u] == T;
      take[u] = valid && (key[u] > T || (eq && eq_before < kr));
      eq_before += eq;
    }
  }
  int n_sel = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) n_sel += take[u];
  int sel_total;
  int r = block_excl_scan(n_sel, s_tmp, &sel_total);
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    sel[u] = take[u] ? r : -1;
    r += take[u];
  }
  return sel_total;
}

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off without cache maintenance. Data that crosses
// workgroups is written and read with device-coherent accesses (agent-scope
// relaxed atomics: stores write through to the device coherence point, loads
// read from it, on every XCD), so no L2 write-back or invalidate is needed.
// The single-launch kernel polls the data itself: a slot holds an empty
// sentinel until its producer's coherent store lands, its one consumer polls
// it with coherent loads and writes the sentinel back, so every call and
// every HIP-graph replay starts from empty slots. Waits are bounded (a poll
// count the host sets); a wait that gives up sets an error bit and turns the
// results it feeds into NaN, and the block proceeds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte device-coherent loads and stores through a buffer resource, with the
// same device-scope cache policy (sc1) as the agent-scope relaxed atomics above.
// The 16 bytes are not one atomic access, but each of their dwords is, so a
// poller checks every dword for the empty sentinel. Offsets are in bytes and
// checked by the hardware against the resource's size.
constexpr int kDeviceScope = 16;  // cache-policy bit of the buffer instructions: device scope (sc1)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld_coh128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kDeviceScope));
}
__device__ __forceinline__ void st_coh128(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kDeviceScope);
}

}  // namespace dev
}  // namespace moe_sel
