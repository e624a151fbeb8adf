// Launch interface between the host runtime and the device kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe_sel {

// Everything one forward call needs; all pointers are device pointers.
struct FwdArgs {
  // prepared layer (read-only)
  const uint32_t* codes;   // packed 2-bit sketch codes
  const float4* stats;     // [E][m] {alpha_gate, alpha_up, down_norm, 0}
  const uint16_t* wch;     // [E][m][3][d] bf16
  const uint16_t* pmat;    // [E][r][d] bf16
  const uint16_t* qmat;    // [E][m][r] bf16
  int d, m, r, n_experts;
  // call
  const uint16_t* x;       // [B][d] bf16
  const float* logits;     // [B][E]
  uint16_t* out;           // [B][d] bf16
  int batch, top_e, k;
  int score_kind;          // 0 full score, 1 gate sketch only, 2 without the down-column norm, 3 full on int16 x
  int thr_mode;            // 1: keep channels with score > thr_bits instead of the top k
  uint32_t thr_bits;       // binary32 bits of the (non-negative) threshold
  // workspace
  int8_t* xq;              // [B][d]
  int* xexp;               // [B]
  int* pair_expert;        // [B*top_e]
  float* pair_w;           // [B*top_e]
  float* hhat;             // [P][m]
  float* score;            // [P][m]
  int* sel_idx;            // [P][m]
  int* sel_count;          // [P]
  float* zvec;             // [P][r]  sum over all channels of h_hat_j Q[j, :]
  float* ypart;            // [kc][P][d] partial outputs of each K split of the down projection
  // expert-grouped multi-kernel path
  int* xqsum;              // [B] sum of the int8 activations
  int* tile_expert;        // [max_tiles]
  int* tile_first;         // [max_tiles] offset into tpair
  int* tile_n;             // [max_tiles] tokens in the tile (1..kTileTokens)
  int* n_tiles;            // [1]
  int* tpair;              // [P] pair indices sorted by (expert, token)
  uint32_t* selbits;       // [P][m/32] selected channels of each pair
  float* gzpart;           // [P][m/64][r] per-group share of Q^T h_hat
  int* ulist;              // [max_tiles][m] union channels of a tile, ascending
  uint64_t* umask;         // [max_tiles][m] which tile tokens selected each union channel
  int* ucount;             // [max_tiles]
  int* slot_ucount;        // [P] union size of the tile of each tile slot (expert tiles)
  int* tile_choff;         // [max_tiles] first gate/up work item of each tile
  int* n_items;            // [1] gate/up work items of the call
  int* gu_items;           // [max_tiles * m/16][kGuItemInts] gate/up work items, tile by tile: tile, chunk,
                           // expert, first slot, tokens, union size, 2 unused, the chunk's 16 union channels
  uint16_t* hbuf;          // [P][kpad] bf16 activations by union position, then z (rows: pairs for one-pair
                           // tiles, tile slots (tile_first + token) for expert tiles)
  float* zsel;             // [P][m/16][r] Q^T h_hat over one gate/up block's selected channels
  int max_tiles, kpad;
};

// expert tiles hold up to this many tokens
constexpr int kTileTokens = 32;
constexpr int kGuItemInts = 24;  // ints per gate/up work item
inline int grouped_max_tiles(int pairs, int n_experts) {
  const int bound = pairs / kTileTokens + (pairs < n_experts ? pairs : n_experts);
  return pairs < bound ? pairs : bound;
}
inline int grouped_kpad(int m, int r) { return (m + r + 31) / 32 * 32; }
bool grouped_supported(int d, int m);
// down projection: outputs per block, and the split of its K range over blocks
constexpr int kDownTargetBlocks = 1024;
constexpr int kDownMaxStages = 6;
constexpr int kMaxDownSplit = 64;
int grouped_down_width(int d);
// kmax: the largest union of channels a tile of the call can hold
int grouped_down_split(int max_tiles, int d, int kmax, int r);
// One routed pair per tile (row kernels, no plan or union launch): batch 1,
// and sparse calls whose routed pairs are at most half the experts, so that
// experts seldom repeat and reading an expert's rows once per pair costs little
// over once per expert tile (at two pairs per expert the tile kernels win).
// Such calls need no more tile slots than expert tiles would.
inline bool grouped_pair_tiles(int batch, int top_e, int n_experts, bool dense) {
  return batch == 1 || (!dense && 2 * batch * top_e <= n_experts);
}
// batch 1 (one token per tile): row-streaming gate/up and down kernels, and
// the down projection's split of the K range
bool grouped_b1_supported(int d);
int grouped_down_split_b1(int kmax, int r);

hipError_t launch_forward(const FwdArgs& a, bool dense, hipStream_t stream);

// Single-launch forward (fused.hip): block roles score / gather / combine.
struct FusedArgs : FwdArgs {
  // hand-off slots, empty = 0xFFFFFFFF
  uint64_t* xscore;  // [P][m]            (score, h_hat) of each pair, read by the pair's gather blocks and z block
  int* readers;      // [P]               consumers that have read each pair's xscore slots; the last one empties
                     //                   them and sets the count back to 0
  float* zpart;      // [P][m/score_ch][r] each score block's share of Q^T h_hat, for the z block
  float* partial;    // [B][d/64][top_e*nc][64] gate-weighted down partials, for combine
  float* zcopy;      // [B][d/32][top_e][r] z of each routed pair, for each combine block
  int* err;          // error bits (1: gather wait timed out, 2: combine wait timed out); sticky until
                     // the host clears them, and while set every combine block writes NaN
  int spin_limit;    // polls before a cross-block wait gives up (0: every wait gives up at once)
  int n_score, n_gather, n_z, n_combine;
  int nc;            // gather blocks per pair
  int ncs;           // readers of a pair's xscore slots: the gather blocks and the z block (if any)
  int chunk;         // channels per gather block
  int score_ch;      // channels per score block: 32, or 64 when the grid of 32 would not fit
};

constexpr int kFusedScoreChMin = 32;  // fewest channels per score block of the single-launch kernel
bool fused_supported(int d, int m, int r, int top_e);
int fused_max_chunk(bool dense);
bool fused_narrow_score_ok(int m, int r);  // kFusedScoreChMin-channel score blocks fit the z block's slots
size_t fused_lds_bytes(int d, int m, int r);
int fused_blocks_per_cu(bool dense, int d, int m, int r);
int fused_grid(const FusedArgs& a, bool dense);  // blocks of a planned call
hipError_t launch_fused(const FusedArgs& a, bool dense, hipStream_t stream);

// polls before a cross-block wait of the single-launch kernel gives up, unless the host sets another limit
constexpr int kDefaultWaitPolls = 1 << 21;

// Inspection and measurement kernels (debug_device.hip)
hipError_t launch_debug_silu(const float* z, float* out, int64_t n, hipStream_t s);
hipError_t launch_debug_score(const int32_t* dg, const int32_t* du, const int32_t* xexp, const float4* stats,
                              int kind, float* h, float* score, int64_t n, hipStream_t s);
hipError_t launch_read_stream(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s);

// Decode-step glue (decode_glue.hip)
hipError_t launch_router(const uint16_t* x, const uint16_t* w, int batch, int d, int n_experts, float* logits,
                         hipStream_t stream);
hipError_t launch_resnorm(const uint16_t* x, const uint16_t* y, int batch, int d, float eps, uint16_t* out,
                          hipStream_t stream);
hipError_t launch_resnorm_router(const uint16_t* x, const uint16_t* y, const uint16_t* w, int batch, int d,
                                 int n_experts, float eps, uint16_t* x_out, float* logits, hipStream_t stream);

}  // namespace moe_sel
