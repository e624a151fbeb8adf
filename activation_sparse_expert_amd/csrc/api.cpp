// C ABI of the library: validation, context lifecycle, preparation and the
// enqueueing of forward calls. See include/moe_sel.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"
#include "kernels.h"
#include "moe_sel.h"

struct moe_sel_ctx {
  moe_sel_config cfg{};
  int device = 0;
  // prepared layer
  uint32_t* codes = nullptr;
  float4* stats = nullptr;
  uint16_t* wch = nullptr;
  uint16_t* pmat = nullptr;
  uint16_t* qmat = nullptr;
  // workspace
  int8_t* xq = nullptr;
  int* xexp = nullptr;
  int* pair_expert = nullptr;
  float* pair_w = nullptr;
  float* hhat = nullptr;
  float* score = nullptr;
  int* sel_idx = nullptr;
  int* sel_count = nullptr;
  float* zvec = nullptr;
  float* ypart = nullptr;
  // expert-grouped path
  int* xqsum = nullptr;
  int* tile_expert = nullptr;
  int* tile_first = nullptr;
  int* tile_n = nullptr;
  int* n_tiles = nullptr;
  int* tpair = nullptr;
  uint32_t* selbits = nullptr;
  float* gzpart = nullptr;
  int* ulist = nullptr;
  uint64_t* umask = nullptr;
  int* ucount = nullptr;
  int* slot_ucount = nullptr;
  int* tile_choff = nullptr;
  int* n_items = nullptr;
  int* gu_items = nullptr;
  uint16_t* hbuf = nullptr;
  float* zsel = nullptr;
  int max_tiles = 0;
  // single-launch path
  uint64_t* xscore = nullptr;
  int* readers = nullptr;
  float* zpart = nullptr;
  float* partial = nullptr;
  float* zcopy = nullptr;
  int* err = nullptr;
  size_t xscore_count = 0, readers_count = 0, zpart_count = 0, partial_count = 0, zcopy_count = 0;
  int fused_max_batch = 0;
  int num_cus = 0;
  int fused_bpc_sparse = 0, fused_bpc_dense = 0;
  int spin_limit = moe_sel::kDefaultWaitPolls;
  moe_sel_path path = MOE_SEL_PATH_AUTO;
  moe_sel_score score_kind = MOE_SEL_SCORE_FULL;
  int last_path = -1;
  std::vector<void*> allocations;
  uint64_t device_bytes = 0;
  // last sparse call (for moe_sel_debug_selection)
  int last_batch = 0, last_top_e = 0, last_k = -1;
  hipStream_t last_stream = nullptr;
};

namespace {

constexpr int kFusedMaxBatch = 8;   // single-launch path: up to this many tokens
constexpr const char* kUnsupportedCall =
    "this call cannot run on the chosen path (a forced single launch that does not fit, or int16 score "
    "activations on a multi-kernel call whose score blocks do not route themselves)";
constexpr int kMinChunk = 8;        // fewest channels per gather block
constexpr int kTargetGather = 512;  // aim for about this many gather blocks

thread_local std::string g_last_error;

moe_sel_status fail(moe_sel_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

moe_sel_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_SEL_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

template <typename T>
moe_sel_status dev_alloc(moe_sel_ctx* c, T** p, size_t count) {
  const size_t bytes = std::max<size_t>(count * sizeof(T), 256);
  void* q = nullptr;
  const hipError_t e = (hipError_t)moe_sel::checked_device_malloc(&q, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_SEL_ENOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  c->allocations.push_back(q);
  c->device_bytes += bytes;
  *p = (T*)q;
  return MOE_SEL_OK;
}

void free_ctx(moe_sel_ctx* c) {
  if (!c) return;
  for (void* p : c->allocations) (void)hipFree(p);
  delete c;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The rank-r maps are built on the device (fp64, batched over experts);
// MOE_SEL_LOWRANK=host builds them on the host instead (the same eigen-solver).
bool lowrank_on_device(const moe_sel_config& c) {
  if (c.rank <= 0) return false;
  const char* env = std::getenv("MOE_SEL_LOWRANK");
  return !(env && std::strcmp(env, "host") == 0);
}

// The sketch codes and statistics are built on the device (bit-identical);
// MOE_SEL_SKETCH=host builds them on the host threads instead.
bool sketch_on_device() {
  const char* env = std::getenv("MOE_SEL_SKETCH");
  return !(env && std::strcmp(env, "host") == 0);
}

struct PrepJob {
  const moe_sel_config* cfg;
  std::atomic<bool>* out_of_memory;
  bool host_lowrank;
  bool host_sketch;
  const uint16_t *wg, *wu, *wd;
  uint32_t* codes;
  float* stats;
  uint16_t* wch;
  uint16_t* pmat;
  uint16_t* qmat;
  std::vector<std::string>* errors;
};

void prep_one(int e, void* arg) {
  PrepJob* j = (PrepJob*)arg;
  const moe_sel_config& c = *j->cfg;
  const size_t md = (size_t)c.m * c.d;
  moe_sel::ExpertPrep out;
  if (j->host_sketch) {
    out.codes = j->codes + (size_t)e * moe_sel::codes_dwords_per_expert(c.d, c.m);
    out.stats = j->stats + (size_t)e * c.m * 4;
  }
  out.wch = j->wch + (size_t)e * 3 * md;
  if (c.rank > 0 && j->host_lowrank) {
    out.p_bf16 = j->pmat + (size_t)e * c.rank * c.d;
    out.q_bf16 = j->qmat + (size_t)e * c.m * c.rank;
  }
  try {
    (*j->errors)[e] = moe_sel::prepare_expert(c, j->wg + (size_t)e * md, j->wu + (size_t)e * md,
                                              j->wd + (size_t)e * md, out);
  } catch (const std::bad_alloc&) {
    (*j->errors)[e] = "host allocation failed";
    j->out_of_memory->store(true);
  } catch (...) {
    (*j->errors)[e] = "unexpected exception";
  }
}

moe_sel_status check_forward(moe_sel_ctx* ctx, const void* x, const void* logits, int32_t batch, int32_t top_e,
                             int32_t k, const void* out) {
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  if (!x || !logits || !out) return fail(MOE_SEL_EINVAL, "x, logits and out must be non-null");
  if (!aligned16(x) || !aligned16(logits) || !aligned16(out))
    return fail(MOE_SEL_EINVAL, "x, logits and out must be 16-byte aligned");
  if (batch < 1 || batch > ctx->cfg.max_batch)
    return fail(MOE_SEL_EINVAL, "batch " + std::to_string(batch) + " outside [1, " +
                                    std::to_string(ctx->cfg.max_batch) + "]");
  if (top_e < 1 || top_e > ctx->cfg.max_top_e)
    return fail(MOE_SEL_EINVAL, "top_e " + std::to_string(top_e) + " outside [1, " +
                                    std::to_string(ctx->cfg.max_top_e) + "]");
  if (k < 0 || k > ctx->cfg.m)
    return fail(MOE_SEL_EINVAL, "k_budget " + std::to_string(k) + " outside [0, " + std::to_string(ctx->cfg.m) + "]");
  return MOE_SEL_OK;
}

bool force_multi_kernel() {
  static const bool v = [] {
    const char* e = std::getenv("MOE_SEL_MULTI_KERNEL");
    return e && e[0] == '1';
  }();
  return v;
}

moe_sel::FwdArgs make_args(moe_sel_ctx* c, const uint16_t* x, const float* logits, int32_t batch, int32_t top_e,
                           int32_t k, uint16_t* out) {
  moe_sel::FwdArgs a{};
  a.codes = c->codes;
  a.stats = c->stats;
  a.wch = c->wch;
  a.pmat = c->pmat;
  a.qmat = c->qmat;
  a.d = c->cfg.d;
  a.m = c->cfg.m;
  a.r = c->cfg.rank;
  a.n_experts = c->cfg.n_experts;
  a.x = x;
  a.logits = logits;
  a.out = out;
  a.batch = batch;
  a.top_e = top_e;
  a.k = k;
  a.score_kind = (int)c->score_kind;
  a.xq = c->xq;
  a.xexp = c->xexp;
  a.pair_expert = c->pair_expert;
  a.pair_w = c->pair_w;
  a.hhat = c->hhat;
  a.score = c->score;
  a.sel_idx = c->sel_idx;
  a.sel_count = c->sel_count;
  a.zvec = c->zvec;
  a.ypart = c->ypart;
  a.xqsum = c->xqsum;
  a.tile_expert = c->tile_expert;
  a.tile_first = c->tile_first;
  a.tile_n = c->tile_n;
  a.n_tiles = c->n_tiles;
  a.tpair = c->tpair;
  a.selbits = c->selbits;
  a.gzpart = c->gzpart;
  a.ulist = c->ulist;
  a.umask = c->umask;
  a.ucount = c->ucount;
  a.slot_ucount = c->slot_ucount;
  a.tile_choff = c->tile_choff;
  a.n_items = c->n_items;
  a.gu_items = c->gu_items;
  a.hbuf = c->hbuf;
  a.zsel = c->zsel;
  a.max_tiles = moe_sel::grouped_max_tiles(batch * top_e, c->cfg.n_experts);
  a.kpad = moe_sel::grouped_kpad(c->cfg.m, c->cfg.rank);
  return a;
}

// The single-launch plan of a call (block counts, chunking) with the context's
// hand-off buffers, or false when the call cannot run as one launch (shape,
// batch, or a grid that would not be resident all at once).
bool plan_fused(moe_sel_ctx* c, const moe_sel::FwdArgs& base, bool dense, moe_sel::FusedArgs* out) {
  const int pairs = base.batch * base.top_e;
  if (!c->fused_max_batch || base.batch > c->fused_max_batch ||
      !moe_sel::fused_supported(base.d, base.m, base.r, base.top_e))
    return false;
  const int count = dense ? base.m : base.k;
  // 8 channels a gather block, or 12 (dense) when that leaves too many blocks
  const int max_chunk = moe_sel::fused_max_chunk(dense);
  int chunk = kMinChunk;
  while (chunk < max_chunk && (size_t)pairs * ((count + chunk - 1) / chunk) > (size_t)kTargetGather)
    chunk = std::min(max_chunk, chunk * 3 / 2);
  moe_sel::FusedArgs f;
  static_cast<moe_sel::FwdArgs&>(f) = base;
  f.xscore = c->xscore;
  f.readers = c->readers;
  f.zpart = c->zpart;
  f.partial = c->partial;
  f.zcopy = c->zcopy;
  f.err = c->err;
  f.spin_limit = c->spin_limit;
  f.chunk = chunk;
  f.nc = std::max(1, (count + chunk - 1) / chunk);
  const bool zblocks = !dense && base.r > 0;
  f.ncs = f.nc + (zblocks ? 1 : 0);
  f.n_z = zblocks ? pairs : 0;
  f.n_gather = pairs * f.nc;
  f.n_combine = base.batch * (base.d / 32);
  const int bpc = dense ? c->fused_bpc_dense : c->fused_bpc_sparse;
  const long capacity = (long)bpc * c->num_cus;
  // score blocks of 32 channels spread the sketch over more CUs; 64 when that
  // grid would not fit. Every block of the grid must be resident at once (the
  // score hand-off waits across blocks).
  for (int sc = moe_sel::kFusedScoreChMin; sc <= 2 * moe_sel::kFusedScoreChMin; sc *= 2) {
    if (!dense && sc == moe_sel::kFusedScoreChMin && !moe_sel::fused_narrow_score_ok(base.m, base.r)) continue;
    f.score_ch = sc;
    f.n_score = dense ? 0 : pairs * (base.m / sc);
    if ((long)moe_sel::fused_grid(f, dense) <= capacity) {
      *out = f;
      return true;
    }
    if (dense) break;
  }
  return false;
}

// The single-launch path when its blocks all fit on the device at once, else
// the one-kernel-per-phase path.
// Returns hipErrorNotSupported when the single-launch path is required but cannot be used, or when the
// multi-kernel path cannot run the call (int16 score activations without self-routing score blocks).
hipError_t launch_any(moe_sel_ctx* c, const moe_sel::FwdArgs& base, bool dense, hipStream_t stream) {
  const bool want_fused = c->path != MOE_SEL_PATH_MULTI_KERNEL && !force_multi_kernel();
  moe_sel::FusedArgs f;
  if (want_fused && c->xscore && plan_fused(c, base, dense, &f)) {
    c->last_path = MOE_SEL_PATH_SINGLE_LAUNCH;
    return moe_sel::launch_fused(f, dense, stream);
  }
  if (c->path == MOE_SEL_PATH_SINGLE_LAUNCH) return hipErrorNotSupported;
  c->last_path = MOE_SEL_PATH_MULTI_KERNEL;
  return moe_sel::launch_forward(base, dense, stream);
}

// every hand-off slot empty (0xFF bytes), error bits clear
hipError_t reset_handoff(moe_sel_ctx* c, hipStream_t s) {
  hipError_t he = hipSuccess;
  const struct {
    void* p;
    size_t bytes;
  } slots[] = {{c->xscore, c->xscore_count * 8},
               {c->zpart, c->zpart_count * 4},
               {c->partial, c->partial_count * 4},
               {c->zcopy, c->zcopy_count * 4}};
  for (const auto& sl : slots)
    if (he == hipSuccess) he = hipMemsetAsync(sl.p, 0xFF, sl.bytes, s);
  if (he == hipSuccess) he = hipMemsetAsync(c->readers, 0, c->readers_count * 4, s);
  if (he == hipSuccess) he = hipMemsetAsync(c->err, 0, 4, s);
  return he;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
    else prev = -1;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace

namespace moe_sel {

int checked_device_malloc(void** p, size_t bytes) {
  if (alloc_fault_hit()) return (int)hipErrorOutOfMemory;
  return (int)hipMalloc(p, bytes);
}

std::string validate_config(const moe_sel_config* c) {
  if (!c) return "config is null";
  if (c->struct_size != sizeof(moe_sel_config))
    return "config.struct_size is " + std::to_string(c->struct_size) + ", expected " +
           std::to_string(sizeof(moe_sel_config));
  if (c->d < 64 || c->d > 16384 || c->d % 64) return "d must be a multiple of 64 in [64, 16384]";
  if (c->m < 64 || c->m > 32768 || c->m % 64) return "m must be a multiple of 64 in [64, 32768]";
  if (c->n_experts < 1 || c->n_experts > 1024) return "n_experts must be in [1, 1024]";
  if (c->rank < 0 || c->rank > 128 || c->rank > c->d || c->rank > c->m) return "rank must be in [0, min(d, m, 128)]";
  if (c->max_top_e < 1 || c->max_top_e > 64 || c->max_top_e > c->n_experts)
    return "max_top_e must be in [1, min(n_experts, 64)]";
  if (c->max_batch < 1 || c->max_batch > 4096) return "max_batch must be in [1, 4096]";
  if (!(c->tern_ratio > 0.0 && c->tern_ratio < 1e3)) return "tern_ratio must be in (0, 1000)";
  return std::string();
}

}  // namespace moe_sel

namespace {

// Every device buffer of a layer: the prepared arrays (left for the caller to
// fill) and the forward workspace sized for cfg.max_batch tokens.
moe_sel_status alloc_layer(moe_sel_ctx* ctx) {
  const moe_sel_config& c = ctx->cfg;
  const size_t E = c.n_experts, d = c.d, m = c.m, r = c.rank;
  const size_t pairs = (size_t)c.max_batch * c.max_top_e;
  const size_t n_codes = E * moe_sel::codes_dwords_per_expert(c.d, c.m);
  moe_sel_status st = MOE_SEL_OK;
#define ALLOC(ptr, n) \
  if (st == MOE_SEL_OK) st = dev_alloc(ctx, &ctx->ptr, (n))
  ALLOC(codes, n_codes);
  ALLOC(stats, E * m);
  ALLOC(wch, E * m * 3 * d);
  ALLOC(pmat, std::max<size_t>(E * r * d, 1));
  ALLOC(qmat, std::max<size_t>(E * m * r, 1));
  ALLOC(xq, (size_t)c.max_batch * d);
  ALLOC(xexp, (size_t)c.max_batch);
  ALLOC(pair_expert, pairs);
  ALLOC(pair_w, pairs);
  ALLOC(hhat, pairs * m);
  ALLOC(score, pairs * m);
  ALLOC(sel_idx, pairs * m);
  ALLOC(sel_count, pairs);
  ALLOC(zvec, pairs * std::max<size_t>(r, 1));
  // partial outputs: the largest split times the pairs of any call size
  size_t ypart_count = 0;
  for (int pp = 1; pp <= c.max_batch * c.max_top_e; ++pp) {
    const size_t need =
        (size_t)moe_sel::grouped_down_split(moe_sel::grouped_max_tiles(pp, c.n_experts), c.d, c.m, c.rank) * pp * d;
    ypart_count = std::max(ypart_count, need);
    if (pp <= c.max_top_e || 2 * pp <= c.n_experts)  // calls with one pair per tile
      ypart_count = std::max(ypart_count, (size_t)moe_sel::grouped_down_split_b1(c.m, c.rank) * pp * d);
  }
  ALLOC(ypart, ypart_count);
  ctx->max_tiles = moe_sel::grouped_max_tiles((int)pairs, c.n_experts);
  const size_t mt = ctx->max_tiles;
  ALLOC(xqsum, (size_t)c.max_batch);
  ALLOC(tile_expert, mt);
  ALLOC(tile_first, mt);
  ALLOC(tile_n, mt);
  ALLOC(n_tiles, 1);
  ALLOC(tpair, pairs);
  ALLOC(selbits, pairs * (m / 32));
  ALLOC(gzpart, pairs * (m / moe_sel::kGroup) * std::max<size_t>(r, 1));
  ALLOC(ulist, mt * m);
  ALLOC(umask, mt * m);
  ALLOC(ucount, mt);
  ALLOC(slot_ucount, pairs);
  ALLOC(tile_choff, mt);
  ALLOC(n_items, 1);
  ALLOC(gu_items, mt * (m / 16) * moe_sel::kGuItemInts);
  ALLOC(hbuf, pairs * moe_sel::grouped_kpad(c.m, c.rank));
  ALLOC(zsel, pairs * (m / 16) * std::max<size_t>(r, 1));

  // single-launch path: sized for up to kFusedMaxBatch tokens and the smallest chunk
  const bool fusable = moe_sel::fused_supported(c.d, c.m, c.rank, c.max_top_e);
  if (fusable) {
    ctx->fused_max_batch = std::min(c.max_batch, kFusedMaxBatch);
    const size_t fp = (size_t)ctx->fused_max_batch * c.max_top_e;
    const size_t nc_max = (m + kMinChunk - 1) / kMinChunk;
    const size_t slices = d / 64;
    ctx->xscore_count = fp * m;
    ctx->readers_count = fp;
    ctx->zpart_count = fp * (m / moe_sel::kFusedScoreChMin) * std::max<size_t>(r, 1);
    ctx->partial_count = (size_t)ctx->fused_max_batch * slices * c.max_top_e * nc_max * 64;
    ctx->zcopy_count = (size_t)ctx->fused_max_batch * 2 * slices * c.max_top_e * std::max<size_t>(r, 1);
    ALLOC(xscore, ctx->xscore_count);
    ALLOC(readers, ctx->readers_count);
    ALLOC(zpart, ctx->zpart_count);
    ALLOC(partial, ctx->partial_count);
    ALLOC(zcopy, ctx->zcopy_count);
    ALLOC(err, 1);
  }
#undef ALLOC
  return st;
}

// ---------------------------------------------------------------------------
// Scratch of moe_sel_forward_noalloc: one file-scope device array, of which each
// GPU holds its own copy until the process ends. Sub-arrays at fixed offsets,
// each sized for the largest call the entry point accepts: the four hand-off
// slot arrays of the single-launch kernel (kept empty between calls), its error
// word, and the arrays it fills for inspection. Host code never passes the
// array's name to a kernel or a copy: set-up looks up each device's copy with
// hipGetSymbolAddress and keeps that pointer.
// ---------------------------------------------------------------------------
constexpr size_t kScrXscore = (size_t)3 << 20;   // (score, h_hat) slots
constexpr size_t kScrZpart = (size_t)256 << 10;  // score-block shares of Q^T h_hat
constexpr size_t kScrPartial = (size_t)3 << 20;  // gather-block down partials
constexpr size_t kScrZcopy = (size_t)256 << 10;  // z for the combine blocks
constexpr size_t kScrErr = 4096;                 // error word, then the reader counts (zeroed)
constexpr size_t kScrInspect = (size_t)1 << 20;  // hhat, score, sel_idx, pair arrays
constexpr size_t kScrSlots = kScrXscore + kScrZpart + kScrPartial + kScrZcopy;
constexpr size_t kScratchBytes = kScrSlots + kScrErr + kScrInspect;
static_assert(kScratchBytes % 256 == 0, "scratch sub-arrays keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};  // device address of each GPU's copy (null until set up)

// Once per device, with that device current: find this GPU's copy of the
// scratch array and empty its slots. Called while a context is created.
moe_sel_status scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_SEL_OK;  // the no-allocation entry point then refuses
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return MOE_SEL_OK;
  unsigned char* p = nullptr;
  hipError_t e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
  if (e == hipSuccess) e = hipMemsetAsync(p, 0xFF, kScrSlots, nullptr);
  if (e == hipSuccess) e = hipMemsetAsync(p + kScrSlots, 0, kScrErr, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_fail(e, "scratch set-up");
  g_scratch_ptr[dev] = p;
  return MOE_SEL_OK;
}

unsigned char* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[dev];
}

// After the prepared arrays are queued on s: empty hand-off slots and the
// device properties of the single-launch path, then wait for s.
moe_sel_status finish_layer(moe_sel_ctx* ctx, hipStream_t s) {
  const moe_sel_config& c = ctx->cfg;
  hipError_t he = hipSuccess;
  if (ctx->xscore) {
    he = reset_handoff(ctx, s);
    if (he == hipSuccess) {
      he = hipDeviceGetAttribute(&ctx->num_cus, hipDeviceAttributeMultiprocessorCount, ctx->device);
      ctx->fused_bpc_sparse = moe_sel::fused_blocks_per_cu(false, c.d, c.m, c.rank);
      ctx->fused_bpc_dense = moe_sel::fused_blocks_per_cu(true, c.d, c.m, c.rank);
    }
    if (he != hipSuccess) return hip_fail(he, "fused path set-up");
  }
  he = hipStreamSynchronize(s);
  if (he != hipSuccess) return hip_fail(he, "hipStreamSynchronize");
  return ctx->xscore ? scratch_setup(ctx->device) : MOE_SEL_OK;
}

// A context for cfg on the current device, with no buffers yet.
moe_sel_status new_ctx(const moe_sel_config& c, moe_sel_ctx** out) {
  moe_sel_ctx* ctx = nullptr;
  try {
    ctx = new moe_sel_ctx();
  } catch (...) {
    return fail(MOE_SEL_ENOMEM, "host allocation failed");
  }
  ctx->cfg = c;
  const hipError_t he = hipGetDevice(&ctx->device);
  if (he != hipSuccess) {
    free_ctx(ctx);
    return hip_fail(he, "hipGetDevice");
  }
  *out = ctx;
  return MOE_SEL_OK;
}


// ---------------------------------------------------------------------------
// Saved layers. A file holds, little-endian:
//   char magic[8] = "MOESELv1"; uint32 format = 1; uint32 zero;
//   int32 d, n_experts, m, rank, max_top_e, max_batch; double tern_ratio;
//   uint64 bytes of each prepared array: codes, stats, wch, pmat, qmat;
//   the five arrays, device layout, in that order;
//   uint64 FNV-1a hash of the arrays taken over 64-bit little-endian words.
// ---------------------------------------------------------------------------
constexpr char kMagic[8] = {'M', 'O', 'E', 'S', 'E', 'L', 'v', '1'};
constexpr uint32_t kFormat = 1;
constexpr size_t kStage = (size_t)64 << 20;  // bytes staged on the host at a time
constexpr uint64_t kFnvBasis = 0xCBF29CE484222325ull, kFnvPrime = 0x100000001B3ull;

struct SavedArray {
  void* dev;
  size_t bytes;
};

// Bytes of the prepared arrays of a layer (all multiples of 8).
void prepared_bytes(const moe_sel_config& c, uint64_t (&b)[5]) {
  const size_t E = c.n_experts, d = c.d, m = c.m, r = c.rank;
  b[0] = E * moe_sel::codes_dwords_per_expert(c.d, c.m) * 4;
  b[1] = E * m * 16;
  b[2] = E * m * 3 * d * 2;
  b[3] = E * r * d * 2;
  b[4] = E * m * r * 2;
}

// The prepared arrays of a context: codes, stats, wch, pmat, qmat.
void prepared_arrays(const moe_sel_ctx* ctx, SavedArray (&arr)[5]) {
  uint64_t b[5];
  prepared_bytes(ctx->cfg, b);
  void* const dev[5] = {ctx->codes, ctx->stats, ctx->wch, ctx->pmat, ctx->qmat};
  for (int i = 0; i < 5; ++i) arr[i] = {dev[i], (size_t)b[i]};
}

uint64_t fnv_words(uint64_t h, const unsigned char* p, size_t bytes) {
  for (size_t i = 0; i + 8 <= bytes; i += 8) {
    uint64_t w;
    std::memcpy(&w, p + i, 8);
    h = (h ^ w) * kFnvPrime;
  }
  return h;
}

struct FileCloser {
  FILE* f;
  ~FileCloser() {
    if (f) std::fclose(f);
  }
};

}  // namespace

extern "C" {

int32_t moe_sel_abi_version(void) { return MOE_SEL_ABI_VERSION; }

const char* moe_sel_status_str(moe_sel_status s) {
  switch (s) {
    case MOE_SEL_OK: return "ok";
    case MOE_SEL_EINVAL: return "invalid argument";
    case MOE_SEL_EUNSUPPORTED: return "unsupported";
    case MOE_SEL_ENOMEM: return "out of memory";
    case MOE_SEL_EDEVICE: return "device error";
    case MOE_SEL_EIO: return "file error";
  }
  return "unknown status";
}

const char* moe_sel_last_error(void) { return g_last_error.c_str(); }

moe_sel_status moe_sel_prepare_expert_host(const moe_sel_config* cfg, const uint16_t* w_gate, const uint16_t* w_up,
                                           const uint16_t* w_down, int8_t* tern_gate, int8_t* tern_up,
                                           float* alpha_gate, float* alpha_up, float* down_norm, int32_t* nnz_gate,
                                           int32_t* nnz_up, uint16_t* p_bf16, uint16_t* q_bf16) {
  g_last_error.clear();
  const std::string bad = moe_sel::validate_config(cfg);
  if (!bad.empty()) return fail(MOE_SEL_EINVAL, bad);
  if (!w_gate || !w_up || !w_down) return fail(MOE_SEL_EINVAL, "weights must be non-null");
  moe_sel::ExpertPrep out;
  out.tern_gate = tern_gate;
  out.tern_up = tern_up;
  out.alpha_gate = alpha_gate;
  out.alpha_up = alpha_up;
  out.down_norm = down_norm;
  out.nnz_gate = nnz_gate;
  out.nnz_up = nnz_up;
  out.p_bf16 = p_bf16;
  out.q_bf16 = q_bf16;
  try {
    const std::string err = moe_sel::prepare_expert(*cfg, w_gate, w_up, w_down, out);
    if (!err.empty()) return fail(MOE_SEL_EINVAL, err);
  } catch (const std::bad_alloc&) {
    return fail(MOE_SEL_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(MOE_SEL_EINVAL, "unexpected exception");
  }
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_prepare(const moe_sel_config* cfg, const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, void* stream, moe_sel_ctx** out) {
  g_last_error.clear();
  const std::string bad = moe_sel::validate_config(cfg);
  if (!bad.empty()) return fail(MOE_SEL_EINVAL, bad);
  if (!w_gate || !w_up || !w_down || !out) return fail(MOE_SEL_EINVAL, "weights and out must be non-null");
  if (!moe_sel::grouped_supported(cfg->d, cfg->m))
    return fail(MOE_SEL_EUNSUPPORTED, "m = " + std::to_string(cfg->m) + " is above the per-pair selection limit (16384)");
  const moe_sel_config c = *cfg;
  const size_t E = c.n_experts, d = c.d, m = c.m, r = c.rank;
  moe_sel_ctx* ctx = nullptr;
  moe_sel_status st = new_ctx(c, &ctx);
  if (st != MOE_SEL_OK) return st;
  hipError_t he = hipSuccess;
  // host staging of the prepared layer
  const bool dev_sketch = sketch_on_device();
  const size_t n_codes = E * moe_sel::codes_dwords_per_expert(c.d, c.m);
  std::vector<uint32_t> h_codes;
  std::vector<float> h_stats;
  std::vector<uint16_t> h_wch, h_p, h_q;
  try {
    if (moe_sel::alloc_fault_hit()) throw std::bad_alloc();
    if (!dev_sketch) {
      h_codes.resize(n_codes);
      h_stats.resize(E * m * 4);
    }
    h_wch.resize(E * m * 3 * d);
    h_p.resize(std::max<size_t>(E * r * d, 1));
    h_q.resize(std::max<size_t>(E * m * r, 1));
  } catch (...) {
    free_ctx(ctx);
    return fail(MOE_SEL_ENOMEM, "host staging allocation failed");
  }
  std::vector<std::string> errors(E);
  std::atomic<bool> out_of_memory{false};
  const bool dev_lowrank = lowrank_on_device(c);
  PrepJob job{&c,           &out_of_memory, !dev_lowrank, !dev_sketch, w_gate,     w_up,       w_down,
              h_codes.data(), h_stats.data(), h_wch.data(), h_p.data(), h_q.data(), &errors};
  moe_sel::parallel_for((int)E, 0, prep_one, &job);
  for (size_t e = 0; e < E; ++e)
    if (!errors[e].empty()) {
      free_ctx(ctx);
      return fail(out_of_memory.load() ? MOE_SEL_ENOMEM : MOE_SEL_EINVAL, "expert " + std::to_string(e) + ": " + errors[e]);
    }
  st = alloc_layer(ctx);
  if (st != MOE_SEL_OK) {
    free_ctx(ctx);
    return st;
  }
  hipStream_t s = (hipStream_t)stream;
  struct Up {
    void* dst;
    const void* src;
    size_t bytes;
  } ups[] = {{ctx->codes, h_codes.data(), h_codes.size() * 4},
             {ctx->stats, h_stats.data(), h_stats.size() * 4},
             {ctx->wch, h_wch.data(), h_wch.size() * 2},
             {ctx->pmat, h_p.data(), h_p.size() * 2},
             {ctx->qmat, h_q.data(), h_q.size() * 2}};
  for (int ui = 0; ui < 5; ++ui) {
    const Up& u = ups[ui];
    if (ui < 2 && dev_sketch) continue;
    if (ui == 3 && dev_sketch) {
      // codes and statistics from the channel rows now on the device
      const std::string err = moe_sel::sketch_stats_device(ctx->wch, c.n_experts, c.d, c.m, c.tern_ratio,
                                                           ctx->codes, (float*)ctx->stats, s);
      if (!err.empty()) {
        free_ctx(ctx);
        return fail(MOE_SEL_EDEVICE, err);
      }
    }
    if (ui == 3 && dev_lowrank) {
      // maps from the channel rows now on the device
      std::string err;
      try {
        err = moe_sel::lowrank_maps_device(ctx->wch, c.n_experts, c.d, c.m, c.rank, h_p.data(), h_q.data(), s);
      } catch (const std::bad_alloc&) {
        err = std::string(moe_sel::kNoDeviceMemory) + "host staging of the low-rank maps";
      }
      if (!err.empty()) {
        free_ctx(ctx);
        return fail(err.rfind(moe_sel::kNoDeviceMemory, 0) == 0 ? MOE_SEL_ENOMEM : MOE_SEL_EDEVICE, err);
      }
    }
    he = hipMemcpyAsync(u.dst, u.src, u.bytes, hipMemcpyHostToDevice, s);
    if (he != hipSuccess) {
      free_ctx(ctx);
      return hip_fail(he, "hipMemcpyAsync");
    }
  }
  st = finish_layer(ctx, s);
  if (st != MOE_SEL_OK) {
    free_ctx(ctx);
    return st;
  }
  *out = ctx;
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_save(const moe_sel_ctx* ctx, const char* path) {
  g_last_error.clear();
  if (!ctx || !path) return fail(MOE_SEL_EINVAL, "ctx and path must be non-null");
  DeviceGuard guard(ctx->device);
  SavedArray arr[5];
  prepared_arrays(ctx, arr);
  std::vector<unsigned char> stage;
  try {
    if (moe_sel::alloc_fault_hit()) throw std::bad_alloc();
    stage.resize(kStage);
  } catch (...) {
    return fail(MOE_SEL_ENOMEM, "host staging allocation failed");
  }
  FileCloser fc{std::fopen(path, "wb")};
  if (!fc.f) return fail(MOE_SEL_EIO, std::string("cannot open ") + path + " for writing");
  const moe_sel_config& c = ctx->cfg;
  const uint32_t head[2] = {kFormat, 0u};
  const int32_t dims[6] = {c.d, c.n_experts, c.m, c.rank, c.max_top_e, c.max_batch};
  uint64_t sizes[5];
  for (int i = 0; i < 5; ++i) sizes[i] = arr[i].bytes;
  bool ok = std::fwrite(kMagic, 1, 8, fc.f) == 8 && std::fwrite(head, 4, 2, fc.f) == 2 &&
            std::fwrite(dims, 4, 6, fc.f) == 6 && std::fwrite(&c.tern_ratio, 8, 1, fc.f) == 1 &&
            std::fwrite(sizes, 8, 5, fc.f) == 5;
  uint64_t h = kFnvBasis;
  for (int i = 0; ok && i < 5; ++i)
    for (size_t off = 0; ok && off < arr[i].bytes; off += kStage) {
      const size_t n = std::min(kStage, arr[i].bytes - off);
      const hipError_t e = hipMemcpy(stage.data(), (const unsigned char*)arr[i].dev + off, n, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
      h = fnv_words(h, stage.data(), n);
      ok = std::fwrite(stage.data(), 1, n, fc.f) == n;
    }
  ok = ok && std::fwrite(&h, 8, 1, fc.f) == 1;
  const int closed = std::fclose(fc.f);
  fc.f = nullptr;
  if (!ok || closed != 0) return fail(MOE_SEL_EIO, std::string("write to ") + path + " failed");
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_load(const char* path, void* stream, moe_sel_ctx** out) {
  g_last_error.clear();
  if (!path || !out) return fail(MOE_SEL_EINVAL, "path and out must be non-null");
  FileCloser fc{std::fopen(path, "rb")};
  if (!fc.f) return fail(MOE_SEL_EIO, std::string("cannot open ") + path);
  const std::string bad_file = std::string(path) + " is not a saved layer: ";
  char magic[8];
  uint32_t head[2];
  int32_t dims[6];
  moe_sel_config c{};
  c.struct_size = sizeof(moe_sel_config);
  uint64_t sizes[5];
  if (std::fread(magic, 1, 8, fc.f) != 8 || std::memcmp(magic, kMagic, 8) != 0)
    return fail(MOE_SEL_EIO, bad_file + "wrong magic");
  if (std::fread(head, 4, 2, fc.f) != 2 || head[0] != kFormat || head[1] != 0u)
    return fail(MOE_SEL_EIO, bad_file + "unknown format version");
  if (std::fread(dims, 4, 6, fc.f) != 6 || std::fread(&c.tern_ratio, 8, 1, fc.f) != 1 ||
      std::fread(sizes, 8, 5, fc.f) != 5)
    return fail(MOE_SEL_EIO, bad_file + "truncated header");
  c.d = dims[0];
  c.n_experts = dims[1];
  c.m = dims[2];
  c.rank = dims[3];
  c.max_top_e = dims[4];
  c.max_batch = dims[5];
  const std::string bad = moe_sel::validate_config(&c);
  if (!bad.empty()) return fail(MOE_SEL_EIO, bad_file + bad);
  if (!moe_sel::grouped_supported(c.d, c.m))
    return fail(MOE_SEL_EUNSUPPORTED, "m = " + std::to_string(c.m) + " is above the per-pair selection limit (16384)");
  uint64_t expect[5];
  prepared_bytes(c, expect);
  for (int i = 0; i < 5; ++i)
    if (sizes[i] != expect[i]) return fail(MOE_SEL_EIO, bad_file + "array sizes do not match its shape");
  moe_sel_ctx* ctx = nullptr;
  moe_sel_status st = new_ctx(c, &ctx);
  if (st != MOE_SEL_OK) return st;
  st = alloc_layer(ctx);
  SavedArray arr[5];
  prepared_arrays(ctx, arr);
  std::vector<unsigned char> stage;
  if (st == MOE_SEL_OK) try {
      if (moe_sel::alloc_fault_hit()) throw std::bad_alloc();
      stage.resize(kStage);
    } catch (...) {
      st = fail(MOE_SEL_ENOMEM, "host staging allocation failed");
    }
  hipStream_t s = (hipStream_t)stream;
  uint64_t h = kFnvBasis;
  for (int i = 0; st == MOE_SEL_OK && i < 5; ++i)
    for (size_t off = 0; st == MOE_SEL_OK && off < arr[i].bytes; off += kStage) {
      const size_t n = std::min(kStage, arr[i].bytes - off);
      if (std::fread(stage.data(), 1, n, fc.f) != n) {
        st = fail(MOE_SEL_EIO, bad_file + "truncated data");
        break;
      }
      h = fnv_words(h, stage.data(), n);
      hipError_t e = hipMemcpyAsync((unsigned char*)arr[i].dev + off, stage.data(), n, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);  // the staging buffer is reused
      if (e != hipSuccess) st = hip_fail(e, "hipMemcpyAsync");
    }
  uint64_t stored = 0;
  if (st == MOE_SEL_OK && (std::fread(&stored, 8, 1, fc.f) != 1 || stored != h))
    st = fail(MOE_SEL_EIO, bad_file + "checksum mismatch");
  if (st == MOE_SEL_OK && std::fgetc(fc.f) != EOF) st = fail(MOE_SEL_EIO, bad_file + "trailing bytes");
  if (st == MOE_SEL_OK) st = finish_layer(ctx, s);
  if (st != MOE_SEL_OK) {
    free_ctx(ctx);
    return st;
  }
  *out = ctx;
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_forward(moe_sel_ctx* ctx, const uint16_t* x, const float* logits, int32_t batch,
                               int32_t top_e, int32_t k_budget, uint16_t* out, void* stream) {
  g_last_error.clear();
  moe_sel_status st = check_forward(ctx, x, logits, batch, top_e, k_budget, out);
  if (st != MOE_SEL_OK) return st;
  DeviceGuard guard(ctx->device);
  const moe_sel::FwdArgs a = make_args(ctx, x, logits, batch, top_e, k_budget, out);
  const hipError_t e = launch_any(ctx, a, false, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(MOE_SEL_EUNSUPPORTED, kUnsupportedCall);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  ctx->last_batch = batch;
  ctx->last_top_e = top_e;
  ctx->last_k = k_budget;
  ctx->last_stream = (hipStream_t)stream;
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_forward_noalloc(moe_sel_ctx* ctx, const uint16_t* x, const float* logits, int32_t batch,
                                       int32_t top_e, int32_t k_budget, uint16_t* out, void* stream) {
  g_last_error.clear();
  moe_sel_status st = check_forward(ctx, x, logits, batch, top_e, k_budget, out);
  if (st != MOE_SEL_OK) return st;
  DeviceGuard guard(ctx->device);
  unsigned char* scr = scratch_ptr(ctx->device);
  if (!scr) return fail(MOE_SEL_EUNSUPPORTED, "no-allocation scratch is not set up on this device (a layer that "
                                              "cannot run as one launch, or a device index above 63)");
  const moe_sel::FwdArgs a = make_args(ctx, x, logits, batch, top_e, k_budget, out);
  moe_sel::FusedArgs f;
  if (!plan_fused(ctx, a, false, &f))
    return fail(MOE_SEL_EUNSUPPORTED, "moe_sel_forward_noalloc runs only calls the single launch can take");
  // the call's share of each scratch sub-array
  const size_t pairs = (size_t)batch * top_e, m = ctx->cfg.m, d = ctx->cfg.d;
  const size_t r1 = std::max(ctx->cfg.rank, 1), slices = d / 64;
  const size_t need_xscore = pairs * m * 8;
  const size_t need_zpart = pairs * (m / f.score_ch) * r1 * 4;
  const size_t need_partial = (size_t)batch * slices * top_e * f.nc * 64 * 4;
  const size_t need_zcopy = (size_t)batch * 2 * slices * top_e * r1 * 4;
  const size_t need_inspect = 3 * pairs * m * 4 + 3 * pairs * 4 + 3 * 256;
  if (need_xscore > kScrXscore || need_zpart > kScrZpart || need_partial > kScrPartial || need_zcopy > kScrZcopy ||
      need_inspect > kScrInspect || 4 * (pairs + 64) > kScrErr)
    return fail(MOE_SEL_EUNSUPPORTED,
                "call needs more scratch than moe_sel_forward_noalloc holds (" + std::to_string(kScratchBytes >> 20) +
                    " MiB per device: hand-off slots " + std::to_string(need_xscore + need_zpart + need_partial + need_zcopy) +
                    " bytes of at most " + std::to_string(kScrSlots) + ")");
  unsigned char* q = scr;
  f.xscore = (uint64_t*)q;
  f.zpart = (float*)(q += kScrXscore);
  f.partial = (float*)(q += kScrZpart);
  f.zcopy = (float*)(q += kScrPartial);
  f.err = (int*)(q += kScrZcopy);
  f.readers = f.err + 64;
  q += kScrErr;
  auto take = [&q](size_t bytes) {
    unsigned char* r = q;
    q += (bytes + 255) / 256 * 256;
    return r;
  };
  f.hhat = (float*)take(pairs * m * 4);
  f.score = (float*)take(pairs * m * 4);
  f.sel_idx = (int*)take(pairs * m * 4);
  f.pair_expert = (int*)take(pairs * 4);
  f.pair_w = (float*)take(pairs * 4);
  f.sel_count = (int*)take(pairs * 4);
  const hipError_t e = moe_sel::launch_fused(f, false, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_forward_threshold(moe_sel_ctx* ctx, const uint16_t* x, const float* logits, int32_t batch,
                                         int32_t top_e, float threshold, uint16_t* out, void* stream) {
  g_last_error.clear();
  moe_sel_status st = check_forward(ctx, x, logits, batch, top_e, 0, out);
  if (st != MOE_SEL_OK) return st;
  if (!(threshold >= 0.0f) || !std::isfinite(threshold))
    return fail(MOE_SEL_EINVAL, "threshold must be finite and non-negative");
  DeviceGuard guard(ctx->device);
  moe_sel::FwdArgs a = make_args(ctx, x, logits, batch, top_e, 0, out);
  a.thr_mode = 1;
  std::memcpy(&a.thr_bits, &threshold, 4);
  const hipError_t e = moe_sel::launch_forward(a, false, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  ctx->last_path = MOE_SEL_PATH_MULTI_KERNEL;
  ctx->last_batch = batch;
  ctx->last_top_e = top_e;
  ctx->last_k = ctx->cfg.m;  // selections vary in length: rows of m entries, chan_count valid
  ctx->last_stream = (hipStream_t)stream;
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_forward_dense(moe_sel_ctx* ctx, const uint16_t* x, const float* logits, int32_t batch,
                                     int32_t top_e, uint16_t* out, void* stream) {
  g_last_error.clear();
  moe_sel_status st = check_forward(ctx, x, logits, batch, top_e, 0, out);
  if (st != MOE_SEL_OK) return st;
  DeviceGuard guard(ctx->device);
  const moe_sel::FwdArgs a = make_args(ctx, x, logits, batch, top_e, ctx->cfg.m, out);
  const hipError_t e = launch_any(ctx, a, true, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(MOE_SEL_EUNSUPPORTED, kUnsupportedCall);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_debug_selection(moe_sel_ctx* ctx, int32_t* expert_ids, float* gate_w, int32_t* chan_idx,
                                       int32_t* chan_count, float* h_hat, float* score) {
  g_last_error.clear();
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  if (ctx->last_k < 0) return fail(MOE_SEL_EINVAL, "no sparse forward has run on this context");
  DeviceGuard guard(ctx->device);
  hipError_t e = hipStreamSynchronize(ctx->last_stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  const size_t pairs = (size_t)ctx->last_batch * ctx->last_top_e;
  const size_t m = ctx->cfg.m, k = ctx->last_k;
  if (expert_ids && (e = hipMemcpy(expert_ids, ctx->pair_expert, pairs * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (gate_w && (e = hipMemcpy(gate_w, ctx->pair_w, pairs * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (chan_count && (e = hipMemcpy(chan_count, ctx->sel_count, pairs * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (chan_idx && k > 0 &&
      (e = hipMemcpy2D(chan_idx, k * 4, ctx->sel_idx, m * 4, k * 4, pairs, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy2D");
  if (h_hat && (e = hipMemcpy(h_hat, ctx->hhat, pairs * m * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (score && (e = hipMemcpy(score, ctx->score, pairs * m * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_export_expert(moe_sel_ctx* ctx, int32_t expert, int8_t* tern_gate, int8_t* tern_up,
                                     float* alpha_gate, float* alpha_up, float* down_norm, int32_t* nnz_gate,
                                     int32_t* nnz_up, uint16_t* p_bf16, uint16_t* q_bf16) {
  g_last_error.clear();
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  if (expert < 0 || expert >= ctx->cfg.n_experts) return fail(MOE_SEL_EINVAL, "expert out of range");
  DeviceGuard guard(ctx->device);
  const int d = ctx->cfg.d, m = ctx->cfg.m, r = ctx->cfg.rank;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  if (tern_gate || tern_up || nnz_gate || nnz_up) {
    const size_t nd = moe_sel::codes_dwords_per_expert(d, m);
    std::vector<uint32_t> codes;
    try {
      codes.resize(nd);
    } catch (const std::bad_alloc&) {
      return fail(MOE_SEL_ENOMEM, "host staging allocation failed");
    }
    if ((e = hipMemcpy(codes.data(), ctx->codes + (size_t)expert * nd, nd * 4, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
    for (int j = 0; j < m; ++j)
      for (int mat = 0; mat < 2; ++mat) {
        int8_t* dst = mat == 0 ? tern_gate : tern_up;
        int32_t* nnz = mat == 0 ? nnz_gate : nnz_up;
        if (!dst && !nnz) continue;
        int32_t kept = 0;
        for (int i = 0; i < d; ++i) {
          const int b = i / moe_sel::kBlock, w = (i % moe_sel::kBlock) / 16, a = (i % 16) / 4, ii = i % 4;
          const uint32_t word = codes[moe_sel::codes_dword_index(d, m, j / moe_sel::kGroup, mat, b,
                                                                 j % moe_sel::kGroup, w)];
          const int t = (int)((word >> (8 * ii + 2 * a)) & 3u) - 1;
          kept += t != 0;
          if (dst) dst[(size_t)j * d + i] = (int8_t)t;
        }
        if (nnz) nnz[j] = kept;
      }
  }
  if (alpha_gate || alpha_up || down_norm) {
    std::vector<float> st((size_t)m * 4);
    if ((e = hipMemcpy(st.data(), ctx->stats + (size_t)expert * m, (size_t)m * 16, hipMemcpyDeviceToHost)) !=
        hipSuccess)
      return hip_fail(e, "hipMemcpy");
    for (int j = 0; j < m; ++j) {
      if (alpha_gate) alpha_gate[j] = st[(size_t)j * 4];
      if (alpha_up) alpha_up[j] = st[(size_t)j * 4 + 1];
      if (down_norm) down_norm[j] = st[(size_t)j * 4 + 2];
    }
  }
  if (p_bf16 && r > 0 &&
      (e = hipMemcpy(p_bf16, ctx->pmat + (size_t)expert * r * d, (size_t)r * d * 2, hipMemcpyDeviceToHost)) !=
          hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (q_bf16 && r > 0 &&
      (e = hipMemcpy(q_bf16, ctx->qmat + (size_t)expert * m * r, (size_t)m * r * 2, hipMemcpyDeviceToHost)) !=
          hipSuccess)
    return hip_fail(e, "hipMemcpy");
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_check_device(moe_sel_ctx* ctx) {
  g_last_error.clear();
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  DeviceGuard guard(ctx->device);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  if (!ctx->err) return MOE_SEL_OK;
  int bits = 0, sbits = 0;
  if ((e = hipMemcpy(&bits, ctx->err, 4, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy");
  unsigned char* scr = scratch_ptr(ctx->device);
  if (scr && (e = hipMemcpy(&sbits, scr + kScrSlots, 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (bits == 0 && sbits == 0) return MOE_SEL_OK;
  // a bounded wait expired: reset the hand-off state so the next call starts clean
  if (bits) (void)reset_handoff(ctx, nullptr);
  if (sbits) {
    (void)hipMemsetAsync(scr, 0xFF, kScrSlots, nullptr);
    (void)hipMemsetAsync(scr + kScrSlots, 0, kScrErr, nullptr);
  }
  (void)hipDeviceSynchronize();
  return fail(MOE_SEL_EDEVICE, "a cross-block wait timed out (bits " + std::to_string(bits | sbits) +
                                   (sbits ? ", in the device's no-allocation scratch" : "") +
                                   "); outputs of the affected calls are invalid");
}

moe_sel_status moe_sel_set_wait_limit(moe_sel_ctx* ctx, int32_t polls) {
  g_last_error.clear();
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  if (polls < 0 || polls > (1 << 30)) return fail(MOE_SEL_EINVAL, "polls must be in [0, 2^30]");
  ctx->spin_limit = polls;
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_set_path(moe_sel_ctx* ctx, moe_sel_path path) {
  g_last_error.clear();
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  if (path != MOE_SEL_PATH_AUTO && path != MOE_SEL_PATH_MULTI_KERNEL && path != MOE_SEL_PATH_SINGLE_LAUNCH)
    return fail(MOE_SEL_EINVAL, "unknown path");
  ctx->path = path;
  return MOE_SEL_OK;
}

int32_t moe_sel_last_path(const moe_sel_ctx* ctx) { return ctx ? ctx->last_path : -1; }

moe_sel_status moe_sel_set_score(moe_sel_ctx* ctx, moe_sel_score kind) {
  g_last_error.clear();
  if (!ctx) return fail(MOE_SEL_EINVAL, "ctx is null");
  if (kind != MOE_SEL_SCORE_FULL && kind != MOE_SEL_SCORE_GATE_ONLY && kind != MOE_SEL_SCORE_NO_DOWN_NORM &&
      kind != MOE_SEL_SCORE_X_INT16)
    return fail(MOE_SEL_EINVAL, "unknown score kind");
  ctx->score_kind = kind;
  return MOE_SEL_OK;
}

moe_sel_status moe_sel_get_config(const moe_sel_ctx* ctx, moe_sel_config* cfg) {
  if (!ctx || !cfg) return fail(MOE_SEL_EINVAL, "ctx and cfg must be non-null");
  *cfg = ctx->cfg;
  return MOE_SEL_OK;
}

uint64_t moe_sel_device_bytes(const moe_sel_ctx* ctx) { return ctx ? ctx->device_bytes : 0; }

void moe_sel_destroy(moe_sel_ctx* ctx) { free_ctx(ctx); }

moe_sel_status moe_sel_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t batch, int32_t d,
                                     int32_t n_experts, float* logits, void* stream) {
  g_last_error.clear();
  if (!x || !w_router || !logits) return fail(MOE_SEL_EINVAL, "x, w_router and logits must be non-null");
  if (!aligned16(x) || !aligned16(w_router) || ((uintptr_t)logits & 3u))
    return fail(MOE_SEL_EINVAL, "x and w_router must be 16-byte aligned, logits 4-byte aligned");
  if (batch < 1 || batch > 65535) return fail(MOE_SEL_EINVAL, "batch must be in [1, 65535]");
  if (d < 64 || d > 16384 || d % 64) return fail(MOE_SEL_EINVAL, "d must be a multiple of 64 in [64, 16384]");
  if (n_experts < 1 || n_experts > 1024) return fail(MOE_SEL_EINVAL, "n_experts must be in [1, 1024]");
  const hipError_t e = moe_sel::launch_router(x, w_router, batch, d, n_experts, logits, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SEL_OK : hip_fail(e, "kernel launch");
}

moe_sel_status moe_sel_residual_rmsnorm(const uint16_t* x, const uint16_t* y, int32_t batch, int32_t d, float eps,
                                        uint16_t* out, void* stream) {
  g_last_error.clear();
  if (!x || !y || !out) return fail(MOE_SEL_EINVAL, "x, y and out must be non-null");
  if (!aligned16(x) || !aligned16(y) || !aligned16(out))
    return fail(MOE_SEL_EINVAL, "x, y and out must be 16-byte aligned");
  if (batch < 1 || batch > 65535) return fail(MOE_SEL_EINVAL, "batch must be in [1, 65535]");
  if (d < 64 || d > 16384 || d % 64) return fail(MOE_SEL_EINVAL, "d must be a multiple of 64 in [64, 16384]");
  if (!(eps > 0.0f) || !(eps < 1.0f)) return fail(MOE_SEL_EINVAL, "eps must be in (0, 1)");
  const hipError_t e = moe_sel::launch_resnorm(x, y, batch, d, eps, out, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SEL_OK : hip_fail(e, "kernel launch");
}

moe_sel_status moe_sel_residual_rmsnorm_router(const uint16_t* x, const uint16_t* y, const uint16_t* w_router,
                                               int32_t batch, int32_t d, int32_t n_experts, float eps, uint16_t* x_out,
                                               float* logits, void* stream) {
  g_last_error.clear();
  if (!x || !y || !w_router || !x_out || !logits)
    return fail(MOE_SEL_EINVAL, "x, y, w_router, x_out and logits must be non-null");
  if (!aligned16(x) || !aligned16(y) || !aligned16(w_router) || !aligned16(x_out) || ((uintptr_t)logits & 3u))
    return fail(MOE_SEL_EINVAL, "x, y, w_router and x_out must be 16-byte aligned, logits 4-byte aligned");
  if (batch < 1 || batch > 65535) return fail(MOE_SEL_EINVAL, "batch must be in [1, 65535]");
  if (d < 64 || d > 4096 || d % 64) return fail(MOE_SEL_EINVAL, "d must be a multiple of 64 in [64, 4096]");
  if (n_experts < 1 || n_experts > 1024) return fail(MOE_SEL_EINVAL, "n_experts must be in [1, 1024]");
  if (!(eps > 0.0f) || !(eps < 1.0f)) return fail(MOE_SEL_EINVAL, "eps must be in (0, 1)");
  const size_t row = (size_t)batch * d * 2;
  auto overlap = [row](const void* p, const void* q) {
    return (const char*)p < (const char*)q + row && (const char*)q < (const char*)p + row;
  };
  if (overlap(x_out, x) || overlap(x_out, y)) return fail(MOE_SEL_EINVAL, "x_out must not overlap x or y");
  const hipError_t e =
      moe_sel::launch_resnorm_router(x, y, w_router, batch, d, n_experts, eps, x_out, logits, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SEL_OK : hip_fail(e, "kernel launch");
}

moe_sel_status moe_sel_debug_silu(const float* z, float* out, int64_t n, void* stream) {
  g_last_error.clear();
  if (n < 0) return fail(MOE_SEL_EINVAL, "n must be non-negative");
  if (n == 0) return MOE_SEL_OK;
  if (!z || !out) return fail(MOE_SEL_EINVAL, "z and out must be non-null");
  if (((uintptr_t)z & 3u) || ((uintptr_t)out & 3u)) return fail(MOE_SEL_EINVAL, "z and out must be 4-byte aligned");
  const hipError_t e = moe_sel::launch_debug_silu(z, out, n, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SEL_OK : hip_fail(e, "kernel launch");
}

moe_sel_status moe_sel_debug_score(const int32_t* dot_gate, const int32_t* dot_up, const int32_t* xexp,
                                   const float* stats, moe_sel_score kind, float* h_hat, float* score, int64_t n,
                                   void* stream) {
  g_last_error.clear();
  if (n < 0) return fail(MOE_SEL_EINVAL, "n must be non-negative");
  if (kind != MOE_SEL_SCORE_FULL && kind != MOE_SEL_SCORE_GATE_ONLY && kind != MOE_SEL_SCORE_NO_DOWN_NORM &&
      kind != MOE_SEL_SCORE_X_INT16)
    return fail(MOE_SEL_EINVAL, "unknown score kind");
  if (n == 0) return MOE_SEL_OK;
  if (!dot_gate || !dot_up || !xexp || !stats || !h_hat || !score)
    return fail(MOE_SEL_EINVAL, "every array must be non-null");
  if (!aligned16(stats)) return fail(MOE_SEL_EINVAL, "stats must be 16-byte aligned");
  const hipError_t e = moe_sel::launch_debug_score(dot_gate, dot_up, xexp, (const float4*)stats, (int)kind, h_hat,
                                                   score, n, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SEL_OK : hip_fail(e, "kernel launch");
}

moe_sel_status moe_sel_read_stream(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  g_last_error.clear();
  if (!buf || !sink) return fail(MOE_SEL_EINVAL, "buf and sink must be non-null");
  if (!aligned16(buf) || bytes % 16) return fail(MOE_SEL_EINVAL, "buf must be 16-byte aligned and bytes a multiple of 16");
  if (((uintptr_t)sink & 3u)) return fail(MOE_SEL_EINVAL, "sink must be 4-byte aligned");
  if (bytes == 0) return MOE_SEL_OK;
  const hipError_t e = moe_sel::launch_read_stream(buf, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? MOE_SEL_OK : hip_fail(e, "kernel launch");
}

moe_sel_status moe_sel_debug_fail_alloc(int32_t nth) {
  g_last_error.clear();
  if (nth < 0) return fail(MOE_SEL_EINVAL, "nth must be non-negative");
  moe_sel::arm_alloc_fault(nth);
  return MOE_SEL_OK;
}

}  // extern "C"
