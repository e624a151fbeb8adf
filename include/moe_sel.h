/*
 * moe_sel.h - C ABI of the routed-MoE block with sketch-based top-k channel
 * selection, for MI355X (gfx950).
 *
 * Method (pages cited by title and section):
 *  - "KAIST drops calibration from MoE decoding, speeds up blocks by up to 2.69x
 *    over vLLM", opening paragraph: decoding at small batch is bound by reading
 *    the routed experts' weights for every token.
 *  - same page, "The threshold promises a budget but does not keep it": inside an
 *    expert a selector predicts which intermediate channels matter for the token
 *    and only those channels' weights are read.
 *  - same page, "Top-k instead of a threshold": each token keeps its k
 *    highest-scoring channels; the read budget is fixed in advance and no
 *    calibration data is needed.
 *  - same page, "A reader built from weights alone": channels are filtered with a
 *    ternary sketch of the weights, and skipped channels are compensated by a
 *    low-rank map that is also built from the weights.
 *  - "Calibration-free top-k MoE selector saves tuning": the reader works from
 *    bf16 weights.
 *
 * Computation of one forward call, per token t and routed expert e (the pages
 * leave the formulas open; the readings used are stated here):
 *   routing   top_e experts with the largest fp32 logits (lower expert index on
 *             equal logits), gate weights = softmax over the chosen logits;
 *   quantise  x_q = round-half-even(x * 2^-s), s the smallest integer with
 *             max|x| * 2^-s <= 127 (int8, exact power-of-two scale);
 *   score     for every channel j: G_j = alpha_g[j] * (t_g[j] . x_q) * 2^s,
 *             U_j = alpha_u[j] * (t_u[j] . x_q) * 2^s (exact integer dots, one
 *             binary32 rounding each), h_hat_j = silu_pinned(G_j) * U_j,
 *             score_j = |h_hat_j| * ||W_down[:, j]||_2, all in binary32 without
 *             fused multiply-add (silu_pinned: Cody-Waite reduction with
 *             ln2 = 2839/4096 + remainder, degree-7 Taylor, z/(1+e^-z), cut at
 *             |z| > 87);
 *   select    S = the k channels with the largest score (lower index first on
 *             equal scores), exactly k per token and expert;
 *   expert    y_e = sum_{j in S} silu(g_j) u_j W_down[:, j] from the bf16 weights
 *             of the selected channels only (fp32 accumulation);
 *   compens.  y_e += P_e (Q_e^T h_hat restricted to the channels not in S), with
 *             P_e Q_e^T the best rank-r approximation of W_down (truncated SVD);
 *   combine   out_t = bf16( sum_e w_{t,e} y_e ).
 * Every token of a batch uses only its own channels; the batch never changes a
 * token's selection or output beyond fp32 summation order.
 *
 * Ownership and threading: the caller owns every buffer it passes. A context is
 * used from one stream at a time (its workspace is reused by every call);
 * different contexts are independent. No function throws; all report a status
 * and leave a thread-local message in moe_sel_last_error().
 */
#ifndef MOE_SEL_H_
#define MOE_SEL_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_SEL_ABI_VERSION 2

typedef struct moe_sel_ctx moe_sel_ctx;

typedef enum moe_sel_status {
  MOE_SEL_OK = 0,
  MOE_SEL_EINVAL = 1,        /* an argument is null, misaligned or out of range */
  MOE_SEL_EUNSUPPORTED = 2,  /* well-formed, but outside what this library implements */
  MOE_SEL_ENOMEM = 3,        /* a host or device allocation failed */
  MOE_SEL_EDEVICE = 4,       /* the HIP runtime reported an error */
  MOE_SEL_EIO = 5            /* a file could not be opened, read or written, or is not a saved layer */
} moe_sel_status;

/* Channel score used to rank a pair's channels (moe_sel_set_score). */
typedef enum moe_sel_score {
  MOE_SEL_SCORE_FULL = 0,          /* |silu(G) U| * ||down column|| (the default reading) */
  MOE_SEL_SCORE_GATE_ONLY = 1,     /* |silu(G)| * ||down column|| */
  MOE_SEL_SCORE_NO_DOWN_NORM = 2,  /* |silu(G) U| */
  MOE_SEL_SCORE_X_INT16 = 3        /* the full score, on int16 instead of int8 activations */
} moe_sel_score;

/* How a forward call is executed on the GPU (same selections either way; outputs
 * differ only in fp32 summation order). */
typedef enum moe_sel_path {
  MOE_SEL_PATH_AUTO = 0,          /* single launch when it fits, else the multi-kernel path */
  MOE_SEL_PATH_MULTI_KERNEL = 1,  /* one kernel per phase. Pairs are grouped by expert into tiles of up
                                     to 32 tokens, and every weight byte an expert needs is read once
                                     per tile (the union of the tile tokens' selections); at batch 1,
                                     and for sparse calls whose routed pairs are at most half the
                                     experts, every pair is a tile of its own */
  MOE_SEL_PATH_SINGLE_LAUNCH = 2  /* one fused kernel; EUNSUPPORTED when it cannot be used */
} moe_sel_path;

/* Shape of one MoE layer. */
typedef struct moe_sel_config {
  uint32_t struct_size;  /* must be sizeof(moe_sel_config) */
  int32_t d;             /* hidden size: multiple of 64, 64 .. 16384 */
  int32_t n_experts;     /* experts E: 1 .. 1024 */
  int32_t m;             /* intermediate channels per expert: multiple of 64, 64 .. 32768
                            (moe_sel_prepare supports m <= 16384: EUNSUPPORTED above) */
  int32_t rank;          /* compensation rank r: 0 .. min(d, m, 128) */
  int32_t max_top_e;     /* experts per token the layer was trained with: 1 .. min(E, 64) */
  int32_t max_batch;     /* largest batch a forward call may pass: 1 .. 4096 */
  double tern_ratio;     /* sketch threshold as a fraction of mean|w| (0.7); 0 < ratio < 1e3 */
} moe_sel_config;

/* Version of this ABI (MOE_SEL_ABI_VERSION of the library that was loaded). */
int32_t moe_sel_abi_version(void);

/* Human-readable name of a status code. Never null. */
const char* moe_sel_status_str(moe_sel_status status);

/* Detail of the last failure on the calling thread ("" if none). Never null. */
const char* moe_sel_last_error(void);

/*
 * Weight-only preparation of ONE expert, on the host, without any GPU.
 * "A reader built from weights alone" (ternary sketch + low-rank map).
 *
 * Inputs (host, bf16 bit patterns, row-major):
 *   w_gate, w_up  [m][d]  row j = intermediate channel j
 *   w_down        [d][m]  column j = channel j's output direction
 * Outputs (host, every pointer may be null to skip that output; P and Q are
 * only computed when either is requested):
 *   tern_gate, tern_up [m][d] int8 in {-1, 0, +1}: t = sign(w) where
 *       |w| > tern_ratio * mean_i |w_ji| (mean over the channel's d weights)
 *   alpha_gate, alpha_up [m] fp32: mean |w| over the kept entries (0 if none)
 *   down_norm [m] fp32: ||W_down[:, j]||_2
 *   nnz_gate, nnz_up [m] int32: kept entries per channel
 *   p_bf16 [rank][d], q_bf16 [m][rank] bf16 bits: P Q^T is the best rank-r
 *       approximation of W_down (the individual factors are not unique; only
 *       their product is specified)
 * Sums are exact and rounded once to double; the threshold, the mean and the
 * scale follow the order mean = S / d, delta = tern_ratio * mean,
 * alpha = (float)(S_kept / nnz), down_norm = (float)sqrt(S_sq).
 * Errors: EINVAL for a null config/weight pointer or an invalid config;
 * ENOMEM if host scratch cannot be allocated. Outputs are undefined on error.
 */
moe_sel_status moe_sel_prepare_expert_host(const moe_sel_config* cfg,
                                           const uint16_t* w_gate, const uint16_t* w_up,
                                           const uint16_t* w_down,
                                           int8_t* tern_gate, int8_t* tern_up,
                                           float* alpha_gate, float* alpha_up, float* down_norm,
                                           int32_t* nnz_gate, int32_t* nnz_up,
                                           uint16_t* p_bf16, uint16_t* q_bf16);

/*
 * Build a context for one MoE layer: per-expert sketches, channel statistics
 * and low-rank maps (as moe_sel_prepare_expert_host), the channel-major weight
 * layout, and a workspace for cfg->max_batch tokens, all in device memory of
 * the current HIP device. The sketches and statistics are computed on the
 * device from the channel-major rows, bit-identical to the host preparation
 * (exact per-binade integer sums, rounded once to double), or on host threads
 * when the environment variable MOE_SEL_SKETCH is "host". The low-rank maps are
 * computed on the device in fp64 for all experts at once (Gram matrices,
 * tridiagonalisation and projection on the GPU, the tridiagonal eigen-solves on
 * host threads), or on the host when MOE_SEL_LOWRANK is "host" (the same
 * eigen-solver).
 *   w_gate, w_up [E][m][d], w_down [E][d][m]: host bf16 bit patterns.
 *   stream: hipStream_t used for the uploads and the device work (null =
 *           default stream). The call synchronises it before returning, so the
 *           caller may free the inputs.
 *   out:    receives the new context (unchanged on error).
 * Errors: EINVAL (null pointer, invalid config), EUNSUPPORTED (m > 16384),
 * ENOMEM (host/device allocation), EDEVICE (HIP error). Nothing is leaked on
 * error.
 */
moe_sel_status moe_sel_prepare(const moe_sel_config* cfg,
                               const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                               void* stream, moe_sel_ctx** out);

/*
 * The block forward with top-k channel selection ("Top-k instead of a threshold"
 * and "A reader built from weights alone").
 *   x       [batch][d] bf16 bits, device, 16-byte aligned
 *   logits  [batch][E] fp32, device, 16-byte aligned (router output)
 *   batch   1 .. max_batch;  top_e 1 .. max_top_e;  k_budget 0 .. m
 *           (k_budget = 0 keeps no channel: the output is the compensation alone;
 *            k_budget = m reads every channel and reproduces the dense expert)
 *   out     [batch][d] bf16 bits, device, 16-byte aligned; overwritten (not
 *           accumulated), no residual added
 *   stream  hipStream_t (null = default stream). Asynchronous: x, logits and out
 *           must stay valid until the stream has passed the call.
 * Errors: EINVAL/EUNSUPPORTED are detected on the host before anything is
 * enqueued, and out is untouched; EDEVICE if a launch fails (out undefined).
 */
moe_sel_status moe_sel_forward(moe_sel_ctx* ctx, const uint16_t* x, const float* logits,
                               int32_t batch, int32_t top_e, int32_t k_budget,
                               uint16_t* out, void* stream);

/*
 * moe_sel_forward without any allocation, for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it). Same arguments, results and errors as moe_sel_forward on the
 * single-launch path (bit-identical outputs); its per-call scratch (hand-off
 * slots, the error word and the inspection arrays) is a fixed 7.5 MiB device
 * array that the library holds on each GPU until the process ends, not the
 * context's workspace. It enqueues one kernel and calls no allocating routine.
 *   Limits: only calls the single launch can run (see moe_sel_set_path), and
 *   at most 3 MiB each of gather hand-off and down-partial slots (the
 *   Qwen3-30B-A3B-shaped layer fits at batch 1); EUNSUPPORTED otherwise,
 *   before anything is enqueued.
 *   Every call on a GPU shares that GPU's array: calls that overlap in time on
 *   one GPU (other streams, other threads) race and must not be issued. A
 *   wait that gives up poisons later calls of this entry point on the GPU, for
 *   every context, until moe_sel_check_device on a context of that GPU.
 *   moe_sel_debug_selection does not see these calls.
 */
moe_sel_status moe_sel_forward_noalloc(moe_sel_ctx* ctx, const uint16_t* x, const float* logits,
                                       int32_t batch, int32_t top_e, int32_t k_budget,
                                       uint16_t* out, void* stream);

/*
 * The threshold selector the pages contrast with top-k ("KAIST drops
 * calibration from MoE decoding...", section "The threshold promises a budget
 * but does not keep it"): each routed pair keeps every channel whose score
 * (the same score as moe_sel_forward) is strictly above `threshold`, so the
 * number of channels read varies from token to token. Everything else (scores,
 * compensation of the skipped channels, combine) is as in moe_sel_forward.
 * Runs on the multi-kernel path. moe_sel_debug_selection afterwards returns
 * rows of m channel indices of which the first chan_count are valid.
 *   threshold  finite, >= 0 (scores are non-negative)
 * Other arguments and errors as moe_sel_forward.
 */
moe_sel_status moe_sel_forward_threshold(moe_sel_ctx* ctx, const uint16_t* x, const float* logits,
                                         int32_t batch, int32_t top_e, float threshold,
                                         uint16_t* out, void* stream);

/*
 * The dense routed block on the same layout (every channel of every routed
 * expert is read, no sketch and no compensation): the baseline the selective
 * block is measured against. Arguments and errors as moe_sel_forward.
 */
moe_sel_status moe_sel_forward_dense(moe_sel_ctx* ctx, const uint16_t* x, const float* logits,
                                     int32_t batch, int32_t top_e, uint16_t* out, void* stream);

/*
 * Routing and selection of the last moe_sel_forward on this context, copied to
 * host buffers (synchronises that call's stream). Sizes use the last call's
 * batch B, top_e and k; every pointer may be null.
 *   expert_ids [B][top_e] int32 (best first), gate_w [B][top_e] fp32,
 *   chan_idx [B][top_e][k] int32 ascending, chan_count [B][top_e] int32,
 *   h_hat [B][top_e][m] fp32, score [B][top_e][m] fp32.
 * Errors: EINVAL if ctx is null or no sparse forward has run; EDEVICE.
 */
moe_sel_status moe_sel_debug_selection(moe_sel_ctx* ctx, int32_t* expert_ids, float* gate_w,
                                       int32_t* chan_idx, int32_t* chan_count,
                                       float* h_hat, float* score);

/*
 * Read back what moe_sel_prepare stored for one expert (synchronous, host
 * buffers, same layouts and nullability as moe_sel_prepare_expert_host): the
 * ternary sketch ("A reader built from weights alone") with its kept-entry
 * counts nnz_gate / nnz_up [m] (counted from the stored codes), the channel
 * statistics and the rank-r maps.
 * Errors: EINVAL (null ctx, expert out of range), ENOMEM, EDEVICE.
 */
moe_sel_status moe_sel_export_expert(moe_sel_ctx* ctx, int32_t expert,
                                     int8_t* tern_gate, int8_t* tern_up,
                                     float* alpha_gate, float* alpha_up, float* down_norm,
                                     int32_t* nnz_gate, int32_t* nnz_up,
                                     uint16_t* p_bf16, uint16_t* q_bf16);

/*
 * Synchronise the device and report whether any enqueued call on this context
 * hit a bounded cross-workgroup wait that gave up (single-launch path). Such a
 * call writes NaN to the outputs of the tokens it could not finish, and from
 * then on every single-launch call on the context writes NaN to all of its
 * outputs (a producer that was waited for may still store into the context's
 * hand-off slots), until this function clears the error and resets the
 * hand-off state. Callers that run many forward calls back to back (a timed
 * region, a captured graph) should call it after them.
 * Errors: EINVAL (null ctx), EDEVICE (a wait gave up, or a HIP error).
 */
moe_sel_status moe_sel_check_device(moe_sel_ctx* ctx);

/*
 * Polls a cross-workgroup wait of the single-launch path makes before it gives
 * up (default 2^21, about a second). polls = 0 makes every wait give up at
 * once, so that the failure handling can be tested with every kernel still
 * finishing normally. Errors: EINVAL (null ctx, polls outside [0, 2^30]).
 */
moe_sel_status moe_sel_set_wait_limit(moe_sel_ctx* ctx, int32_t polls);

/*
 * Choose the execution path of later forward calls on this context (default
 * MOE_SEL_PATH_AUTO). The single-launch path needs d <= 4096, m <= 4096,
 * top_e * rank <= 256, rank dividing 256 and a multiple of 8, batch <= 8, and
 * every workgroup of its grid resident at once (the grid grows with batch *
 * top_e; the occupancy query decides). For the Qwen3-30B-A3B shape (d = 2048,
 * 128 experts, top-8, m = 768, r = 32) on a 256-CU MI355X that holds for batch
 * <= 2 (768 workgroups fit at three per CU; at k = 138 batch 1 takes 408 and
 * batch 2 takes 624 with 64-channel score blocks, batch 3 would take 936).
 * Larger batches run the multi-kernel path, and a forced single launch there
 * fails with EUNSUPPORTED.
 * Errors: EINVAL (null ctx or unknown path).
 */
moe_sel_status moe_sel_set_path(moe_sel_ctx* ctx, moe_sel_path path);

/*
 * Channel score used by later forward calls on this context (default
 * MOE_SEL_SCORE_FULL). The pages leave the score open ("KAIST drops calibration
 * from MoE decoding...", section "A reader built from weights alone": channels
 * are filtered with a ternary sketch); the alternatives are ablations of the
 * default reading. For the first three only the ranking changes: the sketch
 * activations used by the compensation are the same for them.
 *   MOE_SEL_SCORE_FULL          |silu(G) * U| * ||W_down[:, j]||_2
 *   MOE_SEL_SCORE_GATE_ONLY     |silu(G)| * ||W_down[:, j]||_2 (up sketch ignored)
 *   MOE_SEL_SCORE_NO_DOWN_NORM  |silu(G) * U|
 *   MOE_SEL_SCORE_X_INT16       the full score with G and U from int16
 *                               activations: q = rint(x 2^-e), max|q| <= 32767
 *                               (h_hat changes with it). Runs on the single
 *                               launch and on multi-kernel calls with one pair
 *                               per tile whose score blocks route themselves
 *                               (n_experts <= 256); other calls fail with
 *                               EUNSUPPORTED.
 * Errors: EINVAL (null ctx or unknown kind).
 */
moe_sel_status moe_sel_set_score(moe_sel_ctx* ctx, moe_sel_score kind);

/* Path taken by the last forward call on this context (MOE_SEL_PATH_MULTI_KERNEL
 * or MOE_SEL_PATH_SINGLE_LAUNCH), or -1 if none ran yet or ctx is null. */
int32_t moe_sel_last_path(const moe_sel_ctx* ctx);

/* Shape the context was prepared with (copied into *cfg). EINVAL on null. */
moe_sel_status moe_sel_get_config(const moe_sel_ctx* ctx, moe_sel_config* cfg);

/* Device bytes owned by the context (weights, sketch, maps and workspace). */
uint64_t moe_sel_device_bytes(const moe_sel_ctx* ctx);

/*
 * Write the prepared layer of ctx to a file: its shape (the config) and the
 * arrays moe_sel_prepare built from the weights alone (page "KAIST drops
 * calibration from MoE decoding, speeds up blocks by up to 2.69x over vLLM",
 * section "A reader built from weights alone"): the 2-bit sketch codes, the
 * per-channel statistics, the channel-major bf16 weights and the rank-r maps,
 * in their device layouts, followed by a 64-bit FNV-1a hash of the arrays. The
 * forward workspace is not saved. An existing file is replaced.
 *   path: file name (host string).
 * Synchronous (copies the arrays from the device). Errors: EINVAL (null
 * argument), EIO (the file cannot be written), ENOMEM, EDEVICE.
 */
moe_sel_status moe_sel_save(const moe_sel_ctx* ctx, const char* path);

/*
 * Build a context on the current HIP device from a file written by
 * moe_sel_save, without preparing again: forward calls on it give the same
 * results as on the context that was saved (its path and score settings start
 * at their defaults).
 *   stream: hipStream_t used for the uploads (null = default stream); the call
 *           synchronises it before returning.
 *   out:    receives the new context (unchanged on error).
 * Errors: EINVAL (null argument), EIO (the file cannot be opened, is not a
 * saved layer, is truncated, has trailing bytes or fails its hash check),
 * EUNSUPPORTED (m > 16384), ENOMEM, EDEVICE. Nothing is leaked on error.
 */
moe_sel_status moe_sel_load(const char* path, void* stream, moe_sel_ctx** out);

/* Release a context and all its device memory. Null is a no-op. The caller
 * must make sure no enqueued call on it is still running. */
void moe_sel_destroy(moe_sel_ctx* ctx);

/*
 * Decode-step glue for stacking blocks over layers. The pages measure MoE
 * blocks inside decoding ("KAIST drops calibration from MoE decoding, speeds
 * up blocks by up to 2.69x over vLLM", opening paragraph); these two calls
 * chain blocks into a many-layer decode step with a router per layer and the
 * residual stream renormalised between layers; the third does both at once.
 *
 * moe_sel_router_logits: logits[t][e] = sum_i x[t][i] * w_router[e][i], fp32
 * accumulation of the bf16 products.
 *   x        [batch][d] bf16 bits, device, 16-byte aligned
 *   w_router [n_experts][d] bf16 bits, device, 16-byte aligned (caller-owned)
 *   logits   [batch][n_experts] fp32, device, written
 *   batch 1..65535, d a multiple of 64 in [64, 16384], n_experts 1..1024.
 * Asynchronous on stream. Errors: EINVAL (checked before enqueueing), EDEVICE.
 */
moe_sel_status moe_sel_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t batch, int32_t d,
                                     int32_t n_experts, float* logits, void* stream);

/*
 * moe_sel_residual_rmsnorm: out[t] = bf16(v / sqrt(mean_i v_i^2 + eps)) with
 * v = x[t] + y[t] in fp32 (round to nearest even into bf16). out may alias x.
 *   x, y, out [batch][d] bf16 bits, device, 16-byte aligned
 *   batch 1..65535, d a multiple of 64 in [64, 16384], eps in (0, 1).
 * Asynchronous on stream. Errors: EINVAL (checked before enqueueing), EDEVICE.
 */
moe_sel_status moe_sel_residual_rmsnorm(const uint16_t* x, const uint16_t* y, int32_t batch, int32_t d, float eps,
                                        uint16_t* out, void* stream);

/*
 * moe_sel_residual_rmsnorm_router: both calls above in one launch, for the step
 * from one layer to the next: x_out = the renormalised residual stream (as
 * moe_sel_residual_rmsnorm, the mean square summed in another order, so an
 * element may differ by one bf16 step) and logits = the next layer's router
 * applied to x_out (as moe_sel_router_logits).
 *   x, y      [batch][d] bf16 bits, device, 16-byte aligned
 *   w_router  [n_experts][d] bf16 bits, device, 16-byte aligned (caller-owned)
 *   x_out     [batch][d] bf16 bits, device, 16-byte aligned; must not overlap x or y
 *   logits    [batch][n_experts] fp32, device, written
 *   batch 1..65535, d a multiple of 64 in [64, 4096], n_experts 1..1024, eps in (0, 1).
 * Asynchronous on stream. Errors: EINVAL (checked before enqueueing), EDEVICE.
 */
moe_sel_status moe_sel_residual_rmsnorm_router(const uint16_t* x, const uint16_t* y, const uint16_t* w_router,
                                               int32_t batch, int32_t d, int32_t n_experts, float eps,
                                               uint16_t* x_out, float* logits, void* stream);

/*
 * Inspection and measurement entry points.
 *
 * moe_sel_debug_silu: out[i] = silu_pinned(z[i]), the binary32 silu inside the
 * channel score (the score formula at the top of this header), evaluated by
 * the same device function the forward kernels use, so a test can compare it
 * bit for bit with another implementation.
 *   z, out  [n] fp32, device, 4-byte aligned; n >= 0.
 * moe_sel_debug_score: the pinned score of n channels from given exact
 * integer sketch dots: G = alpha_g * dot_gate * 2^xexp, U = alpha_u * dot_up *
 * 2^xexp, h_hat = silu_pinned(G) * U, score per `kind` (moe_sel_set_score).
 *   dot_gate, dot_up, xexp [n] int32; stats [n][4] fp32 {alpha_g, alpha_u,
 *   ||down column||, unused}, 16-byte aligned; h_hat, score [n] fp32; device.
 * moe_sel_read_stream: reads every byte of buf once with 16-byte loads and
 * folds them into *sink (device), so that timing it gives the device's
 * measured HBM read bandwidth, the ceiling the forward's bytes are set against.
 *   buf device, 16-byte aligned; bytes a multiple of 16.
 * All three are asynchronous on stream. Errors: EINVAL (checked before
 * enqueueing), EDEVICE.
 */
moe_sel_status moe_sel_debug_silu(const float* z, float* out, int64_t n, void* stream);
moe_sel_status moe_sel_debug_score(const int32_t* dot_gate, const int32_t* dot_up, const int32_t* xexp,
                                   const float* stats, moe_sel_score kind, float* h_hat, float* score,
                                   int64_t n, void* stream);
moe_sel_status moe_sel_read_stream(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

/*
 * Allocation fault injection, for tests of the out-of-memory paths: with
 * nth >= 1, the nth host or device allocation this library attempts from now
 * on (in any thread) fails as if memory were exhausted, and the injector
 * disarms; nth = 0 disarms it. The entry point that hits it returns
 * MOE_SEL_ENOMEM and frees everything it had allocated.
 * Errors: EINVAL (nth < 0).
 */
moe_sel_status moe_sel_debug_fail_alloc(int32_t nth);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SEL_H_ */
