/*
 * lora_mi355x.h -- C ABI of the MI355X (gfx950) multi-adapter LoRA library.
 *
 * The library applies, for every token t of a mixed batch and one linear
 * module m,
 *
 *     y[t,:] += s_k * (x[t,:] . A_k) . B_k          with k = token_slot_idx[t]
 *
 * where slot k holds an adapter of rank r_k <= max_rank and
 * s_k = lora_alpha / r_k, or lora_alpha / sqrt(r_k) with rsLoRA.  Those adapter
 * fields (r, lora_alpha, use_rslora, target_modules) are the ones of the
 * example PEFT adapter_config.json in "vLLM LoRA Resolver plugins explained"
 * (blog.gitcode.com), section 3.2 "directory structure requirements".  The
 * slot count and the padded rank are vLLM's max_loras and max_lora_rank of the
 * parameter table in "Multi-LoRA adapter cache in production" (oh-bug.com),
 * section "GPU, CPU and disk form the adapter storage hierarchy"; max_loras
 * bounds the adapters one batch may use, not the adapters a server knows.
 *
 * Conventions shared by every call:
 *  - Every call returns an int status (LORA_OK or a negative LORA_ERR_*).  No
 *    call aborts or throws across the ABI.  All argument checks run on the
 *    host before anything is enqueued, so an error has no partial effect.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).  A
 *    stream the ctx has launched on must stay valid until lora_slots_destroy:
 *    later loads record events on it and query it.
 *  - x, y and token_slot_idx are device pointers owned by the caller, who
 *    keeps them alive until the stream has passed the call.
 *  - A lora_ctx is used from one host thread at a time.  Calls that launch
 *    kernels for one ctx (lora_plan_prepare, lora_shrink, lora_expand,
 *    lora_apply) share the ctx's plan and intermediate buffers, so they must be
 *    issued on one stream, or ordered by the caller.
 *  - Element type of x, y, A and B is the ctx dtype: bf16 (raw 16-bit
 *    patterns) or fp32.  Accumulation is fp32 (for fp32 data, the sums over
 *    d_in run in fp64, so large scales keep ~1e-5 relative); a bf16 y is rounded once,
 *    to nearest even.
 *  - Graph capture: the launching calls may be captured into a HIP graph
 *    (hipStreamBeginCapture on a non-null stream) and the graph replayed.
 *    Each launch takes the slot metadata (rank, scale, target modules) by
 *    value when it is enqueued, so a replay uses the metadata as of the
 *    capture and the adapter weights as they are at the replay.  Loads must be
 *    complete before the capture starts (lora_sync_loads), else the first
 *    captured launch fails with LORA_ERR_INVALID_ARGUMENT.  Launches under
 *    capture are never timed (lora_profile_begin).  No load or clear may be
 *    issued while a capture is open.
 *    The library does not see replays, so it cannot order loads against them:
 *    the caller must (1) make sure no replay that reads a slot is in flight
 *    when it loads into that slot (e.g. synchronise the replaying stream
 *    first), and (2) call lora_sync_loads after the load and before a replay
 *    that must see the new weights.  Under those two rules a slot reloaded
 *    with an adapter of the same rank, lora_alpha and target modules is seen
 *    by later replays; any other load or clear needs a new capture.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lora_ctx lora_ctx;

typedef enum { LORA_BF16 = 0, LORA_FP32 = 1 } lora_dtype;

typedef struct {
    int32_t d_in;   /* input features of the linear (x row length), multiple of 8 */
    int32_t d_out;  /* output features (y row length), multiple of 8 */
} lora_module_shape;

enum {
    LORA_OK = 0,
    LORA_ERR_INVALID_ARGUMENT = -1,
    LORA_ERR_RANK_EXCEEDS_MAX = -2,   /* r > max_rank ("LoRA rank exceeds maximum",
                                         "vLLM LoRA Resolver plugins explained", 6.1) */
    LORA_ERR_SLOT_OUT_OF_RANGE = -3,
    LORA_ERR_BAD_MODULE = -4,
    LORA_ERR_TOO_MANY_TOKENS = -5,
    LORA_ERR_HOST_NOT_PINNED = -6,
    LORA_ERR_OUT_OF_MEMORY = -7,
    LORA_ERR_HIP = -8,
    LORA_ERR_NO_PLAN = -9
};

/* Library limits. */
#define LORA_MAX_SLOTS 256   /* max_loras */
#define LORA_MAX_RANK 128    /* max_rank */
#define LORA_MAX_GROUP 8     /* modules of one grouped shrink / expand / apply call */

/* Sticky device-side flags, read with lora_get_device_flags. */
#define LORA_FLAG_SLOT_INDEX_TOO_LARGE 0x1u  /* a token carried idx >= max_loras (skipped) */
#define LORA_FLAG_FUSED_TIMEOUT 0x2u         /* a fused decode launch gave up waiting for a
                                                tile's partials (its rows were left untouched) */

typedef struct {
    int64_t loads;          /* lora_slot_load calls that succeeded */
    int64_t clears;         /* lora_slot_clear calls that succeeded */
    int64_t bytes_loaded;   /* sum over loads of sum_m (d_in + d_out) * r * bytes_per_elem */
    int64_t plans;          /* plan kernels launched */
    int64_t shrinks;        /* lora_shrink launches (including those inside lora_apply) */
    int64_t expands;        /* lora_expand launches (including those inside lora_apply) */
    int64_t tokens;         /* sum of n_tokens over planned batches */
} lora_stats;

/*
 * Create a slot pool on `device`.  The two sizes are vLLM's max_loras (the
 * adapters one batch may use) and max_lora_rank (the largest rank served, to
 * which every slot is padded) of the parameter table in "Multi-LoRA adapter
 * cache in production" (oh-bug.com), section "GPU, CPU and disk form the
 * adapter storage hierarchy".
 *   max_loras   slots, 1..LORA_MAX_SLOTS
 *   max_rank    padded rank of every slot, 1..LORA_MAX_RANK
 *   modules     n_modules shapes; a module index in later calls refers to this array
 *   dtype       element type of x, y and the adapter weights: a lora_dtype value
 *               (LORA_BF16 or LORA_FP32), passed as int32_t so that any other
 *               value is rejected rather than read as an enum
 *   max_tokens  largest n_tokens of a batch, >= 1
 * Allocates and zeroes, per module, A^T storage [max_loras][R][d_in] and B
 * storage for [max_loras][R][d_out] (R = max_rank rounded up to 16), an fp32
 * intermediate, plan buffers, and a side stream for loads (the memory is
 * zeroed on that stream, which the call waits for; no device-wide
 * synchronisation).  Every slot starts empty.  On success *out owns all of it
 * until lora_slots_destroy.
 * Errors: sizes out of range or d_in / d_out not a positive multiple of 8 ->
 * LORA_ERR_INVALID_ARGUMENT (max_rank > LORA_MAX_RANK ->
 * LORA_ERR_RANK_EXCEEDS_MAX); allocation failure -> LORA_ERR_OUT_OF_MEMORY,
 * with nothing left allocated; *out is NULL on every error.
 */
int lora_slots_create(lora_ctx **out, int32_t max_loras, int32_t max_rank,
                      const lora_module_shape *modules, int32_t n_modules,
                      int32_t dtype, int32_t max_tokens, int32_t device);

/* Wait for the streams the ctx has launched on and for its side stream (not
 * for the whole device), then free everything it owns.  NULL is accepted. */
int lora_slots_destroy(lora_ctx *ctx);

/*
 * Load one adapter into `slot` (the CPU-to-GPU upload of a "CPU hit",
 * "Multi-LoRA adapter cache in production", section on cold-load tiers).
 *   A_t[m]   r x d_in_m, row-major (A transposed: row j is rank j), or NULL when
 *            module m is not in the adapter's target_modules
 *   B[m]     r x d_out_m, row-major, NULL exactly when A_t[m] is NULL
 *            Both must be pinned host memory or device memory, and must stay
 *            unmodified until lora_sync_loads returns (or a later call on a
 *            stream that waited for the load has completed).
 *   r        adapter rank, 1..max_rank (r > max_rank -> LORA_ERR_RANK_EXCEEDS_MAX)
 *   lora_alpha, use_rslora   give s = lora_alpha / r or lora_alpha / sqrt(r),
 *            computed in double and rounded to fp32 once
 * Asynchronous, on the ctx's side stream: a kernel reads the weights in place
 * where the device can (16-byte aligned pinned host memory mapped at its host
 * address, over the link; memory of the ctx's device; managed memory) and
 * writes the slot; other weights are first copied to a stage buffer.  The same
 * holds for the output terms of lora_slot_load_ex.  Before
 * overwriting the slot the side stream waits for every kernel already enqueued
 * by this ctx, so
 * an adapter in use by an in-flight batch is never overwritten ("an adapter in
 * use must not be evicted", same page, data-plane section).  Later
 * lora_plan_prepare / lora_shrink / lora_expand / lora_apply calls make their
 * stream wait for the load.  Rows r..R-1 are zeroed, so padding changes nothing.
 * A load while a stream this ctx has launched on is under graph capture fails
 * with LORA_ERR_INVALID_ARGUMENT (its fences would join the capture).
 * The bytes moved are sum_m (d_in_m + d_out_m) * r * bytes_per_elem over the
 * targeted modules, the page's adapter size estimate.
 */
int lora_slot_load(lora_ctx *ctx, int32_t slot, const void *const *A_t, const void *const *B,
                   int32_t r, double lora_alpha, int32_t use_rslora);

/*
 * lora_slot_load with the two per-adapter output terms of the "bias" and
 * "use_dora" fields of the example adapter_config.json ("vLLM LoRA Resolver
 * plugins explained", section 3.2; off in that example).  For a token of this
 * slot the update of module m becomes
 *
 *     y[t,n] = round( g_m[n] * ( y[t,n] + s * (x[t,:] . A) . B[:,n] ) + c_m[n] )
 *
 *   bias        NULL (c = 0), or [n_modules] pointers: c_m, d_out_m values of
 *               the ctx dtype, non-NULL for every targeted module.  The bias is
 *               added as given: a bias trained with the adapter enters as its
 *               difference to the base bias, a bias of lora_B scaled by s.
 *   dora_scale  NULL (g = 1), or [n_modules] pointers: g_m, d_out_m floats,
 *               non-NULL for every targeted module: DoRA's factor
 *               m[n] / ||W0 + s B^T A||_n per output feature ("DoRA:
 *               Weight-Decomposed Low-Rank Adaptation", Liu et al. 2024), which
 *               the caller forms from the base weight W0.  With DoRA, y must be
 *               the base product x W0^T without the base bias.
 * Same memory rules, ordering and errors as lora_slot_load; a NULL entry for a
 * targeted module -> LORA_ERR_INVALID_ARGUMENT.  The extra bytes are not part of
 * the page's size estimate and are not counted in bytes_loaded.
 */
int lora_slot_load_ex(lora_ctx *ctx, int32_t slot, const void *const *A_t, const void *const *B,
                      const void *const *bias, const float *const *dora_scale, int32_t r,
                      double lora_alpha, int32_t use_rslora);

/*
 * Give the adapter in `slot` a whole trained copy of one module, the
 * "modules_to_save" field of the example adapter_config.json in "vLLM LoRA
 * Resolver plugins explained", section 3.2 (null in that example).  For every
 * token of the slot, the launches of that module then write
 *
 *     y[t,n] = round( sum_i x[t,i] * W[n,i] + bias[n] )
 *
 * in place of the base output the caller put in y (the copy takes the base
 * module's place).  Tokens of other slots are untouched.
 *   module  the module index; the adapter in the slot must not target it with
 *           its low-rank update (a module is either targeted or saved), else
 *           LORA_ERR_INVALID_ARGUMENT
 *   W       d_out x d_in, row-major (a linear layer's weight: row n is output
 *           feature n), ctx dtype, pinned host or device memory
 *   bias    d_out values of the ctx dtype, or NULL for none
 * The slot must hold an adapter (lora_slot_load first), else
 * LORA_ERR_INVALID_ARGUMENT; a later lora_slot_load or lora_slot_clear of the
 * slot drops its saved modules.  Storage: the first saved load of a module
 * allocates that module's pool for every slot (max_loras x d_out x (d_in + 1)
 * elements; LORA_ERR_OUT_OF_MEMORY on failure).  The copy runs on the side
 * stream with the ordering, memory rules and capture rule of lora_slot_load.
 * lora_expand (and lora_apply) run the product after the low-rank update of
 * the same call, reading the x given to the matching lora_shrink, which must
 * therefore stay valid until the stream has passed the lora_expand.
 */
int lora_slot_load_saved(lora_ctx *ctx, int32_t slot, int32_t module, const void *W,
                         const void *bias);

/* Mark `slot` empty for every module.  Batches enqueued after this call skip
 * the slot; batches already enqueued still apply the adapter it held.  Host-only:
 * no device work is enqueued. */
int lora_slot_clear(lora_ctx *ctx, int32_t slot);

/* Host waits until every load issued so far has completed; launches after it
 * need not wait for those loads on the device (required before a graph
 * capture). */
int lora_sync_loads(lora_ctx *ctx);

/*
 * Group the batch's tokens by slot on the device (no host synchronisation).
 * token_slot_idx is the per-request adapter choice of a mixed batch, each
 * value a slot of the pool: max_loras bounds how many adapters one batch may
 * use ("Multi-LoRA adapter cache in production", parameter table and section
 * "common misconceptions", item 1).  The grouping is
 * a stable counting sort of token_slot_idx (int32[n_tokens], device) into a
 * permutation, per-slot segments and tiles of up to 64 tokens.  Tokens with
 * idx < 0 are not listed; idx >= max_loras are not listed and set
 * LORA_FLAG_SLOT_INDEX_TOO_LARGE.  For bf16 batches of at most 1024 tokens the
 * grouping runs inside each lora_shrink launch instead of a launch of its own,
 * with tiles of up to 32 tokens (max_rank up to 16) or 48 (above).
 * The plan stays valid for lora_shrink,
 * lora_expand and lora_apply calls with the same (token_slot_idx, n_tokens)
 * until the next lora_plan_prepare; the caller must not change the contents of
 * token_slot_idx meanwhile.  n_tokens == 0 is allowed.
 */
int lora_plan_prepare(lora_ctx *ctx, const int32_t *token_slot_idx, int32_t n_tokens,
                      void *stream);

/*
 * lora_plan_prepare, and a declaration of the slots the batch reads:
 * used_slots is a host array of n_used slot indices (0..max_loras-1; repeats
 * allowed).  The launches of this plan treat every other slot as empty (its
 * tokens leave y untouched), so they read only the listed slots.  The library
 * then records, per listed slot, an event after each lora_expand of the plan,
 * and a later lora_slot_load into a slot waits only for the last such event of
 * that slot instead of for every launch issued since the previous load.  A
 * load into a slot that the batches in flight do not read therefore overlaps
 * them: the next step's misses can be uploaded while this step computes.  The
 * rule kept is that of "Multi-LoRA adapter cache in production" (oh-bug.com),
 * section "GPU, CPU and disk form the adapter storage hierarchy": an adapter
 * that in-flight work uses is never overwritten; the upload of a CPU hit is
 * the H2D tier of the same section.
 * Errors: a used_slots entry out of range -> LORA_ERR_SLOT_OUT_OF_RANGE;
 * used_slots NULL with n_used > 0, or n_used < 0 -> LORA_ERR_INVALID_ARGUMENT.
 * Under graph capture the declaration still limits the slots read, and loads
 * fall back to waiting for every launch on the capturing stream.
 */
int lora_plan_prepare_slots(lora_ctx *ctx, const int32_t *token_slot_idx, int32_t n_tokens,
                            const int32_t *used_slots, int32_t n_used, void *stream);

/*
 * lora_shrink: h = x . A_k for every planned token (fp32 intermediate of rank
 * R, held in the ctx), the first factor of the update with A of shape
 * d_in x r as the adapter size estimate of "Multi-LoRA adapter cache in
 * production" (section "adapter capacity cannot be planned by count alone")
 * implies; r is the "r" of the adapter_config.json in "vLLM LoRA Resolver
 * plugins explained", section 3.2.  x is [n_tokens][d_in] (row-major, device,
 * ctx dtype) of the prepared plan.  Requires a prepared plan (else
 * LORA_ERR_NO_PLAN); a bad module -> LORA_ERR_BAD_MODULE; x NULL with
 * n_tokens > 0 -> LORA_ERR_INVALID_ARGUMENT.
 */
int lora_shrink(lora_ctx *ctx, const void *x, int32_t module, void *stream);

/*
 * lora_expand: y[t,:] = round(y[t,:] + s_k * h[t,:] . B_k) for every planned
 * token whose slot holds an adapter targeting `module` (its "target_modules",
 * with s_k from "lora_alpha", "r" and "use_rslora" of the adapter_config.json
 * in "vLLM LoRA Resolver plugins explained", section 3.2; B is r x d_out as
 * in the size estimate of "Multi-LoRA adapter cache in production"); every
 * other row of y is left bit-identical.  Must follow lora_shrink of the same
 * module on the same plan, with no lora_slot_load or lora_slot_clear in
 * between (else LORA_ERR_INVALID_ARGUMENT).  y is [n_tokens][d_out]
 * (row-major, device, ctx dtype), read and written in place.
 */
int lora_expand(lora_ctx *ctx, void *y, int32_t module, void *stream);

/*
 * One module's update in one call: plan (unless lora_plan_prepare was called
 * for the same token_slot_idx and n_tokens), shrink, expand.  The update is
 * the one the adapter fields "r", "lora_alpha", "use_rslora" and
 * "target_modules" of the example adapter_config.json in "vLLM LoRA Resolver
 * plugins explained", section 3.2, describe, for slots of the pool sized by
 * max_loras / max_lora_rank ("Multi-LoRA adapter cache in production",
 * parameter table).  x: [n_tokens][d_in], y: [n_tokens][d_out] (read and
 * written in place), token_slot_idx: int32[n_tokens], all device memory owned
 * by the caller.  Tokens with
 * idx == -1 (base model only), any other negative idx, idx >= max_loras, an
 * empty slot, or a slot whose adapter does not target `module` leave their row
 * of y bit-identical.  n_tokens == 0 is a no-op; n_tokens > max_tokens returns
 * LORA_ERR_TOO_MANY_TOKENS.
 */
int lora_apply(lora_ctx *ctx, const void *x, void *y, const int32_t *token_slot_idx,
               int32_t n_tokens, int32_t module, void *stream);

/*
 * Grouped forms: the same operations for n (1..LORA_MAX_GROUP) modules of one
 * batch in one kernel launch per phase, e.g. the q, k and v projections of a
 * layer.  modules[i] is a module index, x[i] / y[i] that module's
 * [n_tokens][d_in] input and [n_tokens][d_out] output.  A module may appear more
 * than once (with its own x and y); the y buffers must not overlap (identical
 * pointers are rejected with LORA_ERR_INVALID_ARGUMENT).  lora_expand_group must
 * follow lora_shrink_group with the same module list.  Results equal n
 * single-module calls.
 */
int lora_shrink_group(lora_ctx *ctx, int32_t n, const int32_t *modules, const void *const *x,
                      void *stream);
int lora_expand_group(lora_ctx *ctx, int32_t n, const int32_t *modules, void *const *y,
                      void *stream);
int lora_apply_group(lora_ctx *ctx, int32_t n, const int32_t *modules, const void *const *x,
                     void *const *y, const int32_t *token_slot_idx, int32_t n_tokens,
                     void *stream);

/*
 * lora_apply_group with the shrink and the expand of a decode batch in one
 * launch (the two kernels of the update fused, h kept between workgroups of
 * one launch instead of between launches).  Applies to bf16 batches of at most
 * 1024 tokens on a device that deals the workgroups of a launch to its XCDs
 * in turn, so that workgroups whose indices agree mod 8 share an XCD (MI355X;
 * lora_slots_create checks this once per device); other batches, and
 * every batch elsewhere, take the two launches of lora_apply_group.  All
 * workgroups of a tile run on one XCD, and the expand workgroups wait for
 * their tile's K-split partials through per-(tile, module) counts in that
 * XCD's L2 that every launch returns to zero, so the call can be captured into
 * a graph and replayed.  The wait is bounded: if it ever gives
 * up, the rows it covers are left untouched and LORA_FLAG_FUSED_TIMEOUT is set.
 * Results equal lora_apply_group bit for bit.  Same arguments, ordering and
 * errors as lora_apply_group.
 */
int lora_apply_group_fused(lora_ctx *ctx, int32_t n, const int32_t *modules,
                           const void *const *x, void *const *y,
                           const int32_t *token_slot_idx, int32_t n_tokens, void *stream);

/*
 * lora_apply_group for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The batch's plan and its fp32 h partials live in the library's static
 * scratch array (LORA_NOALLOC_SCRATCH_BYTES on each device, a __device__ array
 * whose address lora_slots_create looks up once per device) instead of the
 * ctx's buffers; the ctx's prepared plan is neither used nor changed, and no
 * device memory is allocated.  Same arguments, results, ordering and errors as
 * lora_apply_group, except that a batch whose plan and partials do not fit the
 * array (about 4 * n * n_tokens * R bytes of partials, R = max_rank rounded up
 * to 16, plus the plan) returns LORA_ERR_TOO_MANY_TOKENS before anything is
 * enqueued.  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents: calls that overlap on one GPU (on other streams, from
 * other ctxs or host threads) race, and the caller must order them.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (16u << 20)
int lora_apply_group_noalloc(lora_ctx *ctx, int32_t n, const int32_t *modules,
                             const void *const *x, void *const *y,
                             const int32_t *token_slot_idx, int32_t n_tokens, void *stream);

/* Wait for the streams the ctx has launched on (not for the whole device),
 * return the sticky LORA_FLAG_* bits in *flags and clear them. */
int lora_get_device_flags(lora_ctx *ctx, uint32_t *flags);

/* Counters since creation. */
int lora_get_stats(lora_ctx *ctx, lora_stats *out);

/*
 * Kernel timing.  Between lora_profile_begin and lora_profile_end, each of the
 * ctx's dispatches (up to max_launches of them) carries a start and a stop
 * event recorded with the dispatch itself, so the elapsed time is that
 * kernel's execution.  lora_profile_end waits for the timed dispatches and
 * returns, per kind, how many were timed and their summed duration.  Events
 * are created by lora_profile_begin, outside any timed region.
 */
typedef struct {
    int64_t launches[5];   /* [0] plan, [1] shrink, [2] expand, [3] saved-module
                              product, [4] fused decode dispatches timed */
    double total_ms[5];    /* their summed kernel time, milliseconds */
    int64_t untimed;       /* dispatches past max_launches (not timed) */
} lora_profile;

int lora_profile_begin(lora_ctx *ctx, int32_t max_launches);
int lora_profile_end(lora_ctx *ctx, lora_profile *out);

/* Static text for a status code. */
const char *lora_status_string(int status);

/* Detail of the last error on ctx (or of the last failed lora_slots_create
 * when ctx is NULL); empty string if none.  Valid until the next call. */
const char *lora_last_error(lora_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
