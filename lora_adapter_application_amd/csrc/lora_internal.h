// lora_internal.h -- launch interface between the C-ABI runtime and the HIP
// kernels of the multi-adapter LoRA path.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lora_mi355x.h"

namespace lora {

// Tokens per tile: a tile is a run of at most kTileTokens tokens of one slot.
constexpr int kTileTokens = 64;
// Tiles of the plan a bf16 shrink forms inline (batches of at most
// kInlinePlanTokens tokens) hold at most inline_tile_tokens(R_pad) tokens: a
// decode kernel ends with its slowest workgroup, and a 64-token tile moves four
// times the x bytes of a 16-token one; every tile also re-reads its slot's A^T,
// a larger share of the bytes at higher rank.
constexpr int kInlineTileTokensMax = 48;
inline int inline_tile_tokens(int R_pad) { return R_pad <= 16 ? 32 : 48; }
// Columns of y one expand workgroup covers.
constexpr int kExpandCols = 256;
// K elements one shrink wave consumes per step (4 MFMA steps of 32).
constexpr int kShrinkKBlock = 128;
// Upper bound of shrink K-splits (the expand sums at most this many partials).
constexpr int kMaxSplits = 16;
// Rank blocks of 16 a kernel instance is compiled for: the padded rank's block
// count rounded up to 1, 2, 4 or 8.
constexpr int nb_template(int R_pad) { return R_pad <= 16 ? 1 : R_pad <= 32 ? 2 : R_pad <= 64 ? 4 : 8; }
// K-splits the expand can sum for a kernel instance of NB rank blocks (keeps
// the partials of one thread at kMaxSplits float4 registers).
constexpr int splits_cap(int NB) { return kMaxSplits / NB > 0 ? kMaxSplits / NB : 1; }
// Largest padded rank (LORA_MAX_RANK rounded up to 16).
#define LORA_MAX_RANK_PAD 128

struct alignas(16) Tile {
    int32_t slot;
    int32_t start;  // first position in the slot-sorted order
    int32_t len;    // 1..kTileTokens
    int32_t rank;   // rank of the slot's adapter, written by the shrink for the expand
    float scale;    // the slot's scale, written with rank
    int32_t pad[3];
};

struct PlanBuffers {
    int32_t *counts;     // [S] tokens per slot
    int32_t *seg_start;  // [S] first position of each slot's run
    Tile *tiles;         // [max_tiles]
    int32_t *tile_tok;   // [max_tiles][kTileTokens]: token index of each tile row
    int32_t *n_tiles;    // scalar
    int32_t *n_active;   // scalar
    uint32_t *flags;     // scalar, sticky
    int32_t *chunk_counts;  // [ceil(max_tokens/1024)][S], batches above 1024 tokens
};

// Batches up to this many tokens are planned inside the bf16 kernels.
constexpr int kInlinePlanTokens = 1024;
// How a bf16 launch finds its tiles: kPlanTiles reads the tiles a plan kernel
// or an earlier launch published; kPlanInline derives each workgroup's tile in
// the kernel (batches of at most kInlinePlanTokens) and publishes it.
enum PlanMode { kPlanTiles = 0, kPlanInline = 1 };
// Modules one grouped shrink / expand launch covers (blockIdx.z = member).
constexpr int kMaxGroup = 8;

// Slot metadata of one launch, passed by value: per slot its adapter's rank
// (0 = empty) and scale, and per group member one bit per slot telling whether
// that adapter targets the member's module.  Launches capture it when they are
// enqueued, so a kernel sees exactly the slots loaded before it.
struct SlotMeta {
    float scale[LORA_MAX_SLOTS];
    uint8_t rank[LORA_MAX_SLOTS];
    uint8_t flags[LORA_MAX_SLOTS];      // kSlotBias | kSlotDora
    uint32_t target[kMaxGroup][LORA_MAX_SLOTS / 32];
};
// Output terms an adapter may carry (lora_slot_load_ex).
enum SlotFlags { kSlotBias = 1, kSlotDora = 2 };

// Optional events around one dispatch (both null: untimed), recorded with the
// dispatch itself so they bracket exactly the kernel's execution.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

inline int max_tiles_for(int T, int S, int cap = kTileTokens)
{
    return (T + cap - 1) / cap + (S < T ? S : T);
}

// A plan of more than 1024 tokens takes two launches; t[0] and t[1] time them.
hipError_t launch_plan(const int32_t *idx, int32_t T, int32_t S, const PlanBuffers &pb,
                       hipStream_t st, const LaunchTiming *t /* [2] or null */);

// Element type: bf16 (uint16_t bit patterns) or fp32.
struct ShrinkArgs {
    int32_t n;                          // group members
    const void *x[kMaxGroup];           // [T][d_in]
    const void *A[kMaxGroup];           // module base: [S][R_pad][d_in]
    int64_t slot_stride_A[kMaxGroup];   // elements
    int32_t d_in[kMaxGroup];
    int32_t k_chunk[kMaxGroup];
    int32_t splits[kMaxGroup];
    PlanBuffers plan;                   // read, or written by an inline plan
    const int32_t *idx;                 // token slot index (inline plan)
    int32_t T;
    int32_t S;
    int32_t plan_mode;                  // PlanMode
    float *hpart;                       // [member][split][T][R_pad]
    int64_t member_stride;              // elements
    int64_t split_stride;               // T * R_pad
    int32_t R_pad;
    int32_t grid_tiles;
    int32_t grid_splits;                // max splits over the members
    int32_t mixed;                      // batch above 1024 tokens: long tiles take the segment path
    int32_t warm;                       // kWarmX | kWarmA: L2 warm-up of the split's blocks (inline plan)
    int32_t warm_rows;                  // rows of the warm-up block per workgroup
    int32_t tile_cap;                   // inline plan: tokens per tile
};

// What the inline-plan shrink warms in L2 while its plan is formed.
enum WarmFlags { kWarmX = 1, kWarmA = 2 };

struct ExpandArgs {
    int32_t n;
    void *y[kMaxGroup];                 // [T][d_out]
    const void *Bi[kMaxGroup];          // module base: [S][R_pad/8][d_out][8]
    int64_t slot_stride_B[kMaxGroup];
    int32_t d_out[kMaxGroup];
    int32_t splits[kMaxGroup];
    const Tile *tiles;
    const int32_t *tile_tok;
    const int32_t *n_tiles;
    const float *hpart;
    int64_t member_stride;
    int64_t split_stride;
    int32_t R_pad;
    int32_t grid_tiles;
    int32_t grid_cols;                  // max column chunks over the members
    int32_t col_start[kMaxGroup + 1];   // bf16 kernel: chunks of the members before member i
    int32_t xcd_group;                  // work items per XCD group (bf16 kernel); < 0: tile t on residue t % 8
    int32_t tile_major;                 // bf16 kernel: chunks of a tile are consecutive items
    const void *bias[kMaxGroup];        // module base: [S][d_out], ctx dtype
    const float *dora[kMaxGroup];       // module base: [S][d_out]
    int32_t terms;                      // some slot of the launch has output terms
    int32_t tile_cap;                   // tokens per tile of the plan (at most kTileTokens)
};

hipError_t launch_shrink(bool bf16, const ShrinkArgs &a, const SlotMeta &m, hipStream_t st,
                         const LaunchTiming &t);

// Fused decode (bf16, batches of at most kInlinePlanTokens, on a device that
// deals the workgroups of a launch to its XCDs in turn): the shrink and the expand of
// one group in one launch; expand workgroups wait for the K-split partials of
// their tile through per-(tile, member) counts in `sync`, which every launch
// leaves at zero.  The counts of a tile fill a 128-byte line of their own
// (kSyncWordsPerTile words: partials stored and consumers past the wait, per
// member), so no line is shared by tiles of two XCDs.
constexpr int kSyncWordsPerTile = 32;
static_assert(2 * kMaxGroup <= kSyncWordsPerTile, "a tile's counts fit its line");
struct FusedArgs {
    ShrinkArgs s;
    ExpandArgs e;
    uint32_t *sync;              // [max_tiles][kSyncWordsPerTile]
    int32_t spin_limit;          // polls of a waiting workgroup before it gives up
};
hipError_t launch_fused(const FusedArgs &f, const SlotMeta &m, hipStream_t st, const LaunchTiming &t);
hipError_t launch_expand(bool bf16, const ExpandArgs &a, const SlotMeta &m, hipStream_t st,
                         const LaunchTiming &t);

// Slot maintenance, on the side stream: one launch finishes the loads of up to
// kFinalizeBatch modules (A^T copy and B repack, read in place or from a staged
// copy, and zero padding rows).
constexpr int kFinalizeBatch = 16;
struct FinalizeItem {
    void *A_slot;            // the slot's A^T block of the module
    void *Bi_slot;           // the slot's repacked B block
    const void *A_src;       // r x d_in, row-major: the caller's weights or their staged copy
    const void *B_src;       // r x d_out, row-major: the same
    void *bias_dst;          // the slot's bias row (d_out, ctx dtype), or null
    const void *bias_src;    // the caller's bias, read in place, or null
    float *dora_dst;         // the slot's DoRA factors (d_out), or null
    const float *dora_src;   // the caller's factors, read in place, or null
    int32_t d_in, d_out;
};
struct FinalizeBatch {
    int32_t n, r, R_pad;
    FinalizeItem it[kFinalizeBatch];
};
hipError_t launch_slot_finalize(bool bf16, const FinalizeBatch &b, hipStream_t st);

// Whole modules an adapter saves (lora_slot_load_saved): for the tokens of a
// slot that saves member m's module, y = round(x . W^T + c) replaces the base
// output; a segmented GEMM over the plan's tiles, kSavedCols columns per
// workgroup (bf16 on MFMA; fp32 on VALU).
constexpr int kSavedCols = 256;
struct SavedArgs {
    int32_t n;                          // group members
    const void *x[kMaxGroup];           // [T][d_in]
    void *y[kMaxGroup];                 // [T][d_out]
    const void *W[kMaxGroup];           // module base: [S][d_out][d_in]
    const void *bias[kMaxGroup];        // module base: [S][d_out]
    int64_t slot_stride_W[kMaxGroup];   // elements
    int32_t d_in[kMaxGroup];
    int32_t d_out[kMaxGroup];
    int32_t col_start[kMaxGroup + 1];   // bf16: kSavedCols chunks of the members before member i
    const Tile *tiles;
    const int32_t *tile_tok;
    const int32_t *n_tiles;
    int32_t grid_tiles;
    int32_t T;                          // tokens of the batch
    int32_t per_xcd;                    // bf16: work items per XCD (set by launch_saved)
    uint32_t saved[kMaxGroup][LORA_MAX_SLOTS / 32];     // slot k saves member m's module
    uint32_t has_bias[kMaxGroup][LORA_MAX_SLOTS / 32];  // ... with a bias
};
hipError_t launch_saved(bool bf16, const SavedArgs &a, hipStream_t st, const LaunchTiming &t);

// Scratch memory of lora_apply_group_noalloc: a static __device__ array of
// this size in the library's code object, so each device the library runs on
// holds one copy until the process ends.  It takes one batch's plan buffers and
// h partials in place of the ctx's own allocation.
constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;
// Device address of the scratch array on `device`, which must be the current
// device: looked up with hipGetSymbolAddress at the first call for the device,
// then kept.
hipError_t scratch_address(int device, void **ptr);
// Whether the workgroups of a launch whose indices agree mod 8 run on one XCD
// on `device` (the current device); probed once per device with two launches
// on `st`, then kept.
hipError_t xcd_dispatch_check(int device, hipStream_t st, bool *ok);

}  // namespace lora
