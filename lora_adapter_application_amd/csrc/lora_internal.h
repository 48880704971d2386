// lora_internal.h -- launch interface between the C-ABI runtime and the HIP
// kernels of the multi-adapter LoRA path.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lora_mi355x.h"

namespace lora {

// Tokens per tile: a tile is a run of at most kTileTokens tokens of one slot.
constexpr int kTileTokens = 64;
// Columns of y one expand workgroup covers.
constexpr int kExpandCols = 256;
// K elements one shrink wave consumes per step (4 MFMA steps of 32).
constexpr int kShrinkKBlock = 128;
// Upper bound of shrink K-splits (the expand sums at most this many partials).
constexpr int kMaxSplits = 16;
// Largest padded rank (LORA_MAX_RANK rounded up to 16).
#define LORA_MAX_RANK_PAD 128

struct alignas(16) Tile {
    int32_t slot;
    int32_t start;  // first position in the permutation
    int32_t len;    // 1..kTileTokens
    int32_t pad;
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

// Per-launch slot metadata, passed by value: rank of each slot for the module
// being applied (0 = empty slot or module not targeted) and the slot's scale.
struct SlotMeta {
    float scale[LORA_MAX_SLOTS];
    uint8_t rank[LORA_MAX_SLOTS];
};

inline int max_tiles_for(int T, int S) { return (T + kTileTokens - 1) / kTileTokens + (S < T ? S : T); }


hipError_t launch_plan(const int32_t *idx, int32_t T, int32_t S, const PlanBuffers &pb,
                       hipStream_t st);

// bf16 (elem = uint16_t bit patterns) and fp32 (elem = float) entry points.
struct ShrinkArgs {
    const void *x;          // [T][d_in]
    const void *A;          // module base: [S][R_pad][d_in]
    int64_t slot_stride_A;  // elements
    const int32_t *tile_tok;
    const Tile *tiles;
    const int32_t *n_tiles;
    float *hpart;           // [splits][T][R_pad]
    int64_t split_stride;   // elements
    int32_t d_in;
    int32_t R_pad;
    int32_t k_chunk;
    int32_t splits;
    int32_t grid_tiles;
    int32_t mixed;          // batch above 1024 tokens: long tiles take the segment path
};

struct ExpandArgs {
    void *y;                // [T][d_out]
    const void *Bi;         // module base: [S][R_pad/8][d_out][8]
    int64_t slot_stride_B;  // elements
    const int32_t *tile_tok;
    const Tile *tiles;
    const int32_t *n_tiles;
    const float *hpart;
    int64_t split_stride;
    int32_t d_out;
    int32_t R_pad;
    int32_t splits;
    int32_t grid_tiles;
};

hipError_t launch_shrink(bool bf16, const ShrinkArgs &a, const SlotMeta &m, hipStream_t st);
hipError_t launch_expand(bool bf16, const ExpandArgs &a, const SlotMeta &m, hipStream_t st);

// Slot maintenance, on the side stream.
hipError_t launch_slot_finalize(bool bf16, void *A_slot, int32_t d_in, void *Bi_slot,
                                const void *B_stage, int32_t d_out, int32_t r, int32_t R_pad,
                                hipStream_t st);

}  // namespace lora
