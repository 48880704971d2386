// lora_kernels.hip -- gfx950 kernels of the multi-adapter LoRA update
//
//   plan     stable counting sort of the per-token slot index into runs of one
//            slot, cut into tiles of up to 64 tokens (32 or 48 when the shrink
//            forms the plan inline); each tile record lists its token indices
//            (device only, no host sync)
//   shrink   h[p, :] = x[tok(p), :] . A_k^T over a K range (fp32 partials)
//   expand   y[t, :] = round(y[t, :] + s_k * h[p, :] . B_k)
//
// The update itself, its scale and the adapter fields it reads are those of the
// example adapter_config.json in "vLLM LoRA Resolver plugins explained",
// section 3.2; the slot count and padded rank are max_loras / max_lora_rank of
// the parameter table in "Multi-LoRA adapter cache in production".
//
// bf16 data runs on the matrix cores: v_mfma_f32_16x16x32_bf16 for the shrink
// (K = d_in) and for the expand (K = a block of 16 ranks, with the fp32
// intermediate split into a bf16 high and low part stacked along K, so the
// expand keeps ~16 bits of h); results are rounded to bf16 by
// v_cvt_pk_bf16_f32 (round to nearest even).  fp32 data runs on plain VALU
// loops (the shrink's K sums in fp64).  One shrink or expand launch covers a group of up to kMaxGroup
// modules.
//
// Operand layout of a 16x16xK MFMA on a 64-wide wave, as used below: lane l
// supplies row (l & 15) of A and column (l & 15) of B, each with the K slice of
// lane group g = l >> 4 (8 values for K=32, 4 for K=16); the 16x16 fp32 result
// leaves rows 4g..4g+3 of column (l & 15) in lane l.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "lora_internal.h"

namespace lora {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Launch, with the dispatch bracketed by t's events when it has them.
template <typename K, typename... Args>
static void launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                   const LaunchTiming &t, Args... args)
{
    if (t.start)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, t.start, t.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

// ----------------------------------------------------------------------------
// plan

// Exclusive scan of two ints per thread over a block of NW waves.
template <int NW>
__device__ void block_excl_scan2(int &a, int &b, int2 *wsum /*[NW + 1]*/, int &total_a, int &total_b)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int sa = a, sb = b;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int oa = __shfl_up(sa, d, 64), ob = __shfl_up(sb, d, 64);
        if (lane >= d) {
            sa += oa;
            sb += ob;
        }
    }
    if (lane == 63)
        wsum[wave] = make_int2(sa, sb);
    __syncthreads();
    if (wave == 0) {
        const int2 w = lane < NW ? wsum[lane] : make_int2(0, 0);
        int ta = w.x, tb = w.y;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            const int oa = __shfl_up(ta, d, 64), ob = __shfl_up(tb, d, 64);
            if (lane >= d) {
                ta += oa;
                tb += ob;
            }
        }
        if (lane < NW)
            wsum[lane] = make_int2(ta - w.x, tb - w.y);
        if (lane == NW - 1)
            wsum[NW] = make_int2(ta, tb);
    }
    __syncthreads();
    const int2 base = wsum[wave], tot = wsum[NW];
    a = sa - a + base.x;
    b = sb - b + base.y;
    total_a = tot.x;
    total_b = tot.y;
}

__device__ __forceinline__ void block_excl_scan2_1024(int &a, int &b, int2 *wsum, int &ta, int &tb)
{
    block_excl_scan2<16>(a, b, wsum, ta, tb);
}

// Rank of this thread's token among the earlier tokens of its wave with the
// same slot (one ballot per distinct slot in the wave); the first lane of each
// slot writes the wave's count of that slot to row[slot].
__device__ __forceinline__ int wave_stable_rank_row(int v, bool valid, int32_t *row)
{
    const int lane = threadIdx.x & 63;
    uint64_t act = __ballot(valid);
    int my_rank = 0;
    while (act) {
        const int leader = __ffsll((unsigned long long)act) - 1;
        const int lv = __shfl(v, leader, 64);
        const bool mine = valid && v == lv;
        const uint64_t m = __ballot(mine);
        if (mine)
            my_rank = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == leader)
            row[lv] = __popcll(m);
        act &= ~m;
    }
    return my_rank;
}

__device__ __forceinline__ int wave_stable_rank(int v, bool valid, int32_t *wcnt, int S)
{
    return wave_stable_rank_row(v, valid, wcnt + (threadIdx.x >> 6) * S);
}

// Batches of at most 1024 tokens: one token per thread, one ballot pass gives
// both the per-slot counts and each token's rank among equal slots.
__global__ __launch_bounds__(1024) void plan_small_kernel(const int32_t *__restrict__ idx,
                                                          int32_t T, int32_t S, PlanBuffers pb)
{
    extern __shared__ int32_t sm[];
    int32_t *wcnt = sm;             // [16][S]: count, then offset within the slot's run
    int32_t *tbase = sm + 16 * S;   // [S]: first tile of slot s
    __shared__ int2 wsum[17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v = tid < T ? idx[tid] : -1;
    for (int i = tid; i < 16 * S; i += 1024)
        wcnt[i] = 0;
    const bool valid = v >= 0 && v < S;
    const uint64_t too_large = __ballot(v >= S);
    if (too_large && lane == 0)
        atomicOr(pb.flags, 1u);
    __syncthreads();
    const int my_rank = wave_stable_rank(v, valid, wcnt, S);
    __syncthreads();
    int c = 0;
    if (tid < S) {
        for (int w = 0; w < 16; ++w) {
            const int k = wcnt[w * S + tid];
            wcnt[w * S + tid] = c;
            c += k;
        }
    }
    int start = c, tstart = (c + kTileTokens - 1) / kTileTokens, n_active, n_tiles;
    const int nt = tstart;
    block_excl_scan2_1024(start, tstart, wsum, n_active, n_tiles);
    if (tid < S) {
        tbase[tid] = tstart;
        pb.counts[tid] = c;
        pb.seg_start[tid] = start;
        for (int j = 0; j < nt; ++j) {
            Tile t;
            t.slot = tid;
            t.start = start + j * kTileTokens;
            t.len = min(kTileTokens, c - j * kTileTokens);
            t.rank = 0;
            t.scale = 0.f;
            t.pad[0] = t.pad[1] = t.pad[2] = 0;
            pb.tiles[tstart + j] = t;
        }
    }
    if (tid == 0) {
        *pb.n_tiles = n_tiles;
        *pb.n_active = n_active;
    }
    __syncthreads();
    if (valid) {
        const int rel = wcnt[wave * S + v] + my_rank;          // position within the slot's run
        pb.tile_tok[(int64_t)(tbase[v] + rel / kTileTokens) * kTileTokens + rel % kTileTokens] = tid;
    }
}

// Batches above 1024 tokens run in two launches over chunks of 1024 tokens:
// count (per chunk and slot), then scatter, where every workgroup derives its
// chunk's offsets and the slot runs from all chunk counts (workgroup 0 also
// writes the tile list).
__global__ __launch_bounds__(1024) void plan_count_kernel(const int32_t *__restrict__ idx,
                                                          int32_t T, int32_t S, PlanBuffers pb)
{
    extern __shared__ int32_t wcnt[];   // [16][S]
    const int tid = threadIdx.x, lane = tid & 63;
    const int i = blockIdx.x * 1024 + tid;
    const int v = i < T ? idx[i] : -1;
    for (int k = tid; k < 16 * S; k += 1024)
        wcnt[k] = 0;
    const bool valid = v >= 0 && v < S;
    if (__ballot(v >= S) && lane == 0)
        atomicOr(pb.flags, 1u);
    __syncthreads();
    (void)wave_stable_rank(v, valid, wcnt, S);
    __syncthreads();
    for (int sl = tid; sl < S; sl += 1024) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w)
            c += wcnt[w * S + sl];
        pb.chunk_counts[(int64_t)blockIdx.x * S + sl] = c;
    }
}

__global__ __launch_bounds__(1024) void plan_scatter_kernel(const int32_t *__restrict__ idx,
                                                            int32_t T, int32_t S, int32_t n_chunks,
                                                            PlanBuffers pb)
{
    extern __shared__ int32_t sm[];
    int32_t *wcnt = sm;              // [16][S]
    int32_t *seg = sm + 16 * S;      // [S] first position of slot s
    int32_t *tbase = sm + 17 * S;    // [S] first tile of slot s
    int32_t *scnt = sm + 18 * S;     // [S] tokens of slot s
    __shared__ int2 wsum[17];
    __shared__ int32_t n_tiles_sh;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int chunk = blockIdx.x;
    const int i = chunk * 1024 + tid;
    const int v = i < T ? idx[i] : -1;
    for (int k = tid; k < 16 * S; k += 1024)
        wcnt[k] = 0;
    const bool valid = v >= 0 && v < S;
    // this slot's tokens in earlier chunks, and in all chunks
    int pre = 0, tot = 0;
    if (tid < S) {
        for (int ch0 = 0; ch0 < n_chunks; ch0 += 16) {
            int k[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                k[u] = ch0 + u < n_chunks ? pb.chunk_counts[(int64_t)(ch0 + u) * S + tid] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                pre += ch0 + u < chunk ? k[u] : 0;
                tot += k[u];
            }
        }
    }
    __syncthreads();
    const int my_rank = wave_stable_rank(v, valid, wcnt, S);
    int start = tot, tstart = (tot + kTileTokens - 1) / kTileTokens, n_active, n_tiles;
    block_excl_scan2_1024(start, tstart, wsum, n_active, n_tiles);
    if (tid < S) {
        seg[tid] = start;
        tbase[tid] = tstart;
        scnt[tid] = tot;
        int run = start + pre;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int k = wcnt[w * S + tid];
            wcnt[w * S + tid] = run;
            run += k;
        }
        if (chunk == 0) {
            pb.counts[tid] = tot;
            pb.seg_start[tid] = start;
        }
    }
    if (tid == 0) {
        n_tiles_sh = n_tiles;
        if (chunk == 0) {
            *pb.n_tiles = n_tiles;
            *pb.n_active = n_active;
        }
    }
    __syncthreads();
    if (chunk == 0) {
        // the tile list, one tile per thread: tile j belongs to the last slot
        // whose first tile is at most j (an empty slot shares its first tile
        // index with the next slot, so that slot is never empty)
        for (int j = tid; j < n_tiles_sh; j += 1024) {
            int lo = 0, hi = S - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tbase[mid] <= j)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int q = j - tbase[lo];
            Tile t;
            t.slot = lo;
            t.start = seg[lo] + q * kTileTokens;
            t.len = min(kTileTokens, scnt[lo] - q * kTileTokens);
            t.rank = 0;
            t.scale = 0.f;
            t.pad[0] = t.pad[1] = t.pad[2] = 0;
            pb.tiles[j] = t;
        }
    }
    if (valid) {
        const int rel = wcnt[wave * S + v] + my_rank - seg[v];
        pb.tile_tok[(int64_t)(tbase[v] + rel / kTileTokens) * kTileTokens + rel % kTileTokens] = i;
    }
}

hipError_t launch_plan(const int32_t *idx, int32_t T, int32_t S, const PlanBuffers &pb,
                       hipStream_t st, const LaunchTiming *t)
{
    const LaunchTiming none;
    if (T <= 1024) {
        launch(plan_small_kernel, dim3(1), dim3(1024), sizeof(int32_t) * (size_t)S * 17, st,
               t ? t[0] : none, idx, T, S, pb);
    } else {
        const int n_chunks = (T + 1023) / 1024;
        launch(plan_count_kernel, dim3(n_chunks), dim3(1024), sizeof(int32_t) * (size_t)S * 16, st,
               t ? t[0] : none, idx, T, S, pb);
        launch(plan_scatter_kernel, dim3(n_chunks), dim3(1024), sizeof(int32_t) * (size_t)S * 19,
               st, t ? t[1] : none, idx, T, S, n_chunks, pb);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// shrink, bf16 on MFMA
//
// One workgroup (4 waves) = one tile (<= 64 tokens of one slot) x one K split x
// one group member.  Output: the member's h partial of the split
// as [rank][token] blocks, lane l holding ranks 4g..4g+3 of token (l & 15),
// stored as one 16-byte write.

// Two fp32 values to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *(const uint4 *)p; }

__device__ __forceinline__ int member_rank(const SlotMeta &meta, int m, int slot)
{
    return ((meta.target[m][slot >> 5] >> (slot & 31)) & 1u) ? (int)meta.rank[slot] : 0;
}

// Slot metadata fetched at kernel start, independent of the tile: lane l holds
// the ranks and the output-term flags of slots 4l .. 4l+3 (rk, fl), word l % 8
// of group member l / 8's target mask (tw) and the scales of slots l, l+64,
// l+128, l+192 (sc).  A lookup for a
// wave-uniform slot reads one lane (v_readlane), with no memory access.
struct MetaRegs {
    uint32_t rk;
    uint32_t fl;
    uint32_t tw;
    float sc[LORA_MAX_SLOTS / 64];
};

__device__ __forceinline__ MetaRegs load_meta_regs(const SlotMeta &meta)
{
    const int lane = threadIdx.x & 63;
    MetaRegs r;
    r.rk = ((const uint32_t *)meta.rank)[lane];
    r.fl = ((const uint32_t *)meta.flags)[lane];
    r.tw = ((const uint32_t *)meta.target)[lane];
#pragma unroll
    for (int i = 0; i < LORA_MAX_SLOTS / 64; ++i)
        r.sc[i] = meta.scale[lane + 64 * i];
    return r;
}

__device__ __forceinline__ int meta_rank(const MetaRegs &r, int slot)
{
    slot = __builtin_amdgcn_readfirstlane(slot);
    return (__builtin_amdgcn_readlane(r.rk, slot >> 2) >> ((slot & 3) * 8)) & 0xff;
}

__device__ __forceinline__ int meta_flags(const MetaRegs &r, int slot)
{
    slot = __builtin_amdgcn_readfirstlane(slot);
    return (__builtin_amdgcn_readlane(r.fl, slot >> 2) >> ((slot & 3) * 8)) & 0xff;
}

__device__ __forceinline__ bool meta_targets(const MetaRegs &r, int m, int slot)
{
    slot = __builtin_amdgcn_readfirstlane(slot);
    return (__builtin_amdgcn_readlane(r.tw, m * (LORA_MAX_SLOTS / 32) + (slot >> 5)) >> (slot & 31)) & 1u;
}

// The lookups read other lanes' registers: call them where every lane of the
// wave is active, or the compiler may compute those registers in fewer lanes.
__device__ __forceinline__ float meta_scale(const MetaRegs &r, int slot)
{
    slot = __builtin_amdgcn_readfirstlane(slot);
    int v[LORA_MAX_SLOTS / 64];
#pragma unroll
    for (int i = 0; i < LORA_MAX_SLOTS / 64; ++i)
        v[i] = __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.sc[i]), slot & 63);
    const int i = slot >> 6;
    return __builtin_bit_cast(float, i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then the totals of rows 0 and 2 into rows
// 1 and 3 (row_bcast:15) and of rows 0-1 into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// One member's view of a shrink launch.
struct ShrinkView {
    const uint16_t *x;
    const uint16_t *A;      // slot's A^T block
    int64_t d_in;
    int k0, k1;             // K range of this split
    float *h;               // this member's split partial: [T][R_pad]
    int R_pad;
};

// Gather path (BGMV): waves split the tile's subtiles and the K range.  A K
// block is 128 elements; MFMA step q of a block takes elements 32q .. 32q+31,
// lane group g holding 8g .. 8g+7 of them, so the four lanes of a row read 64
// contiguous bytes per instruction, of the token's x row and of the rank's A^T
// row alike.  A K chunk past the split's end is zero; a row beyond the tile
// reads token 0's row (it only reaches h rows that are not stored).  tokv:
// lane l of every wave holds the token of tile row l.
template <int NB>
struct KBlock {
    uint4 x[4];
    uint4 a[NB][4];
};

template <int NB>
__device__ __forceinline__ void load_kblock(KBlock<NB> &blk, const uint16_t *xrow,
                                            const uint16_t *arow0, int64_t d_in, int kb, int k1, int nb)
{
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ke = kb + q * 32 + g * 8;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            blk.a[b][q] = (b < nb && ke < k1) ? ld16(arow0 + b * 16 * d_in + ke) : make_uint4(0, 0, 0, 0);
        blk.x[q] = ke < k1 ? ld16(xrow + ke) : make_uint4(0, 0, 0, 0);
    }
}

template <int NB>
__device__ __forceinline__ void mfma_kblock(f32x4_t (&acc)[NB], const KBlock<NB> &blk, int nb)
{
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (b < nb) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, blk.a[b][q]),
                    __builtin_bit_cast(bf16x8_t, blk.x[q]), acc[b], 0, 0, 0);
        }
    }
}

template <int NB, bool DOUBLE_BUFFER>
__device__ __forceinline__ void shrink_bgmv(const ShrinkView &v, const Tile &tile, int tokv, int nb,
                                            unsigned char *smem)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane & 15, g = lane >> 4;
    const int nsub = (tile.len + 15) >> 4;
    const int nsub_pad = nsub == 3 ? 4 : nsub;
    const int kparts = 4 / nsub_pad;
    const int sub = wave % nsub_pad, kp = wave / nsub_pad;
    const bool wave_on = sub < nsub;
    const int t_in = sub * 16 + row;
    const bool tok_ok = wave_on && t_in < tile.len;
    const int tok = __shfl(tokv, t_in & 63, 64);
    const uint16_t *xrow = v.x + (int64_t)(tok_ok ? tok : 0) * v.d_in;
    const uint16_t *arow0 = v.A + (int64_t)row * v.d_in;

    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (wave_on) {
        // this wave's K blocks: k0 + kp*128, then every kparts*128
        const int kstep = kparts * kShrinkKBlock;
        const int kb0 = v.k0 + kp * kShrinkKBlock;
        const int nblk = kb0 < v.k1 ? (v.k1 - kb0 + kstep - 1) / kstep : 0;
        if (DOUBLE_BUFFER) {
            // two K blocks in flight per round
            for (int i = 0; i < nblk; i += 2) {
                KBlock<NB> b0, b1;
                load_kblock<NB>(b0, xrow, arow0, v.d_in, kb0 + i * kstep, v.k1, nb);
                if (i + 1 < nblk)
                    load_kblock<NB>(b1, xrow, arow0, v.d_in, kb0 + (i + 1) * kstep, v.k1, nb);
                mfma_kblock<NB>(acc, b0, nb);
                if (i + 1 < nblk)
                    mfma_kblock<NB>(acc, b1, nb);
            }
        } else {
            for (int i = 0; i < nblk; ++i) {
                KBlock<NB> cur;
                load_kblock<NB>(cur, xrow, arow0, v.d_in, kb0 + i * kstep, v.k1, nb);
                mfma_kblock<NB>(acc, cur, nb);
            }
        }
    }
    f32x4_t (*red)[NB][64] = (f32x4_t (*)[NB][64])smem;
    if (kparts > 1) {
        if (wave_on && kp > 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                red[wave][b][lane] = acc[b];
        }
        __syncthreads();
        if (wave_on && kp == 0) {
            for (int k = 1; k < kparts; ++k) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[b] += red[sub + k * nsub_pad][b][lane];
            }
        }
    }
    if (kp == 0 && tok_ok) {
        float *hrow = v.h + (int64_t)(tile.start + t_in) * v.R_pad;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < nb)
                *(f32x4_t *)(hrow + b * 16 + g * 4) = acc[b];
    }
}

// Segment path (SGMV) for tiles of 17..64 tokens: wave w owns subtile w over
// the whole K range.  Each K block of A^T (nb*16 ranks x 128) is loaded once per
// workgroup into LDS (double buffered) and shared by the 4 waves.  The loads of
// the next D blocks (x in registers, A^T in registers until staged) are in
// flight while a block is multiplied, so a workgroup keeps D blocks of memory
// requests outstanding instead of waiting one round trip per block.  The ring
// of D register sets is indexed statically (the loop is unrolled by D), so no
// register holding an outstanding load is ever copied.  K order as on the gather
// path: MFMA step q takes elements 32q .. 32q+31 of the block, lane group g
// 8g .. 8g+7, so each x load instruction reads 64 contiguous bytes of a row
// (a quarter of its 256-byte block) rather than four 16-byte pieces 64 bytes
// apart: 3% less time for the prefill shrink.
constexpr int kLdsRow = kShrinkKBlock + 8;   // bf16 elements per staged A row (padded)

// Blocks in flight of the segment path: deeper for low rank, where the
// register sets are small.
constexpr int sgmv_depth(int NB) { return NB <= 2 ? 4 : NB == 4 ? 3 : 2; }

template <int NB>
__device__ __forceinline__ void shrink_sgmv(const ShrinkView &v, const Tile &tile, int tokv, int nb,
                                            uint16_t *lds)
{
    constexpr int D = sgmv_depth(NB);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, g = lane >> 4;
    const int t_in = wave * 16 + row;
    const bool tok_ok = t_in < tile.len;
    const int tok = __shfl(tokv, t_in, 64);
    const uint16_t *xrow = v.x + (int64_t)(tok_ok ? tok : 0) * v.d_in;
    const int k0 = v.k0, k1 = v.k1;
    const int nkb = (k1 - k0 + kShrinkKBlock - 1) / kShrinkKBlock;
    constexpr int buf_elems = NB * 16 * kLdsRow;

    // Loads are unconditional, with addresses clamped into the operands (rank
    // rows below nb*16, K below k1): a branch around a load would make the
    // compiler wait for every outstanding load at the loop head.  A^T values
    // past k1 are zeroed when staged, so the x values read there (clamped, finite)
    // contribute nothing; rows past the tile read token 0 and are not stored.
    const int r_last = nb * 16 - 1;
    auto load_a = [&](uint4 (&ra)[NB], int kb) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int c = tid + 256 * i;
            const int r = min(c >> 4, r_last), col = (c & 15) * 8;
            ra[i] = ld16(v.A + (int64_t)r * v.d_in + min(kb + col, k1 - 8));
        }
    };
    auto store_a = [&](const uint4 (&ra)[NB], int buf, int kb) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < nb) {
                const int c = tid + 256 * i;
                const int r = c >> 4, col = (c & 15) * 8;
                *(uint4 *)(lds + buf * buf_elems + r * kLdsRow + col) =
                    kb + col < k1 ? ra[i] : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto load_x = [&](uint4 (&xv)[4], int kb) {
        const int kk = kb + g * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xv[q] = ld16(xrow + min(kk + q * 32, k1 - 8));
    };

    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // ring slot j holds block i + j of the current pass (x) and, for A^T, the
    // block after the one staged in LDS
    uint4 xr[D][4], ar[D][NB];
    auto mma = [&](int b, const uint4 (&xv)[4]) {
        const uint16_t *L = lds + (b & 1) * buf_elems;
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            if (rb < nb) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 av = *(const uint4 *)(L + (rb * 16 + row) * kLdsRow + q * 32 + g * 8);
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, xv[q]), acc[rb], 0,
                        0, 0);
                }
            }
        }
    };
    int i = 0;
    if (nkb >= 2 * D) {
        // Steady state: every refill of the first nkb - D blocks is in range,
        // so the prologue and the loop issue their loads without a branch, in
        // a fixed order, and the compiler counts them exactly; a branch around
        // a load would make it wait for all of them at the loop head.
#pragma unroll
        for (int j = 0; j < D; ++j) {
            load_x(xr[j], k0 + j * kShrinkKBlock);
            load_a(ar[j], k0 + j * kShrinkKBlock);
            __builtin_amdgcn_sched_barrier(0);
        }
        store_a(ar[0], 0, k0);
        __syncthreads();
        for (; i + 2 * D <= nkb; i += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int b = i + j;
                mma(b, xr[j]);
                load_x(xr[j], k0 + (b + D) * kShrinkKBlock);
                store_a(ar[(j + 1) % D], (b + 1) & 1, k0 + (b + 1) * kShrinkKBlock);
                load_a(ar[j], k0 + (b + D) * kShrinkKBlock);
                __syncthreads();
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (j < nkb) {
                load_a(ar[j], k0 + j * kShrinkKBlock);
                load_x(xr[j], k0 + j * kShrinkKBlock);
            }
        }
        store_a(ar[0], 0, k0);
        __syncthreads();
    }
    // the last blocks: refills only while in range
    for (; i < nkb; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int b = i + j;          // block multiplied in this step
            if (b < nkb) {
                mma(b, xr[j]);
                // slot j is free (A^T block b is in LDS, x block b consumed):
                // refill it with block b + D
                if (b + D < nkb)
                    load_x(xr[j], k0 + (b + D) * kShrinkKBlock);
                // stage block b + 1 (slot j + 1) into the other LDS buffer
                if (b + 1 < nkb)
                    store_a(ar[(j + 1) % D], (b + 1) & 1, k0 + (b + 1) * kShrinkKBlock);
                if (b + D < nkb)
                    load_a(ar[j], k0 + (b + D) * kShrinkKBlock);
                __syncthreads();
            }
        }
    }
    if (tok_ok) {
        float *hrow = v.h + (int64_t)(tile.start + t_in) * v.R_pad;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < nb)
                *(f32x4_t *)(hrow + b * 16 + g * 4) = acc[b];
    }
}

// Inline plan (batches of at most kInlinePlanTokens tokens): every workgroup
// derives its own tile of the stable slot-sorted plan the plan kernels make,
// without sorting the batch: per-slot token counts (an LDS histogram), per-slot
// tile and position offsets (one wave scans them), then the sorted positions of
// its own slot's tokens (one ballot per 64 tokens, in token order).  One
// workgroup per tile publishes it, and one workgroup the totals, so that later
// launches on the same plan can read them.
struct TilePlanLds {
    int32_t cnt[LORA_MAX_SLOTS];                 // tokens per slot
    int32_t wc[kInlinePlanTokens / 64];          // tokens of the tile's slot per 64 tokens
    int32_t list[kTileTokens];                   // token ids of the tile
    int32_t slot, j, start, count, n_tiles, ticket;
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// The chip dispatches the workgroups of a launch to its 8 XCDs in turn
// (workgroup i to XCD i mod 8), and each XCD has an L2 of its own.  Work items
// are taken in groups of G consecutive items; group k runs on XCD k mod 8, its
// items one after the other, so they share that XCD's L2, while consecutive
// groups still spread over all XCDs.  The launch has xcd_grid(n, G)
// workgroups; items >= n are padding.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_item(int G, int blk)
{
    const int xcd = blk % kXcds, j = blk / kXcds;
    return ((j / G) * kXcds + xcd) * G + j % G;
}

constexpr int kPlanPerThread = kInlinePlanTokens / 256;

// Kernel arguments are read with scalar loads where the code first needs a
// field, and a field whose 64-byte line is not yet in the scalar cache costs a
// memory round trip at that point; the compiler spreads these loads through
// the plan and the tile code.  Touching every line of the argument struct at
// entry brings them all in behind a single wait.
template <typename Args>
__device__ __forceinline__ void touch_args()
{
    const __attribute__((address_space(4))) uint32_t *p =
        (const __attribute__((address_space(4))) uint32_t *)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < (int)((sizeof(Args) + 63) / 64); ++i)
        s ^= p[i * 16];
    asm volatile("" ::"s"(s));
}

// The batch's slot indices, thread tid holding tokens c*256 + tid (-1 past T).
__device__ __forceinline__ void plan_load_idx(const int32_t *idx, int T, int (&v)[kPlanPerThread])
{
#pragma unroll
    for (int c = 0; c < kPlanPerThread; ++c) {
        // unconditional load (clamped index), so that waiting for these
        // loads need not wait for loads issued after them
        const int i = c * 256 + threadIdx.x;
        const int raw = idx[min(i, T - 1)];
        v[c] = i < T ? raw : -1;
    }
}

// Tile b of the plan, from the slot indices v (plan_load_idx); a slot's tokens
// are cut into tiles of at most cap tokens.  publish: write the tile and its
// token ids to the plan buffers; first: write the totals and the flag.  Returns
// false past the last tile.
__device__ bool plan_tile(const int (&v)[kPlanPerThread], int T, int S, int cap, const MetaRegs &mr,
                          const PlanBuffers &pb, TilePlanLds &L, int b, bool publish, bool first,
                          Tile &tile, int &tokv)
{
    constexpr int NC = kPlanPerThread;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ncu = (T + 255) >> 8;             // entries c of v that hold tokens
    if (tid < S)
        L.cnt[tid] = 0;
    __syncthreads();
    bool big = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c < ncu) {
            if (v[c] >= 0 && v[c] < S)
                atomicAdd(&L.cnt[v[c]], 1);
            big |= v[c] >= S;
        }
    }
    if (first) {
        const uint64_t bigm = __ballot(big);
        if (bigm && lane == 0)
            atomicOr(pb.flags, LORA_FLAG_SLOT_INDEX_TOO_LARGE);
    }
    __syncthreads();
    if (wave == 0) {
        if (S <= 64) {
            // lane l takes slot l: count, tiles, and exclusive prefixes
            const int c1 = lane < S ? L.cnt[lane] : 0;
            const int n1 = (c1 + cap - 1) / cap;
            const int ic = wave_incl_scan(c1), in = wave_incl_scan(n1);
            const int pc = ic - c1, pn = in - n1;
            if (lane < S && b >= pn && b < pn + n1) {
                L.slot = lane;
                L.j = b - pn;
                L.start = pc;
                L.count = c1;
            }
            if (first && lane < S) {
                pb.counts[lane] = c1;
                pb.seg_start[lane] = pc;
            }
            if (lane == 63) {
                L.n_tiles = in;
                if (first) {
                    *pb.n_tiles = in;
                    *pb.n_active = ic;
                }
            }
        } else {
            // lane l takes slots 4l .. 4l+3
            int c4[4], n4[4], sc = 0, sn = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int sl = 4 * lane + k;
                c4[k] = sl < S ? L.cnt[sl] : 0;
                n4[k] = (c4[k] + cap - 1) / cap;
                sc += c4[k];
                sn += n4[k];
            }
            const int ic = wave_incl_scan(sc), in = wave_incl_scan(sn);
            int pc = ic - sc, pn = in - sn;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int sl = 4 * lane + k;
                if (sl < S) {
                    if (b >= pn && b < pn + n4[k]) {
                        L.slot = sl;
                        L.j = b - pn;
                        L.start = pc;
                        L.count = c4[k];
                    }
                    if (first) {
                        pb.counts[sl] = c4[k];
                        pb.seg_start[sl] = pc;
                    }
                }
                pc += c4[k];
                pn += n4[k];
            }
            if (lane == 63) {
                L.n_tiles = in;
                if (first) {
                    *pb.n_tiles = in;
                    *pb.n_active = ic;
                }
            }
        }
    }
    __syncthreads();
    if (b >= L.n_tiles)
        return false;
    const int sl = L.slot, j = L.j;
    uint64_t mk[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        mk[c] = 0;
        if (c < ncu) {
            mk[c] = __ballot(v[c] == sl);
            if (lane == 0)
                L.wc[c * 4 + wave] = __popcll(mk[c]);
        }
    }
    __syncthreads();
    // window c*4 + wave holds tokens c*256 + 64*wave .. +63, so windows in index
    // order are tokens in order
    int pre[NC], before = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c)
        pre[c] = 0;
#pragma unroll
    for (int w = 0; w < kInlinePlanTokens / 64; ++w) {
        if (w < 4 * ncu) {
            const int k = L.wc[w];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (w == c * 4 + wave)
                    pre[c] = before;
            before += k;
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c < ncu && v[c] == sl) {
            const int r = pre[c] - j * cap +
                          (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk[c] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mk[c], 0u));
            if (r >= 0 && r < cap)
                L.list[r] = c * 256 + tid;
        }
    }
    __syncthreads();
    tile.slot = sl;
    tile.start = L.start + j * cap;
    tile.len = min(cap, L.count - j * cap);
    tile.rank = meta_rank(mr, sl);
    tile.scale = meta_scale(mr, sl);
    tokv = lane < tile.len ? L.list[lane] : 0;
    if (publish) {
        if (tid == 0)
            pb.tiles[b] = tile;
        if (tid < tile.len)
            pb.tile_tok[(int64_t)b * kTileTokens + tid] = L.list[tid];
    }
    return true;
}

// Tiles of more than this many tokens take the segment path: their A^T blocks
// are shared by two to four waves, so staging them once in LDS saves the L2
// reads of the other waves.
constexpr int kSegmentMinTokens = 16;

// LDS of a shrink workgroup: K-split reduction, or the segment path's A stage.
constexpr int shrink_smem_bytes(int NB)
{
    return cmax(4 * NB * 64 * 16, 2 * NB * 16 * kLdsRow * 2);
}

// The shrink of one tile for K split `split` of member m: writes the member's h
// partial of that split for the tile's rows.  Requires 0 < tile.rank.
template <int NB, bool MIXED>
__device__ __forceinline__ void shrink_tile(const ShrinkArgs &a, int m, int split, const Tile &tile,
                                            int tokv, unsigned char *smem)
{
    const int nb = (tile.rank + 15) >> 4;
    ShrinkView v;
    v.d_in = a.d_in[m];
    v.x = (const uint16_t *)a.x[m];
    v.A = (const uint16_t *)a.A[m] + (int64_t)tile.slot * a.slot_stride_A[m];
    v.k0 = split * a.k_chunk[m];
    v.k1 = min((int)v.d_in, v.k0 + a.k_chunk[m]);
    v.h = a.hpart + m * a.member_stride + (int64_t)split * a.split_stride;
    v.R_pad = a.R_pad;
    if (tile.len > kSegmentMinTokens) {
        // the segment loop sized to the tile's own rank blocks: a wider one
        // would load (clamped) A^T rows past them on every K block
        if (NB >= 2 && nb <= 1)
            shrink_sgmv<1>(v, tile, tokv, nb, (uint16_t *)smem);
        else if (NB >= 4 && nb <= 2)
            shrink_sgmv<(NB >= 4 ? 2 : NB)>(v, tile, tokv, nb, (uint16_t *)smem);
        else if (NB >= 8 && nb <= 4)
            shrink_sgmv<(NB >= 8 ? 4 : NB)>(v, tile, tokv, nb, (uint16_t *)smem);
        else
            shrink_sgmv<NB>(v, tile, tokv, nb, (uint16_t *)smem);
    } else
        shrink_bgmv<NB, !MIXED && NB <= 4>(v, tile, tokv, nb, smem);
}

// L2 warm-up of one (K split, member) block while the inline plan is formed.
// The workgroups of a split all run on one XCD (the host asks for this only
// when the split count is a multiple of 8), so what they touch here is in that
// XCD's L2 when their tiles load x and A^T after the plan.  The block is a list
// of rows over the split's K range: x rows of every token, then A^T rows of
// every slot (slot s, rank j is row s * R_pad + j, contiguous at stride d_in).
// Workgroup bt takes a.warm_rows of them; lane l touches one 4-byte word in
// 64-byte piece (l & 7) + 8 pj of row (l >> 3) + 32 ri.  Returns the words
// read, to be consumed by keep_warm.
constexpr int kWarmRowIters = 4, kWarmPieceIters = 2;
constexpr int kWarmLoads = kWarmRowIters * kWarmPieceIters;

__device__ __forceinline__ void warm_split(const ShrinkArgs &a, int m, int split, int bt,
                                           uint32_t (&wv)[kWarmLoads])
{
    const int d_in = a.d_in[m];
    const int k0 = split * a.k_chunk[m];
    const int lpr = split < a.splits[m] ? (min(d_in, k0 + a.k_chunk[m]) - k0 + 31) >> 5 : 0;
    const int nx = (a.warm & kWarmX) ? a.T : 0;
    const int rows = nx + ((a.warm & kWarmA) ? a.S * a.R_pad : 0);
    const int r0 = bt * a.warm_rows, r1 = min(rows, r0 + a.warm_rows);
    const uint16_t *x = (const uint16_t *)a.x[m] + k0;
    const uint16_t *A = (const uint16_t *)a.A[m] + k0;
#pragma unroll
    for (int ri = 0; ri < kWarmRowIters; ++ri) {
#pragma unroll
        for (int pj = 0; pj < kWarmPieceIters; ++pj) {
            const int row = r0 + (threadIdx.x >> 3) + 32 * ri;
            const int piece = (threadIdx.x & 7) + 8 * pj;
            // unconditional (a lane with nothing to touch reads x's first
            // word), so that the plan's wait for the slot indices need not
            // wait for these loads as well
            const bool ok = row < r1 && piece < lpr;
            const uint16_t *p = !ok ? (const uint16_t *)a.x[m]
                                : row < nx ? x + (int64_t)row * d_in + piece * 32
                                           : A + (int64_t)(row - nx) * d_in + piece * 32;
            wv[ri * kWarmPieceIters + pj] = *(const uint32_t *)p;
        }
    }
}

// Consumes the warm-up words (waits for them; no instruction is emitted).
__device__ __forceinline__ void keep_warm(const uint32_t (&wv)[kWarmLoads])
{
#pragma unroll
    for (int i = 0; i < kWarmLoads; ++i)
        asm volatile("" ::"v"(wv[i]));
}

// Tiles of 17..64 tokens take the segment path, shorter ones the gather path:
// single-buffered when MIXED (batches above 1024 tokens), else double-buffered
// when the rank allows.  PLAN: how the workgroup finds its tile (PlanMode).
// WARM: the split's block is warmed in L2 meanwhile (warm_split).
// Work item w = (tile * grid_splits + split) * n + member, in groups of n: the
// members of one (tile, K split) run back to back on one XCD, so when they
// share x (q, k and v of a layer) x comes from HBM once and from L2 after.
template <int NB, bool MIXED, int PLAN, bool WARM>
__global__ __launch_bounds__(256) void shrink_bf16_kernel(ShrinkArgs a, SlotMeta meta)
{
    touch_args<ShrinkArgs>();
    const int w = xcd_item(a.n, (int)blockIdx.x);
    if (w >= a.grid_tiles * a.grid_splits * a.n)
        return;
    const int m = w % a.n, split = (w / a.n) % a.grid_splits, bt = w / (a.n * a.grid_splits);
    const int lane = threadIdx.x & 63;
    const MetaRegs mr = load_meta_regs(meta);
    __shared__ __attribute__((aligned(16))) unsigned char lds[shrink_smem_bytes(NB)];
    Tile tile;
    int tokv;
    const bool lead = split == 0 && m == 0;     // publishes the tile
    uint32_t wv[kWarmLoads];
    if constexpr (PLAN == kPlanInline) {
        __shared__ TilePlanLds P;
        int v[kPlanPerThread];
        plan_load_idx(a.idx, a.T, v);
        if constexpr (WARM)
            warm_split(a, m, split, bt, wv);
        const bool has_tile = plan_tile(v, a.T, a.S, a.tile_cap, mr, a.plan, P, bt, lead, lead && bt == 0, tile, tokv);
        if constexpr (WARM)
            keep_warm(wv);
        if (!has_tile)
            return;
    } else {
        const int n_tiles = *a.plan.n_tiles;
        tile = a.plan.tiles[bt];              // in bounds: the tile buffer covers the grid
        tokv = a.plan.tile_tok[(int64_t)bt * kTileTokens + lane];
        // warm the split while the tile record arrives; the words are consumed
        // at the end, so no wait is added
        if constexpr (WARM)
            warm_split(a, m, split, bt, wv);
        if (bt >= n_tiles) {
            if constexpr (WARM)
                keep_warm(wv);
            return;
        }
        // lookups in code every lane runs (see meta_scale), stores by one lane
        tile.rank = meta_rank(mr, tile.slot);
        tile.scale = meta_scale(mr, tile.slot);
        if (lead && threadIdx.x == 0) {
            a.plan.tiles[bt].rank = tile.rank;
            a.plan.tiles[bt].scale = tile.scale;
        }
    }
    if (split >= a.splits[m] || tile.rank == 0 || !meta_targets(mr, m, tile.slot)) {
        if constexpr (WARM && PLAN != kPlanInline)
            keep_warm(wv);
        return;
    }
    shrink_tile<NB, MIXED>(a, m, split, tile, tokv, lds);
    if constexpr (WARM && PLAN != kPlanInline)
        keep_warm(wv);
}

// ----------------------------------------------------------------------------
// expand, bf16 on MFMA
//
// One workgroup = one tile (<= 64 tokens of one slot) x 256 columns of y x one
// group member; wave w owns the 64 columns 64w..64w+63 for every subtile of the
// tile.  The product is formed transposed, out[n][t] = sum_j B[j][n] h[t][j].
// B is stored in groups of 8 ranks, Bi[j/8][n][j%8], so the rank slice an MFMA
// lane needs is contiguous; rows of the 16x16 output blocks are mapped to
// columns so that lane group g of a wave owns 16 adjacent columns of one token,
// and y is read and written 32 bytes per lane.  Every global load of the wave
// (token ids, B, y, h partials) is issued before any arithmetic.  The K-split
// partials of h are summed once per workgroup and split into a bf16 high part
// and a bf16 low part (h - high) in LDS.  One v_mfma_f32_16x16x32_bf16 covers a
// block of 16 ranks with both parts stacked along K (lane groups 0-1 the high
// part of ranks 0-7 / 8-15, lane groups 2-3 the low part, against the same B
// values), which keeps ~16 bits of h.

// Operand loads of the expand are unconditional: a lane whose element lies
// outside the data reads the first element instead, and that value only reaches
// outputs that are never stored (rank blocks >= nb are skipped, columns >= d_out
// and rows beyond the tile are not written).  With no branch around a load the
// compiler can count outstanding loads exactly and wait only for the ones an
// instruction needs.

// B operands of one wave's 64 columns cb..cb+63: lane row -> column
// cb + (row/4)*16 + b*4 + row%4, ranks kst*16 + 8(g&1) .. +7 (one 16-byte
// group of the repacked B; lane groups g and g+2 read the same bytes).
template <int NB>
__device__ __forceinline__ void load_b_ops(uint4 (&bop)[NB][4], const uint16_t *Bslot, int d_out,
                                           int cb, int nb, bool cols_ok)
{
    const int lane = threadIdx.x & 63, row = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kst = 0; kst < NB; ++kst) {
        const int G = kst * 2 + (g & 1);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = cb + (row >> 2) * 16 + b * 4 + (row & 3);
            const bool ok = kst < nb && cols_ok && n < d_out;
            bop[kst][b] = *(const uint4 *)(Bslot + (ok ? ((int64_t)G * d_out + n) * 8 : 0));
        }
    }
}

// y of one wave: 16 adjacent columns cb + 16g.. of one token per lane and subtile.
template <int NSUB>
__device__ __forceinline__ void load_y(uint4 (&yv)[NSUB][2], const uint16_t *ybase, int d_out,
                                       int cb, const int (&tok)[NSUB], const bool (&tok_ok)[NSUB])
{
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
#pragma unroll
        for (int piece = 0; piece < 2; ++piece) {
            const int col = cb + g * 16 + piece * 8;
            const bool ok = tok_ok[st] && col < d_out;
            yv[st][piece] = *(const uint4 *)(ybase + (ok ? (int64_t)tok[st] * d_out + col : 0));
        }
    }
}

// Four h values to packed bf16 high halves and bf16 low halves (h - high).
__device__ __forceinline__ void split_hi_lo(const f32x4_t h, uint2 &hi, uint2 &lo)
{
    const uint32_t hi01 = pack_bf16x2(h[0], h[1]), hi23 = pack_bf16x2(h[2], h[3]);
    hi = make_uint2(hi01, hi23);
    lo = make_uint2(pack_bf16x2(h[0] - bf16_bits_to_f32(hi01 & 0xffffu), h[1] - bf16_bits_to_f32(hi01 >> 16)),
                    pack_bf16x2(h[2] - bf16_bits_to_f32(hi23 & 0xffffu), h[3] - bf16_bits_to_f32(hi23 >> 16)));
}

// out[n][t] = sum_j B[j][n] h[t][j] for the wave's 64 columns and the tile's
// subtiles, then y = round(y + s * out) for the rows of the tile.  hs_hi / hs_lo:
// the tile's h as bf16 high / low halves in LDS, row stride HS elements.  Rows
// beyond the tile hold stale LDS; they only reach output columns of tokens that
// are not stored.
// The output terms of an adapter for the 16 columns cb + 16g .. of a lane:
// DoRA factors (fp32) and bias (bf16), loaded only when the slot has them.
struct OutTerms {
    int fl;
    float g[16];
    uint4 c[2];
};

template <int NB, int NSUB, int HS, bool TERMS>
__device__ __forceinline__ void expand_store(const uint16_t *hs_hi, const uint16_t *hs_lo,
                                             const uint4 (&bop)[NB][4], const uint4 (&yv)[NSUB][2],
                                             const int (&tok)[NSUB], const bool (&tok_ok)[NSUB],
                                             int nsub, int nb, float s, uint16_t *ybase, int d_out,
                                             int cb, const OutTerms &ot)
{
    const int lane = threadIdx.x & 63, row = lane & 15, g = lane >> 4;
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
        if (st >= nsub)
            break;
        f32x4_t acc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kst = 0; kst < NB; ++kst) {
            if (kst < nb) {
                // lane groups 0-1: high part, 2-3: low part, of ranks kst*16 + 8(g&1) ..
                const int o = (st * 16 + row) * HS + kst * 16 + (g & 1) * 8;
                const bf16x8_t hv = __builtin_bit_cast(bf16x8_t, *(const uint4 *)((g < 2 ? hs_hi : hs_lo) + o));
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bop[kst][b]),
                                                                     hv, acc[b], 0, 0, 0);
            }
        }
        if (tok_ok[st]) {
            uint16_t *yrow = ybase + (int64_t)tok[st] * d_out;
#pragma unroll
            for (int piece = 0; piece < 2; ++piece) {
                const int col = cb + g * 16 + piece * 8;
                if (col < d_out) {
                    const uint4 yw = yv[st][piece];
                    uint32_t w[4] = {yw.x, yw.y, yw.z, yw.w};
                    const uint32_t cws[4] = {ot.c[piece].x, ot.c[piece].y, ot.c[piece].z, ot.c[piece].w};
#pragma unroll
                    for (int h2 = 0; h2 < 4; ++h2) {
                        const int e0 = piece * 8 + h2 * 2, e1 = e0 + 1;
                        float v0 = bf16_bits_to_f32(w[h2] & 0xffffu) + s * acc[e0 >> 2][e0 & 3];
                        float v1 = bf16_bits_to_f32(w[h2] >> 16) + s * acc[e1 >> 2][e1 & 3];
                        if constexpr (TERMS) {
                            if (ot.fl & kSlotDora) {
                                v0 = ot.g[e0] * v0;
                                v1 = ot.g[e1] * v1;
                            }
                            if (ot.fl & kSlotBias) {
                                v0 = v0 + bf16_bits_to_f32(cws[h2] & 0xffffu);
                                v1 = v1 + bf16_bits_to_f32(cws[h2] >> 16);
                            }
                        }
                        w[h2] = pack_bf16x2(v0, v1);
                    }
                    *(uint4 *)(yrow + col) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    }
}

// h partials of a tile for the expand, summed over the K splits in split
// order: thread tid owns quads e = tid + 256 i (i < NB) of the len x nb*16 block.
template <int NB>
__device__ __forceinline__ void load_h_sums(f32x4_t (&hsum)[NB], const ExpandArgs &a, int m,
                                            const Tile &tile, int nb)
{
    const int tid = threadIdx.x;
    const int quads = nb * 4;
    const int n_el = tile.len * quads;
    const int splits = a.splits[m];
    const float *hbase = a.hpart + m * a.member_stride;
    if (splits == 1) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int e = tid + 256 * i;
            const int t = e / quads, q = e - t * quads;
            hsum[i] = e < n_el ? *(const f32x4_t *)(hbase + (int64_t)(tile.start + t) * a.R_pad + q * 4)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    } else {
        // at most splits_cap(NB) partials per quad (the host caps the K-split so)
        constexpr int MS = splits_cap(NB);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int e = tid + 256 * i;
            const int t = e / quads, q = e - t * quads;
            f32x4_t pv[MS];
            const float *hp = hbase + (int64_t)(tile.start + t) * a.R_pad + q * 4;
#pragma unroll
            for (int u = 0; u < MS; ++u)
                pv[u] = (e < n_el && u < splits) ? *(const f32x4_t *)(hp + (int64_t)u * a.split_stride)
                                                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
            f32x4_t sum = pv[0];
#pragma unroll
            for (int u = 1; u < MS; ++u)
                sum += pv[u];
            hsum[i] = sum;
        }
    }
}

// Hand-over of a tile's h partials inside one fused launch (fused_xcd_kernel).
// A shrink workgroup, once its partial is stored and every one of its stores
// has completed, adds one to the (tile, member) count.  An expand workgroup
// waits until the count reaches the member's K-split count, with a bounded
// number of polls; past the bound it sets LORA_FLAG_FUSED_TIMEOUT and leaves
// its rows of y untouched.  Every expand workgroup of the (tile, member) then
// adds one to the consumer count, and the last one returns both counts to
// zero, so the next launch (or the next replay of a captured graph) starts
// from zero.
struct FusedWait {
    uint32_t *cnt;          // K-split partials stored so far
    uint32_t *consumed;     // expand workgroups past the wait
    int expected;           // K-splits of the member
    int consumers;          // expand workgroups of the (tile, member)
    int limit;              // polls before giving up
    uint32_t *flags;        // sticky device flags
};

// Hand-over inside one XCD (fused_xcd_kernel, where every workgroup of a tile
// runs on the tile's XCD).  The L2 is shared by the CUs of an XCD, global
// stores pass the write-through L1 into it, and atomics execute in it, so a
// count kept with workgroup-scope atomics (no cache bypass) and partials
// written with plain stores are seen by the other workgroups of the XCD at L2
// latency.  The shrink side waits until its own stores are acknowledged (they
// are in L2) before the count moves.
__device__ __forceinline__ void xcd_signal(uint32_t *cnt)
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The expand side polls the count with an atomic compare-and-swap that never
// succeeds (the count never reaches ~0u): an atomic executes in L2 and returns
// its value there, where a load could be served by a stale line of the CU's
// L1.  The partials it reads afterwards were not read on this CU earlier in
// the launch (every line of a tile's rows is read only once its count is
// complete, and tiles of adjacent rows run on other XCDs), and the L1 starts
// the launch empty of them, so plain loads return the L2 copy.
__device__ __forceinline__ bool xcd_wait(const FusedWait &fw)
{
    __shared__ int ok;
    if (threadIdx.x == 0) {
        bool done = false;
        for (int n = 0; n <= fw.limit; ++n) {
            uint32_t seen = ~0u;
            __hip_atomic_compare_exchange_strong(fw.cnt, &seen, ~0u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
            if ((int)seen >= fw.expected) {
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!done)
            atomicOr(fw.flags, LORA_FLAG_FUSED_TIMEOUT);
        const uint32_t prev = __hip_atomic_fetch_add(fw.consumed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((int)prev + 1 == fw.consumers) {
            __hip_atomic_store(fw.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(fw.consumed, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        ok = done ? 1 : 0;
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return ok != 0;
}

// The expand of one tile for the 256 columns of chunk `chunk` of member m.
// Requires 0 < tile.rank and an adapter that targets the member.  Every global
// load (h partials, B, y) is issued before any arithmetic.  FUSED (the fused
// decode kernel): B, y and the output terms are loaded first, then the
// workgroup waits for the tile's partials (fw) and reads them from the L2 of
// its XCD.
template <int NB, bool TERMS, int SUB, bool FUSED = false>
__device__ __forceinline__ void expand_tile(const ExpandArgs &a, int m, int chunk, const Tile &tile,
                                            int tokv, int flags, uint16_t *hs_hi, uint16_t *hs_lo,
                                            const FusedWait *fw = nullptr)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int d_out = a.d_out[m];
    const int cb = chunk * kExpandCols + wave * 64;
    const int nb = (tile.rank + 15) >> 4;
    const int row = lane & 15;
    const bool cols_ok = cb < d_out;
    const int nsub = (tile.len + 15) >> 4;
    uint16_t *ybase = (uint16_t *)a.y[m];

    // tokens of this lane in each subtile
    int tok[SUB];
    bool tok_ok[SUB];
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
        const int t = st * 16 + row;
        tok_ok[st] = cols_ok && t < tile.len;
        const int tv = __shfl(tokv, t, 64);
        tok[st] = tok_ok[st] ? tv : 0;
    }
    f32x4_t hsum[NB];
    if constexpr (!FUSED)
        load_h_sums<NB>(hsum, a, m, tile, nb);
    uint4 bop[NB][4];
    load_b_ops<NB>(bop, (const uint16_t *)a.Bi[m] + (int64_t)tile.slot * a.slot_stride_B[m], d_out,
                   cb, nb, cols_ok);
    uint4 yv[SUB][2];
    load_y<SUB>(yv, ybase, d_out, cb, tok, tok_ok);
    // output terms of the slot for this lane's 16 columns (clamped like y)
    OutTerms ot;
    ot.fl = flags;
    ot.c[0] = ot.c[1] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int piece = 0; piece < (TERMS ? 2 : 0); ++piece) {
        // columns col .. col+7; past d_out the slot's first columns are read
        // instead, and those outputs are not stored
        const int col = cb + (lane >> 4) * 16 + piece * 8;
        const int64_t o = (int64_t)tile.slot * d_out + (cols_ok && col < d_out ? col : 0);
        if (flags & kSlotDora) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const f32x4_t gq = *(const f32x4_t *)(a.dora[m] + o + q * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ot.g[piece * 8 + q * 4 + e] = gq[e];
            }
        }
        if (flags & kSlotBias)
            ot.c[piece] = *(const uint4 *)((const uint16_t *)a.bias[m] + o);
    }
    if constexpr (FUSED) {
        if (!xcd_wait(*fw))
            return;
        load_h_sums<NB>(hsum, a, m, tile, nb);
    }
    // h -> bf16 high and low halves in LDS
    constexpr int HS = NB * 16 + 8;             // row stride (bf16 elements, 16-byte multiple)
    const int quads = nb * 4;
    const int n_el = tile.len * quads;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int e = tid + 256 * i;
        if (e < n_el) {
            const int t = e / quads, q = e - t * quads;
            split_hi_lo(hsum[i], *(uint2 *)&hs_hi[t * HS + q * 4], *(uint2 *)&hs_lo[t * HS + q * 4]);
        }
    }
    __syncthreads();
    if (cols_ok)
        expand_store<NB, SUB, HS, TERMS>(hs_hi, hs_lo, bop, yv, tok, tok_ok, nsub, nb, tile.scale, ybase,
                                       d_out, cb, ot);
}

// LDS rows of h for SUB subtiles of 16 tokens
constexpr int expand_hs_elems(int NB, int SUB) { return SUB * 16 * (NB * 16 + 8); }

// Tiles as the shrink published them, with rank and scale of the slot as that
// shrink saw them.  Member m has its own number of 256-column chunks,
// a.col_start[m + 1] - a.col_start[m].  A small batch (a.xcd_group < 0) puts
// tile t on residue t % 8 of the grid, as the fused decode does: every (member,
// chunk) of a tile runs on one XCD, which fetches the tile's K-split partials
// from HBM once instead of once per XCD (0.3 us less per Llama-7B-shaped and
// 0.6 us per Qwen-shaped decode step than dealing the items round-robin).
// Otherwise work items cover exactly the (tile, member, chunk) triples, member
// by member, so a group of members of unequal widths (q next to k and v)
// launches no empty workgroups, and are taken in XCD groups of a.xcd_group: a
// large batch gives each XCD one contiguous run of items, numbered
// chunk * grid_tiles + tile, or, with long slot segments (a.tile_major),
// tile * chunks + chunk: then all column chunks of a tile run on one XCD, so
// the tile's h is fetched from HBM once, and consecutive tiles (mostly of one
// slot) read that slot's B from the same L2.
template <int NB, bool TERMS, int SUB>
__global__ __launch_bounds__(256) void expand_bf16_kernel(ExpandArgs a, SlotMeta meta)
{
    int m = 0, bt, chunk;
    if (a.xcd_group < 0) {
        // tile t on residue t % 8: every chunk of a tile on one XCD, which
        // fetches the tile's partials once
        const int x = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
        const int e_per = a.col_start[a.n];
        const int c = j % e_per;
        bt = (j / e_per) * kXcds + x;
        if (bt >= a.grid_tiles)
            return;
        while (m + 1 < a.n && c >= a.col_start[m + 1])
            ++m;
        chunk = c - a.col_start[m];
    } else {
        const int n_items = a.grid_tiles * a.col_start[a.n];
        const int w = xcd_item(a.xcd_group, (int)blockIdx.x);
        if (w >= n_items)
            return;
        while (m + 1 < a.n && w >= a.grid_tiles * a.col_start[m + 1])
            ++m;
        const int local = w - a.grid_tiles * a.col_start[m];
        const int chunks = a.col_start[m + 1] - a.col_start[m];
        bt = a.tile_major ? local / chunks : local % a.grid_tiles;
        chunk = a.tile_major ? local % chunks : local / a.grid_tiles;
    }
    const int lane = threadIdx.x & 63;
    const MetaRegs mr = load_meta_regs(meta);
    const int n_tiles = *a.n_tiles;
    const Tile tile = a.tiles[bt];              // in bounds: the tile buffer covers the grid
    const int tokv = a.tile_tok[(int64_t)bt * kTileTokens + lane];
    if (bt >= n_tiles || chunk * kExpandCols >= a.d_out[m])
        return;
    const int flags = meta_flags(mr, tile.slot);
    if (tile.rank == 0 || !meta_targets(mr, m, tile.slot))
        return;
    __shared__ __attribute__((aligned(16))) uint16_t hs_hi[expand_hs_elems(NB, SUB)];
    __shared__ __attribute__((aligned(16))) uint16_t hs_lo[expand_hs_elems(NB, SUB)];
    expand_tile<NB, TERMS, SUB>(a, m, chunk, tile, tokv, flags, hs_hi, hs_lo);
}

// ----------------------------------------------------------------------------
// fused decode with the hand-over inside each XCD.  The chip deals the
// workgroups of a launch to its XCDs in turn: workgroup i to XCD i % 8 on an
// idle chip (checked once per device at ctx creation), and to XCD (i + c) % 8
// for some c when other kernels run beside the launch.  Either way workgroups
// whose indices agree mod 8 share an XCD, which is all the hand-over needs (a
// placement that broke it would show as waits that give up, flagged, never as
// partials read before they are in).  Tile t belongs to residue t % 8, and on
// each XCD the workgroups come in the order: the
// shrink of its tiles ((K split, member) pairs, tile after tile), then their
// expand ((member, column chunk) pairs, tile after tile).  So every workgroup
// of a tile shares one L2, and the partials and counts move at L2 latency
// (xcd_signal / xcd_wait); an expand workgroup waits only for shrink
// workgroups dispatched before it on its own XCD.
template <int NB, bool TERMS, int SUB, int PLAN>
__device__ __forceinline__ void fused_xcd_body(const FusedArgs &f, const SlotMeta &meta)
{
    constexpr int kExpandLds = 2 * expand_hs_elems(NB, SUB) * 2;
    __shared__ __attribute__((aligned(16))) unsigned char lds[cmax(shrink_smem_bytes(NB), kExpandLds)];
    __shared__ TilePlanLds P;
    const int lane = threadIdx.x & 63;
    const MetaRegs mr = load_meta_regs(meta);
    const int x = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
    const int n_x = (f.s.grid_tiles - x + kXcds - 1) / kXcds;      // tiles x, x + 8, ...
    const int s_per = f.s.grid_splits * f.s.n, e_per = f.e.col_start[f.e.n];
    Tile tile;
    int tokv;
    if (j < n_x * s_per) {
        const ShrinkArgs &a = f.s;
        const int r = j % s_per;
        const int m = r % a.n, split = r / a.n, bt = (j / s_per) * kXcds + x;
        const bool lead = split == 0 && m == 0;     // publishes the tile
        if constexpr (PLAN == kPlanInline) {
            int v[kPlanPerThread];
            plan_load_idx(a.idx, a.T, v);
            if (!plan_tile(v, a.T, a.S, a.tile_cap, mr, a.plan, P, bt, lead, lead && bt == 0, tile, tokv))
                return;
        } else {
            const int n_tiles = *a.plan.n_tiles;
            tile = a.plan.tiles[bt];              // in bounds: the tile buffer covers the grid
            tokv = a.plan.tile_tok[(int64_t)bt * kTileTokens + lane];
            if (bt >= n_tiles)
                return;
            tile.rank = meta_rank(mr, tile.slot);
            tile.scale = meta_scale(mr, tile.slot);
        }
        if (split >= a.splits[m] || tile.rank == 0 || !meta_targets(mr, m, tile.slot))
            return;
        shrink_tile<NB, false>(a, m, split, tile, tokv, lds);
        xcd_signal(f.sync + (int64_t)bt * kSyncWordsPerTile + 2 * m);
    } else if (j < n_x * (s_per + e_per)) {
        const ExpandArgs &a = f.e;
        const int jj = j - n_x * s_per;
        const int c = jj % e_per, bt = (jj / e_per) * kXcds + x;
        int m = 0;
        while (m + 1 < a.n && c >= a.col_start[m + 1])
            ++m;
        const int chunk = c - a.col_start[m];
        const int chunks = a.col_start[m + 1] - a.col_start[m];
        if constexpr (PLAN == kPlanInline) {
            int v[kPlanPerThread];
            plan_load_idx(f.s.idx, f.s.T, v);
            if (!plan_tile(v, f.s.T, f.s.S, f.s.tile_cap, mr, f.s.plan, P, bt, false, false, tile, tokv))
                return;
        } else {
            const int n_tiles = *a.n_tiles;
            tile = a.tiles[bt];
            tokv = a.tile_tok[(int64_t)bt * kTileTokens + lane];
            if (bt >= n_tiles)
                return;
            tile.rank = meta_rank(mr, tile.slot);
            tile.scale = meta_scale(mr, tile.slot);
        }
        const int flags = meta_flags(mr, tile.slot);
        if (chunk * kExpandCols >= a.d_out[m] || tile.rank == 0 || !meta_targets(mr, m, tile.slot))
            return;
        uint32_t *cnt = f.sync + (int64_t)bt * kSyncWordsPerTile + 2 * m;
        const FusedWait fw{cnt, cnt + 1, a.splits[m], chunks, f.spin_limit, f.s.plan.flags};
        uint16_t *hs_hi = (uint16_t *)lds, *hs_lo = hs_hi + expand_hs_elems(NB, SUB);
        expand_tile<NB, TERMS, SUB, true>(a, m, chunk, tile, tokv, flags, hs_hi, hs_lo, &fw);
    }
}

template <int NB, bool TERMS, int SUB, int PLAN>
__global__ __launch_bounds__(256) void fused_xcd_kernel(FusedArgs f, SlotMeta meta)
{
    fused_xcd_body<NB, TERMS, SUB, PLAN>(f, meta);
}

// The same for rank blocks of 16, tiles of 32 tokens and no output terms, held
// to 128 registers a lane so that four waves fit each SIMD: four workgroups a
// CU, so the whole grid of a Llama-7B-shaped decode group is resident at once
// (at three, a quarter of its expand workgroups started only as shrink
// workgroups retired).  This instance fits without spilling; the wider ones
// do not.
template <int PLAN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void fused_xcd_r16_kernel(
    FusedArgs f, SlotMeta meta)
{
    fused_xcd_body<1, false, 2, PLAN>(f, meta);
}

// ----------------------------------------------------------------------------
// fp32 on VALU (same grids and h layout as the bf16 kernels)

__global__ __launch_bounds__(256) void shrink_f32_kernel(ShrinkArgs a, SlotMeta meta)
{
    const int n_tiles = *a.plan.n_tiles;
    const Tile tile = a.plan.tiles[blockIdx.x];
    const int m = blockIdx.z;
    if ((int)blockIdx.x >= n_tiles || (int)blockIdx.y >= a.splits[m])
        return;
    const int rank = member_rank(meta, m, tile.slot);
    if (rank == 0)
        return;
    const int d_in = a.d_in[m];
    const int k0 = blockIdx.y * a.k_chunk[m];
    const int k1 = min(d_in, k0 + a.k_chunk[m]);
    const int tid = threadIdx.x;
    const float *x = (const float *)a.x[m];
    const float *Aslot = (const float *)a.A[m] + (int64_t)tile.slot * a.slot_stride_A[m];
    const int32_t *tok_row = a.plan.tile_tok + (int64_t)blockIdx.x * kTileTokens;
    __shared__ float xs[kTileTokens][33];
    __shared__ float as[LORA_MAX_RANK_PAD][33];
    __shared__ int toks[kTileTokens];
    if (tid < kTileTokens)
        toks[tid] = tid < tile.len ? tok_row[tid] : 0;
    const int npairs = tile.len * rank;   // <= 64 * 128 = 32 per thread
    // fp64 accumulation over the split's K range (products of two fp32 values
    // are exact in fp64): with fp32 sums the rounding error of h, multiplied by
    // a large scale (rsLoRA at high rank, s = alpha / sqrt(r) ~ 20), exceeds
    // 1e-5 of y in the tails of a batch
    double acc[32];
#pragma unroll
    for (int q = 0; q < 32; ++q)
        acc[q] = 0.0;
    __syncthreads();
    for (int kc = k0; kc < k1; kc += 32) {
        for (int e = tid; e < kTileTokens * 32; e += 256) {
            const int t = e >> 5, kk = e & 31;
            xs[t][kk] = (t < tile.len && kc + kk < k1) ? x[(int64_t)toks[t] * d_in + kc + kk] : 0.f;
        }
        for (int e = tid; e < rank * 32; e += 256) {
            const int j = e >> 5, kk = e & 31;
            as[j][kk] = kc + kk < k1 ? Aslot[(int64_t)j * d_in + kc + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int e = tid + q * 256;
            if (e < npairs) {
                const int t = e / rank, j = e % rank;
                double sacc = acc[q];
                for (int kk = 0; kk < 32; ++kk)
                    sacc = fma((double)xs[t][kk], (double)as[j][kk], sacc);
                acc[q] = sacc;
            }
        }
        __syncthreads();
    }
    float *hp = a.hpart + m * a.member_stride + (int64_t)blockIdx.y * a.split_stride;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
        const int e = tid + q * 256;
        if (e < npairs) {
            const int t = e / rank, j = e % rank;
            hp[(int64_t)(tile.start + t) * a.R_pad + j] = (float)acc[q];
        }
    }
}

__global__ __launch_bounds__(256) void expand_f32_kernel(ExpandArgs a, SlotMeta meta)
{
    const int n_tiles = *a.n_tiles;
    const Tile tile = a.tiles[blockIdx.x];
    const int m = blockIdx.z;
    const int d_out = a.d_out[m];
    if ((int)blockIdx.x >= n_tiles || (int)blockIdx.y * kExpandCols >= d_out)
        return;
    const int rank = member_rank(meta, m, tile.slot);
    if (rank == 0)
        return;
    const float s = meta.scale[tile.slot];
    const int tid = threadIdx.x;
    const float *hbase = a.hpart + m * a.member_stride;
    __shared__ float hs[kTileTokens][LORA_MAX_RANK_PAD + 1];
    for (int e = tid; e < tile.len * rank; e += 256) {
        const int t = e / rank, j = e % rank;
        const float *hp = hbase + (int64_t)(tile.start + t) * a.R_pad + j;
        float v = 0.f;
        for (int sp = 0; sp < a.splits[m]; ++sp)
            v += hp[(int64_t)sp * a.split_stride];
        hs[t][j] = v;
    }
    __syncthreads();
    const int n = blockIdx.y * kExpandCols + tid;
    if (n >= d_out)
        return;
    const float *Bslot = (const float *)a.Bi[m] + (int64_t)tile.slot * a.slot_stride_B[m];
    const int32_t *tok_row = a.tile_tok + (int64_t)blockIdx.x * kTileTokens;
    float acc[kTileTokens];
#pragma unroll
    for (int t = 0; t < kTileTokens; ++t)
        acc[t] = 0.f;
    for (int j = 0; j < rank; ++j) {
        const float bj = Bslot[((int64_t)(j >> 3) * d_out + n) * 8 + (j & 7)];
#pragma unroll
        for (int t = 0; t < kTileTokens; ++t)
            if (t < tile.len)
                acc[t] += hs[t][j] * bj;
    }
    float *y = (float *)a.y[m];
    const int fl = meta.flags[tile.slot];
    const float gn = (fl & kSlotDora) ? a.dora[m][(int64_t)tile.slot * d_out + n] : 1.f;
    const float cn = (fl & kSlotBias) ? ((const float *)a.bias[m])[(int64_t)tile.slot * d_out + n] : 0.f;
#pragma unroll
    for (int t = 0; t < kTileTokens; ++t) {
        if (t < tile.len) {
            const int64_t o = (int64_t)tok_row[t] * d_out + n;
            float v = y[o] + s * acc[t];
            if (fl & kSlotDora)
                v = gn * v;
            if (fl & kSlotBias)
                v = v + cn;
            y[o] = v;
        }
    }
}

// ----------------------------------------------------------------------------
// launches

// Workgroups for n work items in XCD groups of G (xcd_item): whole rounds of
// 8 groups.
static dim3 xcd_grid(int64_t n, int G)
{
    const int64_t groups = (n + G - 1) / G;
    return dim3((unsigned)((groups + kXcds - 1) / kXcds * kXcds * G));
}

template <bool MIXED, int PLAN, bool WARM = false>
static void launch_shrink_bf16(const ShrinkArgs &a, const SlotMeta &m, dim3 grid, hipStream_t st,
                               const LaunchTiming &t)
{
    const int nbmax = a.R_pad / 16;
    if (nbmax <= 1)
        launch(shrink_bf16_kernel<1, MIXED, PLAN, WARM>, grid, dim3(256), 0, st, t, a, m);
    else if (nbmax <= 2)
        launch(shrink_bf16_kernel<2, MIXED, PLAN, WARM>, grid, dim3(256), 0, st, t, a, m);
    else if (nbmax <= 4)
        launch(shrink_bf16_kernel<4, MIXED, PLAN, WARM>, grid, dim3(256), 0, st, t, a, m);
    else
        launch(shrink_bf16_kernel<8, MIXED, PLAN, WARM>, grid, dim3(256), 0, st, t, a, m);
}

hipError_t launch_shrink(bool bf16, const ShrinkArgs &a, const SlotMeta &m, hipStream_t st,
                         const LaunchTiming &t)
{
    const dim3 grid(a.grid_tiles, a.grid_splits, a.n), block(256);
    const dim3 g = xcd_grid((int64_t)a.grid_tiles * a.grid_splits * a.n, a.n);
    if (!bf16)
        launch(shrink_f32_kernel, grid, block, 0, st, t, a, m);
    else if (a.plan_mode == kPlanInline)
        a.warm ? launch_shrink_bf16<false, kPlanInline, true>(a, m, g, st, t)
               : launch_shrink_bf16<false, kPlanInline, false>(a, m, g, st, t);
    else if (a.mixed)
        launch_shrink_bf16<true, kPlanTiles>(a, m, g, st, t);
    else if (a.warm)
        launch_shrink_bf16<false, kPlanTiles, true>(a, m, g, st, t);
    else
        launch_shrink_bf16<false, kPlanTiles>(a, m, g, st, t);
    return hipGetLastError();
}

// SUB: 16-token subtiles per tile, from the plan's tile size (a tile never
// holds more than 16 SUB tokens).  Tiles of 32 tokens come only with rank 16
// (one rank block), tiles of 48 only above it.
template <bool TERMS>
static void launch_expand_bf16(const ExpandArgs &a, const SlotMeta &m, dim3 grid, hipStream_t st,
                               const LaunchTiming &t)
{
    const int nbmax = a.R_pad / 16;
    const int sub = (a.tile_cap + 15) / 16;
    const dim3 block(256);
    if (nbmax <= 1) {
        if (sub <= 2)
            launch(expand_bf16_kernel<1, TERMS, 2>, grid, block, 0, st, t, a, m);
        else
            launch(expand_bf16_kernel<1, TERMS, 4>, grid, block, 0, st, t, a, m);
    } else if (nbmax <= 2) {
        if (sub <= 3)
            launch(expand_bf16_kernel<2, TERMS, 3>, grid, block, 0, st, t, a, m);
        else
            launch(expand_bf16_kernel<2, TERMS, 4>, grid, block, 0, st, t, a, m);
    } else if (nbmax <= 4) {
        if (sub <= 3)
            launch(expand_bf16_kernel<4, TERMS, 3>, grid, block, 0, st, t, a, m);
        else
            launch(expand_bf16_kernel<4, TERMS, 4>, grid, block, 0, st, t, a, m);
    } else {
        if (sub <= 3)
            launch(expand_bf16_kernel<8, TERMS, 3>, grid, block, 0, st, t, a, m);
        else
            launch(expand_bf16_kernel<8, TERMS, 4>, grid, block, 0, st, t, a, m);
    }
}

hipError_t launch_expand(bool bf16, const ExpandArgs &a, const SlotMeta &m, hipStream_t st,
                         const LaunchTiming &t)
{
    const dim3 grid(a.grid_tiles, a.grid_cols, a.n), block(256);
    if (!bf16) {
        launch(expand_f32_kernel, grid, block, 0, st, t, a, m);
    } else {
        const dim3 g = a.xcd_group < 0
                           ? dim3((unsigned)(((a.grid_tiles + kXcds - 1) / kXcds) * a.col_start[a.n] * kXcds))
                           : xcd_grid((int64_t)a.grid_tiles * a.col_start[a.n], a.xcd_group);
        // the output-term epilogue only in launches where some slot has terms
        if (a.terms)
            launch_expand_bf16<true>(a, m, g, st, t);
        else
            launch_expand_bf16<false>(a, m, g, st, t);
    }
    return hipGetLastError();
}

template <bool TERMS, int PLAN>
static void launch_fused_xcd(const FusedArgs &f, const SlotMeta &m, dim3 grid, hipStream_t st,
                             const LaunchTiming &t)
{
    const int nbmax = f.s.R_pad / 16;
    const int sub = (f.e.tile_cap + 15) / 16;
    const dim3 block(256);
    if (nbmax <= 1) {
        if (sub <= 2 && !TERMS)
            launch(fused_xcd_r16_kernel<PLAN>, grid, block, 0, st, t, f, m);
        else if (sub <= 2)
            launch(fused_xcd_kernel<1, TERMS, 2, PLAN>, grid, block, 0, st, t, f, m);
        else
            launch(fused_xcd_kernel<1, TERMS, 4, PLAN>, grid, block, 0, st, t, f, m);
    } else if (nbmax <= 2) {
        if (sub <= 3)
            launch(fused_xcd_kernel<2, TERMS, 3, PLAN>, grid, block, 0, st, t, f, m);
        else
            launch(fused_xcd_kernel<2, TERMS, 4, PLAN>, grid, block, 0, st, t, f, m);
    } else if (nbmax <= 4) {
        if (sub <= 3)
            launch(fused_xcd_kernel<4, TERMS, 3, PLAN>, grid, block, 0, st, t, f, m);
        else
            launch(fused_xcd_kernel<4, TERMS, 4, PLAN>, grid, block, 0, st, t, f, m);
    } else {
        if (sub <= 3)
            launch(fused_xcd_kernel<8, TERMS, 3, PLAN>, grid, block, 0, st, t, f, m);
        else
            launch(fused_xcd_kernel<8, TERMS, 4, PLAN>, grid, block, 0, st, t, f, m);
    }
}

hipError_t launch_fused(const FusedArgs &f, const SlotMeta &m, hipStream_t st, const LaunchTiming &t)
{
    // every XCD runs the shrink and expand items of ceil(grid_tiles / 8) tiles
    // (XCDs with fewer tiles leave their last items idle)
    const int64_t per_xcd = (int64_t)((f.s.grid_tiles + kXcds - 1) / kXcds) *
                            (f.s.grid_splits * f.s.n + f.e.col_start[f.e.n]);
    const dim3 grid((unsigned)(per_xcd * kXcds));
    const bool inl = f.s.plan_mode == kPlanInline;
    if (f.e.terms)
        inl ? launch_fused_xcd<true, kPlanInline>(f, m, grid, st, t)
            : launch_fused_xcd<true, kPlanTiles>(f, m, grid, st, t);
    else
        inl ? launch_fused_xcd<false, kPlanInline>(f, m, grid, st, t)
            : launch_fused_xcd<false, kPlanTiles>(f, m, grid, st, t);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// slot maintenance

// Copy A^T (r x d_in) into the slot, repack B (r x d_out, row-major) into
// groups of 8 ranks, Bi[j/8][n][j%8], zero ranks r..R_pad-1 of both, and copy
// the output terms given in place; module blockIdx.y of the batch.  The
// sources are the caller's weights when the device can read them in place (pinned host memory over the link, or
// device memory), else their staged copies.  Every read is a 16-byte piece of
// a source row, consecutive lanes taking consecutive pieces, so a wave reads
// 1 KB of one row per instruction: link reads need such runs.  Rows are
// 16-byte multiples (d_in, d_out multiples of 8).
template <typename E>
__global__ void slot_finalize_kernel(FinalizeBatch fb)
{
    constexpr int C = 16 / (int)sizeof(E);          // columns per 16-byte piece
    const FinalizeItem &it = fb.it[blockIdx.y];
    E *A_slot = (E *)it.A_slot, *Bi_slot = (E *)it.Bi_slot;
    const int d_in = it.d_in, d_out = it.d_out, r = fb.r, R_pad = fb.R_pad;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nA16 = (int64_t)r * d_in * (int64_t)sizeof(E) / 16;
    for (int64_t o = first; o < nA16; o += stride)
        ((uint4 *)A_slot)[o] = ((const uint4 *)it.A_src)[o];
    // B: item o = (rank group G, column piece q); it reads piece q of the group's
    // rows below r and writes Bi[G][qC .. qC+C-1][0..7], C * 16 contiguous bytes
    const int pieces = d_out / C;
    const int64_t nB = (int64_t)(R_pad / 8) * pieces;
    const E *B_src = (const E *)it.B_src;
    for (int64_t o = first; o < nB; o += stride) {
        const int G = (int)(o / pieces), q = (int)(o - (int64_t)G * pieces);
        union Piece {
            uint4 u;
            E e[C];
        } row[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int j = G * 8 + w;
            row[w].u = j < r ? *(const uint4 *)(B_src + (int64_t)j * d_out + (int64_t)q * C)
                             : make_uint4(0, 0, 0, 0);
        }
        E *out = Bi_slot + ((int64_t)G * d_out + (int64_t)q * C) * 8;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            union Piece lo, hi;         // ranks 0..7 of column qC + c (hi: fp32 ranks 4..7)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                if (w < C)
                    lo.e[w] = row[w].e[c];
                else
                    hi.e[w - C] = row[w].e[c];
            }
            *(uint4 *)(out + c * 8) = lo.u;
            if (C < 8)
                *(uint4 *)(out + c * 8 + C) = hi.u;
        }
    }
    const int64_t nZ16 = (int64_t)(R_pad - r) * d_in * (int64_t)sizeof(E) / 16;
    uint4 *A_pad = (uint4 *)(A_slot + (int64_t)r * d_in);
    for (int64_t o = first; o < nZ16; o += stride)
        A_pad[o] = make_uint4(0, 0, 0, 0);
    // output terms read in place: d_out values each, in 16-byte pieces
    if (it.bias_src) {
        const int64_t n16 = (int64_t)d_out * (int64_t)sizeof(E) / 16;
        for (int64_t o = first; o < n16; o += stride)
            ((uint4 *)it.bias_dst)[o] = ((const uint4 *)it.bias_src)[o];
    }
    if (it.dora_src) {
        const int64_t n16 = (int64_t)d_out * 4 / 16;
        for (int64_t o = first; o < n16; o += stride)
            ((uint4 *)it.dora_dst)[o] = ((const uint4 *)it.dora_src)[o];
    }
}

// ----------------------------------------------------------------------------
// static scratch of the calls that allocate nothing

// One batch's plan buffers and h partials for lora_apply_group_noalloc.  The
// host never uses this name as an address: it is a host-side stand-in.  The
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};
}  // namespace

// Placement probe.  state[r] (r < 8) records 1 + the XCD of the first
// workgroup of residue r mod 8 to get there; state[8] counts workgroups that
// find their residue on another XCD.  The XCD of the executing wave is
// HW_REG_XCC_ID (hardware register 20), bits 3:0.
__global__ void xcd_check_kernel(uint32_t *state)
{
    if (threadIdx.x == 0) {
        const uint32_t id = 1u + (__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 0xfu);
        const uint32_t seen = atomicCAS(&state[blockIdx.x % kXcds], 0u, id);
        if (seen != 0u && seen != id)
            atomicAdd(&state[kXcds], 1u);
    }
}

namespace {
std::mutex g_xcd_mu;
int g_xcd_state[kScratchDevices] = {};     // 0 unknown, 1 holds, 2 does not
}  // namespace

// Whether the workgroups of a launch whose indices agree mod 8 share an XCD
// (the deal may start at any XCD when other kernels run, so the probe checks
// that, not i % 8 itself): two launches of several workgroups per CU, with
// workgroups of 256 and of 1024 threads, each against cleared state.
hipError_t xcd_dispatch_check(int device, hipStream_t st, bool *ok)
{
    if (device < 0 || device >= kScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_xcd_mu);
    if (g_xcd_state[device] == 0) {
        constexpr size_t kWords = kXcds + 1;
        uint32_t *d = nullptr, h[2][kWords] = {};
        hipError_t e = hipMalloc(&d, 2 * kWords * sizeof(uint32_t));
        if (e == hipSuccess)
            e = hipMemsetAsync(d, 0, 2 * kWords * sizeof(uint32_t), st);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(xcd_check_kernel, dim3(4096), dim3(256), 0, st, d);
            hipLaunchKernelGGL(xcd_check_kernel, dim3(1024), dim3(1024), 0, st, d + kWords);
            e = hipGetLastError();
        }
        if (e == hipSuccess)
            e = hipMemcpyAsync(h, d, sizeof h, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess)
            e = hipStreamSynchronize(st);
        if (d)
            (void)hipFree(d);
        if (e != hipSuccess)
            return e;
        g_xcd_state[device] = h[0][kXcds] == 0 && h[1][kXcds] == 0 ? 1 : 2;
    }
    *ok = g_xcd_state[device] == 1;
    return hipSuccess;
}

hipError_t scratch_address(int device, void **ptr)
{
    if (device < 0 || device >= kScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

hipError_t launch_slot_finalize(bool bf16, const FinalizeBatch &b, hipStream_t st)
{
    if (b.n <= 0)
        return hipSuccess;
    // about 256 workgroups in all: reads over the link run fastest with about one
    // workgroup per CU (more of them measured up to 20% slower)
    int64_t work = 0;
    for (int i = 0; i < b.n; ++i) {
        const int64_t w = (int64_t)b.R_pad * (b.it[i].d_out > b.it[i].d_in ? b.it[i].d_out : b.it[i].d_in) / 8;
        work = w > work ? w : work;
    }
    int blocks = (int)((work + 255) / 256);
    const int cap = (256 + b.n - 1) / b.n;
    if (blocks > cap)
        blocks = cap;
    if (bf16)
        hipLaunchKernelGGL(slot_finalize_kernel<uint16_t>, dim3(blocks, b.n), dim3(256), 0, st, b);
    else
        hipLaunchKernelGGL(slot_finalize_kernel<float>, dim3(blocks, b.n), dim3(256), 0, st, b);
    return hipGetLastError();
}

}  // namespace lora
