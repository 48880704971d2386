// lora_saved.hip -- gfx950 kernels for modules an adapter saves whole
// ("modules_to_save" of the example adapter_config.json in "vLLM LoRA Resolver
// plugins explained", section 3.2).  A saved module is a complete trained copy
// of a linear; for the tokens of its adapter it takes the base module's place:
//
//     y[t, :] = round( x[t, :] . W_k^T + c_k )        (W_k: d_out x d_in)
//
// Unlike the low-rank update this is a dense contraction over d_in, so the bf16
// kernel is a segmented GEMM on the matrix cores over the batch's plan (tiles of
// at most 64 tokens of one slot, the same tiles the shrink and the expand use).
//
// bf16, any d_in (saved_bf16_kernel): one workgroup = a pair of consecutive
// plan tiles x kSavedCols output columns x one group member; wave w owns
// columns 64w .. 64w+63 for all of the run's 16-token subtiles.  The product is
// formed transposed, out[n][t] = sum_k W[n][k] x[t][k], with
// v_mfma_f32_16x16x32_bf16 (lane l gives row l & 15 of the A operand and column
// l & 15 of the B operand with the K slice 8g .. 8g+7 of lane group g = l >> 4;
// the result's rows 4g .. 4g+3 of column l & 15 land in lane l).  MFMA row i of
// block b is output column (i / 4) * 16 + b * 4 + i % 4 of the wave's 64, so
// lane group g owns 16 adjacent columns of one token and y is written 32 bytes
// per lane.  The tile's x rows (gathered by token id) are staged in LDS one
// 64-wide K block at a time, double buffered, and shared by the four waves;
// each wave streams its own W rows straight into registers, also double
// buffered.  Loads use clamped addresses, never a branch.  A launch whose
// modules all have d_in a multiple of 64 takes saved_bf16_quad_kernel instead:
// 256 x 256 tiles with x and W both staged in LDS by direct-to-LDS loads.
//
// fp32: VALU, fp64 sums (products of two fp32 values are exact in fp64), the
// same tiles; it serves fp32 contexts and exactness checks.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_internal.h"

namespace lora {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bool saved_bit(const uint32_t (&bits)[LORA_MAX_SLOTS / 32], int slot)
{
    return (bits[slot >> 5] >> (slot & 31)) & 1u;
}

// Launch, with the dispatch bracketed by t's events when it has them.
template <typename K, typename... Args>
void launch(K kernel, dim3 grid, dim3 block, hipStream_t st, const LaunchTiming &t, Args... args)
{
    if (t.start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, t.start, t.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

constexpr int kXcds = 8;
constexpr int kBK = 64;                     // K elements per staged block
constexpr int kXRow = kBK + 8;              // LDS row of the x stage (bf16 elements, padded)

// Work item of workgroup blockIdx.x: the grid is dealt round-robin to the 8
// XCDs, and XCD j takes the j-th contiguous eighth of the items, so
// consecutive items of one (member, column chunk) share that chunk's W rows in
// the XCD's L2.
__device__ __forceinline__ int saved_item(int per_xcd)
{
    return (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
}

// The member, column chunk and tile pair of work item w (pair fastest).
__device__ __forceinline__ void saved_decode(const SavedArgs &a, int w, int &m, int &chunk, int &pair)
{
    const int pairs = (a.grid_tiles + 1) / 2;
    m = 0;
    while (m + 1 < a.n && w >= pairs * a.col_start[m + 1])
        ++m;
    const int local = w - pairs * a.col_start[m];
    chunk = local / pairs;
    pair = local - chunk * pairs;
}

// One run of at most 16 SUB tokens of one slot against the slot's W: rows
// 0 .. lenA-1 are the tokens of tile A (lane l of every wave holds its row l's
// token in tokA), rows lenA .. len-1 those of tile B (tokB; SUB = 8 only).
// Each wave owns 64 of the chunk's columns; out[n][t] = sum_k W[n][k] x[t][k].
template <int SUB>
__device__ __forceinline__ void saved_run(const SavedArgs &a, int m, int chunk, int slot, int len,
                                          int lenA, int tokA, int tokB, uint16_t *xs_base)
{
    // token of run row t: both lanes' values are fetched, then one is chosen
    // (a shuffled value is the source lane's, so the choice cannot be made
    // inside the shuffle)
    auto run_tok = [&](int t) {
        const int ta = __shfl(tokA, min(t, 63), 64);
        const int tb = __shfl(tokB, max(t - lenA, 0) & 63, 64);
        return t < lenA ? ta : tb;
    };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, g = lane >> 4;
    constexpr int kRows = SUB * 16;
    constexpr int kXBuf = kRows * kXRow;
    // token of this lane's row in each subtile, and of the x rows this thread stages
    // (shuffled where every lane of the wave is active)
    int toks[SUB];
#pragma unroll
    for (int st = 0; st < SUB; ++st)
        toks[st] = run_tok(st * 16 + row);
    constexpr int kXRowsPerThread = kRows / 64;    // x rows each thread stages per block
    const int xk = (tid & 3) * 16;
    const int d_in = a.d_in[m], d_out = a.d_out[m];
    const int cb = chunk * kSavedCols + wave * 64;
    const uint16_t *x = (const uint16_t *)a.x[m];
    const uint16_t *W = (const uint16_t *)a.W[m] + (int64_t)slot * a.slot_stride_W[m];
    const uint16_t *xsrc[kXRowsPerThread];
    int xr[kXRowsPerThread];
#pragma unroll
    for (int h2 = 0; h2 < kXRowsPerThread; ++h2) {
        xr[h2] = (tid >> 2) + 64 * h2;
        const int tok = run_tok(xr[h2]);
        // rows past the run read token 0's row (finite; those outputs are not stored)
        xsrc[h2] = x + (int64_t)(xr[h2] < len ? tok : 0) * d_in;
    }
    // W rows of this lane: block b, MFMA row `row` -> column cb + (row/4)*16 + b*4 + row%4
    // (rows past d_out read the last row; those outputs are not stored)
    const uint16_t *wrow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int n = min(cb + (row >> 2) * 16 + b * 4 + (row & 3), d_out - 1);
        wrow[b] = W + (int64_t)n * d_in;
    }
    const int nkb = (d_in + kBK - 1) / kBK;
    const int kmax = d_in - 8;                          // last 16-byte piece of a row

    uint4 wr[2][2][4];     // [stage][K step of 32][block]
    uint4 xv[kXRowsPerThread][2];
    auto load_w = [&](uint4 (&dst)[2][4], int kb) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                dst[s][b] = *(const uint4 *)(wrow[b] + min(kb + s * 32 + g * 8, kmax));
    };
    auto load_x = [&](int kb) {
#pragma unroll
        for (int h2 = 0; h2 < kXRowsPerThread; ++h2)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                xv[h2][h] = *(const uint4 *)(xsrc[h2] + min(kb + xk + h * 8, kmax));
    };
    auto store_x = [&](int buf, int kb) {
#pragma unroll
        for (int h2 = 0; h2 < kXRowsPerThread; ++h2)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *(uint4 *)(&xs_base[buf * kXBuf + xr[h2] * kXRow + xk + h * 8]) =
                    kb + xk + h * 8 < d_in ? xv[h2][h] : make_uint4(0, 0, 0, 0);
    };
    f32x4_t acc[SUB][4];     // [subtile][block]
#pragma unroll
    for (int st = 0; st < SUB; ++st)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[st][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nsub = (len + 15) >> 4;
    auto mma = [&](const uint4 (&wv)[2][4], int buf) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int st = 0; st < SUB; ++st) {
                if (st < nsub) {
                    const bf16x8_t xb = __builtin_bit_cast(
                        bf16x8_t, *(const uint4 *)(&xs_base[buf * kXBuf + (st * 16 + row) * kXRow + s * 32 + g * 8]));
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc[st][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, wv[s][b]), xb, acc[st][b], 0, 0, 0);
                }
            }
        }
    };
    // prologue: block 0 into stage 0 and LDS buffer 0
    load_w(wr[0], 0);
    load_x(0);
    store_x(0, 0);
    __syncthreads();
    // two blocks per pass, so the register stages are indexed statically; the
    // loads of block i + 1 are in flight while block i is multiplied (their
    // addresses are clamped, so the last pass loads in-range data it ignores)
    for (int i = 0; i < nkb; i += 2) {
        const int k1 = (i + 1) * kBK, k2 = (i + 2) * kBK;
        load_w(wr[1], min(k1, (nkb - 1) * kBK));
        load_x(min(k1, (nkb - 1) * kBK));
        mma(wr[0], 0);
        if (i + 1 >= nkb)
            break;
        store_x(1, k1);
        __syncthreads();
        load_w(wr[0], min(k2, (nkb - 1) * kBK));
        load_x(min(k2, (nkb - 1) * kBK));
        mma(wr[1], 1);
        if (i + 2 >= nkb)
            break;
        store_x(0, k2);
        __syncthreads();
    }
    // epilogue: lane group g owns columns cb + 16g .. +15 of token st*16 + row
    const bool has_bias = saved_bit(a.has_bias[m], slot);
    const uint16_t *bias = (const uint16_t *)a.bias[m] + (int64_t)slot * d_out;
    uint16_t *y = (uint16_t *)a.y[m];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int col = cb + g * 16 + p * 8;
        if (col >= d_out)
            continue;
        uint4 cw = make_uint4(0, 0, 0, 0);
        if (has_bias)
            cw = *(const uint4 *)(bias + col);
        const uint32_t c[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int st = 0; st < SUB; ++st) {
            const int t = st * 16 + row;
            if (t >= len)
                continue;
            // columns col .. col+7 are rows 4g..4g+3 of blocks 2p and 2p+1
            const f32x4_t v0 = acc[st][2 * p], v1 = acc[st][2 * p + 1];
            uint4 o;
            o.x = pack_bf16x2(v0[0] + bf16_lo(c[0]), v0[1] + bf16_hi(c[0]));
            o.y = pack_bf16x2(v0[2] + bf16_lo(c[1]), v0[3] + bf16_hi(c[1]));
            o.z = pack_bf16x2(v1[0] + bf16_lo(c[2]), v1[1] + bf16_hi(c[2]));
            o.w = pack_bf16x2(v1[2] + bf16_lo(c[3]), v1[3] + bf16_hi(c[3]));
            *(uint4 *)(y + (int64_t)toks[st] * d_out + col) = o;
        }
    }
}

// Work item = (member, column chunk, pair of consecutive plan tiles).  A
// slot's tiles are consecutive in the plan (tiles hold up to 32, 48 or 64
// tokens), so when both tiles of a pair belong to one slot they form one run
// of up to 128 tokens, and the slot's W rows, read once per K block, serve twice the tokens
// (the kernel is bound by those reads: 0.011 instead of 0.019 bytes per flop).
// Otherwise each tile is a run of its own.
__global__ __launch_bounds__(256, 2) void saved_bf16_kernel(SavedArgs a)
{
    const int pairs = (a.grid_tiles + 1) / 2;
    const int n_items = pairs * a.col_start[a.n];
    const int w = saved_item(a.per_xcd);
    if (w >= n_items)
        return;
    int m, chunk, pair;
    saved_decode(a, w, m, chunk, pair);
    const int lane = threadIdx.x & 63;
    const int n_tiles = *a.n_tiles;
    const int bt0 = 2 * pair, bt1 = min(2 * pair + 1, a.grid_tiles - 1);   // in bounds of the tile buffer
    const Tile t0 = a.tiles[bt0], t1 = a.tiles[bt1];
    const int tok0 = a.tile_tok[(int64_t)bt0 * kTileTokens + lane];
    const int tok1 = a.tile_tok[(int64_t)bt1 * kTileTokens + lane];
    if (bt0 >= n_tiles)
        return;
    const bool has1 = 2 * pair + 1 < n_tiles;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2 * 128 * kXRow];
    if (has1 && t1.slot == t0.slot) {
        if (saved_bit(a.saved[m], t0.slot))
            saved_run<8>(a, m, chunk, t0.slot, t0.len + t1.len, t0.len, tok0, tok1, xs);
        return;
    }
    if (saved_bit(a.saved[m], t0.slot))
        saved_run<4>(a, m, chunk, t0.slot, t0.len, t0.len, tok0, tok0, xs);
    if (has1 && saved_bit(a.saved[m], t1.slot)) {
        __syncthreads();                     // the first run's last LDS reads are done
        saved_run<4>(a, m, chunk, t1.slot, t1.len, t1.len, tok1, tok1, xs);
    }
}

// One global_load_lds_dwordx4 with a wave-uniform 64-bit base and a 32-bit
// byte offset per lane, written as asm so that the compiler does not track it:
// its own tracking cannot tell the stages apart and would wait for every load
// in flight before each LDS read.  The waits for these loads are explicit
// (s_waitcnt vmcnt in the kernel); lane l writes the 16 bytes at LDS offset
// 16 l of the instruction's 1 KB, whose wave-uniform address is lds.  m0 is
// not named as clobbered: the compiler reserves it and sets it before each of
// its own uses.
__device__ __forceinline__ void dma16_off(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory");
}

// ----------------------------------------------------------------------------
// bf16 on 256 x 256 tiles, both operands staged in LDS by direct-to-LDS loads
// (modules whose d_in is a multiple of 64).
//
// Work item = (member, column chunk of 256, quad of four consecutive plan
// tiles).  The quad's consecutive tiles of one slot form a run, and run row r is
// row r % 64 of the run's tile r / 64 (rows past a tile's length are computed
// and not stored).  Eight waves (two per SIMD, so that one wave's LDS reads run
// under the other's MFMAs) tile 256 run rows x 256 columns 2 x 4: wave w takes
// rows 128 (w & 1) .. + 127 and columns 64 (w >> 1) .. + 63, 32 accumulators of
// four.  Against the 128 x 256 tile above, a CU pulls two thirds of the L2
// bytes per flop.
//
// Stage: 512 rows of 128 bytes (K = 64), so that every load request covers a
// whole 128-byte line (64-byte rows, with twice the stages, ran 10% slower).
// Rows 0 .. 255 are the run's x rows; rows 256 .. 511 the chunk's W rows in
// MFMA order: stage row 256 + c*64 + b*16 + i holds column c*64 + (i/4)*16 +
// b*4 + i%4 of the chunk, so that each MFMA operand is 16 consecutive stage rows
// and lane group g of a result owns 16 adjacent output columns.  16-byte piece p
// of stage row r sits in slot p ^ qswz(r), qswz(r) = (r & 7) ^ ((r >> 3) & 1):
// the 16 rows of an operand read fall on distinct banks whether the LDS serves
// 16 consecutive lanes of a 16-byte read together, or lanes 0-7 with lanes
// 16-23.  Two 64 KB stages alternate: halfway through block k (its second
// 32-deep half is in registers by then) the loads of block k + 2 go into block
// k's stage.
constexpr int kQRows = 256;                                  // run rows of a work item
constexpr int kQBK = 64;                                     // K elements per stage row
constexpr int kQStageBytes = (kQRows + kSavedCols) * kQBK * 2;   // 64 KB
constexpr int kQThreads = 512;
constexpr int kQBlockQuads = 4, kQBlockCols = 8;             // an L2 block of work items
constexpr int kQBlockItems = kQBlockQuads * kQBlockCols;
// direct-to-LDS loads per wave per block (1 KB each: 8 stage rows)
constexpr int kQLoads = (kQRows + kSavedCols) * kQBK * 2 / 1024 / (kQThreads / 64);
static_assert(kQLoads == 8, "loads per wave per block");

__device__ __forceinline__ int qswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Work item w -> (member, column chunk, quad).  Per member, the (quad, chunk)
// grid is padded to whole blocks of kQBlockQuads x kQBlockCols and laid out
// block after block, chunk fastest inside a block: the items an XCD runs at one
// time (one per CU) then share four quads of x rows and eight chunks of W rows
// in its L2.  Returns false for padding.
__device__ __forceinline__ bool quad_decode(const SavedArgs &a, int w, int &m, int &chunk, int &quad)
{
    const int quads = (a.grid_tiles + 3) >> 2;
    const int qb = (quads + kQBlockQuads - 1) / kQBlockQuads;
    int base = 0;
    for (m = 0; m < a.n; ++m) {
        const int cols = a.col_start[m + 1] - a.col_start[m];
        const int cb = (cols + kQBlockCols - 1) / kQBlockCols;
        const int items = qb * cb * kQBlockItems;
        if (w < base + items) {
            const int local = w - base;
            const int blk = local / kQBlockItems, in = local % kQBlockItems;
            quad = (blk / cb) * kQBlockQuads + in / kQBlockCols;
            chunk = (blk % cb) * kQBlockCols + in % kQBlockCols;
            return quad < quads && chunk < cols;
        }
        base += items;
    }
    return false;
}

__global__ __launch_bounds__(kQThreads, 1) void saved_bf16_quad_kernel(SavedArgs a)
{
    int m, chunk, quad;
    if (!quad_decode(a, saved_item(a.per_xcd), m, chunk, quad))
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = lane & 15, g = lane >> 4;
    const int n_tiles = *a.n_tiles;
    const int bt0 = 4 * quad;
    if (bt0 >= n_tiles)
        return;
    __shared__ __attribute__((aligned(16))) unsigned char stages[2 * kQStageBytes];
    __shared__ int32_t qtok[4][kTileTokens];
    __shared__ int32_t qslot[4], qlen[4];
    if (tid < 4 * kTileTokens) {
        // tile q of the quad (clamped into the tile buffer): tokens, slot, length
        const int q = tid >> 6, bt = min(bt0 + q, a.grid_tiles - 1);
        qtok[q][lane] = a.tile_tok[(int64_t)bt * kTileTokens + lane];
        if (lane == 0) {
            const Tile t = a.tiles[bt];
            qslot[q] = t.slot;
            qlen[q] = t.len;
        }
    }
    __syncthreads();
    const int nq = min(4, n_tiles - bt0);
    const int d_in = a.d_in[m], d_out = a.d_out[m];
    const int nkb = d_in / kQBK;
    const int th = wave & 1, cq = wave >> 1;
    const uint32_t sbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)stages;
    const uint16_t *x = (const uint16_t *)a.x[m];
    int q0 = 0;
    while (q0 < nq) {
        const int slot = qslot[q0];
        int q1 = q0 + 1;
        while (q1 < nq && qslot[q1] == slot)
            ++q1;
        if (!saved_bit(a.saved[m], slot)) {
            q0 = q1;
            continue;
        }
        // run row r -> token, or -1 past the run or its tile
        auto run_tok = [&](int r) {
            const int q = q0 + (r >> 6), p = r & 63;
            return (q < q1 && p < qlen[q]) ? qtok[q][p] : -1;
        };
        // this lane's rows of the wave's direct-to-LDS loads of a block:
        // load i fills stage rows 8 j .. 8 j + 7, j = wave + 8 i, lane l row
        // 8 j + l / 8 and slot l % 8 (piece (l % 8) ^ qswz(row))
        // (byte offsets from the x or the slot's W base, kept in 32 bits: the
        // launch takes this kernel only when both fit)
        uint32_t src[kQLoads];
        const uint16_t *W = (const uint16_t *)a.W[m] + (int64_t)slot * a.slot_stride_W[m];
#pragma unroll
        for (int i = 0; i < kQLoads; ++i) {
            const int srow = 8 * (wave + 8 * i) + (lane >> 3);
            const int piece = (lane & 7) ^ qswz(srow);
            if (srow < kQRows) {
                const int tok = run_tok(srow);
                src[i] = ((uint32_t)(tok < 0 ? 0 : tok) * (uint32_t)d_in + piece * 8) * 2u;
            } else {
                const int rho = srow - kQRows, c = rho >> 6, b = (rho >> 4) & 3, ii = rho & 15;
                const int n = min(chunk * kSavedCols + c * 64 + (ii >> 2) * 16 + b * 4 + (ii & 3), d_out - 1);
                src[i] = ((uint32_t)n * (uint32_t)d_in + piece * 8) * 2u;
            }
        }
        auto dma_block = [&](int stage, int kb) __attribute__((always_inline)) {
            const uint32_t base = sbase + (uint32_t)stage * kQStageBytes + (uint32_t)wave * 1024u;
#pragma unroll
            for (int i = 0; i < kQLoads; ++i)
                dma16_off(8 * (wave + 8 * i) < kQRows ? (const void *)x : (const void *)W,
                          src[i] + (uint32_t)kb * 2u, base + (uint32_t)i * 8192u);
        };
        // fragments: x subtile st of a block (run rows th*128 + st*16 ..) and
        // W block b (stage rows 256 + cq*64 + b*16 ..)
        auto x_frag = [&](int stage, int st, int s) __attribute__((always_inline)) {
            const int r = th * 128 + st * 16 + row;
            return *(const uint4 *)(stages + stage * kQStageBytes + r * 128 + (((s * 4 + g) ^ qswz(r)) << 4));
        };
        auto w_frag = [&](int stage, int b, int s) __attribute__((always_inline)) {
            const int r = kQRows + cq * 64 + b * 16 + row;
            return *(const uint4 *)(stages + stage * kQStageBytes + r * 128 + (((s * 4 + g) ^ qswz(r)) << 4));
        };
        f32x4_t acc[8][4];     // [x subtile][W block]
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[st][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint4 X[8], Wf[4];
        // Block k, with the fragments of its first 32-deep half in X and Wf:
        // multiply that half subtile by subtile, reading the second half's x
        // fragment of each subtile once the subtile is done with the first's
        // (its W fragments before); then wait for this wave's loads of block
        // k + 1 and its reads of block k, meet the other waves (their loads of
        // block k + 1 are in, their reads of block k are done), load block
        // k + 2 into block k's stage, and multiply the second half while
        // reading block k + 1's first.  After the last block those reads fetch
        // a stale stage that nothing uses, and a wave whose rows are all past
        // the run multiplies what is never stored, so the multiply code has no
        // branches.
        if (q0 > 0)
            __syncthreads();     // the previous run's last fragment reads are done
        dma_block(0, 0);
        if (nkb > 1)
            dma_block(1, kQBK);
        if (nkb > 1)
            asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int st = 0; st < 8; ++st)
            X[st] = x_frag(0, st, 0);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            Wf[b] = w_frag(0, b, 0);
        for (int k = 0; k < nkb; ++k) {
            const int cs = k & 1, ns = cs ^ 1;
            uint4 Wn[4];
            // sub-step 0 of block k; read sub-step 1's fragments
#pragma unroll
            for (int b = 0; b < 4; ++b)
                Wn[b] = w_frag(cs, b, 1);
#pragma unroll
            for (int st = 0; st < 8; ++st) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[st][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, Wf[b]), __builtin_bit_cast(bf16x8_t, X[st]), acc[st][b],
                        0, 0, 0);
                X[st] = x_frag(cs, st, 1);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b)
                Wf[b] = Wn[b];
            // block k + 1 landed everywhere, block k read everywhere
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (k + 2 < nkb)
                dma_block(cs, (k + 2) * kQBK);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                Wn[b] = w_frag(ns, b, 0);
#pragma unroll
            for (int st = 0; st < 8; ++st) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[st][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, Wf[b]), __builtin_bit_cast(bf16x8_t, X[st]), acc[st][b],
                        0, 0, 0);
                X[st] = x_frag(ns, st, 0);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b)
                Wf[b] = Wn[b];
        }
        // epilogue: lane group g owns columns cq*64 + g*16 .. +15 of the chunk
        // for run rows th*128 + st*16 + row
        if (q0 + 2 * th < q1) {
            uint16_t *y = (uint16_t *)a.y[m];
            const bool has_bias = saved_bit(a.has_bias[m], slot);
            const uint16_t *bias = (const uint16_t *)a.bias[m] + (int64_t)slot * d_out;
            const int col = chunk * kSavedCols + cq * 64 + g * 16;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                if (col + p * 8 >= d_out)
                    continue;
                uint4 cw = make_uint4(0, 0, 0, 0);
                if (has_bias)
                    cw = *(const uint4 *)(bias + col + p * 8);
                const uint32_t c[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    const int tok = run_tok(th * 128 + st * 16 + row);
                    if (tok < 0)
                        continue;
                    // columns col + 8p .. +7: rows 4g..4g+3 of blocks 2p and 2p + 1
                    const f32x4_t v0 = acc[st][2 * p], v1 = acc[st][2 * p + 1];
                    uint4 o;
                    o.x = pack_bf16x2(v0[0] + bf16_lo(c[0]), v0[1] + bf16_hi(c[0]));
                    o.y = pack_bf16x2(v0[2] + bf16_lo(c[1]), v0[3] + bf16_hi(c[1]));
                    o.z = pack_bf16x2(v1[0] + bf16_lo(c[2]), v1[1] + bf16_hi(c[2]));
                    o.w = pack_bf16x2(v1[2] + bf16_lo(c[3]), v1[3] + bf16_hi(c[3]));
                    *(uint4 *)(y + (int64_t)tok * d_out + col + p * 8) = o;
                }
            }
        }
        q0 = q1;
    }
}

// fp32: one workgroup = one tile x 64 columns x one member; thread tid takes
// column tid % 64 for the 16 tokens (tid / 64) * 16 .. +15, with fp64 sums.
constexpr int kF32Cols = 64;

__global__ __launch_bounds__(256) void saved_f32_kernel(SavedArgs a)
{
    const int bt = blockIdx.x, chunk = blockIdx.y, m = blockIdx.z;
    if (m >= a.n || chunk * kF32Cols >= a.d_out[m])
        return;
    const int n_tiles = *a.n_tiles;
    const Tile tile = a.tiles[bt];
    if (bt >= n_tiles || !saved_bit(a.saved[m], tile.slot))
        return;
    const int d_in = a.d_in[m], d_out = a.d_out[m];
    const int tid = threadIdx.x;
    const float *x = (const float *)a.x[m];
    const float *W = (const float *)a.W[m] + (int64_t)tile.slot * a.slot_stride_W[m];
    const int32_t *toks = a.tile_tok + (int64_t)bt * kTileTokens;
    __shared__ float xs[kTileTokens][33];
    __shared__ float ws[kF32Cols][33];
    const int c = tid & 63, q = tid >> 6;
    const int n = chunk * kF32Cols + c;
    double acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        acc[j] = 0.0;
    for (int k0 = 0; k0 < d_in; k0 += 32) {
        for (int e = tid; e < kTileTokens * 32; e += 256) {
            const int t = e >> 5, kk = e & 31;
            xs[t][kk] = (t < tile.len && k0 + kk < d_in) ? x[(int64_t)toks[t] * d_in + k0 + kk] : 0.f;
        }
        for (int e = tid; e < kF32Cols * 32; e += 256) {
            const int cc = e >> 5, kk = e & 31, nn = chunk * kF32Cols + cc;
            ws[cc][kk] = (nn < d_out && k0 + kk < d_in) ? W[(int64_t)nn * d_in + k0 + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            double s = acc[j];
            for (int kk = 0; kk < 32; ++kk)
                s = fma((double)xs[q * 16 + j][kk], (double)ws[c][kk], s);
            acc[j] = s;
        }
        __syncthreads();
    }
    if (n >= d_out)
        return;
    const double cn = saved_bit(a.has_bias[m], tile.slot)
                          ? (double)((const float *)a.bias[m])[(int64_t)tile.slot * d_out + n] : 0.0;
    float *y = (float *)a.y[m];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = q * 16 + j;
        if (t < tile.len)
            y[(int64_t)toks[t] * d_out + n] = (float)(acc[j] + cn);
    }
}

}  // namespace

// The 256 x 256 kernel takes a launch whose modules all have d_in a multiple
// of 64, whose x buffers are 16-byte aligned (its direct-to-LDS loads move
// aligned 16-byte pieces) and whose x and per-slot W are under 4 GB (they are
// addressed by 32-bit byte offsets); any other bf16 launch takes
// saved_bf16_kernel.
static bool quad_fits(const SavedArgs &a)
{
    for (int i = 0; i < a.n; ++i) {
        const uint64_t d_in = (uint64_t)a.d_in[i];
        if (d_in % kQBK || ((uintptr_t)a.x[i] & 15) || (uint64_t)a.T * d_in * 2 > UINT32_MAX ||
            (uint64_t)a.d_out[i] * d_in * 2 > UINT32_MAX)
            return false;
    }
    return true;
}

hipError_t launch_saved(bool bf16, const SavedArgs &a, hipStream_t st, const LaunchTiming &t)
{
    if (bf16) {
        SavedArgs b = a;
        if (quad_fits(a)) {
            // work items as quad_decode lays them out (whole blocks per member)
            const int64_t quads = (a.grid_tiles + 3) / 4;
            const int64_t qb = (quads + kQBlockQuads - 1) / kQBlockQuads;
            int64_t items = 0;
            for (int i = 0; i < a.n; ++i) {
                const int64_t cols = a.col_start[i + 1] - a.col_start[i];
                items += qb * ((cols + kQBlockCols - 1) / kQBlockCols) * kQBlockItems;
            }
            b.per_xcd = (int)((items + kXcds - 1) / kXcds);
            launch(saved_bf16_quad_kernel, dim3((unsigned)(b.per_xcd * kXcds)), dim3(kQThreads), st, t, b);
            return hipGetLastError();
        }
        const int64_t items = (int64_t)((a.grid_tiles + 1) / 2) * a.col_start[a.n];
        b.per_xcd = (int)((items + kXcds - 1) / kXcds);
        launch(saved_bf16_kernel, dim3((unsigned)(b.per_xcd * kXcds)), dim3(256), st, t, b);
    } else {
        int cols = 1;
        for (int i = 0; i < a.n; ++i)
            cols = cols > (a.d_out[i] + kF32Cols - 1) / kF32Cols ? cols : (a.d_out[i] + kF32Cols - 1) / kF32Cols;
        launch(saved_f32_kernel, dim3(a.grid_tiles, cols, a.n), dim3(256), st, t, a);
    }
    return hipGetLastError();
}

}  // namespace lora
