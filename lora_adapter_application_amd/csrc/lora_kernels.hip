// lora_kernels.hip -- gfx950 kernels of the multi-adapter LoRA update
//
//   plan     stable counting sort of the per-token slot index into runs of one
//            slot, cut into tiles of up to 64 tokens (device only, no host sync)
//   shrink   h[p, :] = x[perm[p], :] . A_k^T over a K range (fp32 partials)
//   expand   y[t, :] = round(y[t, :] + s_k * h[p, :] . B_k)
//
// The update itself, its scale and the adapter fields it reads are those of the
// example adapter_config.json in "vLLM LoRA Resolver plugins explained",
// section 3.2; the slot count and padded rank are max_loras / max_lora_rank of
// the parameter table in "Multi-LoRA adapter cache in production".
//
// bf16 data runs on the matrix cores: v_mfma_f32_16x16x32_bf16 for shrink
// (K = d_in) and v_mfma_f32_16x16x16_bf16 for expand (K = rank), with the fp32
// intermediate split into a bf16 high and low part so the expand keeps ~16
// bits of h.  fp32 data runs on plain VALU loops.
//
// Operand layout of a 16x16xK MFMA on a 64-wide wave, as used below: lane l
// supplies row (l & 15) of A and column (l & 15) of B, each with the K slice of
// lane group g = l >> 4 (8 values for K=32, 4 for K=16); the 16x16 fp32 result
// leaves rows 4g..4g+3 of column (l & 15) in lane l.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_internal.h"

namespace lora {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ----------------------------------------------------------------------------
// plan

// Exclusive scan of one int per thread over a 1024-thread block.
__device__ int block_excl_scan_1024(int v, int *wsum /*[17]*/, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int s = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(s, d, 64);
        if (lane >= d)
            s += o;
    }
    if (lane == 63)
        wsum[wave] = s;
    __syncthreads();
    if (wave == 0) {
        int ws = lane < 16 ? wsum[lane] : 0;
        int t = ws;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
            int o = __shfl_up(t, d, 64);
            if (lane >= d)
                t += o;
        }
        if (lane < 16)
            wsum[lane] = t - ws;
        if (lane == 15)
            wsum[16] = t;
    }
    __syncthreads();
    int excl = s - v + wsum[wave];
    *total = wsum[16];
    __syncthreads();
    return excl;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *__restrict__ idx, int32_t T,
                                                    int32_t S, PlanBuffers pb)
{
    extern __shared__ int32_t sm[];
    int32_t *cnt = sm;             // [S]
    int32_t *base = sm + S;        // [S]
    int32_t *wcnt = sm + 2 * S;    // [16][S] tokens of slot s in wave w of the chunk
    int32_t *woff = sm + 18 * S;   // [16][S] first position for them
    __shared__ int32_t wsum[17];
    __shared__ int32_t bad;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int i = tid; i < S; i += 1024)
        cnt[i] = 0;
    for (int i = tid; i < 16 * S; i += 1024)
        wcnt[i] = 0;
    if (tid == 0)
        bad = 0;
    __syncthreads();
    for (int i = tid; i < T; i += 1024) {
        int v = idx[i];
        if (v >= S)
            bad = 1;
        else if (v >= 0)
            atomicAdd(&cnt[v], 1);
    }
    __syncthreads();

    // Runs and tiles, one slot per thread (S <= 1024).
    const int c = tid < S ? cnt[tid] : 0;
    int n_active, n_tiles;
    const int start = block_excl_scan_1024(c, wsum, &n_active);
    const int nt = (c + kTileTokens - 1) / kTileTokens;
    const int tstart = block_excl_scan_1024(nt, wsum, &n_tiles);
    if (tid < S) {
        base[tid] = start;
        pb.counts[tid] = c;
        pb.seg_start[tid] = start;
        for (int j = 0; j < nt; ++j) {
            Tile t;
            t.slot = tid;
            t.start = start + j * kTileTokens;
            t.len = min(kTileTokens, c - j * kTileTokens);
            t.pad = 0;
            pb.tiles[tstart + j] = t;
        }
    }
    if (tid == 0) {
        *pb.n_tiles = n_tiles;
        *pb.n_active = n_active;
        if (bad)
            atomicOr(pb.flags, 1u);
    }
    __syncthreads();

    // Stable scatter, 1024 tokens per pass in index order.  Within a wave, a
    // token's rank among equal slots comes from ballots, one per distinct slot.
    for (int c0 = 0; c0 < T; c0 += 1024) {
        const int i = c0 + tid;
        const int v = i < T ? idx[i] : -1;
        const bool valid = v >= 0 && v < S;
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
                wcnt[wave * S + lv] = __popcll(m);
            act &= ~m;
        }
        __syncthreads();
        for (int s = tid; s < S; s += 1024) {
            int run = base[s];
            for (int w = 0; w < 16; ++w) {
                const int k = wcnt[w * S + s];
                wcnt[w * S + s] = 0;
                woff[w * S + s] = run;
                run += k;
            }
            base[s] = run;
        }
        __syncthreads();
        if (valid)
            pb.perm[woff[wave * S + v] + my_rank] = i;
        __syncthreads();
    }
}

hipError_t launch_plan(const int32_t *idx, int32_t T, int32_t S, const PlanBuffers &pb,
                       hipStream_t st)
{
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), plan_lds_bytes(S), st, idx, T, S, pb);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// shrink, bf16 on MFMA
//
// One workgroup (4 waves) = one tile (<= 64 tokens of one slot) x one K split.
// A tile has nsub = ceil(len/16) subtiles of 16 tokens; waves split the work as
// (subtile, K part) so short tiles still keep all 4 waves loading.  Per step a
// lane loads 64 contiguous bytes of its token's x row and of its rank's A^T row
// and feeds them to 4 MFMAs; both operands use the same K order, so the sum is
// the plain dot product over that K block.  Output: h as [rank][token] blocks,
// lane l holding ranks 4g..4g+3 of token (l & 15) -> one 16-byte store.

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *(const uint4 *)p; }

template <int NB>
__global__ __launch_bounds__(256) void shrink_bf16_kernel(ShrinkArgs a)
{
    if ((int)blockIdx.x >= *a.n_tiles)
        return;
    const Tile tile = a.tiles[blockIdx.x];
    const int rank = a.rank[tile.slot];
    if (rank <= 0)
        return;
    const int nb = (rank + 15) >> 4;
    const int split = blockIdx.y;
    const int k0 = split * a.k_chunk;
    const int k1 = min(a.d_in, k0 + a.k_chunk);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = lane & 15, g = lane >> 4;
    const int nsub = (tile.len + 15) >> 4;
    const int nsub_pad = nsub == 3 ? 4 : nsub;
    const int kparts = 4 / nsub_pad;
    const int sub = wave % nsub_pad, kp = wave / nsub_pad;
    const bool wave_on = sub < nsub;
    const int tok_in_tile = sub * 16 + row;
    const bool tok_ok = wave_on && tok_in_tile < tile.len;
    const int p = tile.start + tok_in_tile;

    const uint16_t *xrow = (const uint16_t *)a.x + (int64_t)(tok_ok ? a.perm[p] : 0) * a.d_in;
    const uint16_t *Aslot = (const uint16_t *)a.A + (int64_t)tile.slot * a.slot_stride_A;

    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (wave_on) {
        for (int kb = k0 + kp * kShrinkKBlock; kb < k1; kb += kparts * kShrinkKBlock) {
            const int kk = kb + g * 32;
            uint4 xv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ke = kk + q * 8;
                xv[q] = (tok_ok && ke < k1) ? ld16(xrow + ke) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b < nb) {
                    const uint16_t *arow = Aslot + (int64_t)(b * 16 + row) * a.d_in;
                    uint4 av[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int ke = kk + q * 8;
                        av[q] = ke < k1 ? ld16(arow + ke) : make_uint4(0, 0, 0, 0);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, av[q]), __builtin_bit_cast(bf16x8_t, xv[q]),
                            acc[b], 0, 0, 0);
                }
            }
        }
    }

    __shared__ f32x4_t red[4][NB][64];
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
        float *hrow = a.hpart + (int64_t)split * a.split_stride + (int64_t)p * a.R_pad;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b < nb)
                *(f32x4_t *)(hrow + b * 16 + g * 4) = acc[b];
    }
}

// ----------------------------------------------------------------------------
// expand, bf16 on MFMA
//
// One workgroup = one tile x 256 columns of y.  The product is formed
// transposed, out[n][t] = sum_j B[j][n] h[t][j], so the result of one lane is
// four columns of one token.  B is stored in groups of 8 ranks,
// Bi[j/8][n][j%8], so the rank slice an MFMA lane needs is contiguous.  Rows
// of the 16x16 output blocks are mapped to columns so that lane group g of a
// wave owns 16 adjacent columns: y is read and written 32 bytes per lane.

template <int NB>
__global__ __launch_bounds__(256) void expand_bf16_kernel(ExpandArgs a)
{
    if ((int)blockIdx.x >= *a.n_tiles)
        return;
    const Tile tile = a.tiles[blockIdx.x];
    const int rank = a.rank[tile.slot];
    if (rank <= 0)
        return;
    const int nb = (rank + 15) >> 4;
    const float s = a.scale[tile.slot];
    const int c0 = blockIdx.y * kExpandCols;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = lane & 15, g = lane >> 4;
    const int nsub = (tile.len + 15) >> 4;
    const int nsub_pad = nsub == 3 ? 4 : nsub;
    const int cparts = 4 / nsub_pad;
    const int sub = wave % nsub_pad, cp = wave / nsub_pad;
    if (sub >= nsub)
        return;
    const int tok_in_tile = sub * 16 + row;
    const bool tok_ok = tok_in_tile < tile.len;
    const int p = tile.start + tok_in_tile;

    // h for this lane's token, ranks kst*16 + 4g .. +3, summed over K splits,
    // split into bf16 high and low halves.
    s16x4_t hhi[NB], hlo[NB];
#pragma unroll
    for (int kst = 0; kst < NB; ++kst) {
        f32x4_t hs = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (kst < nb && tok_ok) {
            const float *hp = a.hpart + (int64_t)p * a.R_pad + kst * 16 + g * 4;
            for (int sp = 0; sp < a.splits; ++sp)
                hs += *(const f32x4_t *)(hp + (int64_t)sp * a.split_stride);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t hi = f32_to_bf16_bits(hs[e]);
            const uint32_t lo = f32_to_bf16_bits(hs[e] - bf16_bits_to_f32(hi));
            hhi[kst][e] = (short)hi;
            hlo[kst][e] = (short)lo;
        }
    }

    const int tok = tok_ok ? a.perm[p] : 0;
    uint16_t *yrow = (uint16_t *)a.y + (int64_t)tok * a.d_out;
    const uint16_t *Bslot = (const uint16_t *)a.Bi + (int64_t)tile.slot * a.slot_stride_B;

    for (int cg = cp; cg < 4; cg += cparts) {
        const int cb = c0 + cg * 64;
        if (cb >= a.d_out)
            break;
        f32x4_t acc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kst = 0; kst < NB; ++kst) {
            if (kst < nb) {
                const int G = kst * 2 + (g >> 1);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int n = cb + (row >> 2) * 16 + b * 4 + (row & 3);
                    uint2 bv = make_uint2(0, 0);
                    if (n < a.d_out)
                        bv = *(const uint2 *)(Bslot + ((int64_t)G * a.d_out + n) * 8 + (g & 1) * 4);
                    const s16x4_t bop = __builtin_bit_cast(s16x4_t, bv);
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bop, hhi[kst], acc[b], 0, 0, 0);
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bop, hlo[kst], acc[b], 0, 0, 0);
                }
            }
        }
        if (tok_ok) {
#pragma unroll
            for (int piece = 0; piece < 2; ++piece) {
                const int col = cb + g * 16 + piece * 8;
                if (col < a.d_out) {
                    uint4 yv = *(const uint4 *)(yrow + col);
                    uint32_t w[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
                    for (int h2 = 0; h2 < 4; ++h2) {
                        const int e0 = piece * 8 + h2 * 2, e1 = e0 + 1;
                        const float v0 = bf16_bits_to_f32(w[h2] & 0xffffu) + s * acc[e0 >> 2][e0 & 3];
                        const float v1 = bf16_bits_to_f32(w[h2] >> 16) + s * acc[e1 >> 2][e1 & 3];
                        w[h2] = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
                    }
                    *(uint4 *)(yrow + col) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
// fp32 on VALU

__global__ __launch_bounds__(256) void shrink_f32_kernel(ShrinkArgs a)
{
    if ((int)blockIdx.x >= *a.n_tiles)
        return;
    const Tile tile = a.tiles[blockIdx.x];
    const int rank = a.rank[tile.slot];
    if (rank <= 0)
        return;
    const int split = blockIdx.y;
    const int k0 = split * a.k_chunk;
    const int k1 = min(a.d_in, k0 + a.k_chunk);
    const int tid = threadIdx.x;
    const float *x = (const float *)a.x;
    const float *Aslot = (const float *)a.A + (int64_t)tile.slot * a.slot_stride_A;
    __shared__ float xs[kTileTokens][33];
    __shared__ float as[LORA_MAX_RANK_PAD][33];
    __shared__ int toks[kTileTokens];
    if (tid < kTileTokens)
        toks[tid] = tid < tile.len ? a.perm[tile.start + tid] : 0;
    const int npairs = tile.len * rank;   // <= 64 * 128 = 32 per thread
    float acc[32];
#pragma unroll
    for (int q = 0; q < 32; ++q)
        acc[q] = 0.f;
    __syncthreads();
    for (int kc = k0; kc < k1; kc += 32) {
        for (int e = tid; e < kTileTokens * 32; e += 256) {
            const int t = e >> 5, kk = e & 31;
            xs[t][kk] = (t < tile.len && kc + kk < k1) ? x[(int64_t)toks[t] * a.d_in + kc + kk] : 0.f;
        }
        for (int e = tid; e < rank * 32; e += 256) {
            const int j = e >> 5, kk = e & 31;
            as[j][kk] = kc + kk < k1 ? Aslot[(int64_t)j * a.d_in + kc + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int e = tid + q * 256;
            if (e < npairs) {
                const int t = e / rank, j = e % rank;
                float sacc = acc[q];
                for (int kk = 0; kk < 32; ++kk)
                    sacc += xs[t][kk] * as[j][kk];
                acc[q] = sacc;
            }
        }
        __syncthreads();
    }
    float *hp = a.hpart + (int64_t)split * a.split_stride;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
        const int e = tid + q * 256;
        if (e < npairs) {
            const int t = e / rank, j = e % rank;
            hp[(int64_t)(tile.start + t) * a.R_pad + j] = acc[q];
        }
    }
}

__global__ __launch_bounds__(256) void expand_f32_kernel(ExpandArgs a)
{
    if ((int)blockIdx.x >= *a.n_tiles)
        return;
    const Tile tile = a.tiles[blockIdx.x];
    const int rank = a.rank[tile.slot];
    if (rank <= 0)
        return;
    const float s = a.scale[tile.slot];
    const int tid = threadIdx.x;
    __shared__ float hs[kTileTokens][LORA_MAX_RANK_PAD + 1];
    for (int e = tid; e < tile.len * rank; e += 256) {
        const int t = e / rank, j = e % rank;
        const float *hp = a.hpart + (int64_t)(tile.start + t) * a.R_pad + j;
        float v = 0.f;
        for (int sp = 0; sp < a.splits; ++sp)
            v += hp[(int64_t)sp * a.split_stride];
        hs[t][j] = v;
    }
    __syncthreads();
    const int n = blockIdx.y * kExpandCols + tid;
    if (n >= a.d_out)
        return;
    const float *Bslot = (const float *)a.Bi + (int64_t)tile.slot * a.slot_stride_B;
    float acc[kTileTokens];
#pragma unroll
    for (int t = 0; t < kTileTokens; ++t)
        acc[t] = 0.f;
    for (int j = 0; j < rank; ++j) {
        const float bj = Bslot[((int64_t)(j >> 3) * a.d_out + n) * 8 + (j & 7)];
#pragma unroll
        for (int t = 0; t < kTileTokens; ++t)
            if (t < tile.len)
                acc[t] += hs[t][j] * bj;
    }
    float *y = (float *)a.y;
#pragma unroll
    for (int t = 0; t < kTileTokens; ++t) {
        if (t < tile.len) {
            const int64_t o = (int64_t)a.perm[tile.start + t] * a.d_out + n;
            y[o] = y[o] + s * acc[t];
        }
    }
}

// ----------------------------------------------------------------------------
// launches

hipError_t launch_shrink(bool bf16, const ShrinkArgs &a, hipStream_t st)
{
    const dim3 grid(a.grid_tiles, a.splits), block(256);
    if (!bf16) {
        hipLaunchKernelGGL(shrink_f32_kernel, grid, block, 0, st, a);
    } else {
        const int nbmax = a.R_pad / 16;
        if (nbmax <= 1)
            hipLaunchKernelGGL(shrink_bf16_kernel<1>, grid, block, 0, st, a);
        else if (nbmax <= 2)
            hipLaunchKernelGGL(shrink_bf16_kernel<2>, grid, block, 0, st, a);
        else if (nbmax <= 4)
            hipLaunchKernelGGL(shrink_bf16_kernel<4>, grid, block, 0, st, a);
        else
            hipLaunchKernelGGL(shrink_bf16_kernel<8>, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_expand(bool bf16, const ExpandArgs &a, hipStream_t st)
{
    const dim3 grid(a.grid_tiles, (a.d_out + kExpandCols - 1) / kExpandCols), block(256);
    if (!bf16) {
        hipLaunchKernelGGL(expand_f32_kernel, grid, block, 0, st, a);
    } else {
        const int nbmax = a.R_pad / 16;
        if (nbmax <= 1)
            hipLaunchKernelGGL(expand_bf16_kernel<1>, grid, block, 0, st, a);
        else if (nbmax <= 2)
            hipLaunchKernelGGL(expand_bf16_kernel<2>, grid, block, 0, st, a);
        else if (nbmax <= 4)
            hipLaunchKernelGGL(expand_bf16_kernel<4>, grid, block, 0, st, a);
        else
            hipLaunchKernelGGL(expand_bf16_kernel<8>, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// slot maintenance

__global__ void slot_reset_kernel(int32_t *rank_all, int32_t n_modules, int32_t S, int32_t slot)
{
    for (int m = blockIdx.x * blockDim.x + threadIdx.x; m < n_modules; m += gridDim.x * blockDim.x)
        rank_all[(int64_t)m * S + slot] = 0;
}

hipError_t launch_slot_reset(int32_t *rank_all, int32_t n_modules, int32_t S, int32_t slot,
                             hipStream_t st)
{
    const int blocks = (n_modules + 255) / 256;
    hipLaunchKernelGGL(slot_reset_kernel, dim3(blocks), dim3(256), 0, st, rank_all, n_modules, S,
                       slot);
    return hipGetLastError();
}

// Repack B (r x d_out, row-major, staged on the device) into groups of 8 ranks,
// Bi[j/8][n][j%8], zero ranks r..R_pad-1 of both A^T and B, then publish the
// rank and scale of the slot for this module.
template <typename E>
__global__ void slot_finalize_kernel(E *A_slot, int32_t d_in, E *Bi_slot, const E *B_stage,
                                     int32_t d_out, int32_t r, int32_t R_pad, int32_t *rank_entry,
                                     float *scale_entry, float s)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_group = (int64_t)d_out * 8;
    const int64_t nB = (int64_t)R_pad * d_out;
    for (int64_t o = first; o < nB; o += stride) {
        const int G = (int)(o / per_group);
        const int64_t rem = o - (int64_t)G * per_group;
        const int n = (int)(rem >> 3), w = (int)(rem & 7);
        const int j = G * 8 + w;
        Bi_slot[o] = j < r ? B_stage[(int64_t)j * d_out + n] : E(0);
    }
    const int64_t nA = (int64_t)(R_pad - r) * d_in;
    for (int64_t o = first; o < nA; o += stride)
        A_slot[(int64_t)r * d_in + o] = E(0);
    if (first == 0) {
        *rank_entry = r;
        *scale_entry = s;
    }
}

hipError_t launch_slot_finalize(bool bf16, void *A_slot, int32_t d_in, void *Bi_slot,
                                const void *B_stage, int32_t d_out, int32_t r, int32_t R_pad,
                                int32_t *rank_entry, float *scale_entry, float s, hipStream_t st)
{
    const int64_t work = (int64_t)R_pad * (d_out > d_in ? d_out : d_in);
    int blocks = (int)((work + 255) / 256);
    if (blocks > 2048)
        blocks = 2048;
    if (bf16)
        hipLaunchKernelGGL(slot_finalize_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                           (uint16_t *)A_slot, d_in, (uint16_t *)Bi_slot,
                           (const uint16_t *)B_stage, d_out, r, R_pad, rank_entry, scale_entry, s);
    else
        hipLaunchKernelGGL(slot_finalize_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           (float *)A_slot, d_in, (float *)Bi_slot, (const float *)B_stage, d_out,
                           r, R_pad, rank_entry, scale_entry, s);
    return hipGetLastError();
}

}  // namespace lora
