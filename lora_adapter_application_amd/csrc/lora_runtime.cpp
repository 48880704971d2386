// lora_runtime.cpp -- the C ABI declared in include/lora_mi355x.h: slot pool,
// asynchronous slot loads on a side stream, device-side plan, and the
// shrink / expand launches of the multi-adapter LoRA update.
//
// Slot pool ("GPU active slots" of the cache hierarchy in "Multi-LoRA adapter
// cache in production", section "GPU, CPU and disk form the adapter storage
// hierarchy"): per module m, A^T as [S][R_pad][d_in] (rank-major, rank j of a
// slot is one contiguous row) and B as [S][R_pad/8][d_out][8] (groups of eight
// ranks interleaved per output column, the order the expand MFMA consumes).
// Rows r..R_pad-1 of a slot are kept zero.  The host keeps, per (module, slot),
// the rank (0 = nothing to apply) and per slot the fp32 scale; every launch gets
// the module's table by value, so a kernel sees exactly the slots that were
// loaded before it was enqueued.
//
// Ordering without host synchronisation:
//  - a load records an event on the side stream; a later kernel launch on a
//    compute stream waits for it once (read after write);
//  - before a load overwrites a slot, the side stream waits for the
//    current tail of every compute stream this ctx has launched on since the
//    previous load, so weights an in-flight batch reads are never overwritten
//    ("an adapter in use must not be evicted", same page, data-plane section).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/lora_mi355x.h"
#include "lora_internal.h"

using namespace lora;

namespace {

thread_local std::string g_create_error;

struct StreamState {
    hipStream_t stream;
    uint64_t waited_gen;    // load generation this stream has waited for
    bool used_since_load;   // launched on since the last load
    bool since_fence;       // launched on since the side stream last waited for it
    hipEvent_t tail;        // recorded at load time to fence the stream's tail
};

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess)
            prev = -1;
        if (prev != dev)
            ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard()
    {
        if (prev >= 0)
            (void)hipSetDevice(prev);
    }
};

int round_up(int v, int m) { return (v + m - 1) / m * m; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Where one batch's plan and h partials live: the ctx's own allocation, or the
// library's static scratch array (lora_apply_group_noalloc).
struct Workspace {
    PlanBuffers plan{};
    float *hpart = nullptr;
    int hbuf_rows = 0;       // rows of one group member's block of h partials
    uint32_t *sync = nullptr;   // fused decode counts [max_tiles][kSyncWordsPerTile], kept at zero
                                // between launches (null: no fused launches on this workspace)
};

// Polls of a fused decode workgroup waiting for its tile's partials before it
// gives up (about 20 ms; a launch normally waits a few microseconds).
constexpr int kFusedSpinLimit = 20000;

// The plan of the current batch, and the module list of the last shrink (which
// the expand must repeat).
struct BatchState {
    bool hinted = false;     // the batch declared its slots (lora_plan_prepare_slots)
    int plan_mode = kPlanTiles;   // PlanMode of the next bf16 launch on this plan
    int tile_cap = kTileTokens;   // tokens per tile of the plan
    const int32_t *idx = nullptr;
    int32_t T = 0;
    int last_n = 0;
    int last_modules[kMaxGroup] = {};
    int last_splits[kMaxGroup] = {};
    const void *last_x[kMaxGroup] = {};   // inputs of the last shrink (saved modules read them)
};

}  // namespace

struct lora_ctx {
    int device = 0;
    lora_dtype dtype = LORA_BF16;
    int S = 0, R = 0, R_pad = 0, n_modules = 0, max_tokens = 0, elem = 2;
    std::vector<lora_module_shape> shapes;
    std::vector<void *> A, Bi;
    std::vector<void *> bias;                // per module: [max_loras][d_out], ctx dtype
    std::vector<float *> dora;               // per module: [max_loras][d_out]
    std::vector<uint8_t> slot_flags;         // [S]: kSlotBias | kSlotDora
    // saved modules (lora_slot_load_saved): per module a pool [S][d_out][d_in] and
    // its biases [S][d_out], allocated at the module's first saved load
    std::vector<void *> saved_W, saved_bias;
    std::vector<uint8_t> saved_host;         // [n_modules][S]: 1 = the slot saves the module
    std::vector<uint8_t> saved_bias_host;    // [n_modules][S]: ... with a bias
    std::vector<int64_t> strideA, strideB;   // per-slot element strides
    std::vector<int32_t> rank_host;          // [n_modules][S]: r if the slot's adapter targets m
    std::vector<int32_t> slot_rank;          // [S]: rank of the adapter in the slot (0 = empty)
    std::vector<float> scale_host;
    void *stage = nullptr;                   // A^T and B staging for the modules of one load
    int64_t stage_elems = 0;
    Workspace ws;                            // the ctx's plan buffers and h partials
    int max_tiles = 0;
    void *scratch = nullptr;                 // this device's static scratch array (no-alloc calls)
    bool xcd_local = false;                  // workgroups equal mod 8 share an XCD (fused decode hand-over in L2)
    hipStream_t side = nullptr;
    hipEvent_t load_done = nullptr;
    uint64_t load_gen = 0;
    uint64_t synced_gen = 0;                 // loads the host has seen complete (lora_sync_loads)
    // slots the prepared plan reads (lora_plan_prepare_slots, bs.hinted); else every slot
    std::vector<uint8_t> hint;               // [S]
    // per slot, the number of the last use event recorded after a launch of a
    // declared plan that reads it (0: none since the slot's last load)
    std::vector<uint64_t> last_use;          // [S]
    static constexpr int kUseEvents = 64;    // ring; a reused entry only waits longer
    hipEvent_t use_ev[kUseEvents] = {};
    uint64_t use_seq = 0;
    std::vector<StreamState> streams;
    // plan state of the ctx's workspace; an inline plan is computed by the
    // first shrink launch itself
    bool plan_valid = false, plan_prepared = false;
    BatchState bs;
    uint64_t slot_epoch = 0, shrink_epoch = 0;   // loads + clears, and their count at the last shrink
    lora_stats stats{};
    // kernel timing (lora_profile_begin / lora_profile_end)
    bool profiling = false;
    std::vector<LaunchTiming> prof_events;
    std::vector<int> prof_kind;
    size_t prof_used = 0, prof_cap = 0;
    int64_t prof_untimed = 0;
    std::string last_error;
    std::vector<void *> allocations;
    uint32_t flags_host = 0;                 // lora_get_device_flags' copy of the sticky word
};

namespace {

int fail(lora_ctx *c, int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (c)
        c->last_error = buf;
    else
        g_create_error = buf;
    return status;
}

int hip_fail(lora_ctx *c, hipError_t e, const char *what)
{
    return fail(c, LORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(ctx, expr)                                   \
    do {                                                     \
        hipError_t e_ = (expr);                              \
        if (e_ != hipSuccess)                                \
            return hip_fail((ctx), e_, #expr);               \
    } while (0)

StreamState *stream_state(lora_ctx *c, hipStream_t s)
{
    for (auto &st : c->streams)
        if (st.stream == s)
            return &st;
    StreamState st{s, 0, false, false, nullptr};
    if (hipEventCreateWithFlags(&st.tail, hipEventDisableTiming) != hipSuccess)
        return nullptr;
    c->streams.push_back(st);
    return &c->streams.back();
}

// Whether s is being captured into a graph.
bool stream_capturing(hipStream_t s)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();   // a query error must not surface at a later call
        return false;
    }
    return cs != hipStreamCaptureStatusNone;
}

// Make stream s wait for all loads issued so far, and mark it as in use.  A
// stream that is being captured into a graph cannot wait for the load event,
// which was recorded outside the capture: loads must be complete (on the host,
// lora_sync_loads) before a capture starts.
// reads_slots: the launch reads slot data (shrink, expand); plan kernels read
// only the slot indices, so a later load need not wait for them.
int before_launch(lora_ctx *c, hipStream_t s, bool reads_slots, bool hinted)
{
    StreamState *st = stream_state(c, s);
    if (!st)
        return fail(c, LORA_ERR_HIP, "hipEventCreateWithFlags failed");
    if (st->waited_gen < c->load_gen && c->synced_gen < c->load_gen) {
        if (stream_capturing(s))
            return fail(c, LORA_ERR_INVALID_ARGUMENT,
                        "slot loads pending on a stream under graph capture: call lora_sync_loads "
                        "before the capture");
        HIP_TRY(c, hipStreamWaitEvent(s, c->load_done, 0));
        st->waited_gen = c->load_gen;
    }
    // a launch of a declared plan is fenced per slot (after its expand), except
    // under capture, where no event is recorded
    if (reads_slots && (!hinted || stream_capturing(s)))
        st->used_since_load = true;
    st->since_fence = true;
    return LORA_OK;
}

// After an expand of a declared plan: one event, the last use of every declared slot.
int record_slot_use(lora_ctx *c, hipStream_t s, bool hinted)
{
    if (!hinted || stream_capturing(s))
        return LORA_OK;
    const uint64_t seq = ++c->use_seq;
    hipEvent_t &ev = c->use_ev[seq % lora_ctx::kUseEvents];
    if (!ev)
        HIP_TRY(c, hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    HIP_TRY(c, hipEventRecord(ev, s));
    for (int k = 0; k < c->S; ++k)
        if (c->hint[k])
            c->last_use[k] = seq;
    return LORA_OK;
}

// Side stream waits for the current tail of every stream used since the last load.
int fence_compute_streams(lora_ctx *c)
{
    for (auto &st : c->streams) {
        if (!st.used_since_load)
            continue;
        HIP_TRY(c, hipEventRecord(st.tail, st.stream));
        HIP_TRY(c, hipStreamWaitEvent(c->side, st.tail, 0));
        st.used_since_load = false;
        st.since_fence = false;
    }
    return LORA_OK;
}

// A load source must be pinned host, device or managed memory.  *in_place:
// the finalize kernel on `device` may read it at its own address (memory of
// that device, managed memory, or pinned host memory mapped at its host
// address) and it is 16-byte aligned; otherwise it is staged by a copy.
int check_source(const void *p, int device, bool *in_place = nullptr)
{
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return LORA_ERR_HOST_NOT_PINNED;
    }
    if (attr.type != hipMemoryTypeHost && attr.type != hipMemoryTypeDevice &&
        attr.type != hipMemoryTypeManaged)
        return LORA_ERR_HOST_NOT_PINNED;
    if (in_place) {
        const bool mapped = attr.type == hipMemoryTypeManaged ||
                            (attr.type == hipMemoryTypeDevice && attr.device == device) ||
                            (attr.type == hipMemoryTypeHost && attr.devicePointer == p);
        *in_place = mapped && ((uintptr_t)p & 15) == 0;
    }
    return LORA_OK;
}

void free_all(lora_ctx *c)
{
    for (auto &t : c->prof_events) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    c->prof_events.clear();
    for (void *p : c->allocations)
        (void)hipFree(p);
    c->allocations.clear();
    for (auto &st : c->streams)
        if (st.tail)
            (void)hipEventDestroy(st.tail);
    c->streams.clear();
    for (auto &ev : c->use_ev)
        if (ev) {
            (void)hipEventDestroy(ev);
            ev = nullptr;
        }
    if (c->load_done)
        (void)hipEventDestroy(c->load_done);
    if (c->side)
        (void)hipStreamDestroy(c->side);
    c->load_done = nullptr;
    c->side = nullptr;
}

// Device allocation owned by the ctx, zeroed on the ctx's side stream (the
// creating call waits for that stream before it returns).
template <typename T>
hipError_t dalloc(lora_ctx *c, T **p, size_t bytes)
{
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, bytes ? bytes : 16);
    if (e != hipSuccess)
        return e;
    c->allocations.push_back(q);
    e = hipMemsetAsync(q, 0, bytes ? bytes : 16, c->side);
    *p = (T *)q;
    return e;
}

// Host waits for every stream this ctx has launched on and for its side
// stream; unrelated streams of the process are not waited for.
hipError_t sync_ctx_streams(lora_ctx *c)
{
    hipError_t first = hipSuccess;
    for (auto &st : c->streams) {
        const hipError_t e = hipStreamSynchronize(st.stream);
        if (e != hipSuccess && first == hipSuccess)
            first = e;
    }
    if (c->side) {
        const hipError_t e = hipStreamSynchronize(c->side);
        if (e != hipSuccess && first == hipSuccess)
            first = e;
    }
    return first;
}

// K-split of the shrink for a batch of T tokens in a group of n modules:
// enough workgroups to cover the chip when the batch is small, none when it is
// large.  A batch whose tiles times members already fill the chip's resident
// workgroups (512) is not split even when the ctx has room for more partials:
// a split saves the prefill shrink a few us and costs the expand, which sums
// the partials, more (0.759 against 0.744 ms per Llama-7B prefill step).
void choose_splits(const lora_ctx *c, const Workspace &ws, const BatchState &bs, int T, int d_in,
                   int n, int *splits, int *kchunk)
{
    const int tiles = max_tiles_for(T, c->S, bs.tile_cap);
    int want = ceil_div(1024, std::max(tiles, 1));
    if (T > kInlinePlanTokens && tiles * n >= 512)
        want = 1;
    int cap = std::min(kMaxSplits, std::max(1, d_in / 256));
    cap = std::min(cap, splits_cap(nb_template(c->R_pad)));
    cap = std::min(cap, std::max(1, ws.hbuf_rows / std::max(T, 1)));
    int sp = std::max(1, std::min(want, cap));
    int kc = round_up(ceil_div(d_in, sp), kShrinkKBlock);
    *kchunk = kc;
    *splits = ceil_div(d_in, kc);
}

int check_ctx(lora_ctx *c) { return c ? LORA_OK : LORA_ERR_INVALID_ARGUMENT; }

enum { PROF_PLAN = 0, PROF_SHRINK = 1, PROF_EXPAND = 2, PROF_SAVED = 3, PROF_FUSED = 4 };

// Events for the next dispatch while profiling (none once the reserve is used
// up, and none for a dispatch captured into a graph).
LaunchTiming next_timing(lora_ctx *c, int kind, hipStream_t s)
{
    if (!c->profiling)
        return LaunchTiming{};
    if (c->prof_used >= c->prof_cap || stream_capturing(s)) {
        c->prof_untimed += 1;
        return LaunchTiming{};
    }
    c->prof_kind[c->prof_used] = kind;
    return c->prof_events[c->prof_used++];
}

SlotMeta group_meta(const lora_ctx *c, int n, const int32_t *modules, bool hinted)
{
    SlotMeta m;
    std::memset(&m, 0, sizeof m);
    for (int k = 0; k < c->S; ++k) {
        const bool readable = !hinted || c->hint[k];
        m.scale[k] = c->scale_host[k];
        m.rank[k] = readable ? (uint8_t)c->slot_rank[k] : 0;
        m.flags[k] = readable ? c->slot_flags[k] : 0;
    }
    for (int i = 0; i < n; ++i) {
        const int32_t *r = c->rank_host.data() + (size_t)modules[i] * c->S;
        for (int k = 0; k < c->S; ++k)
            if (r[k] > 0 && (!hinted || c->hint[k]))
                m.target[i][k >> 5] |= 1u << (k & 31);
    }
    return m;
}

int run_plan(lora_ctx *c, const Workspace &ws, BatchState &bs, const int32_t *idx, int32_t T,
             hipStream_t s)
{
    bs.hinted = false;
    bs.plan_mode = c->dtype == LORA_BF16 && T <= kInlinePlanTokens ? kPlanInline : kPlanTiles;
    bs.tile_cap = bs.plan_mode == kPlanInline ? inline_tile_tokens(c->R_pad) : kTileTokens;
    if (T > 0 && bs.plan_mode == kPlanTiles) {
        int rc = before_launch(c, s, false, false);
        if (rc)
            return rc;
        LaunchTiming t[2];
        t[0] = next_timing(c, PROF_PLAN, s);
        if (T > 1024)
            t[1] = next_timing(c, PROF_PLAN, s);
        HIP_TRY(c, launch_plan(idx, T, c->S, ws.plan, s, t));
    }
    if (T > 0)
        c->stats.plans += 1;
    c->stats.tokens += T;
    bs.idx = idx;
    bs.T = T;
    bs.last_n = 0;
    return LORA_OK;
}

// Launch arguments of a shrink of the planned batch for a group of modules
// (records the K-splits for the expand that follows).
ShrinkArgs shrink_args(lora_ctx *c, const Workspace &ws, BatchState &bs, int n,
                       const int32_t *modules, const void *const *x)
{
    const int T = bs.T;
    ShrinkArgs a;
    std::memset(&a, 0, sizeof a);
    a.n = n;
    a.grid_splits = 1;
    for (int i = 0; i < n; ++i) {
        const int mod = modules[i];
        const lora_module_shape sh = c->shapes[mod];
        int splits = 1, kchunk = 0;
        choose_splits(c, ws, bs, T, sh.d_in, n, &splits, &kchunk);
        a.x[i] = x[i];
        a.A[i] = c->A[mod];
        a.slot_stride_A[i] = c->strideA[mod];
        a.d_in[i] = sh.d_in;
        a.k_chunk[i] = kchunk;
        a.splits[i] = splits;
        a.grid_splits = std::max(a.grid_splits, splits);
        bs.last_splits[i] = splits;
    }
    a.plan = ws.plan;
    a.idx = bs.idx;
    a.T = T;
    a.S = c->S;
    a.plan_mode = bs.plan_mode;
    a.hpart = ws.hpart;
    a.member_stride = (int64_t)ws.hbuf_rows * c->R_pad;
    a.split_stride = (int64_t)T * c->R_pad;
    a.R_pad = c->R_pad;
    a.grid_tiles = max_tiles_for(T, c->S, bs.tile_cap);
    a.tile_cap = bs.tile_cap;
    a.mixed = T > 1024;
    // A small batch with a multiple of 8 K-splits runs every tile of one split
    // on one XCD: its workgroups warm that split's x block (all tokens) and,
    // when it is small, its A^T block (all slots) in that XCD's L2 while they
    // form the plan or read the published tile.
    a.warm = 0;
    if (c->dtype == LORA_BF16 && T <= kInlinePlanTokens && a.grid_splits % 8 == 0) {
        a.warm = kWarmX;
        int64_t a_bytes = 0;
        for (int i = 0; i < n; ++i)
            a_bytes = std::max<int64_t>(a_bytes, (int64_t)c->S * c->R_pad * a.k_chunk[i] * c->elem);
        if (a_bytes <= (256 << 10))
            a.warm |= kWarmA;
        const int rows = T + ((a.warm & kWarmA) ? c->S * c->R_pad : 0);
        a.warm_rows = ceil_div(rows, a.grid_tiles);
    }
    return a;
}

// Launch arguments of the expand matching the last shrink_args.
ExpandArgs expand_args(lora_ctx *c, const Workspace &ws, const BatchState &bs, int n,
                       const int32_t *modules, void *const *y)
{
    const int T = bs.T;
    ExpandArgs a;
    std::memset(&a, 0, sizeof a);
    a.n = n;
    a.grid_cols = 1;
    for (int i = 0; i < n; ++i) {
        const int mod = modules[i];
        const lora_module_shape sh = c->shapes[mod];
        a.y[i] = y[i];
        a.Bi[i] = c->Bi[mod];
        a.bias[i] = c->bias[mod];
        a.dora[i] = c->dora[mod];
        a.slot_stride_B[i] = c->strideB[mod];
        a.d_out[i] = sh.d_out;
        a.splits[i] = bs.last_splits[i];
        a.grid_cols = std::max(a.grid_cols, ceil_div(sh.d_out, kExpandCols));
        a.col_start[i + 1] = a.col_start[i] + ceil_div(sh.d_out, kExpandCols);
    }
    a.tiles = ws.plan.tiles;
    a.tile_tok = ws.plan.tile_tok;
    a.n_tiles = ws.plan.n_tiles;
    a.hpart = ws.hpart;
    a.member_stride = (int64_t)ws.hbuf_rows * c->R_pad;
    a.split_stride = (int64_t)T * c->R_pad;
    a.R_pad = c->R_pad;
    a.grid_tiles = max_tiles_for(T, c->S, bs.tile_cap);
    // large batches: one contiguous run of items per XCD.  With long slot
    // segments (prefill) the run is tile-major, every column chunk of a tile on
    // one XCD: the tile's h comes from HBM once and consecutive tiles of a slot
    // share its B in L2 (0.74 vs 0.81 ms per Llama-7B prefill step).  With about
    // one tile per slot it is chunk-major, which measured 4% faster on the churn
    // workload (8192 tokens over 128 slots).  Small batches: round-robin.
    const int64_t items = (int64_t)a.grid_tiles * a.col_start[n];
    const bool large = T > kInlinePlanTokens;
    a.tile_major = large && T >= 128 * c->S;
    a.tile_cap = bs.tile_cap;
    a.xcd_group = large ? (int)((items + 7) / 8) : -1;
    a.terms = 0;
    for (int k = 0; k < c->S; ++k)
        if (c->slot_flags[k] && (!bs.hinted || c->hint[k]))
            a.terms = 1;
    return a;
}

int run_shrink(lora_ctx *c, const Workspace &ws, BatchState &bs, int n, const int32_t *modules,
               const void *const *x, hipStream_t s)
{
    const int T = bs.T;
    if (T > 0) {
        int rc = before_launch(c, s, true, bs.hinted);
        if (rc)
            return rc;
        const ShrinkArgs a = shrink_args(c, ws, bs, n, modules, x);
        HIP_TRY(c, launch_shrink(c->dtype == LORA_BF16, a, group_meta(c, n, modules, bs.hinted), s,
                                 next_timing(c, PROF_SHRINK, s)));
        if (bs.plan_mode == kPlanInline)
            bs.plan_mode = kPlanTiles;   // later launches read the plan this one published
        c->stats.shrinks += n;
    }
    bs.last_n = n;
    c->shrink_epoch = c->slot_epoch;
    for (int i = 0; i < n; ++i) {
        bs.last_modules[i] = modules[i];
        bs.last_x[i] = x[i];
    }
    return LORA_OK;
}

// Launch arguments of the saved-module products of a group, or false when no
// slot the batch may read saves any member's module.
bool saved_args(const lora_ctx *c, const Workspace &ws, const BatchState &bs, int n,
                const int32_t *modules, void *const *y, SavedArgs *out)
{
    SavedArgs &a = *out;
    std::memset(&a, 0, sizeof a);
    bool any = false;
    a.n = n;
    for (int i = 0; i < n; ++i) {
        const int mod = modules[i];
        const lora_module_shape sh = c->shapes[mod];
        a.x[i] = bs.last_x[i];
        a.y[i] = y[i];
        a.W[i] = c->saved_W[mod];
        a.bias[i] = c->saved_bias[mod];
        a.slot_stride_W[i] = (int64_t)sh.d_out * sh.d_in;
        a.d_in[i] = sh.d_in;
        a.d_out[i] = sh.d_out;
        a.col_start[i + 1] = a.col_start[i] + ceil_div(sh.d_out, kSavedCols);
        if (!c->saved_W[mod])
            continue;
        const uint8_t *sv = c->saved_host.data() + (size_t)mod * c->S;
        const uint8_t *sb = c->saved_bias_host.data() + (size_t)mod * c->S;
        for (int k = 0; k < c->S; ++k) {
            if (!sv[k] || (bs.hinted && !c->hint[k]))
                continue;
            a.saved[i][k >> 5] |= 1u << (k & 31);
            if (sb[k])
                a.has_bias[i][k >> 5] |= 1u << (k & 31);
            any = true;
        }
    }
    a.tiles = ws.plan.tiles;
    a.tile_tok = ws.plan.tile_tok;
    a.n_tiles = ws.plan.n_tiles;
    a.grid_tiles = max_tiles_for(bs.T, c->S, bs.tile_cap);
    a.T = bs.T;
    return any;
}

int run_expand(lora_ctx *c, const Workspace &ws, const BatchState &bs, int n,
               const int32_t *modules, void *const *y, hipStream_t s)
{
    const int T = bs.T;
    if (T > 0) {
        int rc = before_launch(c, s, true, bs.hinted);
        if (rc)
            return rc;
        const ExpandArgs a = expand_args(c, ws, bs, n, modules, y);
        HIP_TRY(c, launch_expand(c->dtype == LORA_BF16, a, group_meta(c, n, modules, bs.hinted), s,
                                 next_timing(c, PROF_EXPAND, s)));
        c->stats.expands += n;
        // saved modules replace the base output of their slots' tokens (disjoint
        // from the tokens the low-rank update touches for the same module)
        SavedArgs sa;
        if (saved_args(c, ws, bs, n, modules, y, &sa))
            HIP_TRY(c, launch_saved(c->dtype == LORA_BF16, sa, s, next_timing(c, PROF_SAVED, s)));
        int rc2 = record_slot_use(c, s, bs.hinted);
        if (rc2)
            return rc2;
    }
    return LORA_OK;
}

// Shrink and expand of one group in one launch (bf16 batches of at most
// kInlinePlanTokens on a workspace with fused counts, on a device that places
// workgroups whose indices agree mod 8 on one XCD), then the saved-module
// products of the group.
int run_fused(lora_ctx *c, const Workspace &ws, BatchState &bs, int n, const int32_t *modules,
              const void *const *x, void *const *y, hipStream_t s)
{
    const int T = bs.T;
    for (int i = 0; i < n; ++i) {
        bs.last_modules[i] = modules[i];
        bs.last_x[i] = x[i];
    }
    bs.last_n = n;
    c->shrink_epoch = c->slot_epoch;
    if (T == 0)
        return LORA_OK;
    int rc = before_launch(c, s, true, bs.hinted);
    if (rc)
        return rc;
    FusedArgs f;
    std::memset(&f, 0, sizeof f);
    f.s = shrink_args(c, ws, bs, n, modules, x);     // records the K-splits for the expand
    f.e = expand_args(c, ws, bs, n, modules, y);
    f.sync = ws.sync;
    f.spin_limit = kFusedSpinLimit;
    HIP_TRY(c, launch_fused(f, group_meta(c, n, modules, bs.hinted), s, next_timing(c, PROF_FUSED, s)));
    if (bs.plan_mode == kPlanInline)
        bs.plan_mode = kPlanTiles;   // later launches read the plan this one published
    c->stats.shrinks += n;
    c->stats.expands += n;
    SavedArgs sa;
    if (saved_args(c, ws, bs, n, modules, y, &sa))
        HIP_TRY(c, launch_saved(c->dtype == LORA_BF16, sa, s, next_timing(c, PROF_SAVED, s)));
    return record_slot_use(c, s, bs.hinted);
}

bool fused_applies(const lora_ctx *c, const Workspace &ws, const BatchState &bs)
{
    return c->dtype == LORA_BF16 && c->xcd_local && ws.sync && bs.T <= kInlinePlanTokens;
}

int check_group(lora_ctx *c, int32_t n, const int32_t *modules)
{
    if (n < 1 || n > LORA_MAX_GROUP || !modules)
        return fail(c, LORA_ERR_INVALID_ARGUMENT, "group size %d not in 1..%d", n, LORA_MAX_GROUP);
    for (int i = 0; i < n; ++i)
        if (modules[i] < 0 || modules[i] >= c->n_modules)
            return fail(c, LORA_ERR_BAD_MODULE, "module %d not in 0..%d", modules[i],
                        c->n_modules - 1);
    return LORA_OK;
}

int check_ptrs(lora_ctx *c, int32_t n, const void *const *p, const char *what, bool distinct)
{
    if (!p)
        return fail(c, LORA_ERR_INVALID_ARGUMENT, "%s array is NULL", what);
    for (int i = 0; i < n; ++i) {
        if (!p[i])
            return fail(c, LORA_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", what, i);
        if (distinct)
            for (int j = 0; j < i; ++j)
                if (p[j] == p[i])
                    return fail(c, LORA_ERR_INVALID_ARGUMENT, "%s[%d] and %s[%d] are the same buffer",
                                what, j, what, i);
    }
    return LORA_OK;
}

// One batch's workspace carved out of this device's scratch array: the plan
// buffers first, the rest for the h partials of n group members.  The flags
// word stays the ctx's own.  *need is the bytes the batch takes; false when
// they exceed the array.
bool scratch_workspace(const lora_ctx *c, int T, int n, Workspace *ws, size_t *need)
{
    char *base = (char *)c->scratch;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base + off;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    const int tiles = std::max(max_tiles_for(T, c->S),
                               max_tiles_for(std::min(T, (int)kInlinePlanTokens), c->S,
                                             inline_tile_tokens(c->R_pad)));
    ws->plan.counts = (int32_t *)take(sizeof(int32_t) * (size_t)c->S);
    ws->plan.seg_start = (int32_t *)take(sizeof(int32_t) * (size_t)c->S);
    ws->plan.tiles = (Tile *)take(sizeof(Tile) * (size_t)tiles);
    ws->plan.tile_tok = (int32_t *)take(sizeof(int32_t) * (size_t)tiles * kTileTokens);
    ws->plan.n_tiles = (int32_t *)take(sizeof(int32_t));
    ws->plan.n_active = (int32_t *)take(sizeof(int32_t));
    ws->plan.chunk_counts = (int32_t *)take(sizeof(int32_t) * (size_t)ceil_div(T, 1024) * c->S);
    ws->plan.flags = c->ws.plan.flags;
    const size_t row = sizeof(float) * (size_t)c->R_pad * n;    // one token's h, all members
    *need = off + row * (size_t)T;
    if (*need > kScratchBytes)
        return false;
    ws->hpart = (float *)(base + off);
    ws->hbuf_rows = (int)((kScratchBytes - off) / row);
    return true;
}

}  // namespace

extern "C" {

const char *lora_status_string(int status)
{
    switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LORA_ERR_RANK_EXCEEDS_MAX: return "LoRA rank exceeds maximum (r > max_rank)";
    case LORA_ERR_SLOT_OUT_OF_RANGE: return "slot out of range";
    case LORA_ERR_BAD_MODULE: return "module index out of range";
    case LORA_ERR_TOO_MANY_TOKENS: return "n_tokens exceeds max_tokens";
    case LORA_ERR_HOST_NOT_PINNED: return "adapter weights are not in pinned host or device memory";
    case LORA_ERR_OUT_OF_MEMORY: return "device out of memory";
    case LORA_ERR_HIP: return "HIP runtime error";
    case LORA_ERR_NO_PLAN: return "no prepared plan (call lora_plan_prepare first)";
    default: return "unknown status";
    }
}

const char *lora_last_error(lora_ctx *ctx)
{
    return ctx ? ctx->last_error.c_str() : g_create_error.c_str();
}

int lora_slots_create(lora_ctx **out, int32_t max_loras, int32_t max_rank,
                      const lora_module_shape *modules, int32_t n_modules, int32_t dtype_arg,
                      int32_t max_tokens, int32_t device)
{
    g_create_error.clear();
    if (!out)
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    if (max_loras < 1 || max_loras > LORA_MAX_SLOTS)
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "max_loras %d not in 1..%d", max_loras,
                    LORA_MAX_SLOTS);
    if (max_rank < 1)
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "max_rank %d < 1", max_rank);
    if (max_rank > LORA_MAX_RANK)
        return fail(nullptr, LORA_ERR_RANK_EXCEEDS_MAX, "max_rank %d > %d", max_rank,
                    LORA_MAX_RANK);
    if (!modules || n_modules < 1)
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "no modules");
    if (dtype_arg != LORA_BF16 && dtype_arg != LORA_FP32)
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype_arg);
    const lora_dtype dtype = dtype_arg == LORA_BF16 ? LORA_BF16 : LORA_FP32;
    if (max_tokens < 1)
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "max_tokens %d < 1", max_tokens);
    for (int m = 0; m < n_modules; ++m) {
        const auto &sh = modules[m];
        if (sh.d_in < 8 || sh.d_out < 8 || sh.d_in % 8 || sh.d_out % 8)
            return fail(nullptr, LORA_ERR_INVALID_ARGUMENT,
                        "module %d: d_in %d / d_out %d must be positive multiples of 8", m,
                        sh.d_in, sh.d_out);
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
        (void)hipGetLastError();
        return fail(nullptr, LORA_ERR_INVALID_ARGUMENT, "device %d not available (%d devices)",
                    device, ndev);
    }
    DeviceGuard guard(device);
    if (!guard.ok)
        return fail(nullptr, LORA_ERR_HIP, "hipSetDevice(%d) failed", device);

    lora_ctx *c = new lora_ctx();
    c->device = device;
    c->dtype = dtype;
    c->S = max_loras;
    c->R = max_rank;
    c->R_pad = round_up(max_rank, 16);
    c->n_modules = n_modules;
    c->max_tokens = max_tokens;
    c->elem = dtype == LORA_BF16 ? 2 : 4;
    c->shapes.assign(modules, modules + n_modules);
    c->rank_host.assign((size_t)n_modules * max_loras, 0);
    c->scale_host.assign(max_loras, 0.f);

    // the side stream first: allocations are zeroed on it
    hipError_t e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
    int max_out = 0;
    for (int m = 0; m < n_modules && e == hipSuccess; ++m) {
        const auto &sh = modules[m];
        const int64_t sa = (int64_t)c->R_pad * sh.d_in, sb = (int64_t)c->R_pad * sh.d_out;
        void *a = nullptr, *b = nullptr;
        e = dalloc(c, &a, (size_t)(sa * max_loras * c->elem));
        if (e == hipSuccess)
            e = dalloc(c, &b, (size_t)(sb * max_loras * c->elem));
        void *cb = nullptr;
        float *gb = nullptr;
        if (e == hipSuccess)
            e = dalloc(c, &cb, (size_t)sh.d_out * max_loras * c->elem);
        if (e == hipSuccess)
            e = dalloc(c, &gb, sizeof(float) * (size_t)sh.d_out * max_loras);
        c->A.push_back(a);
        c->Bi.push_back(b);
        c->bias.push_back(cb);
        c->dora.push_back(gb);
        c->strideA.push_back(sa);
        c->strideB.push_back(sb);
        max_out = std::max(max_out, sh.d_out);
    }
    c->ws.hbuf_rows = std::max(max_tokens, 16384);
    c->slot_rank.assign(max_loras, 0);
    c->slot_flags.assign(max_loras, 0);
    c->saved_W.assign(n_modules, nullptr);
    c->saved_bias.assign(n_modules, nullptr);
    c->saved_host.assign((size_t)n_modules * max_loras, 0);
    c->saved_bias_host.assign((size_t)n_modules * max_loras, 0);
    c->hint.assign(max_loras, 0);
    c->last_use.assign(max_loras, 0);
    c->max_tiles = std::max(max_tiles_for(max_tokens, max_loras),
                            max_tiles_for(std::min(max_tokens, (int)kInlinePlanTokens), max_loras,
                                          inline_tile_tokens(c->R_pad)));
    // A^T and B of every module of a load side by side, within 64 MB (at least
    // one module)
    int64_t sum_io = 0, max_io = 0;
    for (int m = 0; m < n_modules; ++m) {
        sum_io += modules[m].d_in + modules[m].d_out;
        max_io = std::max<int64_t>(max_io, modules[m].d_in + modules[m].d_out);
    }
    c->stage_elems = std::max<int64_t>((int64_t)c->R_pad * max_io,
                                       std::min<int64_t>((int64_t)c->R_pad * sum_io,
                                                         (64ll << 20) / c->elem));
    if (e == hipSuccess) e = dalloc(c, &c->stage, (size_t)c->stage_elems * c->elem);
    if (e == hipSuccess)
        e = dalloc(c, &c->ws.hpart, sizeof(float) * (size_t)kMaxGroup * c->ws.hbuf_rows * c->R_pad);
    if (e == hipSuccess) e = dalloc(c, &c->ws.plan.counts, sizeof(int32_t) * (size_t)max_loras);
    if (e == hipSuccess) e = dalloc(c, &c->ws.plan.seg_start, sizeof(int32_t) * (size_t)max_loras);
    if (e == hipSuccess) e = dalloc(c, &c->ws.plan.tiles, sizeof(Tile) * (size_t)c->max_tiles);
    if (e == hipSuccess)
        e = dalloc(c, &c->ws.plan.tile_tok, sizeof(int32_t) * (size_t)c->max_tiles * kTileTokens);
    if (e == hipSuccess)
        e = dalloc(c, &c->ws.sync, sizeof(uint32_t) * kSyncWordsPerTile * (size_t)c->max_tiles);
    if (e == hipSuccess) e = dalloc(c, &c->ws.plan.n_tiles, sizeof(int32_t));
    if (e == hipSuccess) e = dalloc(c, &c->ws.plan.n_active, sizeof(int32_t));
    if (e == hipSuccess) e = dalloc(c, &c->ws.plan.flags, sizeof(uint32_t));
    if (e == hipSuccess)
        e = dalloc(c, &c->ws.plan.chunk_counts,
                   sizeof(int32_t) * (size_t)ceil_div(max_tokens, 1024) * max_loras);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->load_done, hipEventDisableTiming);
    // this device's static scratch array (lora_apply_group_noalloc), looked up
    // once per device with the device current
    if (e == hipSuccess) e = scratch_address(device, &c->scratch);
    if (e == hipSuccess) e = xcd_dispatch_check(device, c->side, &c->xcd_local);
    if (e == hipSuccess) e = hipStreamSynchronize(c->side);
    if (e != hipSuccess) {
        int status = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
                         ? LORA_ERR_OUT_OF_MEMORY : LORA_ERR_HIP;
        fail(nullptr, status, "slot pool allocation: %s", hipGetErrorString(e));
        (void)hipGetLastError();
        free_all(c);
        delete c;
        return status;
    }
    *out = c;
    return LORA_OK;
}

int lora_slots_destroy(lora_ctx *ctx)
{
    if (!ctx)
        return LORA_OK;
    DeviceGuard guard(ctx->device);
    (void)sync_ctx_streams(ctx);
    (void)hipGetLastError();
    free_all(ctx);
    delete ctx;
    return LORA_OK;
}

int lora_slot_load(lora_ctx *ctx, int32_t slot, const void *const *A_t, const void *const *B,
                   int32_t r, double lora_alpha, int32_t use_rslora)
{
    return lora_slot_load_ex(ctx, slot, A_t, B, nullptr, nullptr, r, lora_alpha, use_rslora);
}

int lora_slot_load_ex(lora_ctx *ctx, int32_t slot, const void *const *A_t, const void *const *B,
                      const void *const *bias, const float *const *dora_scale, int32_t r,
                      double lora_alpha, int32_t use_rslora)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    if (slot < 0 || slot >= ctx->S)
        return fail(ctx, LORA_ERR_SLOT_OUT_OF_RANGE, "slot %d not in 0..%d", slot, ctx->S - 1);
    if (r > ctx->R)
        return fail(ctx, LORA_ERR_RANK_EXCEEDS_MAX, "rank %d exceeds max_rank %d", r, ctx->R);
    if (r < 1)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "rank %d < 1", r);
    if (!A_t || !B)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "A_t / B arrays are NULL");
    const double sd = use_rslora ? lora_alpha / std::sqrt((double)r) : lora_alpha / (double)r;
    const float s = (float)sd;
    if (!std::isfinite(s))
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "scale is not finite (lora_alpha %g)",
                    lora_alpha);
    std::vector<uint8_t> in_place, bias_in, dora_in;   // per module: read by the finalize in place
    {
        DeviceGuard guard(ctx->device);
        in_place.assign(ctx->n_modules, 0);
        bias_in.assign(ctx->n_modules, 0);
        dora_in.assign(ctx->n_modules, 0);
        for (int m = 0; m < ctx->n_modules; ++m) {
            if ((A_t[m] == nullptr) != (B[m] == nullptr))
                return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                            "module %d: A_t and B must both be given or both be NULL", m);
            bool ia = false, ib = false;
            if (A_t[m] && (check_source(A_t[m], ctx->device, &ia) || check_source(B[m], ctx->device, &ib)))
                return fail(ctx, LORA_ERR_HOST_NOT_PINNED,
                            "module %d: weights must be pinned host or device memory", m);
            in_place[m] = ia && ib;
            if (A_t[m] && bias && !bias[m])
                return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "module %d: bias entry is NULL", m);
            if (A_t[m] && dora_scale && !dora_scale[m])
                return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "module %d: dora_scale entry is NULL", m);
            bool ic = false, ig = false;
            if (A_t[m] && ((bias && check_source(bias[m], ctx->device, &ic)) ||
                           (dora_scale && check_source(dora_scale[m], ctx->device, &ig))))
                return fail(ctx, LORA_ERR_HOST_NOT_PINNED,
                            "module %d: bias / dora_scale must be pinned host or device memory", m);
            bias_in[m] = bias && ic;
            dora_in[m] = dora_scale && ig;
        }
    }
    DeviceGuard guard(ctx->device);
    // The fences below record events on the compute streams; on a stream under
    // capture that would pull the load into the graph.
    for (auto &st : ctx->streams)
        if (stream_capturing(st.stream))
            return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                        "slot load while a stream this ctx launched on is under graph capture");
    // A load that may run beside kernels it does not wait for (batches of
    // declared plans in flight on a stream this ctx launched on) stages its
    // weights with the copy engine: the in-place finalize streams over the link
    // on the CUs and would take them from those kernels (measured: a pipelined
    // churn step 1.32 -> 1.61 ms).  The side stream waits in full for streams
    // fenced below or at an earlier load with no launch since.
    bool beside_compute = false;
    for (auto &st : ctx->streams) {
        if (st.used_since_load || !st.since_fence)
            continue;
        const hipError_t q = hipStreamQuery(st.stream);
        if (q != hipSuccess)
            (void)hipGetLastError();   // not-ready is an answer, not an error to keep
        if (q == hipErrorNotReady)
            beside_compute = true;
    }
    if (beside_compute) {
        std::fill(in_place.begin(), in_place.end(), 0);
        std::fill(bias_in.begin(), bias_in.end(), 0);
        std::fill(dora_in.begin(), dora_in.end(), 0);
    }
    int rc = fence_compute_streams(ctx);
    if (rc)
        return rc;
    if (ctx->last_use[slot]) {
        HIP_TRY(ctx, hipStreamWaitEvent(ctx->side, ctx->use_ev[ctx->last_use[slot] % lora_ctx::kUseEvents], 0));
        ctx->last_use[slot] = 0;
    }
    int64_t bytes = 0;
    const bool bf16 = ctx->dtype == LORA_BF16;
    // One finalize launch per batch of modules moves A^T into the slot and
    // repacks B.  It reads weights the device can reach in place directly (over
    // the link for pinned host memory, at about the rate of a copy engine, and
    // with no copy-to-kernel hand-over per load).  Other weights go to the stage
    // first, in module order, A^T then B; ranges that follow each other both in
    // the source and in the stage are moved by one copy, and the finalize runs
    // in stream order after its copies.
    FinalizeBatch fb;
    std::memset(&fb, 0, sizeof fb);
    fb.r = r;
    fb.R_pad = ctx->R_pad;
    int64_t stage_used = 0;
    const char *run_src = nullptr;
    char *run_dst = nullptr;
    size_t run_bytes = 0;
    auto flush_run = [&]() -> hipError_t {
        hipError_t e = hipSuccess;
        if (run_bytes)
            e = hipMemcpyAsync(run_dst, run_src, run_bytes, hipMemcpyDefault, ctx->side);
        run_bytes = 0;
        return e;
    };
    auto add_range = [&](const void *src, char *dst, size_t n) -> hipError_t {
        if (run_bytes && (const char *)src == run_src + run_bytes && dst == run_dst + run_bytes) {
            run_bytes += n;
            return hipSuccess;
        }
        hipError_t e = flush_run();
        run_src = (const char *)src;
        run_dst = dst;
        run_bytes = n;
        return e;
    };
    for (int m = 0; m < ctx->n_modules; ++m) {
        if (!A_t[m])
            continue;
        const auto sh = ctx->shapes[m];
        const int64_t a_elems = (int64_t)r * sh.d_in, b_elems = (int64_t)r * sh.d_out;
        char *Aslot = (char *)ctx->A[m] + (size_t)slot * ctx->strideA[m] * ctx->elem;
        char *Bslot = (char *)ctx->Bi[m] + (size_t)slot * ctx->strideB[m] * ctx->elem;
        const size_t abytes = (size_t)a_elems * ctx->elem, bbytes = (size_t)b_elems * ctx->elem;
        bytes += (int64_t)abytes + (int64_t)bbytes;
        void *cdst = bias_in[m] ? (char *)ctx->bias[m] + (size_t)slot * sh.d_out * ctx->elem : nullptr;
        float *gdst = dora_in[m] ? ctx->dora[m] + (size_t)slot * sh.d_out : nullptr;
        const void *csrc = bias_in[m] ? bias[m] : nullptr;
        const float *gsrc = dora_in[m] ? dora_scale[m] : nullptr;
        if (in_place[m]) {
            if (fb.n == kFinalizeBatch) {
                HIP_TRY(ctx, flush_run());
                HIP_TRY(ctx, launch_slot_finalize(bf16, fb, ctx->side));
                fb.n = 0;
                stage_used = 0;
            }
            fb.it[fb.n++] = FinalizeItem{Aslot, Bslot, A_t[m], B[m], cdst, csrc, gdst, gsrc,
                                         sh.d_in, sh.d_out};
            continue;
        }
        if (fb.n == kFinalizeBatch || stage_used + a_elems + b_elems > ctx->stage_elems) {
            HIP_TRY(ctx, flush_run());
            HIP_TRY(ctx, launch_slot_finalize(bf16, fb, ctx->side));
            fb.n = 0;
            stage_used = 0;
        }
        char *Ast = (char *)ctx->stage + (size_t)stage_used * ctx->elem;
        char *Bst = Ast + abytes;
        HIP_TRY(ctx, add_range(A_t[m], Ast, abytes));
        HIP_TRY(ctx, add_range(B[m], Bst, bbytes));
        fb.it[fb.n++] = FinalizeItem{Aslot, Bslot, Ast, Bst, cdst, csrc, gdst, gsrc, sh.d_in, sh.d_out};
        stage_used += a_elems + b_elems;
    }
    HIP_TRY(ctx, flush_run());
    HIP_TRY(ctx, launch_slot_finalize(bf16, fb, ctx->side));
    // output terms the finalize did not read in place, straight into the slot's rows
    for (int m = 0; m < ctx->n_modules && (bias || dora_scale); ++m) {
        if (!A_t[m])
            continue;
        const int d_out = ctx->shapes[m].d_out;
        if (bias && !bias_in[m])
            HIP_TRY(ctx, hipMemcpyAsync((char *)ctx->bias[m] + (size_t)slot * d_out * ctx->elem, bias[m],
                                        (size_t)d_out * ctx->elem, hipMemcpyDefault, ctx->side));
        if (dora_scale && !dora_in[m])
            HIP_TRY(ctx, hipMemcpyAsync(ctx->dora[m] + (size_t)slot * d_out, dora_scale[m],
                                        sizeof(float) * (size_t)d_out, hipMemcpyDefault, ctx->side));
    }
    HIP_TRY(ctx, hipEventRecord(ctx->load_done, ctx->side));
    ctx->load_gen += 1;
    for (int m = 0; m < ctx->n_modules; ++m) {
        ctx->rank_host[(size_t)m * ctx->S + slot] = A_t[m] ? r : 0;
        ctx->saved_host[(size_t)m * ctx->S + slot] = 0;      // the new adapter saves nothing yet
        ctx->saved_bias_host[(size_t)m * ctx->S + slot] = 0;
    }
    ctx->slot_rank[slot] = r;
    ctx->slot_flags[slot] = (uint8_t)((bias ? kSlotBias : 0) | (dora_scale ? kSlotDora : 0));
    ctx->scale_host[slot] = s;
    ctx->slot_epoch += 1;
    ctx->stats.loads += 1;
    ctx->stats.bytes_loaded += bytes;
    return LORA_OK;
}

int lora_slot_clear(lora_ctx *ctx, int32_t slot)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    if (slot < 0 || slot >= ctx->S)
        return fail(ctx, LORA_ERR_SLOT_OUT_OF_RANGE, "slot %d not in 0..%d", slot, ctx->S - 1);
    // Launches capture the rank table by value, so clearing needs no device work:
    // batches already enqueued keep the adapter, later ones skip the slot.
    for (int m = 0; m < ctx->n_modules; ++m) {
        ctx->rank_host[(size_t)m * ctx->S + slot] = 0;
        ctx->saved_host[(size_t)m * ctx->S + slot] = 0;
        ctx->saved_bias_host[(size_t)m * ctx->S + slot] = 0;
    }
    ctx->slot_rank[slot] = 0;
    ctx->slot_flags[slot] = 0;
    ctx->slot_epoch += 1;
    ctx->stats.clears += 1;
    return LORA_OK;
}

int lora_slot_load_saved(lora_ctx *ctx, int32_t slot, int32_t module, const void *W,
                         const void *bias)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    if (slot < 0 || slot >= ctx->S)
        return fail(ctx, LORA_ERR_SLOT_OUT_OF_RANGE, "slot %d not in 0..%d", slot, ctx->S - 1);
    if (module < 0 || module >= ctx->n_modules)
        return fail(ctx, LORA_ERR_BAD_MODULE, "module %d not in 0..%d", module, ctx->n_modules - 1);
    if (!W)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "W is NULL");
    if (ctx->slot_rank[slot] == 0)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                    "slot %d holds no adapter: load the adapter before its saved modules", slot);
    if (ctx->rank_host[(size_t)module * ctx->S + slot] > 0)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                    "module %d is a low-rank target of the adapter in slot %d; a module is either "
                    "targeted or saved", module, slot);
    DeviceGuard guard(ctx->device);
    if (check_source(W, ctx->device) || (bias && check_source(bias, ctx->device)))
        return fail(ctx, LORA_ERR_HOST_NOT_PINNED, "W / bias must be pinned host or device memory");
    for (auto &st : ctx->streams)
        if (stream_capturing(st.stream))
            return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                        "slot load while a stream this ctx launched on is under graph capture");
    const lora_module_shape sh = ctx->shapes[module];
    const size_t wbytes = (size_t)sh.d_out * sh.d_in * ctx->elem;
    if (!ctx->saved_W[module]) {
        // the module's pool, at its first saved load (all slots at once)
        void *wp = nullptr, *bp = nullptr;
        hipError_t e = hipMalloc(&wp, wbytes * ctx->S);
        if (e == hipSuccess)
            e = hipMalloc(&bp, (size_t)sh.d_out * ctx->elem * ctx->S);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            if (wp)
                (void)hipFree(wp);
            return fail(ctx, (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
                                 ? LORA_ERR_OUT_OF_MEMORY : LORA_ERR_HIP,
                        "saved-module pool of module %d (%zu bytes): %s", module,
                        wbytes * ctx->S, hipGetErrorString(e));
        }
        ctx->allocations.push_back(wp);
        ctx->allocations.push_back(bp);
        ctx->saved_W[module] = wp;
        ctx->saved_bias[module] = bp;
    }
    // the same write-after-read fences as a low-rank load of the slot
    int rc = fence_compute_streams(ctx);
    if (rc)
        return rc;
    if (ctx->last_use[slot]) {
        HIP_TRY(ctx, hipStreamWaitEvent(ctx->side, ctx->use_ev[ctx->last_use[slot] % lora_ctx::kUseEvents], 0));
        ctx->last_use[slot] = 0;
    }
    HIP_TRY(ctx, hipMemcpyAsync((char *)ctx->saved_W[module] + wbytes * slot, W, wbytes,
                                hipMemcpyDefault, ctx->side));
    if (bias)
        HIP_TRY(ctx, hipMemcpyAsync((char *)ctx->saved_bias[module] + (size_t)sh.d_out * ctx->elem * slot,
                                    bias, (size_t)sh.d_out * ctx->elem, hipMemcpyDefault, ctx->side));
    HIP_TRY(ctx, hipEventRecord(ctx->load_done, ctx->side));
    ctx->load_gen += 1;
    ctx->saved_host[(size_t)module * ctx->S + slot] = 1;
    ctx->saved_bias_host[(size_t)module * ctx->S + slot] = bias ? 1 : 0;
    ctx->slot_epoch += 1;
    return LORA_OK;
}

int lora_sync_loads(lora_ctx *ctx)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(ctx->device);
    HIP_TRY(ctx, hipStreamSynchronize(ctx->side));
    ctx->synced_gen = ctx->load_gen;
    return LORA_OK;
}

int lora_plan_prepare(lora_ctx *ctx, const int32_t *token_slot_idx, int32_t n_tokens,
                      void *stream)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    if (n_tokens < 0)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "n_tokens %d < 0", n_tokens);
    if (n_tokens > ctx->max_tokens)
        return fail(ctx, LORA_ERR_TOO_MANY_TOKENS, "n_tokens %d > max_tokens %d", n_tokens,
                    ctx->max_tokens);
    if (n_tokens > 0 && !token_slot_idx)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "token_slot_idx is NULL");
    DeviceGuard guard(ctx->device);
    int rc = run_plan(ctx, ctx->ws, ctx->bs, token_slot_idx, n_tokens, (hipStream_t)stream);
    if (rc) {
        ctx->plan_valid = ctx->plan_prepared = false;
        return rc;
    }
    ctx->plan_valid = ctx->plan_prepared = true;
    return LORA_OK;
}

int lora_plan_prepare_slots(lora_ctx *ctx, const int32_t *token_slot_idx, int32_t n_tokens,
                            const int32_t *used_slots, int32_t n_used, void *stream)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    if (n_used < 0 || (n_used > 0 && !used_slots))
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "used_slots: %d entries at %p", n_used,
                    (const void *)used_slots);
    for (int i = 0; i < n_used; ++i)
        if (used_slots[i] < 0 || used_slots[i] >= ctx->S)
            return fail(ctx, LORA_ERR_SLOT_OUT_OF_RANGE, "used_slots[%d] = %d not in 0..%d", i,
                        used_slots[i], ctx->S - 1);
    int rc = lora_plan_prepare(ctx, token_slot_idx, n_tokens, stream);
    if (rc)
        return rc;
    std::fill(ctx->hint.begin(), ctx->hint.end(), 0);
    for (int i = 0; i < n_used; ++i)
        ctx->hint[used_slots[i]] = 1;
    ctx->bs.hinted = true;
    return LORA_OK;
}

int lora_shrink_group(lora_ctx *ctx, int32_t n, const int32_t *modules, const void *const *x,
                      void *stream)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    int rc = check_group(ctx, n, modules);
    if (rc)
        return rc;
    if (!ctx->plan_valid)
        return fail(ctx, LORA_ERR_NO_PLAN, "lora_shrink needs a prepared plan");
    if (ctx->bs.T > 0 && (rc = check_ptrs(ctx, n, x, "x", false)))
        return rc;
    DeviceGuard guard(ctx->device);
    return run_shrink(ctx, ctx->ws, ctx->bs, n, modules, x, (hipStream_t)stream);
}

int lora_expand_group(lora_ctx *ctx, int32_t n, const int32_t *modules, void *const *y,
                      void *stream)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    int rc = check_group(ctx, n, modules);
    if (rc)
        return rc;
    if (!ctx->plan_valid)
        return fail(ctx, LORA_ERR_NO_PLAN, "lora_expand needs a prepared plan");
    bool same = ctx->bs.last_n == n;
    for (int i = 0; same && i < n; ++i)
        same = ctx->bs.last_modules[i] == modules[i];
    if (!same)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                    "lora_expand must follow lora_shrink of the same module list");
    if (ctx->shrink_epoch != ctx->slot_epoch)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT,
                    "a slot was loaded or cleared between lora_shrink and lora_expand");
    if (ctx->bs.T > 0 && (rc = check_ptrs(ctx, n, (const void *const *)y, "y", true)))
        return rc;
    DeviceGuard guard(ctx->device);
    return run_expand(ctx, ctx->ws, ctx->bs, n, modules, y, (hipStream_t)stream);
}

int lora_shrink(lora_ctx *ctx, const void *x, int32_t module, void *stream)
{
    return lora_shrink_group(ctx, 1, &module, &x, stream);
}

int lora_expand(lora_ctx *ctx, void *y, int32_t module, void *stream)
{
    return lora_expand_group(ctx, 1, &module, &y, stream);
}

namespace {

// lora_apply_group and lora_apply_group_fused: plan unless prepared, then the
// group's update as two launches, or as one fused launch where it applies.
int apply_group(lora_ctx *ctx, int32_t n, const int32_t *modules, const void *const *x,
                void *const *y, const int32_t *token_slot_idx, int32_t n_tokens, void *stream,
                bool fused)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    int rc = check_group(ctx, n, modules);
    if (rc)
        return rc;
    if (n_tokens < 0)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "n_tokens %d < 0", n_tokens);
    if (n_tokens > ctx->max_tokens)
        return fail(ctx, LORA_ERR_TOO_MANY_TOKENS, "n_tokens %d > max_tokens %d", n_tokens,
                    ctx->max_tokens);
    if (n_tokens == 0)
        return LORA_OK;
    if (!token_slot_idx)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "token_slot_idx is NULL");
    if ((rc = check_ptrs(ctx, n, x, "x", false)) ||
        (rc = check_ptrs(ctx, n, (const void *const *)y, "y", true)))
        return rc;
    DeviceGuard guard(ctx->device);
    hipStream_t s = (hipStream_t)stream;
    if (!(ctx->plan_valid && ctx->plan_prepared && ctx->bs.idx == token_slot_idx &&
          ctx->bs.T == n_tokens)) {
        ctx->plan_prepared = false;
        rc = run_plan(ctx, ctx->ws, ctx->bs, token_slot_idx, n_tokens, s);
        if (rc) {
            ctx->plan_valid = false;
            return rc;
        }
        ctx->plan_valid = true;
    }
    if (fused && fused_applies(ctx, ctx->ws, ctx->bs))
        return run_fused(ctx, ctx->ws, ctx->bs, n, modules, x, y, s);
    rc = run_shrink(ctx, ctx->ws, ctx->bs, n, modules, x, s);
    if (rc)
        return rc;
    return run_expand(ctx, ctx->ws, ctx->bs, n, modules, y, s);
}

}  // namespace

int lora_apply_group(lora_ctx *ctx, int32_t n, const int32_t *modules, const void *const *x,
                     void *const *y, const int32_t *token_slot_idx, int32_t n_tokens,
                     void *stream)
{
    return apply_group(ctx, n, modules, x, y, token_slot_idx, n_tokens, stream, false);
}

int lora_apply_group_fused(lora_ctx *ctx, int32_t n, const int32_t *modules, const void *const *x,
                           void *const *y, const int32_t *token_slot_idx, int32_t n_tokens,
                           void *stream)
{
    return apply_group(ctx, n, modules, x, y, token_slot_idx, n_tokens, stream, true);
}

int lora_apply(lora_ctx *ctx, const void *x, void *y, const int32_t *token_slot_idx,
               int32_t n_tokens, int32_t module, void *stream)
{
    return lora_apply_group(ctx, 1, &module, &x, &y, token_slot_idx, n_tokens, stream);
}

int lora_apply_group_noalloc(lora_ctx *ctx, int32_t n, const int32_t *modules,
                             const void *const *x, void *const *y,
                             const int32_t *token_slot_idx, int32_t n_tokens, void *stream)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    int rc = check_group(ctx, n, modules);
    if (rc)
        return rc;
    if (n_tokens < 0)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "n_tokens %d < 0", n_tokens);
    if (n_tokens > ctx->max_tokens)
        return fail(ctx, LORA_ERR_TOO_MANY_TOKENS, "n_tokens %d > max_tokens %d", n_tokens,
                    ctx->max_tokens);
    if (n_tokens == 0)
        return LORA_OK;
    if (!token_slot_idx)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "token_slot_idx is NULL");
    if ((rc = check_ptrs(ctx, n, x, "x", false)) ||
        (rc = check_ptrs(ctx, n, (const void *const *)y, "y", true)))
        return rc;
    Workspace ws;
    size_t need = 0;
    if (!scratch_workspace(ctx, n_tokens, n, &ws, &need))
        return fail(ctx, LORA_ERR_TOO_MANY_TOKENS,
                    "%d tokens x %d modules need %zu bytes of scratch; the static array holds %zu",
                    n_tokens, n, need, (size_t)kScratchBytes);
    DeviceGuard guard(ctx->device);
    hipStream_t s = (hipStream_t)stream;
    // a plan of its own, in the scratch array; the ctx's plan is left as it is
    BatchState bs;
    if ((rc = run_plan(ctx, ws, bs, token_slot_idx, n_tokens, s)))
        return rc;
    const uint64_t shrink_epoch = ctx->shrink_epoch;
    rc = run_shrink(ctx, ws, bs, n, modules, x, s);
    ctx->shrink_epoch = shrink_epoch;
    if (rc)
        return rc;
    return run_expand(ctx, ws, bs, n, modules, y, s);
}

int lora_get_device_flags(lora_ctx *ctx, uint32_t *flags)
{
    if (check_ctx(ctx) || !flags)
        return LORA_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(ctx->device);
    // the kernels that set flags ran on the ctx's streams: wait for those
    // only, then read and clear the word in order on the side stream
    HIP_TRY(ctx, sync_ctx_streams(ctx));
    HIP_TRY(ctx, hipMemcpyAsync(&ctx->flags_host, ctx->ws.plan.flags, sizeof(uint32_t),
                                hipMemcpyDeviceToHost, ctx->side));
    HIP_TRY(ctx, hipMemsetAsync(ctx->ws.plan.flags, 0, sizeof(uint32_t), ctx->side));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->side));
    *flags = ctx->flags_host;
    return LORA_OK;
}

int lora_profile_begin(lora_ctx *ctx, int32_t max_launches)
{
    if (check_ctx(ctx))
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    if (max_launches < 0)
        return fail(ctx, LORA_ERR_INVALID_ARGUMENT, "max_launches %d < 0", max_launches);
    DeviceGuard guard(ctx->device);
    while ((int32_t)ctx->prof_events.size() < max_launches) {
        LaunchTiming t;
        HIP_TRY(ctx, hipEventCreate(&t.start));
        if (hipEventCreate(&t.stop) != hipSuccess) {
            (void)hipEventDestroy(t.start);
            return fail(ctx, LORA_ERR_HIP, "hipEventCreate failed");
        }
        ctx->prof_events.push_back(t);
    }
    ctx->prof_kind.assign(ctx->prof_events.size(), 0);
    ctx->prof_cap = (size_t)max_launches;
    ctx->prof_used = 0;
    ctx->prof_untimed = 0;
    ctx->profiling = true;
    return LORA_OK;
}

int lora_profile_end(lora_ctx *ctx, lora_profile *out)
{
    if (check_ctx(ctx) || !out)
        return LORA_ERR_INVALID_ARGUMENT;
    ctx->last_error.clear();
    std::memset(out, 0, sizeof *out);
    DeviceGuard guard(ctx->device);
    ctx->profiling = false;
    for (size_t i = 0; i < ctx->prof_used; ++i) {
        const LaunchTiming &t = ctx->prof_events[i];
        HIP_TRY(ctx, hipEventSynchronize(t.stop));
        float ms = 0.f;
        HIP_TRY(ctx, hipEventElapsedTime(&ms, t.start, t.stop));
        out->launches[ctx->prof_kind[i]] += 1;
        out->total_ms[ctx->prof_kind[i]] += ms;
    }
    out->untimed = ctx->prof_untimed;
    ctx->prof_used = 0;
    return LORA_OK;
}

int lora_get_stats(lora_ctx *ctx, lora_stats *out)
{
    if (check_ctx(ctx) || !out)
        return LORA_ERR_INVALID_ARGUMENT;
    *out = ctx->stats;
    return LORA_OK;
}

}  // extern "C"
