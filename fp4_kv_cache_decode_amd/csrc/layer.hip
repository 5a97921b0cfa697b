// One Reindex layer in a single cooperative launch.
//
// What is computed: a Reindex layer's indexer re-scores only the positions of
// its group's candidate pool, keeps the top-k of them, and the layer attends
// over those positions plus its 128-token window (origotech.dev deep dive
// "Inside DeepSeek V4.1-Flash", section "How the architecture shrinks the KV
// cache").  That is csa2_index_reindex followed by csa2_decode_attn_ex; this
// kernel runs the same device code (score_dev, topk_dev, attn_dev) on the same
// data in the same order, so its results are bit-identical to those two calls
// whenever they run the tile attention kernel.
//
// The separate calls are four kernels: pool scores, top-k, attention tiles,
// merge.  At decode batch sizes each is latency bound and each kernel
// boundary costs about 2 us.  Here the three boundaries become grid-wide
// barriers inside one launch.
//
// Layout: workgroups of 1,024 threads, all resident at once (cooperative
// launch), enough of them for every stage to finish in one round (loops over
// rounds made the compiler spill registers; larger batches are refused), and
// up to one per scoring run or tile.  Stage by stage:
//   1. scores: 256-thread scoring bodies, up to four side by side (one per
//      quarter of the workgroup), one 256-key run of one query each; they have
//      no barrier;
//   2. top-k: query b's row in workgroup b (the 1,024-thread select core);
//   3. attention: 64-entry tiles, up to four side by side, each quarter with
//      its own LDS; a quarter without a tile passes the tile's barriers;
//   4. merge: (head, query) merges of 128 threads, up to eight side by side.
//
// Grid barrier: the workgroup synchronises, its thread 0 fences (device
// scope) and arrives on a counter.  The last arrival resets the counter and
// then advances a generation word, which the others poll (the two words on
// separate cache lines).  An acquire fence and a workgroup barrier follow.
// The count is zero between barriers, so zero-filled words serve every later
// launch.
// Waits are bounded: a workgroup that has polled max_polls times stops
// waiting, ORs 1 into *status and goes on; its results are then undefined,
// but every wave still reaches the end of the kernel.
#include "attn_dev.h"
#include "csa2_device.h"
#include "csa2_internal.h"
#include "score_dev.h"
#include "topk_dev.h"

namespace csa2 {

namespace {

constexpr int LY_THREADS = 1024;
constexpr int LY_QUARTERS = LY_THREADS / attn_dev::AT_THREADS;     // tiles side by side
constexpr int LY_MERGES = LY_THREADS / D;                          // merges side by side
constexpr int32_t DEFAULT_MAX_POLLS = 1 << 20;
static_assert(score_dev::SC_THREADS == attn_dev::AT_THREADS, "one quarter per scoring body");
static_assert(topk_dev::BIG_T == LY_THREADS, "the select core takes the whole workgroup");

struct LayerArgs {
    score_dev::ScoreArgs sc;
    topk_dev::TopkArgs tk;
    attn_dev::TileArgs at;
    const float* q_idx;
    const uint8_t* idxk;
    float* scores;           // [B][n_blocks * 8] pool scores
    float* out;              // [B][16][128]
    LayerSync* sync;
    int32_t* status;
    int64_t zero;            // 0 (see score_body)
    int32_t B;
    int32_t n_runs;          // 256-key scoring runs per query
    int32_t max_polls;
};

union LayerShared {
    topk_dev::Shared<topk_dev::BIG_T> tk;
    attn_dev::AttnShared at[LY_QUARTERS];
};

// gen: this workgroup's count of completed barriers (its thread 0's copy, kept
// in LDS so that no register holds it through the stages).
__device__ __forceinline__ void grid_barrier(LayerSync* sy, uint32_t n_wg, uint32_t& gen,
                                             int32_t max_polls, int32_t* status) {
    // the workgroup barrier waits for every wave's stores; one device-scope
    // release by thread 0 then publishes them all (one L2 write-back per
    // workgroup, not one per wave)
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        bool wait = true;
        if (__hip_atomic_fetch_add(&sy->count.v, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == n_wg - 1) {
            // last arrival: reset the count, then release the others (release:
            // the reset is seen before the next barrier's arrivals)
            __hip_atomic_store(&sy->count.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&sy->gen.v, gen + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            wait = false;
        }
        if (wait) {
            int32_t polls = 0;
            while (__hip_atomic_load(&sy->gen.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   gen) {
                if (++polls > max_polls) {
                    atomicOr(status, 1);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        ++gen;
    }
    __syncthreads();
}

typedef __attribute__((address_space(4))) const LayerArgs* ArgsPtr;

// The kernel's argument block, read again from the argument segment: the
// empty asm hides where the pointer came from, so each stage loads the
// arguments it uses (scalar loads) instead of keeping every stage's arguments
// in registers for the whole kernel.
__device__ __forceinline__ const LayerArgs& stage_args() {
    ArgsPtr p = (ArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return *(const LayerArgs*)p;
}

__device__ __forceinline__ void barrier(uint32_t n_wg, uint32_t& gen) {
    const LayerArgs& f = stage_args();
    grid_barrier(f.sync, n_wg, gen, f.max_polls, f.status);
}

template <int AM>
__global__ void __launch_bounds__(LY_THREADS) reindex_layer_kernel(LayerArgs) {
    __shared__ LayerShared sh;
    __shared__ uint32_t gen;
    const uint32_t G = gridDim.x;
    // generation word at entry: read before this workgroup's first arrival, so
    // before any barrier of this launch can complete
    if (threadIdx.x == 0)
        gen = __hip_atomic_load(&stage_args().sync->gen.v, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);

    // ---- 1. pool scores: run v % n_runs of query v / n_runs, v = quarter * G +
    // workgroup (quarter 0 of every workgroup first: one body per CU when the
    // grid is wide enough)
    {
        const LayerArgs& f = stage_args();
        const int qt = __builtin_amdgcn_readfirstlane(threadIdx.x / attn_dev::AT_THREADS);
        const int t = threadIdx.x % attn_dev::AT_THREADS;
        const int v = qt * (int)G + blockIdx.x;
        constexpr bool PAGED = AM == attn_dev::AM_PAGED;
        if (v < f.B * f.n_runs)
            score_dev::score_body<true, PAGED, false>(f.sc, f.q_idx, f.idxk, f.scores, f.zero,
                                                      v % f.n_runs, v / f.n_runs, t, nullptr);
    }
    barrier(G, gen);

    // ---- 2. top-k of each query's pool scores: query b in workgroup b
    {
        const LayerArgs& f = stage_args();
        const int b = blockIdx.x;
        if (b < f.B) {
            if (f.tk.n_fixed <= topk_dev::SMALL_MAX)
                topk_dev::topk_small_body(sh.tk, f.tk, b);
            else
                topk_dev::topk_run32_body(sh.tk, f.tk, b);
        }
    }
    barrier(G, gen);

    // ---- 3. attention: tile v % n_tiles of query v / n_tiles, v as above
    {
        const LayerArgs& f = stage_args();
        const int qt = __builtin_amdgcn_readfirstlane(threadIdx.x / attn_dev::AT_THREADS);
        const int t = threadIdx.x % attn_dev::AT_THREADS;
        const int v = qt * (int)G + blockIdx.x;
        if (v < f.B * f.at.n_tiles) {
            attn_dev::tile_body<AM>(f.at, sh.at[qt], v % f.at.n_tiles, v / f.at.n_tiles, t);
        } else {
            // the tile's workgroup barriers, so that the other quarters' pair up
#pragma unroll
            for (int i = 0; i < attn_dev::TILE_BARRIERS; ++i) __syncthreads();
        }
    }
    barrier(G, gen);

    // ---- 4. merge of the tiles' partials: head v % 16 of query v / 16,
    // v = slot * G + workgroup
    {
        const LayerArgs& f = stage_args();
        const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x / D);
        const int v = slot * (int)G + blockIdx.x;
        if (v < f.B * HEADS)
            attn_dev::merge_body(f.at.part, f.at.n_tiles, f.out, v % HEADS, v / HEADS,
                                 threadIdx.x % D);
    }
}

// Workgroups of the kernel that can be resident at once on the current device.
template <int AM>
int resident_limit() {
    int dev = -1, per_cu = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&reindex_layer_kernel<AM>), LY_THREADS, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return per_cu * n_cu;
}

int cdiv(int64_t x, int64_t y) { return (int)((x + y - 1) / y); }

// Workgroups for one round of every stage (at least), and as many as one per
// scoring run or tile would take (at most, within the resident limit): the
// bodies of a workgroup share one CU, so spreading them shortens each stage.
int layer_grid(int32_t B, int32_t n_blocks, int32_t topk, int limit) {
    const int runs = cdiv((int64_t)n_blocks * BLOCK, score_dev::SC_THREADS);
    const int n_tiles = cdiv(topk, attn_dev::TILE) + WINDOW / attn_dev::TILE;
    int need = cdiv((int64_t)B * runs, LY_QUARTERS);
    need = need > B ? need : B;
    const int tiles = cdiv((int64_t)B * n_tiles, LY_QUARTERS);
    need = need > tiles ? need : tiles;
    const int merges = cdiv((int64_t)B * HEADS, LY_MERGES);
    need = need > merges ? need : merges;
    const int64_t spread = (int64_t)B * (runs > n_tiles ? runs : n_tiles);
    const int want = spread < limit ? (int)spread : limit;
    return want > need ? want : need;
}

template <int AM>
hipError_t launch_layer(LayerArgs& f, int grid, hipStream_t stream) {
    void* args[] = {&f};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&reindex_layer_kernel<AM>),
                                      dim3((unsigned)grid), dim3(LY_THREADS), args, 0, stream);
}

int address_mode(const csa2_cache& c) {
    if (c.page_table) return attn_dev::AM_PAGED;
    return (uint64_t)c.cap * RECORD <= 0xffffffffull ? attn_dev::AM_OFF32 : attn_dev::AM_FLAT64;
}

int resident_limit(const csa2_cache& c) {
    switch (address_mode(c)) {
        case attn_dev::AM_PAGED: return resident_limit<attn_dev::AM_PAGED>();
        case attn_dev::AM_OFF32: return resident_limit<attn_dev::AM_OFF32>();
        default: return resident_limit<attn_dev::AM_FLAT64>();
    }
}

}  // namespace

bool reindex_layer_fits(const csa2_cache& c, int32_t B, int32_t n_blocks, int32_t topk) {
    const int limit = resident_limit(c);
    return limit > 0 && layer_grid(B, n_blocks, topk, limit) <= limit;
}

hipError_t launch_reindex_layer(const csa2_cache& c, const csa2_window& w, int32_t layer,
                                const float* q_idx, const float* wts, const float* q,
                                const int32_t* seq, const int64_t* ctx, int32_t B,
                                const int32_t* pool, int32_t n_blocks, int32_t topk,
                                float sm_scale, int32_t* idx, uint8_t* kvg_out, float* out,
                                int32_t max_polls, int32_t* status, LayerSync* sync,
                                float* scores, float* partials, hipStream_t stream) {
    using namespace attn_dev;
    LayerArgs f{};
    const int32_t n_pos = n_blocks * BLOCK;
    // pool scores: one 256-key run per scoring body (one 64-key step per wave)
    score_dev::ScoreArgs& s = f.sc;
    s.idxk = c.idxk;
    s.q_idx = q_idx;
    s.w = wts;
    s.seq = seq;
    s.ctx = ctx;
    s.pool = pool;
    s.out = scores;
    s.cap = c.cap;
    s.max_ctx = c.cap;
    s.out_stride = n_pos;
    s.pm = page_map(c);
    s.n_seq = c.n_seq;
    s.n_blocks = n_blocks;
    s.keys_per_wg = score_dev::SC_THREADS;
    s.scale = c.idxk_scale;
    f.n_runs = (n_pos + score_dev::SC_THREADS - 1) / score_dev::SC_THREADS;
    // top-k over the pool's positions, reported as positions
    topk_dev::TopkArgs& k = f.tk;
    k.vals = scores;
    k.stride = n_pos;
    k.n_fixed = n_pos;
    k.pool = pool;
    k.n_blocks = n_blocks;
    k.k = topk;
    k.out = idx;
    // attention tiles over the selected positions and the window
    TileArgs& a = f.at;
    a.kv = c.kv;
    a.kvg_out = kvg_out;
    a.wk = w.k;
    a.wv = w.v;
    a.q = q;
    a.idx = idx;
    a.seq = seq;
    a.ctx = ctx;
    a.part = partials;
    a.cap = c.cap;
    a.pm = page_map(c);
    a.n_seq = c.n_seq;
    a.w_cap = w.w_cap;
    a.layer = layer;
    a.topk = topk;
    a.n_main = (topk + TILE - 1) / TILE;
    a.n_tiles = a.n_main + WINDOW / TILE;
    a.wk_scale = w.k_scale;
    a.wv_scale = w.v_scale;
    a.sm_scale = sm_scale;
    f.q_idx = q_idx;
    f.idxk = c.idxk;
    f.scores = scores;
    f.out = out;
    f.sync = sync;
    f.status = status;
    f.zero = 0;
    f.B = B;
    f.max_polls = max_polls > 0 ? max_polls : DEFAULT_MAX_POLLS;
    const int grid = layer_grid(B, n_blocks, topk, resident_limit(c));
    switch (address_mode(c)) {
        case AM_PAGED: return launch_layer<AM_PAGED>(f, grid, stream);
        case AM_OFF32: return launch_layer<AM_OFF32>(f, grid, stream);
        default: return launch_layer<AM_FLAT64>(f, grid, stream);
    }
}

}  // namespace csa2
