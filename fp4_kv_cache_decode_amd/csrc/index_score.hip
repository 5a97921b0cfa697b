// Indexer scoring over FP8 E4M3 keys.
//
// What is computed: the indexer of a Full or Reindex layer scores cached
// positions so that top-k selection can run (origotech.dev deep dive "Inside
// DeepSeek V4.1-Flash", section "How the architecture shrinks the KV cache";
// trawling.dev "CSA2 and FP4 KV caching").  The pages do not give the score
// function; this library reads it as
//     score_t = sum_h w_h * max(0, q_h . khat_t),  khat_t = E4M3(code_t) * scale,
// with 4 heads of 64 dims, and a block's score as the max over its 8 positions.
//
// Design (gfx950, wave64): one key per lane, 64 keys (4 KB) per wave step.  A
// workgroup's query (or its four queries, in prefill-sized batches) is the same
// for every lane, so it is read as scalar (SGPR) operands of v_fma_f32 straight
// from the scalar cache, one head (64 floats) at a time: no lane holds a copy
// of it and no cross-lane reduction is needed.
// FP8->fp32 uses the packed converter (2 values per instruction); the dot
// products are plain fp32 FMAs (the 1e-5 relative score budget rules out f16
// query math).  Block maxima come from DPP/swizzle max over the 8 lanes of a
// block, no LDS involved.
//
// Two kernels share this scoring core:
//  - score_kernel<true> scores a Reindex (or the Full layer's second) pass over
//    the pool's 2,048 runs of 8 positions: latency bound, each lane holding its
//    key plus the next one in flight in registers;
//  - scan_kernel scores the whole context of a Full layer, keys streamed
//    through a per-wave LDS ring (below): HBM bound in decode; in a chunked
//    prefill it scores four queries per key pass and is bound by fp32 VALU.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "score_dev.h"

namespace csa2 {

namespace {

using namespace score_dev;

// One workgroup per (run of keys_per_wg keys, query).
template <bool POOL, bool PAGED, bool STAGE>
__global__ void __launch_bounds__(SC_THREADS)
score_kernel(ScoreArgs a, const float* __restrict__ q_all, const uint8_t* __restrict__ idxk,
             float* __restrict__ out_all, int64_t zero) {
    __shared__ int32_t pslice[STAGE ? CSA2_MAX_POOL : 1];
    score_body<POOL, PAGED, STAGE>(a, q_all, idxk, out_all, zero, blockIdx.x, blockIdx.y,
                                   threadIdx.x, pslice);
}

// ---------------------------------------------------------------------------
// Full-context scan with an LDS staging ring.
//
// Each wave streams its own 64-key (4 KB) steps into a private ring of
// SCAN_STAGES LDS slots with global_load_lds_dwordx4: one instruction moves a
// contiguous 1 KB of keys (lane l's 16 bytes land at slot + 16 l), so every
// load is fully coalesced and no VGPR holds data in flight.  The wave then
// reads its own key (64 bytes) from LDS and scores it as above.
// SCAN_STAGES - 1 steps are in flight while one is scored.
//
// Bank-conflict-free reads: a key occupies 64 bytes of LDS, and 16 lanes
// reading the same 16-byte chunk of 16 consecutive keys would hit only four
// distinct 16-byte bank groups.  The 16-byte chunks of key j (j mod 16) are
// therefore stored rotated by chunk_rot(j): chunk m sits at position
// (m + chunk_rot(j)) mod 4 of the key's 64 bytes.  The rotation is applied on
// the load side (each lane fetches the chunk that belongs at its LDS position,
// the same contiguous 1 KB per instruction) and undone by per-lane read
// addresses, so register m still holds channels 16m..16m+15 for every lane.
// chunk_rot is a permutation within every group of 4 keys with equal j mod 4
// (16-lane passes over 64 banks) and within every group of 4 keys of equal
// parity in an aligned run of 8 (8-lane passes over 32 banks).
//
// The loads are written as inline asm so that the compiler neither reorders
// them nor inserts a full vmcnt(0) drain before every LDS read; the waits are
// explicit: with j steps issued after step i, "s_waitcnt vmcnt(4 j)" leaves
// only the later steps' loads outstanding (loads complete in order; the block
// maxima stores in between only make the wait stricter).  The asm statements
// carry a memory clobber, which keeps the LDS reads of a step after its wait
// and before the next refill of the same slot.
constexpr int SCAN_STAGES = 2;   // 16 waves x 2 x 4 KB = 128 KB of LDS per CU
constexpr int SCAN_STEP_BYTES = STEP * IDX_DIM;   // 4096

// chunk_rot, dma_1k and wait_vm live in csa2_device.h (shared with top-k).

// One workgroup per CU: 16 waves (4 per SIMD), each with a private LDS ring.
// (Measured: 16 waves with 2 slots beat 12 waves with 3 slots by about 3%.)
// The workgroup's 64-key steps are handed out by an LDS counter, so a wave
// that the SIMD's issue order favours simply takes more steps and all waves
// of the CU finish within one step of each other (with a static split, the
// oldest wave on a SIMD finishes first and the last one runs alone, with its
// memory latency exposed).
constexpr int SCAN_WAVES = 16;
constexpr int SCAN_THREADS = SCAN_WAVES * 64;
constexpr int SCAN_GROUP = 4;            // queries per key pass in large batches
constexpr int32_t SCAN_GROUP_MIN_B = 1024;

// Scores one key stream, sequence s keys [wg0, min(wg0 + keys_per_wg, N)),
// against NQ queries: rows bq[], visible lengths nq[] (N is the largest).  The
// caller has zeroed next_step and synchronised; every wave calls this with the
// same (uniform) arguments.  NT: non-temporal key loads (keys read once).
template <bool PAGED, int NQ, bool NT>
__device__ __forceinline__ void scan_stream(const ScoreArgs& a, const float* __restrict__ q_all,
                                            const uint8_t* __restrict__ idxk,
                                            float* __restrict__ out_all, int64_t zero,
                                            uint8_t* my_ring, int* next_step, int32_t s,
                                            const int (&bq)[NQ], const int64_t (&nq)[NQ],
                                            int64_t N) {
    const int lane = threadIdx.x & 63;
    const int64_t wg0 = (int64_t)blockIdx.x * a.keys_per_wg;
    const int64_t wg_end = wg0 + a.keys_per_wg < N ? wg0 + a.keys_per_wg : N;
    const int n_steps = (int)((wg_end - wg0 + STEP - 1) / STEP);

    const uint8_t* keys = idxk + (int64_t)s * a.cap * IDX_DIM;
    const float* q[NQ];
    float wh[NQ][4];
    float* out[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        q[j] = q_all + (int64_t)bq[j] * IDX_HEADS * IDX_DIM;
#pragma unroll
        for (int h = 0; h < 4; ++h) wh[j][h] = a.w[(int64_t)bq[j] * IDX_HEADS + h] * a.scale;
        out[j] = out_all + (int64_t)bq[j] * a.out_stride;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)my_ring;

    // load side: lane l fills position l & 3 of key l >> 2 of each 1 KB group
    const int kl = lane >> 2;
    const int chunk_here = ((lane & 3) - chunk_rot(kl)) & 3;
    const uint32_t dma_off = (uint32_t)(64 * kl + 16 * chunk_here);
    // read side: channels 16m..16m+15 of this lane's key
    const uint8_t* rd[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        rd[m] = my_ring + 64 * lane + 16 * ((m + chunk_rot(lane & 15)) & 3);

    // next step of the workgroup for this wave, or -1 when none is left
    auto grab = [&]() -> int {
        int t = 0;
        if (lane == 0) t = atomicAdd(next_step, 1);
        t = __builtin_amdgcn_readfirstlane(t);
        return t < n_steps ? t : -1;
    };
    // issue step t into `slot`; a step that reaches past N loads key N - 1 in
    // place of the missing keys (in bounds; their scores are masked).  A step
    // is 64 aligned keys, so in a paged cache it lies inside one page; the page
    // id is a uniform (scalar-cache) load, and neighbouring steps share it.
    auto issue = [&](int t, int slot) {
        const int64_t kb = wg0 + (int64_t)t * STEP;
        const uint8_t* g =
            PAGED ? idxk + cache_row<true>(a.pm, a.cap, s, kb) * IDX_DIM : keys + kb * IDX_DIM;
        const uint32_t l = lds0 + (uint32_t)(slot * SCAN_STEP_BYTES);
        if (kb + STEP <= N) {
#pragma unroll
            for (int c = 0; c < 4; ++c) dma_1k<NT>(dma_off, g + 1024 * c, l + 1024 * c);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                int64_t j = kb + 16 * c + kl;
                j = j < N ? j : N - 1;
                dma_1k<NT>((uint32_t)((j - kb) * IDX_DIM + 16 * chunk_here), g, l + 1024 * c);
            }
        }
    };

    // sid[slot]: the step held in that slot (-1: none).  Steps are taken in
    // increasing order, so once a grab fails every later one fails too.
    int sid[SCAN_STAGES];
#pragma unroll
    for (int i = 0; i < SCAN_STAGES - 1; ++i) {
        sid[i] = i == 0 || sid[i - 1] >= 0 ? grab() : -1;
        if (sid[i] >= 0) issue(sid[i], i);
    }
    sid[SCAN_STAGES - 1] = -1;

    // score the step held in `slot` after topping up the ring; false when done
    auto step = [&](const int slot) -> bool {
        const int t = sid[slot];
        if (t < 0) return false;
        const int ns = (slot + SCAN_STAGES - 1) % SCAN_STAGES;
        sid[ns] = sid[(slot + SCAN_STAGES - 2) % SCAN_STAGES] >= 0 ? grab() : -1;
        if (sid[ns] >= 0) issue(sid[ns], ns);
        // steps issued after t: the valid ones among the next SCAN_STAGES - 1 slots
        int after = 0;
#pragma unroll
        for (int d = 1; d < SCAN_STAGES; ++d) after += sid[(slot + d) % SCAN_STAGES] >= 0;
        if (after >= SCAN_STAGES - 1) wait_vm<4 * (SCAN_STAGES - 1)>();
        else if (SCAN_STAGES > 2 && after == 1) wait_vm<4>();
        else wait_vm<0>();
        const int64_t k0 = wg0 + (int64_t)t * STEP;
        Raw r;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            r.d[m] = *reinterpret_cast<const uint4*>(rd[m] + slot * SCAN_STEP_BYTES);
        // the key is converted once and scored against every query of the stream
        float kf[64];
        key_f32(r, kf);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float sc = key_dot(kf, q[j] + zero * k0, wh[j]);
            const bool whole = k0 + STEP <= nq[j];    // uniform
            if (!whole) sc = k0 + lane < nq[j] ? sc : NEG_INF;
            float mx = fmaxf(sc, dpp_f32<DPP_XOR1>(sc));
            mx = fmaxf(mx, dpp_f32<DPP_XOR2>(mx));
            mx = fmaxf(mx,
                       __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x101f)));
            // lanes 8m..8m+7 hold block k0/8 + m; a block is visible iff its first key is
            float* ob = out[j] + (k0 >> 3);
            if ((lane & 7) == 0 && (whole || k0 + lane < nq[j])) ob[lane >> 3] = mx;
        }
        return true;
    };
    static_assert(SCAN_STAGES == 2, "the slot rotation below is written out for 2 slots");
    while (step(0) && step(1)) {
    }
}

// QPW = 1: one query per workgroup row (decode batches; keys are read once, so
// their loads are non-temporal).  QPW > 1: the workgroup row serves queries
// QPW*y .. QPW*y + QPW - 1 (chunked prefill, where a chunk's queries read one
// sequence and the keys are re-read from L2 by every row): when they share the
// sequence, each key is loaded and converted once and scored against all of
// them; otherwise they are scanned one after another.
template <bool PAGED, int QPW>
__global__ void __launch_bounds__(SCAN_THREADS)
scan_kernel(ScoreArgs a, const float* __restrict__ q_all, const uint8_t* __restrict__ idxk,
            float* __restrict__ out_all, int64_t zero) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[SCAN_WAVES][SCAN_STAGES][SCAN_STEP_BYTES];
    __shared__ int next_step;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t* const my_ring = &ring[wave][0][0];
    const int64_t wg0 = (int64_t)blockIdx.x * a.keys_per_wg;
    auto start = [&]() {
        if (threadIdx.x == 0) next_step = 0;
        __syncthreads();
    };
    if (QPW == 1) {
        const int bq[1] = {(int)blockIdx.y};
        const int64_t nq[1] = {clamp64(a.ctx[bq[0]], 0, a.max_ctx)};
        const int32_t s = a.seq[bq[0]];
        if (s < 0 || s >= a.n_seq || wg0 >= nq[0]) return;
        start();
        scan_stream<PAGED, 1, QPW == 1>(a, q_all, idxk, out_all, zero, my_ring, &next_step, s, bq, nq,
                              nq[0]);
        return;
    }
    // the group's queries; rows past the batch get length 0 (never written)
    // and borrow the first row's query and weights
    const int b0 = (int)blockIdx.y * QPW;
    int bq[QPW];
    int64_t nq[QPW];
    int32_t sq[QPW];
    bool shared = true;
    int64_t N = 0;
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        const bool in = b0 + j < a.n_queries;
        bq[j] = in ? b0 + j : b0;
        sq[j] = a.seq[bq[j]];
        const bool ok = in && sq[j] >= 0 && sq[j] < a.n_seq;
        nq[j] = ok ? clamp64(a.ctx[bq[j]], 0, a.max_ctx) : 0;
        shared &= !ok || sq[j] == sq[0];
        N = nq[j] > N ? nq[j] : N;
    }
    shared &= sq[0] >= 0 && sq[0] < a.n_seq;
    if (shared) {
        if (wg0 >= N) return;
        start();
        scan_stream<PAGED, QPW, false>(a, q_all, idxk, out_all, zero, my_ring, &next_step, sq[0], bq,
                                nq, N);
        return;
    }
    for (int j = 0; j < QPW; ++j) {
        if (wg0 >= nq[j]) continue;       // also an absent or invalid row (length 0)
        const int bj[1] = {bq[j]};
        const int64_t nj[1] = {nq[j]};
        start();
        scan_stream<PAGED, 1, false>(a, q_all, idxk, out_all, zero, my_ring, &next_step, sq[j], bj, nj,
                              nj[0]);
        __syncthreads();                  // every wave is done with the ring and the counter
    }
}

}  // namespace

// Keys per scan workgroup: one workgroup per CU (256 of them) across all
// rows, each a multiple of one 64-key step.
int32_t scan_keys_per_wg(int32_t B, int64_t max_ctx) {
    const int64_t total = (int64_t)B * max_ctx;
    int64_t kpw = (total + 255) / 256;
    kpw = (kpw + STEP - 1) / STEP * STEP;
    const int64_t row = (max_ctx + STEP - 1) / STEP * STEP;
    if (kpw > row) kpw = row;
    return (int32_t)(kpw < STEP ? STEP : (kpw > (1 << 30) ? (1 << 30) : kpw));
}

hipError_t launch_score_blocks(const csa2_cache& c, const float* q_idx, const float* w,
                               const int32_t* seq, const int64_t* ctx, int32_t B,
                               int64_t max_ctx, int64_t m_stride, float* M,
                               hipStream_t stream) {
    // batches of prefill size score four queries per key pass
    const int qpw = B >= SCAN_GROUP_MIN_B ? SCAN_GROUP : 1;
    const int32_t rows = (B + qpw - 1) / qpw;
    const int32_t keys_per_wg = scan_keys_per_wg(rows, max_ctx);
    ScoreArgs a{};
    a.idxk = c.idxk;
    a.q_idx = q_idx;
    a.w = w;
    a.seq = seq;
    a.ctx = ctx;
    a.out = M;
    a.cap = c.cap;
    a.max_ctx = max_ctx;
    a.out_stride = m_stride;
    a.pm = page_map(c);
    a.n_seq = c.n_seq;
    a.n_queries = B;
    a.keys_per_wg = keys_per_wg;
    a.scale = c.idxk_scale;
    dim3 grid((unsigned)((max_ctx + keys_per_wg - 1) / keys_per_wg), (unsigned)rows);
    if (grid.x == 0) return hipSuccess;
    const dim3 blk(SCAN_THREADS);
    const int64_t z = 0;
    if (qpw == 1) {
        if (c.page_table)
            hipLaunchKernelGGL((scan_kernel<true, 1>), grid, blk, 0, stream, a, q_idx, c.idxk, M, z);
        else
            hipLaunchKernelGGL((scan_kernel<false, 1>), grid, blk, 0, stream, a, q_idx, c.idxk, M, z);
    } else {
        if (c.page_table)
            hipLaunchKernelGGL((scan_kernel<true, SCAN_GROUP>), grid, blk, 0, stream, a, q_idx,
                               c.idxk, M, z);
        else
            hipLaunchKernelGGL((scan_kernel<false, SCAN_GROUP>), grid, blk, 0, stream, a, q_idx,
                               c.idxk, M, z);
    }
    return hipGetLastError();
}

hipError_t launch_score_pool(const csa2_cache& c, const float* q_idx, const float* w,
                             const int32_t* seq, const int64_t* ctx, int32_t B,
                             const int32_t* pool, int32_t n_blocks, float* S,
                             hipStream_t stream) {
    ScoreArgs a{};
    a.idxk = c.idxk;
    a.q_idx = q_idx;
    a.w = w;
    a.seq = seq;
    a.ctx = ctx;
    a.pool = pool;
    a.out = S;
    a.cap = c.cap;
    a.max_ctx = c.cap;
    a.out_stride = (int64_t)n_blocks * BLOCK;
    a.pm = page_map(c);
    a.n_seq = c.n_seq;
    a.n_blocks = n_blocks;
    // few queries: one step per wave (latency); many queries: longer runs per
    // workgroup, so that dispatch does not dominate (about 8 workgroups per CU)
    const int64_t items_all = (int64_t)B * n_blocks * BLOCK;
    int64_t kpw = items_all / (256 * 8);
    kpw = kpw < STEP * WAVES ? STEP * WAVES : (kpw + STEP * WAVES - 1) / (STEP * WAVES) * (STEP * WAVES);
    const int64_t row = ((int64_t)n_blocks * BLOCK + STEP * WAVES - 1) / (STEP * WAVES) * (STEP * WAVES);
    a.keys_per_wg = (int32_t)(kpw > row ? row : kpw);
    a.scale = c.idxk_scale;
    const int64_t items = (int64_t)n_blocks * BLOCK;
    dim3 grid((unsigned)((items + a.keys_per_wg - 1) / a.keys_per_wg), (unsigned)B);
    const bool stage = a.keys_per_wg > STEP * WAVES;      // several steps per wave
    const dim3 blk(SC_THREADS);
    const int64_t z = 0;
    if (c.page_table) {
        if (stage)
            hipLaunchKernelGGL((score_kernel<true, true, true>), grid, blk, 0, stream, a, q_idx,
                               c.idxk, S, z);
        else
            hipLaunchKernelGGL((score_kernel<true, true, false>), grid, blk, 0, stream, a, q_idx,
                               c.idxk, S, z);
    } else {
        if (stage)
            hipLaunchKernelGGL((score_kernel<true, false, true>), grid, blk, 0, stream, a, q_idx,
                               c.idxk, S, z);
        else
            hipLaunchKernelGGL((score_kernel<true, false, false>), grid, blk, 0, stream, a, q_idx,
                               c.idxk, S, z);
    }
    return hipGetLastError();
}

}  // namespace csa2
