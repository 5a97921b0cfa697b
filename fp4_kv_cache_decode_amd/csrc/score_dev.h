// Indexer scoring core shared by the scoring kernels and the fused Reindex
// layer: FP8 E4M3 keys of 64 dims, 4 heads, score_t = sum_h w_h * max(0, q_h . khat_t)
// (the reading of the indexer taken in index_score.hip's header, after
// origotech.dev deep dive "Inside DeepSeek V4.1-Flash", section "How the
// architecture shrinks the KV cache").
#pragma once

#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {
namespace score_dev {

constexpr int SC_THREADS = 256;
constexpr int STEP = 64;                 // keys per wave step
constexpr int WAVES = SC_THREADS / 64;
constexpr float NEG_INF = -__builtin_huge_valf();

struct ScoreArgs {
    const uint8_t* idxk;
    const float* q_idx;
    const float* w;
    const int32_t* seq;
    const int64_t* ctx;
    const int32_t* pool;     // pool mode
    float* out;              // block maxima (full mode) or pool scores (pool mode)
    int64_t cap;
    int64_t max_ctx;
    int64_t out_stride;
    PageMap pm;              // page table of a paged cache (table null otherwise)
    int32_t n_seq;
    int32_t n_queries;       // B (rows of q_idx / out)
    int32_t n_blocks;        // pool mode
    int32_t keys_per_wg;
    float scale;
};

struct Raw {
    uint4 d[4];
};

// Lanes whose key is not visible load key 0 of the sequence (always in bounds)
// and have their score masked later: no branch, no register clearing.
template <bool PAGED>
__device__ __forceinline__ void load_key(Raw& r, const ScoreArgs& a, const uint8_t* idxk,
                                         int32_t s, int64_t t, bool ok) {
    const uint4* p =
        reinterpret_cast<const uint4*>(idxk + cache_row<PAGED>(a.pm, a.cap, s, ok ? t : 0) * IDX_DIM);
    r.d[0] = p[0];
    r.d[1] = p[1];
    r.d[2] = p[2];
    r.d[3] = p[3];
}

// One key's 64 E4M3 codes as fp32 (exact).
__device__ __forceinline__ void key_f32(const Raw& r, float (&kf)[64]) {
    const uint32_t dw[16] = {r.d[0].x, r.d[0].y, r.d[0].z, r.d[0].w, r.d[1].x, r.d[1].y,
                             r.d[1].z, r.d[1].w, r.d[2].x, r.d[2].y, r.d[2].z, r.d[2].w,
                             r.d[3].x, r.d[3].y, r.d[3].z, r.d[3].w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float2 lo = e4m3x2_to_f32<false>(dw[i]);
        const float2 hi = e4m3x2_to_f32<true>(dw[i]);
        kf[4 * i] = lo.x;
        kf[4 * i + 1] = lo.y;
        kf[4 * i + 2] = hi.x;
        kf[4 * i + 3] = hi.y;
    }
}

// Score of one key against one query; wh already carries the key scale
// (w_h * max(0, s*d) = (w_h * s) * max(0, d) for s > 0).
__device__ __forceinline__ float key_dot(const float (&kf)[64], const float* __restrict__ q,
                                         const float (&wh)[4]) {
    // two accumulator chains per head (a single 64-long chain measured slower)
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float* qh = q + 64 * h;
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int d = 0; d < 64; d += 2) {
            a0 = fmaf(qh[d], kf[d], a0);
            a1 = fmaf(qh[d + 1], kf[d + 1], a1);
        }
        s = fmaf(wh[h], fmaxf(a0 + a1, 0.0f), s);
    }
    return s + 0.0f;
}

__device__ __forceinline__ float key_score(const Raw& r, const float* __restrict__ q,
                                           const float (&wh)[4]) {
    float kf[64];
    key_f32(r, kf);
    return key_dot(kf, q, wh);
}

// Body of one scoring workgroup (bx, b) of SC_THREADS threads, t the thread's
// index in it, bx and b uniform.  q, keys and out are distinct buffers
// (restrict), so the query loads are provably unclobbered and can be scalar
// loads.  `zero` is 0 at run time; adding zero * step to the query address
// makes it loop-variant, so the compiler reloads one head at a time (64 SGPRs)
// instead of hoisting all 256 floats.
// STAGE (pool mode, several steps per wave): the workgroup's slice of the
// block list is copied to LDS first (pslice, CSA2_MAX_POOL entries), so that a
// step's key loads wait on an LDS read of their block instead of a global
// load.  Without STAGE the body has no barrier, so several bodies can run side
// by side in one larger workgroup.
template <bool POOL, bool PAGED, bool STAGE>
__device__ __forceinline__ void score_body(const ScoreArgs& a, const float* __restrict__ q_all,
                                           const uint8_t* __restrict__ idxk,
                                           float* __restrict__ out_all, int64_t zero, int bx,
                                           int b, int t, int32_t* pslice) {
    const int lane = t & 63;
    // wave index is uniform per wave; say so, so that k0 and the query address are SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t N = clamp64(a.ctx[b], 0, a.max_ctx);
    const int32_t s = a.seq[b];
    if (s < 0 || s >= a.n_seq) return;
    const int64_t n_items = POOL ? (int64_t)a.n_blocks * BLOCK : N;
    const int64_t wg0 = (int64_t)bx * a.keys_per_wg;
    if (wg0 >= n_items) return;
    const int64_t wg_end = wg0 + a.keys_per_wg < n_items ? wg0 + a.keys_per_wg : n_items;

    const float* q = q_all + (int64_t)b * IDX_HEADS * IDX_DIM;
    float wh[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) wh[h] = a.w[(int64_t)b * IDX_HEADS + h] * a.scale;
    float* out = out_all + (int64_t)b * a.out_stride;
    const int32_t* pool = POOL ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    const int64_t blk0 = wg0 >> 3;          // wg0 is a multiple of 256
    if (STAGE) {
        const int cnt = (int)(((wg_end + 7) >> 3) - blk0);
        for (int i = t; i < cnt; i += SC_THREADS) pslice[i] = pool[blk0 + i];
        __syncthreads();
    }

    // position of item i (pool mode maps through the block list); ok = visible
    auto locate = [&](int64_t i, int64_t& t) -> bool {
        if (POOL) {
            const int32_t pb = i < n_items ? (STAGE ? pslice[(i >> 3) - blk0] : pool[i >> 3]) : -1;
            t = (int64_t)pb * BLOCK + (i & 7);
            return pb >= 0 && t < N;
        }
        t = i;
        return i < N;
    };
    auto finish = [&](const Raw& r, int64_t k0, bool ok) {
        float sc = key_score(r, q + zero * k0, wh);
        sc = ok ? sc : NEG_INF;
        const int64_t item = k0 + lane;
        if (POOL) {
            if (item < n_items) out[item] = sc;
        } else {
            // lanes 8m..8m+7 hold block (k0/8 + m)
            float mx = fmaxf(sc, dpp_f32<DPP_XOR1>(sc));
            mx = fmaxf(mx, dpp_f32<DPP_XOR2>(mx));
            mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x101f)));
            const int64_t blk = (k0 >> 3) + (lane >> 3);
            if ((lane & 7) == 0 && blk * BLOCK < N) out[blk] = mx;
        }
    };

    // ping-pong key buffers: the next step's loads are issued first and pinned
    // there (the scheduler may not sink them into the arithmetic), so they are
    // in flight for a whole step of FMAs
    const int64_t stride = (int64_t)STEP * WAVES;
    int64_t k0 = wg0 + (int64_t)wave * STEP;
    Raw A, B;
    int64_t tA = 0, tB = 0;
    bool okA = k0 < wg_end && locate(k0 + lane, tA);
    load_key<PAGED>(A, a, idxk, s, tA, okA);
    for (; k0 < wg_end; k0 += 2 * stride) {
        const int64_t k1 = k0 + stride;
        const bool okB = k1 < wg_end && locate(k1 + lane, tB);
        load_key<PAGED>(B, a, idxk, s, tB, okB);
        __builtin_amdgcn_sched_barrier(0);
        finish(A, k0, okA);
        if (k1 >= wg_end) break;
        const int64_t k2 = k1 + stride;
        okA = k2 < wg_end && locate(k2 + lane, tA);
        load_key<PAGED>(A, a, idxk, s, tA, okA);
        __builtin_amdgcn_sched_barrier(0);
        finish(B, k1, okB);
    }
}

}  // namespace score_dev
}  // namespace csa2
