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
// Design (gfx950, wave64, HBM-bound): a wave scores 64 keys (4 KB) per step.
// Each key is split over a lane pair: lane 2m+r holds dims 32r..32r+31 of keys
// m and 32+m, so a lane keeps only half of the 4x64 query in VGPRs (128 regs)
// and streams its keys with 16-byte loads.  The FP8->fp32 conversion uses the
// packed converter (2 values per instruction) and the dot products are plain
// fp32 FMAs (the 1e-5 relative score budget rules out f16 query math).  One
// DPP exchange per head finishes each key: the lane pair swaps the half-sums of
// the key it does not keep.  Block maxima come from row_ror DPP max over lanes
// of equal parity, so no LDS is touched in the hot loop.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int SC_THREADS = 256;
constexpr int KEYS_PER_STEP = 64;        // per wave
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
    int32_t n_seq;
    int32_t n_blocks;        // pool mode
    int32_t keys_per_wg;
    float scale;
};

// Dot products of one lane's 32 dims of a key with the 4 head half-queries.
__device__ __forceinline__ void half_dots(const uint4& a, const uint4& b, const float (&qv)[4][32],
                                          float (&acc)[4]) {
    const uint32_t dw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float2 lo = e4m3x2_to_f32<false>(dw[i]);
        float2 hi = e4m3x2_to_f32<true>(dw[i]);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            acc[h] = fmaf(qv[h][4 * i + 0], lo.x, acc[h]);
            acc[h] = fmaf(qv[h][4 * i + 1], lo.y, acc[h]);
            acc[h] = fmaf(qv[h][4 * i + 2], hi.x, acc[h]);
            acc[h] = fmaf(qv[h][4 * i + 3], hi.y, acc[h]);
        }
    }
}

// Finish a lane-pair key: returns the score of the key this lane keeps.
__device__ __forceinline__ float finish_score(const float (&accA)[4], const float (&accB)[4],
                                              bool odd, const float (&wh)[4], float scale) {
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        float keep = odd ? accB[h] : accA[h];
        float send = odd ? accA[h] : accB[h];
        float dot = (keep + dpp_f32<DPP_XOR1>(send)) * scale;
        s = fmaf(wh[h], fmaxf(dot, 0.0f), s);
    }
    return s + 0.0f;
}

template <bool POOL>
__global__ void __launch_bounds__(SC_THREADS) score_kernel(ScoreArgs a) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool odd = lane & 1;
    const int m = lane >> 1;
    const int64_t N = clamp64(a.ctx[b], 0, a.max_ctx);
    const int32_t s = a.seq[b];
    if (s < 0 || s >= a.n_seq) return;
    const int64_t n_items = POOL ? (int64_t)a.n_blocks * BLOCK : N;
    const int64_t wg0 = (int64_t)blockIdx.x * a.keys_per_wg;
    if (wg0 >= n_items) return;

    const uint8_t* keys = a.idxk + (int64_t)s * a.cap * IDX_DIM;
    float qv[4][32];
    float wh[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float4* qp = reinterpret_cast<const float4*>(a.q_idx + ((int64_t)b * 4 + h) * 64 + 32 * odd);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 t = qp[i];
            qv[h][4 * i] = t.x;
            qv[h][4 * i + 1] = t.y;
            qv[h][4 * i + 2] = t.z;
            qv[h][4 * i + 3] = t.w;
        }
        wh[h] = a.w[(int64_t)b * 4 + h];
    }
    const int32_t* pool = POOL ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    float* out = a.out + (int64_t)b * a.out_stride;

    const int64_t wg_end = wg0 + a.keys_per_wg < n_items ? wg0 + a.keys_per_wg : n_items;
    for (int64_t k0 = wg0 + (int64_t)wave * KEYS_PER_STEP; k0 < wg_end;
         k0 += (int64_t)KEYS_PER_STEP * (SC_THREADS / 64)) {
        // item indices of the two keys this lane touches
        const int64_t iA = k0 + m, iB = k0 + 32 + m;
        int64_t tA = iA, tB = iB;
        bool vA, vB;
        if (POOL) {
            int32_t pa = iA < n_items ? pool[iA >> 3] : -1;
            int32_t pb = iB < n_items ? pool[iB >> 3] : -1;
            tA = (int64_t)pa * BLOCK + (iA & 7);
            tB = (int64_t)pb * BLOCK + (iB & 7);
            vA = pa >= 0 && tA < N;
            vB = pb >= 0 && tB < N;
        } else {
            vA = iA < N;
            vB = iB < N;
        }
        uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
        if (vA) {
            const uint4* p = reinterpret_cast<const uint4*>(keys + tA * IDX_DIM + 32 * odd);
            a0 = p[0];
            a1 = p[1];
        }
        if (vB) {
            const uint4* p = reinterpret_cast<const uint4*>(keys + tB * IDX_DIM + 32 * odd);
            b0 = p[0];
            b1 = p[1];
        }
        float accA[4], accB[4];
        half_dots(a0, a1, qv, accA);
        half_dots(b0, b1, qv, accB);
        float sc = finish_score(accA, accB, odd, wh, a.scale);
        const bool valid = odd ? vB : vA;     // the kept key
        sc = valid ? sc : NEG_INF;
        if (POOL) {
            const int64_t item = odd ? iB : iA;
            if (item < n_items) out[item] = sc;
        } else {
            // same-parity lanes of a 16-lane row hold one block of 8 keys
            float mx = fmaxf(sc, dpp_f32<DPP_ROR2>(sc));
            mx = fmaxf(mx, dpp_f32<DPP_ROR4>(mx));
            mx = fmaxf(mx, dpp_f32<DPP_ROR8>(mx));
            if ((lane & 14) == 0) {           // lanes 16c and 16c+1
                const int c = lane >> 4;
                const int64_t blk = (k0 >> 3) + c + 4 * odd;
                if (blk * BLOCK < N) out[blk] = mx;
            }
        }
    }
}

}  // namespace

hipError_t launch_score_blocks(const csa2_cache& c, const float* q_idx, const float* w,
                               const int32_t* seq, const int64_t* ctx, int32_t B,
                               int64_t max_ctx, int64_t m_stride, float* M,
                               int32_t keys_per_wg, hipStream_t stream) {
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
    a.n_seq = c.n_seq;
    a.keys_per_wg = keys_per_wg;
    a.scale = c.idxk_scale;
    dim3 grid((unsigned)((max_ctx + keys_per_wg - 1) / keys_per_wg), (unsigned)B);
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL(score_kernel<false>, grid, dim3(SC_THREADS), 0, stream, a);
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
    a.n_seq = c.n_seq;
    a.n_blocks = n_blocks;
    a.keys_per_wg = 1024;
    a.scale = c.idxk_scale;
    const int64_t items = (int64_t)n_blocks * BLOCK;
    dim3 grid((unsigned)((items + a.keys_per_wg - 1) / a.keys_per_wg), (unsigned)B);
    hipLaunchKernelGGL(score_kernel<true>, grid, dim3(SC_THREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
