// Top-k select core shared by the top-k kernels and the fused Reindex layer.
// The algorithm is described at the top of topk.hip: the k largest of a row
// of floats, ties to the lower index, chosen indices ascending and -1 padded,
// -inf entries absent (origotech.dev deep dive "Inside DeepSeek V4.1-Flash",
// section "How the architecture shrinks the KV cache", for where top-k is used).
#pragma once

#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {
namespace topk_dev {

constexpr int NB = 2048;                 // linear bins
constexpr int VPT = 16;                  // values per thread
constexpr int BIG_T = 1024;              // threads: small-row and merge kernels
constexpr int SEG_T = 256;               // threads: segment kernel
constexpr int SMALL_MAX = BIG_T * VPT;   // 16,384
constexpr int RUN2_MAX = 2 * SMALL_MAX;  // 32,768: one workgroup at 32 values per thread
constexpr int SEG = SEG_T * VPT;         // 4,096
constexpr int FAST_MAX_N = 131072;
constexpr int STAGE_WORDS = CSA2_MAX_POOL > RUN2_MAX / 32 ? CSA2_MAX_POOL : RUN2_MAX / 32;
constexpr int CAND_CAP = 4096;
constexpr int RANK_MAX = 256;            // candidate sets ranked directly
constexpr int UNROLL = 8;
constexpr uint32_t KEY_ABSENT = 0x007fffffu;   // order_key(-inf)
constexpr float NEG_INF = -__builtin_huge_valf();

struct TopkArgs {
    const float* vals;       // rows of the input
    int64_t stride;
    const int64_t* ctx;      // block mode (n = ceil(ctx/8)) when non-null
    int64_t max_ctx;
    int32_t n_fixed;         // pool mode row length
    const int32_t* pool;     // report entry i as pool[i/8]*8 + i%8 when non-null
    int32_t n_blocks;
    int32_t k;
    int32_t* out;
    // two-stage path
    float* seg_val;          // [B][SMALL_MAX] chosen values of all segments, dense
    uint32_t* seg_id;        // [B][SMALL_MAX] their indices
    uint32_t* seg_meta;      // [B][n_seg][2]: count | full << 31, worst reported index
    int32_t n_seg;           // segments per row in the grid
};

template <int NT>
struct Shared {
    uint32_t hist[4096];
    uint32_t sel_bits[NT == BIG_T ? RUN2_MAX / 32 : SEG / 32];
    uint32_t eq_bits[NT == BIG_T ? STAGE_WORDS : SEG / 32];   // also the output staging
    uint32_t ckey[CAND_CAP];
    uint32_t cidx[CAND_CAP];
    uint32_t wave_u[NT / 64];
    float wave_f[3][NT / 64];
    uint32_t misc[8];        // [0,1] digit search, [2] candidates, [3] flag, [4] valid count
    int32_t pool[NT == BIG_T ? CSA2_MAX_POOL : 1];   // the row's pool (pool mode), in LDS
};

__device__ __forceinline__ int64_t row_length(const TopkArgs& a, int b) {
    if (a.ctx) {
        const int64_t N = clamp64(a.ctx[b], 0, a.max_ctx);
        return (N + BLOCK - 1) / BLOCK;
    }
    return a.n_fixed;
}

// Per-segment quota of the two-stage path; false if the segments' choices would
// not fit the merge kernel (then the row takes the fallback).
__device__ __forceinline__ bool seg_plan(int64_t n, int32_t k, int32_t* quota) {
    const int64_t expect = ((int64_t)k * SEG + n - 1) / n;   // ceil(k * SEG / n)
    int64_t q = 4 * expect;
    q = q < 256 ? 256 : (q > SEG ? SEG : q);
    *quota = (int32_t)q;
    const int64_t n_seg = (n + SEG - 1) / SEG;
    return n > SMALL_MAX && n <= FAST_MAX_N && n_seg * q <= SMALL_MAX;
}

// ------------------------------------------------------------ block collectives

// Wave collectives on DPP and v_readlane only (no LDS round trips, which a
// chain of shuffles would cost one after another).
// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane
// row (row_shr 1, 2, 4, 8), then row_bcast:15 and row_bcast:31 carry the row
// totals into the rows above.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
    return v;
}

// Min / max over the wave: the four 16-lane rows reduced inside the row by
// DPP, then combined from lanes 0, 16, 32, 48 with v_readlane (wave-uniform).
__device__ __forceinline__ float rows_min(float v) {
    auto rl = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
    v = fminf(v, dpp_f32<DPP_XOR1>(v));
    v = fminf(v, dpp_f32<DPP_XOR2>(v));
    v = fminf(v, dpp_f32<DPP_ROR4>(v));
    v = fminf(v, dpp_f32<DPP_ROR8>(v));
    return fminf(fminf(rl(v, 0), rl(v, 16)), fminf(rl(v, 32), rl(v, 48)));
}
__device__ __forceinline__ float rows_max(float v) {
    auto rl = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
    v = fmaxf(v, dpp_f32<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f32<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f32<DPP_ROR4>(v));
    v = fmaxf(v, dpp_f32<DPP_ROR8>(v));
    return fmaxf(fmaxf(rl(v, 0), rl(v, 16)), fmaxf(rl(v, 32), rl(v, 48)));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
    uint64_t o;
    o = dpp_u64<DPP_XOR1>(v); v = o < v ? o : v;
    o = dpp_u64<DPP_XOR2>(v); v = o < v ? o : v;
    o = dpp_u64<DPP_ROR4>(v); v = o < v ? o : v;
    o = dpp_u64<DPP_ROR8>(v); v = o < v ? o : v;
    uint64_t m = ~0ull;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t x = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
        m = x < m ? x : m;
    }
    return m;
}

template <int NT>
__device__ uint32_t block_incl_scan(uint32_t v, Shared<NT>& sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_incl_scan(v);
    if (lane == 63) sh.wave_u[wave] = v;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        uint32_t x = sh.wave_u[i];
        before += (i < wave) ? x : 0u;
        all += x;
    }
    __syncthreads();
    *total = all;
    return v + before;
}

// Block-wide statistics in one LDS round: count, min and max of the valid
// values, and the smallest per-thread maximum with the number of threads that
// hold a valid value (each such thread has at least one value >= that
// minimum, so it bounds the k-th largest value from below whenever at least k
// threads hold one).  Each wave reduces its own values (cnt is already the
// wave's count), then lanes 0 .. NT/64 - 1 of every wave read the waves'
// partials and a 16-lane DPP reduction leaves the block's result in every lane.
// The partial arrays are next written after at least one more barrier (every
// caller's next phase ends in one before any wave_u / wave_f write).
template <int NT>
__device__ void block_stats(uint32_t cnt, float lo, float hi, Shared<NT>& sh, uint32_t* total,
                            float* mn, float* mx, float* tmax_min, uint32_t* n_thr) {
    static_assert(NT / 64 <= 16, "one 16-lane row holds every wave's partial");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // this thread's maximum if it holds a valid value (-inf never raises hi)
    float fl = hi != NEG_INF ? hi : __builtin_huge_valf();
    const uint32_t thr = (uint32_t)__builtin_popcountll(__ballot(hi != NEG_INF));
    lo = rows_min(lo);
    hi = rows_max(hi);
    fl = rows_min(fl);
    if (lane == 0) {
        sh.wave_f[0][wave] = lo;
        sh.wave_f[1][wave] = hi;
        sh.wave_f[2][wave] = fl;
        sh.wave_u[wave] = cnt | (thr << 16);   // counts < 2^16 (at most 32,768 values)
    }
    __syncthreads();
    const bool mine = lane < NT / 64;
    float a = mine ? sh.wave_f[0][lane] : __builtin_huge_valf();
    float c = mine ? sh.wave_f[1][lane] : NEG_INF;
    float e = mine ? sh.wave_f[2][lane] : __builtin_huge_valf();
    uint32_t n = mine ? sh.wave_u[lane] : 0u;
    a = fminf(a, dpp_f32<DPP_XOR1>(a));
    a = fminf(a, dpp_f32<DPP_XOR2>(a));
    a = fminf(a, dpp_f32<DPP_ROR4>(a));
    a = fminf(a, dpp_f32<DPP_ROR8>(a));
    c = fmaxf(c, dpp_f32<DPP_XOR1>(c));
    c = fmaxf(c, dpp_f32<DPP_XOR2>(c));
    c = fmaxf(c, dpp_f32<DPP_ROR4>(c));
    c = fmaxf(c, dpp_f32<DPP_ROR8>(c));
    e = fminf(e, dpp_f32<DPP_XOR1>(e));
    e = fminf(e, dpp_f32<DPP_XOR2>(e));
    e = fminf(e, dpp_f32<DPP_ROR4>(e));
    e = fminf(e, dpp_f32<DPP_ROR8>(e));
    n += (uint32_t)__builtin_amdgcn_mov_dpp((int)n, DPP_XOR1, 0xf, 0xf, false);
    n += (uint32_t)__builtin_amdgcn_mov_dpp((int)n, DPP_XOR2, 0xf, 0xf, false);
    n += (uint32_t)__builtin_amdgcn_mov_dpp((int)n, DPP_ROR4, 0xf, 0xf, false);
    n += (uint32_t)__builtin_amdgcn_mov_dpp((int)n, DPP_ROR8, 0xf, 0xf, false);
    *mn = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a)));
    *mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)));
    *tmax_min = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(e)));
    n = (uint32_t)__builtin_amdgcn_readfirstlane((int)n);
    *total = n & 0xffffu;
    *n_thr = n >> 16;
}

// Histogram floor: values below it cannot be among the k largest.  With at
// least k threads holding a valid value, every one of them holds a value >= the
// smallest thread maximum, so the k-th largest value is >= that minimum;
// otherwise the floor is the smallest valid value.
__device__ __forceinline__ float hist_floor(uint32_t k, float vmin, float tmax_min,
                                            uint32_t n_thr) {
    return n_thr >= k ? tmax_min : vmin;
}

// Digit d of hist[0..nbins) with count(> d) < kk <= count(>= d); returns d and
// count(> d) through misc[0], misc[1].  Bins are visited top-down.
template <int NT>
__device__ void find_digit(Shared<NT>& sh, uint32_t kk, int nbins) {
    const int t = threadIdx.x;
    const int per = nbins >= NT ? nbins / NT : 1;
    const int p0 = t * per;
    uint32_t sum = 0;
    for (int j = 0; j < per; ++j) {
        const int p = p0 + j;
        if (p < nbins) sum += sh.hist[nbins - 1 - p];
    }
    uint32_t total;
    uint32_t run = block_incl_scan<NT>(sum, sh, &total) - sum;
    for (int j = 0; j < per; ++j) {
        const int p = p0 + j;
        if (p >= nbins) break;
        const uint32_t c = sh.hist[nbins - 1 - p];
        if (run < kk && run + c >= kk) {
            sh.misc[0] = (uint32_t)(nbins - 1 - p);
            sh.misc[1] = run;
        }
        run += c;
    }
    __syncthreads();
}

// ------------------------------------------------------------ select core

template <int NT>
__device__ __forceinline__ bool resolve_candidates(Shared<NT>& sh, uint32_t kk, int words);

// Chooses the k best of the block's register-held values (v, id), -inf absent,
// ties to the lower id.  Marks the choice in sh.sel_bits, bit (id - id_base),
// over `words` bitmap words; leaves the number of valid values in misc[4].
// Returns false if the candidate list overflowed (the caller then needs the
// fallback); true otherwise.
template <int NT>
__device__ bool select_core(Shared<NT>& sh, const float (&v)[VPT], const uint32_t (&id)[VPT],
                            uint32_t k, uint32_t id_base, int words) {
    const int t = threadIdx.x;
    for (int i = t; i < NB; i += NT) sh.hist[i] = 0;
    for (int i = t; i < words; i += NT) {
        sh.sel_bits[i] = 0;
        sh.eq_bits[i] = 0;
    }
    if (t == 0) sh.misc[2] = 0;
    float lo = __builtin_huge_valf(), hi = NEG_INF;
    uint32_t cnt = 0;                    // the wave's valid values (wave-uniform)
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const bool ok = v[j] != NEG_INF;
        cnt += (uint32_t)__builtin_popcountll(__ballot(ok));
        lo = fminf(lo, ok ? v[j] : __builtin_huge_valf());
        hi = fmaxf(hi, v[j]);               // -inf never raises the max
    }
    uint32_t n_valid, n_thr;
    float vmin, vmax, tmax_min;
    block_stats<NT>(cnt, lo, hi, sh, &n_valid, &vmin, &vmax, &tmax_min, &n_thr);
    if (t == 0) sh.misc[4] = n_valid;
    if (n_valid <= k) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const uint32_t rel = id[j] - id_base;
            if (v[j] != NEG_INF) atomicOr(&sh.sel_bits[rel >> 5], 1u << (rel & 31));
        }
        __syncthreads();
        return true;
    }
    // bins linear in value over [floor, max]; values below the floor are absent
    const float floor_ = hist_floor(k, vmin, tmax_min, n_thr);
    float inv = vmax > floor_ ? (float)NB / (vmax - floor_) : 0.0f;
    if (!(inv < __builtin_huge_valf())) inv = 0.0f;     // range overflowed: one bin
    uint32_t bin[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int bb = (int)((v[j] - floor_) * inv);
        bin[j] = !(v[j] >= floor_) ? 0xffffffffu : (uint32_t)(bb < NB - 1 ? bb : NB - 1);
        if (bin[j] != 0xffffffffu) atomicAdd(&sh.hist[bin[j]], 1u);
    }
    __syncthreads();
    find_digit<NT>(sh, k, NB);
    const uint32_t d = sh.misc[0];
    uint32_t kk = k - sh.misc[1];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t rel = id[j] - id_base;
        if (bin[j] != 0xffffffffu && bin[j] > d) {
            atomicOr(&sh.sel_bits[rel >> 5], 1u << (rel & 31));
        } else if (bin[j] == d) {
            const uint32_t slot = atomicAdd(&sh.misc[2], 1u);
            if (slot < (uint32_t)CAND_CAP) {
                sh.ckey[slot] = order_key(v[j]);
                sh.cidx[slot] = rel;
            }
        }
    }
    __syncthreads();
    return resolve_candidates<NT>(sh, kk, words);
}

// Chooses kk of the m = misc[2] candidates of the threshold bin (order keys in
// ckey, bitmap positions in cidx) in (value desc, index asc) order and sets
// their bits in sh.sel_bits.  Expects eq_bits[0, words) zero.  Returns false if
// the candidate list overflowed.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ bool resolve_candidates(Shared<NT>& sh, uint32_t kk, int words) {
    const int t = threadIdx.x;
    const uint32_t m = sh.misc[2];
    if (m > (uint32_t)CAND_CAP) return false;
    if (m <= (uint32_t)RANK_MAX) {
        // few candidates: rank each against all others in (key desc, index asc)
        // order and keep the kk best; the LDS reads are broadcasts
        for (uint32_t j = t; j < m; j += NT) {
            const uint32_t kj = sh.ckey[j], ij = sh.cidx[j];
            uint32_t rank = 0;
            for (uint32_t i = 0; i < m; ++i) {
                const uint32_t ki = sh.ckey[i], ii = sh.cidx[i];
                rank += (ki > kj || (ki == kj && ii < ij)) ? 1u : 0u;
            }
            if (rank < kk) atomicOr(&sh.sel_bits[ij >> 5], 1u << (ij & 31));
        }
        __syncthreads();
        return true;
    }
    // exact threshold among the candidates: 11/11/10-bit radix on their keys
    uint32_t prefix = 0, pmask = 0;
    for (int pass = 0; pass < 3; ++pass) {
        const int shft = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t nbins = pass == 2 ? 1024u : 2048u;
        for (int i = t; i < 2048; i += NT) sh.hist[i] = 0;
        __syncthreads();
        for (uint32_t j = t; j < m; j += NT) {
            const uint32_t key = sh.ckey[j];
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shft) & (nbins - 1)], 1u);
        }
        __syncthreads();
        find_digit<NT>(sh, kk, (int)nbins);
        kk -= sh.misc[1];
        prefix |= sh.misc[0] << shft;
        pmask |= (nbins - 1) << shft;
        __syncthreads();
    }
    for (uint32_t j = t; j < m; j += NT) {
        const uint32_t key = sh.ckey[j], rel = sh.cidx[j];
        if (key > prefix) atomicOr(&sh.sel_bits[rel >> 5], 1u << (rel & 31));
        else if (key == prefix) atomicOr(&sh.eq_bits[rel >> 5], 1u << (rel & 31));
    }
    __syncthreads();
    // keep the kk lowest-index keys equal to T; thread t owns words [t*wpt, +wpt)
    const int wpt = (words + NT - 1) / NT;
    uint32_t c = 0;
    for (int j = 0; j < wpt; ++j) {
        const int wi = t * wpt + j;
        c += wi < words ? __popc(sh.eq_bits[wi]) : 0u;
    }
    uint32_t tot;
    const uint32_t before = block_incl_scan<NT>(c, sh, &tot) - c;
    uint32_t need = kk > before ? kk - before : 0u;
    for (int j = 0; j < wpt; ++j) {
        const int wi = t * wpt + j;
        if (wi >= words) break;
        uint32_t keep = 0, bits = sh.eq_bits[wi];
        while (bits && need) {
            const uint32_t low = bits & (0u - bits);
            keep |= low;
            bits ^= low;
            --need;
        }
        if (keep) sh.sel_bits[wi] |= keep;
    }
    __syncthreads();
    return true;
}

// ------------------------------------------------------------ exact fallback

__device__ __forceinline__ uint32_t key_at(float v, int64_t i, int64_t n) {
    const uint32_t key = order_key(v);
    return i < n ? key : KEY_ABSENT;
}

// Sweep a row in float4 chunks, UNROLL loads in flight per thread; chunks past
// the end re-read the last one (in bounds) and f masks them by index.
template <typename F>
__device__ __forceinline__ void sweep(const float* vals, int64_t n, F&& f) {
    const int64_t nc = (n + 3) >> 2;
    const float4* v4 = reinterpret_cast<const float4*>(vals);
    for (int64_t base = 0; base < nc; base += (int64_t)BIG_T * UNROLL) {
        const int64_t c0 = base + threadIdx.x;
        float4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t c = c0 + (int64_t)u * BIG_T;
            v[u] = v4[c < nc ? c : nc - 1];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) f(c0 + (int64_t)u * BIG_T, v[u]);
    }
}

// Exact fallback over a row in global memory: 11/11/10-bit radix sweeps,
// ordered collection of ties, bitonic sort of the chosen indices (k <= 4096).
__device__ inline void topk_fallback(Shared<BIG_T>& sh, const float* vals, int64_t n, int32_t k,
                              const int32_t* pool, int32_t* out) {
    const int t = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k;
    bool take_all = false;
    __syncthreads();
    for (int pass = 0; pass < 3; ++pass) {
        const int shft = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t nb = pass == 2 ? 1024u : 2048u;
        for (int i = t; i < 4096; i += BIG_T) sh.hist[i] = 0;
        __syncthreads();
        sweep(vals, n, [&](int64_t c, float4 v) {
            const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(x[j], 4 * c + j, n);
                if (key != KEY_ABSENT && (key & pmask) == prefix)
                    atomicAdd(&sh.hist[(key >> shft) & (nb - 1)], 1u);
            }
        });
        __syncthreads();
        if (pass == 0) {
            uint32_t c = sh.hist[2 * t] + sh.hist[2 * t + 1], tot;
            block_incl_scan<BIG_T>(c, sh, &tot);
            if (tot <= (uint32_t)k) {
                take_all = true;
                break;
            }
        }
        find_digit<BIG_T>(sh, kk, (int)nb);
        kk -= sh.misc[1];
        prefix |= sh.misc[0] << shft;
        pmask |= (nb - 1) << shft;
        __syncthreads();
    }
    const uint32_t T = take_all ? KEY_ABSENT : prefix;
    const uint32_t n_eq = take_all ? 0u : sh.hist[prefix & 1023u];
    if (t == 0) sh.misc[2] = 0;
    __syncthreads();
    if (take_all || n_eq == kk) {
        sweep(vals, n, [&](int64_t c, float4 v) {
            const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(x[j], 4 * c + j, n);
                if (take_all ? key != KEY_ABSENT : key >= T) {
                    const uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                    if (slot < (uint32_t)CAND_CAP) sh.cidx[slot] = (uint32_t)(4 * c + j);
                }
            }
        });
    } else {
        // ordered rounds of 4096 entries: thread t owns entries r0 + 4t .. +3
        uint32_t base = 0;
        for (int64_t r0 = 0; r0 < n; r0 += 4 * BIG_T) {
            uint32_t keys[4], ceq = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = r0 + 4 * t + j;
                keys[j] = i < n ? order_key(vals[i]) : KEY_ABSENT;
                ceq += keys[j] == T ? 1u : 0u;
                if (keys[j] != KEY_ABSENT && keys[j] > T) {
                    const uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                    if (slot < (uint32_t)CAND_CAP) sh.cidx[slot] = (uint32_t)i;
                }
            }
            if (base < kk) {
                uint32_t tot;
                uint32_t rank = block_incl_scan<BIG_T>(ceq, sh, &tot) - ceq + base;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (keys[j] == T) {
                        if (rank < kk) {
                            const uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                            if (slot < (uint32_t)CAND_CAP)
                                sh.cidx[slot] = (uint32_t)(r0 + 4 * t + j);
                        }
                        ++rank;
                    }
                }
                base += tot;
            }
        }
    }
    __syncthreads();
    const int cnt = (int)min(sh.misc[2], (uint32_t)k);
    int P = 1;
    while (P < cnt) P <<= 1;
    for (int i = cnt + t; i < P; i += BIG_T) sh.cidx[i] = 0x7fffffffu;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < P / 2; i += BIG_T) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint32_t x = sh.cidx[lo], y = sh.cidx[hi];
                if ((x > y) == up) {
                    sh.cidx[lo] = y;
                    sh.cidx[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int j = t; j < k; j += BIG_T) {
        int32_t val = -1;
        if (j < cnt) {
            const int32_t i = (int32_t)sh.cidx[j];
            val = pool ? pool[i >> 3] * BLOCK + (i & 7) : i;
        }
        out[j] = val;
    }
}

// ------------------------------------------------------------ kernels

// Load VPT values per thread as float4 chunks: thread t, chunk r covers entries
// base + 4*(t + NT*r) .. +3.  Entries outside [base, end) read as -inf; their
// loads re-read the chunk at base (in bounds).  base is a multiple of 4.
template <int NT>
__device__ __forceinline__ void load_values(const float* row, int64_t base, int64_t end,
                                            float (&v)[VPT], uint32_t (&id)[VPT]) {
    const float4* v4 = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int r = 0; r < VPT / 4; ++r) {
        const int64_t e0 = base + 4 * ((int64_t)threadIdx.x + (int64_t)NT * r);
        const float4 x = v4[(e0 < end ? e0 : base) >> 2];
        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[4 * r + j] = e0 + j < end ? xs[j] : NEG_INF;
            id[4 * r + j] = (uint32_t)(e0 + j);
        }
    }
}

// Selection over up to V * 1,024 positions with thread t owning positions
// Vt .. Vt+V-1 (V = 16 or 32; values in registers, -inf absent).  Its share of
// the choice is then a V-bit register mask, and because positions are in output order the
// ascending output is one block scan of the masks' popcounts: on the common
// path no bitmap and no atomics besides the histogram's.  The steps are those
// of select_core: count / min / max, the value-linear histogram and the bin d
// of the k-th value, positions above d chosen, bin d's positions resolved as
// candidates (returned through sel_bits).  id_of(j) is the output value of
// position Vt + j; veto(j) (for chosen positions) may reject the whole choice.
// Writes out[0, k) ascending with -1 padding and returns true, or returns false
// (nothing written) when the candidate list overflowed or a veto fired.
// STATIC_J visits the chosen positions with compile-time j (for id_of / veto
// that index register arrays, which a runtime j would move to scratch).
template <int NT, int V, bool STATIC_J, typename IdOf, typename Veto>
__device__ bool select_run(Shared<NT>& sh, const float (&v)[V], int64_t n_pos, uint32_t k,
                           int32_t* out, IdOf id_of, Veto veto) {
    static_assert(V == 16 || V == 32, "a thread's choice is one 32-bit mask word or half of one");
    static_assert(NT == BIG_T || NT == SEG_T, "the block sizes Shared is laid out for");
    const int t = threadIdx.x;
    const int words = (int)((n_pos + 31) >> 5);
    for (int i = t; i < NB; i += NT) sh.hist[i] = 0;
    if (t < words) {
        sh.sel_bits[t] = 0;
        sh.eq_bits[t] = 0;
    }
    if (t == 0) {
        sh.misc[2] = 0;
        sh.misc[3] = 0;
    }

    // ---- count / min / max of the valid values
    float lo = __builtin_huge_valf(), hi = NEG_INF;
    uint32_t cnt = 0;                    // the wave's valid values (wave-uniform)
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const bool ok = v[j] != NEG_INF;
        cnt += (uint32_t)__builtin_popcountll(__ballot(ok));
        lo = fminf(lo, ok ? v[j] : __builtin_huge_valf());
        hi = fmaxf(hi, v[j]);               // -inf never raises the max
    }
    uint32_t n_valid, n_thr;
    float vmin, vmax, tmax_min;
    block_stats<NT>(cnt, lo, hi, sh, &n_valid, &vmin, &vmax, &tmax_min, &n_thr);

    uint32_t mask = 0;                   // bit j: position Vt + j chosen
    if (n_valid <= k) {
#pragma unroll
        for (int j = 0; j < V; ++j) mask |= v[j] != NEG_INF ? 1u << j : 0u;
        __syncthreads();                 // block_stats' partials read before the scan reuses them
    } else {
        // ---- histogram over [floor, max] (values below the floor cannot be
        // chosen and stay out of it) and the bin d holding the k-th largest
        const float floor_ = hist_floor(k, vmin, tmax_min, n_thr);
        float inv = vmax > floor_ ? (float)NB / (vmax - floor_) : 0.0f;
        if (!(inv < __builtin_huge_valf())) inv = 0.0f;     // range overflowed: one bin
        uint32_t bin[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int bb = (int)((v[j] - floor_) * inv);
            bin[j] = !(v[j] >= floor_) ? 0xffffffffu : (uint32_t)(bb < NB - 1 ? bb : NB - 1);
            if (bin[j] != 0xffffffffu) atomicAdd(&sh.hist[bin[j]], 1u);
        }
        __syncthreads();
        find_digit<NT>(sh, k, NB);
        const uint32_t d = sh.misc[0];
        const uint32_t kk = k - sh.misc[1];
        __syncthreads();
        // ---- above d: chosen; in d: candidates
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if (bin[j] != 0xffffffffu && bin[j] > d) {
                mask |= 1u << j;
            } else if (bin[j] == d) {
                const uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                if (slot < (uint32_t)CAND_CAP) {
                    sh.ckey[slot] = order_key(v[j]);
                    sh.cidx[slot] = (uint32_t)(V * t + j);
                }
            }
        }
        __syncthreads();
        if (!resolve_candidates<NT>(sh, kk, words)) return false;
        const uint32_t bit0 = (uint32_t)(V * t);
        mask |= V == 32 ? sh.sel_bits[t] : (sh.sel_bits[bit0 >> 5] >> (bit0 & 31)) & 0xffffu;
    }

    // ---- veto, then ranks from a block scan (its barriers also publish the
    // veto flag), staged in LDS (k <= 4096 entries fit eq_bits), then one
    // coalesced store with -1 padding
    if (STATIC_J) {
        bool vetoed = false;
#pragma unroll
        for (int j = 0; j < V; ++j) vetoed |= ((mask >> j) & 1u) && veto(j);
        if (vetoed) sh.misc[3] = 1;
    } else {
        for (uint32_t m = mask; m; m &= m - 1)
            if (veto(__ffs(m) - 1)) sh.misc[3] = 1;
    }
    const uint32_t c = (uint32_t)__popc(mask);
    uint32_t total;
    uint32_t pos = block_incl_scan<NT>(c, sh, &total) - c;
    if (sh.misc[3]) return false;
    // staging: eq_bits holds k <= 4096 entries at BIG_T; the smaller block's
    // eq_bits is one word per 32 entries, so it stages in ckey (free again
    // once the candidates are resolved)
    int32_t* stage = NT == BIG_T ? reinterpret_cast<int32_t*>(sh.eq_bits)
                                 : reinterpret_cast<int32_t*>(sh.ckey);
    if (STATIC_J) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if ((mask >> j) & 1u) {
                if (pos < k) stage[pos] = id_of(j);
                ++pos;
            }
        }
    } else {
        while (mask) {
            const int j = __ffs(mask) - 1;
            mask &= mask - 1;
            if (pos < k) stage[pos] = id_of(j);
            ++pos;
        }
    }
    __syncthreads();
    for (int j = t; j < (int)k; j += NT) out[j] = j < (int)total ? stage[j] : -1;
    return true;
}

// Entries Vt .. Vt+V-1 of a row of n entries as float4 loads; entries past the
// end read as -inf (their loads stay in bounds).
template <int V>
__device__ __forceinline__ void load_run(const float* row, int64_t n, float (&v)[V]) {
    const float4* v4 = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int r = 0; r < V / 4; ++r) {
        const int64_t e0 = (int64_t)V * threadIdx.x + 4 * r;
        const float4 x = v4[(e0 < n ? e0 : 0) >> 2];
        v[4 * r] = e0 < n ? x.x : NEG_INF;
        v[4 * r + 1] = e0 + 1 < n ? x.y : NEG_INF;
        v[4 * r + 2] = e0 + 2 < n ? x.z : NEG_INF;
        v[4 * r + 3] = e0 + 3 < n ? x.w : NEG_INF;
    }
}

// Rows of up to SMALL_MAX entries (longer rows: the exact fallback).
// Body of row b's workgroup of BIG_T threads (uniform b, thread index
// threadIdx.x), sh its LDS.
__device__ __forceinline__ void topk_small_body(Shared<BIG_T>& sh, const TopkArgs& a, int b) {
    const int t = threadIdx.x;
    const int64_t n = row_length(a, b);
    const float* row = a.vals + (int64_t)b * a.stride;
    int32_t* out = a.out + (int64_t)b * a.k;
    const int32_t* pool = a.pool ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    if (n > SMALL_MAX) {
        topk_fallback(sh, row, n, a.k, pool, out);
        return;
    }
    // entries 16t .. 16t+15; in pool mode they lie in pool blocks 2t and 2t + 1
    float v[VPT];
    load_run<VPT>(row, n, v);
    int32_t pb[2] = {0, 0};
    if (pool) {
        pb[0] = 2 * t < a.n_blocks ? pool[2 * t] : 0;
        pb[1] = 2 * t + 1 < a.n_blocks ? pool[2 * t + 1] : 0;
    }
    const bool done = select_run<BIG_T, VPT, false>(
        sh, v, n, (uint32_t)a.k, out,
        [&](int j) -> int32_t { return pool ? pb[j >> 3] * BLOCK + (j & 7) : VPT * t + j; },
        [](int) { return false; });
    if (!done) topk_fallback(sh, row, n, a.k, pool, out);
}

// Rows of up to SEG entries (4,096) in a workgroup of SEG_T threads, 16 values
// per thread: the steps of topk_small_body with a quarter of the waves, so each
// block-wide step is shorter and about three such workgroups fit a CU (LDS
// ~50 KB, against one of the 1,024-thread kind), which large batches of short
// rows need.  With n <= CAND_CAP the candidate list cannot overflow and no veto
// is used, so the selection always completes here.
__device__ __forceinline__ void topk_quarter_body(Shared<SEG_T>& sh, const TopkArgs& a, int b) {
    static_assert(SEG <= CAND_CAP, "a row's candidates always fit");
    const int t = threadIdx.x;
    const int64_t n = row_length(a, b);
    const float* row = a.vals + (int64_t)b * a.stride;
    int32_t* out = a.out + (int64_t)b * a.k;
    const int32_t* pool = a.pool ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    float v[VPT];
    load_run<VPT>(row, n, v);
    int32_t pb[2] = {0, 0};
    if (pool) {
        pb[0] = 2 * t < a.n_blocks ? pool[2 * t] : 0;
        pb[1] = 2 * t + 1 < a.n_blocks ? pool[2 * t + 1] : 0;
    }
    select_run<SEG_T, VPT, false>(
        sh, v, n, (uint32_t)a.k, out,
        [&](int j) -> int32_t { return pool ? pb[j >> 3] * BLOCK + (j & 7) : VPT * t + j; },
        [](int) { return false; });
}

// Rows of up to RUN2_MAX entries in one workgroup, 32 values per thread (rows
// just past SMALL_MAX, e.g. the block maxima of 131,073..262,144 positions,
// need no segment pass).  Entries 32t .. 32t+31 lie in pool blocks 4t .. 4t+3.
__device__ __forceinline__ void topk_run32_body(Shared<BIG_T>& sh, const TopkArgs& a, int b) {
    const int t = threadIdx.x;
    const int64_t n = row_length(a, b);
    const float* row = a.vals + (int64_t)b * a.stride;
    int32_t* out = a.out + (int64_t)b * a.k;
    const int32_t* pool = a.pool ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    if (n > RUN2_MAX) {
        topk_fallback(sh, row, n, a.k, pool, out);
        return;
    }
    float v[2 * VPT];
    load_run<2 * VPT>(row, n, v);
    int32_t pb[4] = {0, 0, 0, 0};
    if (pool) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = 4 * t + i < a.n_blocks ? pool[4 * t + i] : 0;
    }
    const bool done = select_run<BIG_T, 2 * VPT, true>(
        sh, v, n, (uint32_t)a.k, out,
        [&](int j) -> int32_t { return pool ? pb[j >> 3] * BLOCK + (j & 7) : 2 * VPT * t + j; },
        [](int) { return false; });
    if (!done) topk_fallback(sh, row, n, a.k, pool, out);
}

}  // namespace topk_dev
}  // namespace csa2
