// Top-k selection: the k largest of n floats, ties to the lower index, the
// chosen indices written in ascending order and padded with -1.  -inf entries
// are absent (never chosen).
//
// Used twice per Full layer (the 2,048 best blocks of 8 positions forming the
// candidate pool, then the top 512 positions inside the pool) and once per
// Reindex layer (origotech.dev deep dive "Inside DeepSeek V4.1-Flash", section
// "How the architecture shrinks the KV cache").
//
// Select core (one workgroup, values held in registers, 16 per thread):
//   1. min / max / count of the valid values (block reduction);
//   2. an LDS histogram over 2,048 bins linear in value between min and max
//      (a monotone map, so ranks survive; linear bins keep LDS atomics spread
//      even when every value shares one exponent) and the bin d holding the
//      k-th largest value;
//   3. values in bins above d are chosen; bin d's values go to an LDS candidate
//      list.  Up to 256 candidates are ranked directly in (value desc, index
//      asc) order; larger lists take an 11/11/10-bit radix on the exact order
//      keys for the threshold key T and how many keys equal to T to take, and an
//      ordered popcount scan over an "equal" bitmap keeps the lowest-index ones.
// The choice lives in an LDS bitmap over indices; an ordered popcount scan of
// the bitmap writes ascending indices.
//
// Rows of up to 16,384 entries: one workgroup, one read of the row.
// Longer rows (up to 131,072): a segment kernel takes the exact top-q of each
// 4,096-entry segment (q >= 4x a segment's expected share of the top-k); a
// merge kernel selects the top-k of the union and checks that no segment's
// worst reported entry was chosen (else that segment might hide more winners).
// Rows that fail the check, overflow the candidate list (heavy ties), or are
// longer than 131,072 entries take an exact fallback: three radix sweeps over
// the row in global memory, an ordered collection and a bitonic sort.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int NB = 2048;                 // linear bins
constexpr int VPT = 16;                  // values per thread
constexpr int BIG_T = 1024;              // threads: small-row and merge kernels
constexpr int SEG_T = 256;               // threads: segment kernel
constexpr int SMALL_MAX = BIG_T * VPT;   // 16,384
constexpr int SEG = SEG_T * VPT;         // 4,096
constexpr int FAST_MAX_N = 131072;
constexpr int BM_WORDS = FAST_MAX_N / 32;
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
    uint32_t sel_bits[NT == BIG_T ? BM_WORDS : SEG / 32];
    uint32_t eq_bits[NT == BIG_T ? BM_WORDS : SEG / 32];
    uint32_t ckey[CAND_CAP];
    uint32_t cidx[CAND_CAP];
    uint32_t wave_u[NT / 64];
    float wave_f[2][NT / 64];
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

// The four 16-lane rows reduced inside the row by DPP, then combined from
// lanes 0, 16, 32, 48 with v_readlane; the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, DPP_XOR1, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, DPP_XOR2, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, DPP_ROR4, 0xf, 0xf, false);
    v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, DPP_ROR8, 0xf, 0xf, false);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
           (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}
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

// Block-wide count, min and max in one LDS round.
template <int NT>
__device__ void block_stats(uint32_t cnt, float lo, float hi, Shared<NT>& sh, uint32_t* total,
                            float* mn, float* mx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    lo = rows_min(lo);
    hi = rows_max(hi);
    cnt = wave_sum_u32(cnt);
    if (lane == 0) {
        sh.wave_f[0][wave] = lo;
        sh.wave_f[1][wave] = hi;
        sh.wave_u[wave] = cnt;
    }
    __syncthreads();
    float a = sh.wave_f[0][0], c = sh.wave_f[1][0];
    uint32_t n = sh.wave_u[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        a = fminf(a, sh.wave_f[0][i]);
        c = fmaxf(c, sh.wave_f[1][i]);
        n += sh.wave_u[i];
    }
    __syncthreads();
    *mn = a;
    *mx = c;
    *total = n;
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
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const bool ok = v[j] != NEG_INF;
        cnt += ok ? 1u : 0u;
        lo = ok ? fminf(lo, v[j]) : lo;
        hi = ok ? fmaxf(hi, v[j]) : hi;
    }
    uint32_t n_valid;
    float vmin, vmax;
    block_stats<NT>(cnt, lo, hi, sh, &n_valid, &vmin, &vmax);
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
    float inv = vmax > vmin ? (float)NB / (vmax - vmin) : 0.0f;
    if (!(inv < __builtin_huge_valf())) inv = 0.0f;     // range overflowed: one bin
    uint32_t bin[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int bb = (int)((v[j] - vmin) * inv);
        bin[j] = v[j] == NEG_INF ? 0xffffffffu : (uint32_t)(bb < NB - 1 ? bb : NB - 1);
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

// Ordered compaction of the chosen bits into out[0..k), ascending, -1 padded.
template <int NT>
__device__ void write_bitmap(Shared<NT>& sh, int words, bool use_pool, int32_t* out, int32_t k) {
    const int t = threadIdx.x;
    const int wpt = (words + NT - 1) / NT;
    uint32_t c = 0;
    for (int j = 0; j < wpt; ++j) {
        const int wi = t * wpt + j;
        c += wi < words ? __popc(sh.sel_bits[wi]) : 0u;
    }
    uint32_t total;
    uint32_t pos = block_incl_scan<NT>(c, sh, &total) - c;
    for (int j = 0; j < wpt; ++j) {
        const int wi = t * wpt + j;
        if (wi >= words) break;
        uint32_t bits = sh.sel_bits[wi];
        while (bits) {
            const int bit = __ffs(bits) - 1;
            bits &= bits - 1;
            const int32_t i = wi * 32 + bit;
            if (pos < (uint32_t)k) out[pos] = use_pool ? sh.pool[i >> 3] * BLOCK + (i & 7) : i;
            ++pos;
        }
    }
    for (int j = (int)total + t; j < k; j += NT) out[j] = -1;
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
__device__ void topk_fallback(Shared<BIG_T>& sh, const float* vals, int64_t n, int32_t k,
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

// Rows of up to SMALL_MAX entries (longer rows: the exact fallback).
__global__ void __launch_bounds__(BIG_T) topk_small_kernel(TopkArgs a) {
    __shared__ Shared<BIG_T> sh;
    const int b = blockIdx.x;
    const int64_t n = row_length(a, b);
    const float* row = a.vals + (int64_t)b * a.stride;
    int32_t* out = a.out + (int64_t)b * a.k;
    const int32_t* pool = a.pool ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    if (n > SMALL_MAX) {
        topk_fallback(sh, row, n, a.k, pool, out);
        return;
    }
    // the pool is needed only to name the chosen entries; its load overlaps
    // the values' (select_core synchronises before anything reads it)
    if (pool)
        for (int i = threadIdx.x; i < a.n_blocks; i += BIG_T) sh.pool[i] = pool[i];
    float v[VPT];
    uint32_t id[VPT];
    load_values<BIG_T>(row, 0, n, v, id);
    const int words = (int)((n + 31) >> 5);
    if (!select_core<BIG_T>(sh, v, id, (uint32_t)a.k, 0, words)) {
        topk_fallback(sh, row, n, a.k, pool, out);
        return;
    }
    write_bitmap<BIG_T>(sh, words, pool != nullptr, out, a.k);
}

// Stage 1 of long rows: exact top-quota of segment g of row b, written densely
// at slot g * quota of the row's area, with its count and worst entry.
__global__ void __launch_bounds__(SEG_T) topk_seg_kernel(TopkArgs a) {
    __shared__ Shared<SEG_T> sh;
    __shared__ float segv[SEG];
    __shared__ uint64_t wmin[SEG_T / 64];
    const int g = blockIdx.x, b = blockIdx.y;
    const int t = threadIdx.x;
    const int64_t n = row_length(a, b);
    int32_t quota;
    if (!seg_plan(n, a.k, &quota)) return;     // the merge kernel handles this row alone
    uint32_t* meta = a.seg_meta + ((int64_t)b * a.n_seg + g) * 2;
    const int64_t base = (int64_t)g * SEG;
    if (base >= n) {
        if (t == 0) meta[0] = meta[1] = 0;
        return;
    }
    const int64_t end = base + SEG < n ? base + SEG : n;
    const float* row = a.vals + (int64_t)b * a.stride;
    float v[VPT];
    uint32_t id[VPT];
    load_values<SEG_T>(row, base, end, v, id);
#pragma unroll
    for (int j = 0; j < VPT; ++j) segv[id[j] - base] = v[j];
    // never overflows: the candidate list holds a whole segment
    select_core<SEG_T>(sh, v, id, (uint32_t)quota, (uint32_t)base, SEG / 32);
    const uint32_t n_valid = sh.misc[4];
    // ordered write of the chosen (value, index) pairs; track the worst one
    constexpr int W = SEG / 32;
    uint32_t c = t < W ? __popc(sh.sel_bits[t]) : 0u;
    uint32_t total;
    uint32_t pos = block_incl_scan<SEG_T>(c, sh, &total) - c;
    float* ov = a.seg_val + (int64_t)b * SMALL_MAX + (int64_t)g * quota;
    uint32_t* oi = a.seg_id + (int64_t)b * SMALL_MAX + (int64_t)g * quota;
    // min over chosen of (key << 32 | ~index): lowest value, then highest index
    uint64_t worst = ~0ull;
    if (t < W) {
        uint32_t bits = sh.sel_bits[t];
        while (bits) {
            const int bit = __ffs(bits) - 1;
            bits &= bits - 1;
            const uint32_t rel = (uint32_t)(t * 32 + bit);
            const float val = segv[rel];
            const uint32_t gi = (uint32_t)base + rel;
            if (pos < (uint32_t)quota) {
                ov[pos] = val;
                oi[pos] = gi;
            }
            ++pos;
            const uint64_t key = ((uint64_t)order_key(val) << 32) | (uint64_t)(~gi);
            worst = key < worst ? key : worst;
        }
    }
    worst = wave_min_u64(worst);
    if ((t & 63) == 0) wmin[t >> 6] = worst;
    __syncthreads();
    if (t == 0) {
        uint64_t mn = wmin[0];
        for (int i = 1; i < SEG_T / 64; ++i) mn = wmin[i] < mn ? wmin[i] : mn;
        const uint32_t cnt = total < (uint32_t)quota ? total : (uint32_t)quota;
        // full: the segment holds valid entries it did not report
        meta[0] = cnt | (n_valid > cnt ? 0x80000000u : 0u);
        meta[1] = ~(uint32_t)mn;
    }
}

// Stage 2 of long rows: top-k of the union of the segments' choices, checked.
// Rows the segment kernel skipped are selected here directly.
__global__ void __launch_bounds__(BIG_T) topk_merge_kernel(TopkArgs a) {
    __shared__ Shared<BIG_T> sh;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t n = row_length(a, b);
    const float* row = a.vals + (int64_t)b * a.stride;
    int32_t* out = a.out + (int64_t)b * a.k;
    const int32_t* pool = a.pool ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    int32_t quota;
    const bool two_stage = seg_plan(n, a.k, &quota);
    if (!two_stage && n > SMALL_MAX) {
        topk_fallback(sh, row, n, a.k, pool, out);
        return;
    }
    if (pool)
        for (int i = t; i < a.n_blocks; i += BIG_T) sh.pool[i] = pool[i];
    float v[VPT];
    uint32_t id[VPT];
    const uint32_t* meta = a.seg_meta + (int64_t)b * a.n_seg * 2;
    const int n_seg = (int)((n + SEG - 1) / SEG);
    if (!two_stage) {
        load_values<BIG_T>(row, 0, n, v, id);
    } else {
        const float* sv = a.seg_val + (int64_t)b * SMALL_MAX;
        const uint32_t* si = a.seg_id + (int64_t)b * SMALL_MAX;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int e = t + BIG_T * j;           // dense slot, < SMALL_MAX
            const int g = e / quota, r = e % quota;
            const bool ok = g < n_seg && (uint32_t)r < (meta[2 * g] & 0x7fffffffu);
            v[j] = ok ? sv[e] : NEG_INF;
            id[j] = ok ? si[e] : 0u;
        }
    }
    const int words = (int)((n + 31) >> 5);
    bool good = select_core<BIG_T>(sh, v, id, (uint32_t)a.k, 0, words);
    if (good && two_stage) {
        // a full segment whose worst reported entry was chosen may hide winners
        if (t == 0) sh.misc[3] = 0;
        __syncthreads();
        for (int g = t; g < n_seg; g += BIG_T) {
            const uint32_t m0 = meta[2 * g], worst = meta[2 * g + 1];
            if ((m0 & 0x80000000u) && ((sh.sel_bits[worst >> 5] >> (worst & 31)) & 1u))
                sh.misc[3] = 1;
        }
        __syncthreads();
        good = sh.misc[3] == 0;
    }
    if (!good) {
        topk_fallback(sh, row, n, a.k, pool, out);
        return;
    }
    write_bitmap<BIG_T>(sh, words, pool != nullptr, out, a.k);
}

}  // namespace

size_t topk_workspace_bytes(int32_t B, int64_t max_n) {
    if (max_n <= SMALL_MAX || max_n > FAST_MAX_N) return 0;
    const int64_t n_seg = (max_n + SEG - 1) / SEG;
    return (size_t)B * SMALL_MAX * (sizeof(float) + sizeof(uint32_t)) +
           (size_t)B * (size_t)n_seg * 2 * sizeof(uint32_t);
}

hipError_t launch_topk(const float* vals, int64_t stride, const int64_t* ctx,
                       int64_t max_ctx, int32_t n_fixed, const int32_t* pool,
                       int32_t n_blocks, int32_t B, int32_t k, int32_t* out, void* ws,
                       hipStream_t stream) {
    TopkArgs a{};
    a.vals = vals;
    a.stride = stride;
    a.ctx = ctx;
    a.max_ctx = max_ctx;
    a.n_fixed = n_fixed;
    a.pool = pool;
    a.n_blocks = n_blocks;
    a.k = k;
    a.out = out;
    const int64_t max_n = ctx ? (max_ctx + BLOCK - 1) / BLOCK : n_fixed;
    if (max_n <= SMALL_MAX || max_n > FAST_MAX_N) {
        hipLaunchKernelGGL(topk_small_kernel, dim3(B), dim3(BIG_T), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t n_seg = (max_n + SEG - 1) / SEG;
    char* w = static_cast<char*>(ws);
    a.seg_val = reinterpret_cast<float*>(w);
    a.seg_id = reinterpret_cast<uint32_t*>(w + (size_t)B * SMALL_MAX * sizeof(float));
    a.seg_meta = reinterpret_cast<uint32_t*>(w + (size_t)B * SMALL_MAX * 2 * sizeof(float));
    a.n_seg = (int32_t)n_seg;
    hipLaunchKernelGGL(topk_seg_kernel, dim3((unsigned)n_seg, B), dim3(SEG_T), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(B), dim3(BIG_T), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
