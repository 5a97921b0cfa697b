// Top-k selection: the k largest of n floats, ties to the lower index, the
// chosen indices written in ascending order and padded with -1.
//
// Used twice per Full layer (the 2,048 best blocks of 8 positions forming the
// candidate pool, then the top 512 positions inside the pool) and once per
// Reindex layer (origotech.dev deep dive "Inside DeepSeek V4.1-Flash", section
// "How the architecture shrinks the KV cache").
//
// Algorithm: exact radix select on order-preserving uint32 keys with 11/11/10
// bit digits and LDS histograms, one 1024-thread workgroup per row.  Rows of up
// to 32,768 entries are staged once in LDS (128 KiB, gfx950 allows 160 KiB per
// workgroup); longer rows are re-read from global memory for each digit.  The
// threshold key T and the number kk of entries equal to T that must be taken
// come out of the last digit; a collection pass appends every key > T, and the
// kk lowest-index keys == T (an ordered block scan per 4096-entry round runs
// only when more than kk entries tie at T), to an LDS list that a bitonic sort
// puts in ascending order.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int LDS_KEYS = 32768;
constexpr uint32_t KEY_ABSENT = 0x007fffffu;   // order_key(-inf)

struct TopkArgs {
    const float* vals;
    int64_t stride;
    const int64_t* ctx;      // block mode when non-null
    int64_t max_ctx;
    int32_t n_fixed;
    const int32_t* pool;
    int32_t n_blocks;
    int32_t k;
    int32_t* out;
};

struct TopkShared {
    uint32_t hist[2048];
    int32_t sel[2048];
    uint32_t wave_sums[TK_WAVES];
    uint32_t misc[8];
};

// Inclusive block scan over 1024 threads; returns the inclusive prefix and the
// block total through *total.
__device__ uint32_t block_incl_scan(uint32_t v, TopkShared& sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    if (lane == 63) sh.wave_sums[wave] = v;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < TK_WAVES; ++i) {
        uint32_t x = sh.wave_sums[i];
        before += (i < wave) ? x : 0u;
        all += x;
    }
    __syncthreads();
    *total = all;
    return v + before;
}

template <bool IN_LDS>
__device__ __forceinline__ uint32_t get_key(const float* vals, const uint32_t* lk, int64_t i) {
    if (IN_LDS) return lk[i];
    return order_key(vals[i]);
}

// Given hist over the current digit, find the digit d with
// count(> d) < kk <= count(>= d).  Writes d and count(> d) into misc[0..1].
__device__ void find_digit(TopkShared& sh, uint32_t kk, int nbins) {
    const int t = threadIdx.x;
    // thread t owns bins nbins-1-2t and nbins-2-2t (descending order)
    const int b0 = nbins - 1 - 2 * t, b1 = b0 - 1;
    uint32_t c0 = b0 >= 0 ? sh.hist[b0] : 0u;
    uint32_t c1 = b1 >= 0 ? sh.hist[b1] : 0u;
    uint32_t total;
    uint32_t incl = block_incl_scan(c0 + c1, sh, &total);
    uint32_t above0 = incl - c0 - c1;           // count of bins > b0
    if (b0 >= 0 && above0 < kk && above0 + c0 >= kk) {
        sh.misc[0] = (uint32_t)b0;
        sh.misc[1] = above0;
    }
    uint32_t above1 = above0 + c0;
    if (b1 >= 0 && above1 < kk && above1 + c1 >= kk) {
        sh.misc[0] = (uint32_t)b1;
        sh.misc[1] = above1;
    }
    __syncthreads();
}

template <bool IN_LDS>
__global__ void __launch_bounds__(TK_THREADS) topk_kernel(TopkArgs a) {
    extern __shared__ uint32_t lds_keys[];
    __shared__ TopkShared sh;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    int64_t n;
    if (a.ctx) {
        int64_t N = clamp64(a.ctx[b], 0, a.max_ctx);
        n = (N + BLOCK - 1) / BLOCK;
    } else {
        n = a.n_fixed;
    }
    const float* vals = a.vals + (int64_t)b * a.stride;
    const int32_t k = a.k;
    int32_t* out = a.out + (int64_t)b * k;

    if (IN_LDS) {
        for (int64_t i = t; i < n; i += TK_THREADS) lds_keys[i] = order_key(vals[i]);
    }
    // ---- digit passes
    uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k, n_valid = 0;
    bool take_all = false;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int sh_ = shifts[pass];
        const int nb = 1 << widths[pass];
        for (int i = t; i < 2048; i += TK_THREADS) sh.hist[i] = 0;
        __syncthreads();
        for (int64_t i = t; i < n; i += TK_THREADS) {
            uint32_t key = get_key<IN_LDS>(vals, lds_keys, i);
            if (key != KEY_ABSENT && (key & pmask) == prefix)
                atomicAdd(&sh.hist[(key >> sh_) & (nb - 1)], 1u);
        }
        __syncthreads();
        if (pass == 0) {
            uint32_t c = sh.hist[2 * t] + sh.hist[2 * t + 1], tot;
            block_incl_scan(c, sh, &tot);
            n_valid = tot;
            if (n_valid <= (uint32_t)k) {
                take_all = true;
                break;
            }
        }
        find_digit(sh, kk, nb);
        const uint32_t d = sh.misc[0];
        kk -= sh.misc[1];
        prefix |= d << sh_;
        pmask |= (uint32_t)(nb - 1) << sh_;
        __syncthreads();
    }
    // threshold T = prefix; take every key > T and the kk lowest-index keys == T
    const uint32_t T = take_all ? KEY_ABSENT : prefix;
    const uint32_t n_eq = take_all ? 0u : sh.hist[prefix & 1023u];
    if (t == 0) sh.misc[2] = 0;
    __syncthreads();
    if (take_all || n_eq == kk) {
        // every valid key when n_valid <= k; else every key >= T (T itself is
        // a valid key, and absent keys sort below every valid one)
        for (int64_t i = t; i < n; i += TK_THREADS) {
            uint32_t key = get_key<IN_LDS>(vals, lds_keys, i);
            if (take_all ? key != KEY_ABSENT : key >= T) {
                uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                if (slot < 2048u) sh.sel[slot] = (int32_t)i;
            }
        }
    } else {
        // ordered rounds: thread t owns entries r*4096 + 4t .. +3
        uint32_t base = 0;
        for (int64_t r0 = 0; r0 < n; r0 += 4 * TK_THREADS) {
            uint32_t keys[4];
            uint32_t ceq = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int64_t i = r0 + 4 * t + j;
                keys[j] = i < n ? get_key<IN_LDS>(vals, lds_keys, i) : KEY_ABSENT;
                ceq += (keys[j] == T) ? 1u : 0u;
                if (keys[j] != KEY_ABSENT && keys[j] > T) {
                    uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                    if (slot < 2048u) sh.sel[slot] = (int32_t)i;
                }
            }
            if (base < kk) {
                uint32_t tot;
                uint32_t rank = block_incl_scan(ceq, sh, &tot) - ceq + base;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (keys[j] == T) {
                        if (rank < kk) {
                            uint32_t slot = atomicAdd(&sh.misc[2], 1u);
                            if (slot < 2048u) sh.sel[slot] = (int32_t)(r0 + 4 * t + j);
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
    // ---- bitonic sort of sel[0..cnt) ascending, padded with INT_MAX
    int P = 1;
    while (P < cnt) P <<= 1;
    for (int i = cnt + t; i < P; i += TK_THREADS) sh.sel[i] = 0x7fffffff;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < P / 2; i += TK_THREADS) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool up = (lo & size) == 0;
                int x = sh.sel[lo], y = sh.sel[hi];
                if ((x > y) == up) {
                    sh.sel[lo] = y;
                    sh.sel[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    // ---- write
    const int32_t* pool = a.pool ? a.pool + (int64_t)b * a.n_blocks : nullptr;
    for (int j = t; j < k; j += TK_THREADS) {
        int32_t v = -1;
        if (j < cnt) {
            int32_t i = sh.sel[j];
            v = pool ? pool[i >> 3] * BLOCK + (i & 7) : i;
        }
        out[j] = v;
    }
}

}  // namespace

hipError_t launch_topk(const float* vals, int64_t stride, const int64_t* ctx,
                       int64_t max_ctx, int32_t n_fixed, const int32_t* pool,
                       int32_t n_blocks, int32_t B, int32_t k, int32_t* out,
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
    if (max_n <= LDS_KEYS) {
        size_t lds = (size_t)(max_n > 0 ? max_n : 1) * sizeof(uint32_t);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_kernel<true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(topk_kernel<true>, dim3(B), dim3(TK_THREADS), lds, stream, a);
    } else {
        hipLaunchKernelGGL(topk_kernel<false>, dim3(B), dim3(TK_THREADS), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace csa2
