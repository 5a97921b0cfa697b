// Top-k selection: the k largest of n floats, ties to the lower index, the
// chosen indices written in ascending order and padded with -1.  -inf entries
// are absent (never chosen).
//
// Used twice per Full layer (the 2,048 best blocks of 8 positions forming the
// candidate pool, then the top 512 positions inside the pool) and once per
// Reindex layer (origotech.dev deep dive "Inside DeepSeek V4.1-Flash", section
// "How the architecture shrinks the KV cache").
//
// Select core (one workgroup of 1,024 threads, 16 values per thread in registers):
//   1. min / max / count of the valid values and the smallest per-thread
//      maximum (block reduction); when at least k threads hold a valid value,
//      that minimum is a floor the k-th largest value cannot fall below;
//   2. an LDS histogram over 2,048 bins linear in value between the floor and
//      max (a monotone map, so ranks survive; linear bins keep LDS atomics
//      spread even when every value shares one exponent; values below the floor
//      stay out, which for 16 values per thread skips most atomics) and the bin
//      d holding the k-th largest value;
//   3. values in bins above d are chosen; bin d's values go to an LDS candidate
//      list.  Up to 256 candidates are ranked directly in (value desc, index
//      asc) order; larger lists take an 11/11/10-bit radix on the exact order
//      keys for the threshold key T and how many keys equal to T to take, and an
//      ordered popcount scan over an "equal" bitmap keeps the lowest-index ones.
// Thread t holds the 16 consecutive positions 16t .. 16t+15, so its share of
// the choice is a 16-bit register mask and one block scan of the masks'
// popcounts places the chosen indices in ascending order.  Every instruction
// of this core is issued by 16 waves on one CU's 4 SIMDs, so it is written for
// few instructions per value: a single-barrier block reduction, no atomics on
// the chosen path, one coalesced store.
//
// Rows of up to 4,096 entries: the same core in a 256-thread workgroup (each
// block-wide step is shorter, and about three rows share a CU); up to 16,384:
// one 1,024-thread workgroup, one read of the row; up to 32,768: the same with
// 32 values per thread.
// Longer rows (up to 131,072): a segment kernel takes the exact top-q of each
// 4,096-entry segment (q >= 4x a segment's expected share of the top-k) and
// writes it densely in ascending index order; a merge kernel selects the top-k
// of those slots (slot order is index order) and checks that no segment's worst
// reported entry was chosen (else that segment might hide more winners).
// Rows that fail the check, overflow the candidate list (heavy ties), or are
// longer than 131,072 entries take an exact fallback: three radix sweeps over
// the row in global memory, an ordered collection and a bitonic sort.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "topk_dev.h"

namespace csa2 {

namespace {

using namespace topk_dev;

// Rows of up to SMALL_MAX entries (longer rows: the exact fallback).
__global__ void __launch_bounds__(BIG_T) topk_small_kernel(TopkArgs a) {
    __shared__ Shared<BIG_T> sh;
    topk_small_body(sh, a, blockIdx.x);
}

// Rows of up to SEG entries in a quarter-size workgroup.
__global__ void __launch_bounds__(SEG_T) topk_quarter_kernel(TopkArgs a) {
    __shared__ Shared<SEG_T> sh;
    topk_quarter_body(sh, a, blockIdx.x);
}

// Rows of up to RUN2_MAX entries, 32 values per thread.
__global__ void __launch_bounds__(BIG_T) topk_run32_kernel(TopkArgs a) {
    __shared__ Shared<BIG_T> sh;
    topk_run32_body(sh, a, blockIdx.x);
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
// The dense candidate area lists segment 0's choices, then segment 1's, ...,
// each in ascending index order, so slot order is output order and the
// selection runs on slots (select_run) with the slots' indices as output.  A full
// segment whose worst reported entry is chosen may hide winners: that vetoes
// the choice and the row takes the exact fallback.  Rows the segment kernel
// skipped are selected here directly.
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
    float v[VPT];
    uint32_t id[VPT];
    // this thread's slots 16t .. 16t+15 span at most two segments (quota >= 256)
    int g0 = 0, g1 = 0;
    uint2 m0 = make_uint2(0u, 0u), m1 = make_uint2(0u, 0u);
    if (!two_stage) {
        load_run<VPT>(row, n, v);
#pragma unroll
        for (int j = 0; j < VPT; ++j) id[j] = (uint32_t)(VPT * t + j);
    } else {
        // slots past the last segment's area are never loaded (absent)
        const float4* sv = reinterpret_cast<const float4*>(a.seg_val + (int64_t)b * SMALL_MAX);
        const uint4* si = reinterpret_cast<const uint4*>(a.seg_id + (int64_t)b * SMALL_MAX);
        const int n_slots = (int)((n + SEG - 1) / SEG) * quota;   // <= SMALL_MAX
#pragma unroll
        for (int r = 0; r < VPT / 4; ++r) {
            const bool in = VPT * t + 4 * r < n_slots;
            float4 x = make_float4(NEG_INF, NEG_INF, NEG_INF, NEG_INF);
            uint4 y = make_uint4(0u, 0u, 0u, 0u);
            if (in) {
                x = sv[4 * t + r];
                y = si[4 * t + r];
            }
            v[4 * r] = x.x; v[4 * r + 1] = x.y; v[4 * r + 2] = x.z; v[4 * r + 3] = x.w;
            id[4 * r] = y.x; id[4 * r + 1] = y.y; id[4 * r + 2] = y.z; id[4 * r + 3] = y.w;
        }
        // segment of a slot: the quotient of a float reciprocal, exact after
        // one correction (slots < 2^14, quota <= 4096)
        const float inv_q = 1.0f / (float)quota;
        auto seg_of = [&](int e) {
            int g = (int)((float)e * inv_q);
            const int r = e - g * quota;
            return r < 0 ? g - 1 : (r >= quota ? g + 1 : g);
        };
        const int n_seg = (int)((n + SEG - 1) / SEG);
        g0 = seg_of(VPT * t);
        g1 = seg_of(VPT * t + VPT - 1);
        const uint32_t* meta = a.seg_meta + (int64_t)b * a.n_seg * 2;
        if (g0 < n_seg) m0 = *reinterpret_cast<const uint2*>(meta + 2 * g0);
        if (g1 < n_seg) m1 = *reinterpret_cast<const uint2*>(meta + 2 * g1);
    }
    // the pool goes to LDS for the output's lookups; its loads were issued
    // with the values', and select_run orders these writes before any read
    int32_t pv[CSA2_MAX_POOL / BIG_T];
#pragma unroll
    for (int r = 0; r < CSA2_MAX_POOL / BIG_T; ++r)
        pv[r] = pool && t + BIG_T * r < a.n_blocks ? pool[t + BIG_T * r] : 0;
    if (two_stage) {
        // slots past a segment's reported count hold stale data: absent
        const int g1_start = g1 * quota;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int e = VPT * t + j;
            const bool hi_seg = e >= g1_start;
            const uint32_t c = (hi_seg ? m1.x : m0.x) & 0x7fffffffu;
            const int r = e - (hi_seg ? g1_start : g0 * quota);
            v[j] = (uint32_t)r < c ? v[j] : NEG_INF;
        }
    }
    if (pool) {
#pragma unroll
        for (int r = 0; r < CSA2_MAX_POOL / BIG_T; ++r)
            if (t + BIG_T * r < a.n_blocks) sh.pool[t + BIG_T * r] = pv[r];
    }
    const int64_t n_pos = two_stage ? (int64_t)SMALL_MAX : n;
    const int g1_start = g1 * quota;
    const bool done = select_run<BIG_T, VPT, true>(
        sh, v, n_pos, (uint32_t)a.k, out,
        [&](int j) -> int32_t {
            const int32_t i = (int32_t)id[j];
            return pool ? sh.pool[i >> 3] * BLOCK + (i & 7) : i;
        },
        [&](int j) -> bool {
            if (!two_stage) return false;
            const uint2 m = VPT * t + j >= g1_start ? m1 : m0;
            return (m.x & 0x80000000u) && id[j] == m.y;
        });
    if (!done) topk_fallback(sh, row, n, a.k, pool, out);
}

static_assert(CSA2_MAX_POOL % BIG_T == 0, "pool entries per thread");
static_assert(CSA2_MAX_POOL <= STAGE_WORDS && CSA2_MAX_TOPK <= STAGE_WORDS,
              "select_run stages up to k outputs in eq_bits");

}  // namespace

size_t topk_workspace_bytes(int32_t B, int64_t max_n) {
    if (max_n <= RUN2_MAX || max_n > FAST_MAX_N) return 0;
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
    if (max_n <= SEG) {
        hipLaunchKernelGGL(topk_quarter_kernel, dim3(B), dim3(SEG_T), 0, stream, a);
        return hipGetLastError();
    }
    if (max_n <= SMALL_MAX || max_n > FAST_MAX_N) {
        hipLaunchKernelGGL(topk_small_kernel, dim3(B), dim3(BIG_T), 0, stream, a);
        return hipGetLastError();
    }
    if (max_n <= RUN2_MAX) {
        hipLaunchKernelGGL(topk_run32_kernel, dim3(B), dim3(BIG_T), 0, stream, a);
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
