// Quantise-on-write of new tokens into the compressed cache.
//
// What is computed (origotech.dev deep dive "Inside DeepSeek V4.1-Flash",
// sub-section "FP4 and SWA Bounded Replay"; trawling.dev "CSA2 and FP4 KV
// caching"): post-RoPE main K and V go to FP4 E2M1 with one E4M3 scale per 16
// channels; the sliding-window K/V stay FP8 (E4M3); indexer keys are FP8 too
// (this library's reading: one per-tensor fp32 scale for each FP8 store).
//
// Every part of the grid covers the same 16 * QG rows per block, 16 threads per
// row and QG groups of 16 rows per thread.  Part 0 writes the main-KV records (one
// 16-channel group per thread: 8 of K, 8 of V) and, when given, the rows' indexer
// keys (4 channels per thread); part 1+l writes the window rows of layer l (one
// 16-channel group per thread: 8 of K, 8 of V).  A group's thread reads 64
// contiguous bytes of fp32, so a wave streams 4 KB of input per instruction group.
//
// QG = 4 from 1,048,576 rows on, where more loads in flight per thread pay (4M
// rows: 1.17 ms against 1.19 with QG = 1); below that QG = 1, which spreads a call
// over four times the blocks (256K rows: 73 us against 79).  A thread loads seq
// and pos of its rows first and then all of its row data, before it decides where
// any row goes: a wait on a destination then never drains the row loads behind
// it, and the row data is in flight while the destinations are checked.
//
// Compression M (M = 2 for the encoder's CSA2 layers, origotech.dev deep dive,
// section "How the architecture shrinks the KV cache"; this library's reading of
// the operator): part 0 then covers groups of M consecutive input rows, the
// tokens at positions M*e .. M*e + M - 1 of one sequence, and writes entry e from
// the rows' fp32 mean ((r0 + r1) * 0.5: one rounding of the sum, an exact
// halving); the window parts still write every token.  M = 1 is plain
// quantise-on-write: every step that depends on M folds away for it.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int QTHREADS = 256;
constexpr int ROWS_GROUP = QTHREADS / 16;   // rows per group (16 threads per row)
constexpr int QG_BULK = 4;                  // row groups per thread in large calls
constexpr int64_t BULK_BLOCKS = 16384;      // blocks of QG_BULK groups from which to use them

struct QuantArgs {
    uint8_t* kv;
    uint8_t* idxk;
    uint8_t* wk;
    uint8_t* wv;
    const float* k;
    const float* v;
    const float* idx_k;
    const float* win_k;
    const float* win_v;
    const int32_t* seq;
    const int64_t* pos;
    int64_t n;
    int64_t n_main;          // M > 1: groups written to the global store (0: window only)
    int64_t win_limit;       // M > 1: token positions the window accepts (m * cap)
    int64_t cap;
    PageMap pm;              // page table of a paged cache (table null otherwise)
    int32_t n_seq;
    int32_t w_cap;
    float idxk_scale;
    float wk_scale;
    float wv_scale;
};

__device__ __forceinline__ void load16(const float* p, float4* x) {
    const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = p4[i];
}

__device__ __forceinline__ float elem(const float4* x, int i) {
    const float4 t = x[i >> 2];
    return (i & 3) == 0 ? t.x : (i & 3) == 1 ? t.y : (i & 3) == 2 ? t.z : t.w;
}

__device__ __forceinline__ uint32_t fp8_word(float4 x, float scale) {
    return e4m3_encode(x.x / scale) | (e4m3_encode(x.y / scale) << 8) |
           (e4m3_encode(x.z / scale) << 16) | (e4m3_encode(x.w / scale) << 24);
}

// 16 channels -> 16 E4M3 bytes of x/scale.
__device__ __forceinline__ uint4 fp8_group(const float4* x, float scale) {
    return make_uint4(fp8_word(x[0], scale), fp8_word(x[1], scale), fp8_word(x[2], scale),
                      fp8_word(x[3], scale));
}

// Cache row of (s, p), or false when the row is skipped (s or p out of range).
__device__ __forceinline__ bool row_target(const QuantArgs& a, int32_t s, int64_t p, int64_t& dst) {
    if (s < 0 || s >= a.n_seq || p < 0 || p >= a.cap) return false;
    dst = a.pm.table ? cache_row<true>(a.pm, a.cap, s, p) : cache_row<false>(a.pm, a.cap, s, p);
    return true;
}

// Row (or group) g of the thread, clamped to the last of the n_items: loads need
// no branch (a branch around a load makes the compiler wait for every load in
// flight at the join); items past the end are loaded again from the last one
// and never stored.
__device__ __forceinline__ int64_t load_row(int64_t n_items, int64_t row0, int g) {
    const int64_t row = row0 + g * ROWS_GROUP;
    return row < n_items ? row : n_items - 1;
}

// seq and pos of the thread's rows (of the first row of each group of M),
// loaded before anything else so that no later wait for them also waits for
// the row data behind them.
template <int QG, int M>
__device__ __forceinline__ void load_rows(const QuantArgs& a, int64_t n_items, int64_t row0,
                                          int32_t* sq, int64_t* ps) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const int64_t row = load_row(n_items, row0, g) * M;
        sq[g] = a.seq[row];
        ps[g] = a.pos[row];
    }
}

// 16 floats of group e: the row itself (M = 1) or the fp32 mean of its M rows.
template <int M>
__device__ __forceinline__ void load_group16(const float* src, int64_t e, int dim, int off,
                                             float4* x) {
    load16(src + e * M * dim + off, x);
    if (M == 2) {
        float4 y[4];
        load16(src + (e * M + 1) * dim + off, y);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i].x = (x[i].x + y[i].x) * 0.5f;
            x[i].y = (x[i].y + y[i].y) * 0.5f;
            x[i].z = (x[i].z + y[i].z) * 0.5f;
            x[i].w = (x[i].w + y[i].w) * 0.5f;
        }
    }
}
template <int M>
__device__ __forceinline__ float4 load_group4(const float* src, int64_t e, int dim, int off) {
    float4 x = *reinterpret_cast<const float4*>(src + e * M * dim + off);
    if (M == 2) {
        const float4 y = *reinterpret_cast<const float4*>(src + (e * M + 1) * dim + off);
        x.x = (x.x + y.x) * 0.5f;
        x.y = (x.y + y.y) * 0.5f;
        x.z = (x.z + y.z) * 0.5f;
        x.w = (x.w + y.w) * 0.5f;
    }
    return x;
}

template <int QG, int M>
__global__ void __launch_bounds__(QTHREADS) quantize_kernel(QuantArgs a) {
    static_assert(M == 1 || M == 2, "compression 1 or 2");
    const int part = blockIdx.y;
    const int t = threadIdx.x;
    const int u = t & 15;
    const int64_t row0 = (int64_t)blockIdx.x * (ROWS_GROUP * QG) + t / 16;
    int32_t sq[QG];
    int64_t ps[QG];
    float4 x[QG][4];
    if (part == 0) {
        // the grid covers the n tokens; part 0 has n_main = n / M groups (none
        // for a window-only call)
        const int64_t n_g = M > 1 ? a.n_main : a.n;
        if (M > 1 && (int64_t)blockIdx.x * (ROWS_GROUP * QG) >= n_g) return;
        load_rows<QG, M>(a, n_g, row0, sq, ps);
        float4 ik[QG];
#pragma unroll
        for (int g = 0; g < QG; ++g)
            load_group16<M>(u < 8 ? a.k : a.v, load_row(n_g, row0, g), D, 16 * (u & 7), x[g]);
        if (a.idx_k) {
#pragma unroll
            for (int g = 0; g < QG; ++g)
                ik[g] = load_group4<M>(a.idx_k, load_row(n_g, row0, g), IDX_DIM, 4 * u);
        }
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            const int64_t row = row0 + g * ROWS_GROUP;
            int64_t dst = 0;
            const bool ok = row < n_g && ps[g] % M == 0 && row_target(a, sq[g], ps[g] / M, dst);
            uint32_t sc = 0, lo = 0, hi = 0;
            if (ok) {
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(elem(x[g], i)));
                sc = e4m3_encode(amax / 6.0f);      // amax >= 0: positive code
                const float sv = e4m3_value_pos(sc);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float xi = elem(x[g], i);
                    const uint32_t nib = e2m1_mag(fabsf(xi), sv) | ((__float_as_uint(xi) >> 28) & 8u);
                    if (i < 8) lo |= nib << (4 * i);
                    else hi |= nib << (4 * (i - 8));
                }
            }
            // gather the 4 scale bytes of lanes u..u+3 (u % 4 == 0) into one dword
            uint32_t word = sc << (8 * (u & 3));
            word |= (uint32_t)__builtin_amdgcn_mov_dpp((int)word, DPP_XOR1, 0xf, 0xf, false);
            word |= (uint32_t)__builtin_amdgcn_mov_dpp((int)word, DPP_XOR2, 0xf, 0xf, false);
            if (!ok) continue;
            uint8_t* rec = a.kv + dst * RECORD;
            *reinterpret_cast<uint2*>(rec + 8 * u) = make_uint2(lo, hi);   // K codes, then V
            if ((u & 3) == 0) *reinterpret_cast<uint32_t*>(rec + 128 + u) = word;
            if (a.idx_k)
                *reinterpret_cast<uint32_t*>(a.idxk + dst * IDX_DIM + 4 * u) =
                    fp8_word(ik[g], a.idxk_scale);
        }
        return;
    }
    // window rows of layer l
    const int l = part - 1;
    const int64_t n = a.n;
    load_rows<QG, 1>(a, n, row0, sq, ps);
#pragma unroll
    for (int g = 0; g < QG; ++g)
        load16((u < 8 ? a.win_k : a.win_v) + ((int64_t)l * n + load_row(n, row0, g)) * D +
                   16 * (u & 7), x[g]);
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const int64_t row = row0 + g * ROWS_GROUP;
        const int32_t s = sq[g];
        const int64_t p = ps[g];
        // token positions reach m * cap: the global store holds one entry per m
        const int64_t lim = M > 1 ? a.win_limit : a.cap;
        if (row >= n || s < 0 || s >= a.n_seq || p < 0 || p >= lim) continue;
        const int64_t slot = (((int64_t)l * a.n_seq + s) * a.w_cap + p % a.w_cap) * D + 16 * (u & 7);
        uint8_t* dstp = (u < 8 ? a.wk : a.wv) + slot;
        *reinterpret_cast<uint4*>(dstp) = fp8_group(x[g], u < 8 ? a.wk_scale : a.wv_scale);
    }
}

}  // namespace

hipError_t launch_quantize(const csa2_cache& c, const csa2_window* w, const float* k,
                           const float* v, const float* idx_k, const float* win_k,
                           const float* win_v, const int32_t* seq, const int64_t* pos,
                           int64_t n, int32_t m, hipStream_t stream) {
    QuantArgs a{};
    a.kv = c.kv;
    a.idxk = c.idxk;
    a.k = k;
    a.v = v;
    a.idx_k = idx_k;
    a.win_k = win_k;
    a.win_v = win_v;
    a.seq = seq;
    a.pos = pos;
    a.n = n;
    a.cap = c.cap;
    a.pm = page_map(c);
    a.n_seq = c.n_seq;
    a.idxk_scale = c.idxk_scale;
    int parts = 1;
    if (win_k) {
        a.wk = w->k;
        a.wv = w->v;
        a.w_cap = w->w_cap;
        a.wk_scale = w->k_scale;
        a.wv_scale = w->v_scale;
        parts = 1 + w->n_layers;
    }
    // k and v null: window rows only (a compressed store gets its entries from
    // complete groups, the window every token)
    a.n_main = k ? n / m : 0;
    a.win_limit = c.cap * m;
    const int64_t bulk_blocks = (n + ROWS_GROUP * QG_BULK - 1) / (ROWS_GROUP * QG_BULK);
    const dim3 small((unsigned)((n + ROWS_GROUP - 1) / ROWS_GROUP), parts);
    if (m == 2 || !k)
        hipLaunchKernelGGL((quantize_kernel<1, 2>), small, dim3(QTHREADS), 0, stream, a);
    else if (bulk_blocks >= BULK_BLOCKS)
        hipLaunchKernelGGL((quantize_kernel<QG_BULK, 1>), dim3((unsigned)bulk_blocks, parts),
                           dim3(QTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((quantize_kernel<1, 1>), small, dim3(QTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
