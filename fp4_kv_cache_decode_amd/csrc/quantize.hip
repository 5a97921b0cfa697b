// Quantise-on-write of new tokens into the compressed cache.
//
// What is computed (origotech.dev deep dive "Inside DeepSeek V4.1-Flash",
// sub-section "FP4 and SWA Bounded Replay"; trawling.dev "CSA2 and FP4 KV
// caching"): post-RoPE main K and V go to FP4 E2M1 with one E4M3 scale per 16
// channels; the sliding-window K/V stay FP8 (E4M3); indexer keys are FP8 too
// (this library's reading: one per-tensor fp32 scale for each FP8 store).
//
// Every part of the grid covers the same 16 rows per block, 16 threads per row.
// Part 0 writes main-KV records (one 16-channel group per thread: 8 of K, 8 of
// V), part 1 indexer keys (4 channels per thread), part 2+l the window rows of
// layer l (one 16-channel group per thread: 8 of K, 8 of V).  A group's thread
// reads 64 contiguous bytes of fp32, so a wave streams 4 KB of input per
// instruction group.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

constexpr int QTHREADS = 256;
constexpr int ROWS_MAIN = QTHREADS / 16;   // rows per block (16 threads per row)

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
    int64_t cap;
    PageMap pm;              // page table of a paged cache (table null otherwise)
    int32_t n_seq;
    int32_t w_cap;
    float idxk_scale;
    float wk_scale;
    float wv_scale;
};

__device__ __forceinline__ void load16(const float* p, float* x) {
    const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 t = p4[i];
        x[4 * i] = t.x;
        x[4 * i + 1] = t.y;
        x[4 * i + 2] = t.z;
        x[4 * i + 3] = t.w;
    }
}

// 16 channels -> 16 E4M3 bytes of x/scale.
__device__ __forceinline__ uint4 fp8_group(const float* x, float scale) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[i] |= e4m3_encode(x[4 * i + j] / scale) << (8 * j);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ bool row_target(const QuantArgs& a, int64_t row, int64_t& dst) {
    int32_t s = a.seq[row];
    int64_t p = a.pos[row];
    if (s < 0 || s >= a.n_seq || p < 0 || p >= a.cap) return false;
    dst = a.pm.table ? cache_row<true>(a.pm, a.cap, s, p) : cache_row<false>(a.pm, a.cap, s, p);
    return true;
}

__global__ void __launch_bounds__(QTHREADS) quantize_kernel(QuantArgs a) {
    const int part = blockIdx.y;
    const int t = threadIdx.x;
    if (part == 1) {
        // indexer keys: channels 4u .. 4u+3 of the row
        const int64_t row = (int64_t)blockIdx.x * ROWS_MAIN + t / 16;
        const int u = t & 15;
        int64_t dst;
        if (!a.idx_k || row >= a.n || !row_target(a, row, dst)) return;
        const float4 x = *reinterpret_cast<const float4*>(a.idx_k + row * IDX_DIM + 4 * u);
        const float sc = a.idxk_scale;
        const uint32_t w = e4m3_encode(x.x / sc) | (e4m3_encode(x.y / sc) << 8) |
                           (e4m3_encode(x.z / sc) << 16) | (e4m3_encode(x.w / sc) << 24);
        *reinterpret_cast<uint32_t*>(a.idxk + dst * IDX_DIM + 4 * u) = w;
        return;
    }
    int64_t row = (int64_t)blockIdx.x * ROWS_MAIN + t / 16;
    int u = t & 15;
    int64_t dst = 0;
    bool ok = row < a.n && row_target(a, row, dst);
    if (part == 0) {
        float x[16];
        uint32_t sc = 0, lo = 0, hi = 0;
        if (ok) {
            const float* src = (u < 8 ? a.k : a.v) + row * D + 16 * (u & 7);
            load16(src, x);
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
            sc = e4m3_encode(amax / 6.0f);          // amax >= 0: positive code
            float s = e4m3_value_pos(sc);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t nib = e2m1_mag(fabsf(x[i]), s) | ((__float_as_uint(x[i]) >> 28) & 8u);
                if (i < 8) lo |= nib << (4 * i);
                else hi |= nib << (4 * (i - 8));
            }
        }
        // gather the 4 scale bytes of lanes u..u+3 (u % 4 == 0) into one dword
        uint32_t word = sc << (8 * (u & 3));
        word |= (uint32_t)__builtin_amdgcn_mov_dpp((int)word, DPP_XOR1, 0xf, 0xf, false);
        word |= (uint32_t)__builtin_amdgcn_mov_dpp((int)word, DPP_XOR2, 0xf, 0xf, false);
        if (!ok) return;
        uint8_t* rec = a.kv + dst * RECORD;
        *reinterpret_cast<uint2*>(rec + 8 * u) = make_uint2(lo, hi);   // K codes, then V
        if ((u & 3) == 0) *reinterpret_cast<uint32_t*>(rec + 128 + u) = word;
        return;
    }
    // window rows of layer l
    if (!ok) return;
    const int l = part - 2;
    const int64_t n = a.n;
    const float* src = (u < 8 ? a.win_k : a.win_v) + ((int64_t)l * n + row) * D + 16 * (u & 7);
    float x[16];
    load16(src, x);
    int64_t p = a.pos[row];
    int32_t s = a.seq[row];
    int64_t slot = (((int64_t)l * a.n_seq + s) * a.w_cap + p % a.w_cap) * D + 16 * (u & 7);
    uint8_t* dstp = (u < 8 ? a.wk : a.wv) + slot;
    *reinterpret_cast<uint4*>(dstp) = fp8_group(x, u < 8 ? a.wk_scale : a.wv_scale);
}

}  // namespace

hipError_t launch_quantize(const csa2_cache& c, const csa2_window* w, const float* k,
                           const float* v, const float* idx_k, const float* win_k,
                           const float* win_v, const int32_t* seq, const int64_t* pos,
                           int64_t n, hipStream_t stream) {
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
    int parts = idx_k ? 2 : 1;
    if (win_k) {
        a.wk = w->k;
        a.wv = w->v;
        a.w_cap = w->w_cap;
        a.wk_scale = w->k_scale;
        a.wv_scale = w->v_scale;
        parts = 2 + w->n_layers;
    }
    // with windows but no indexer input, part 1 blocks exit at once
    const dim3 grid((unsigned)((n + ROWS_MAIN - 1) / ROWS_MAIN), parts);
    hipLaunchKernelGGL(quantize_kernel, grid, dim3(QTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa2
