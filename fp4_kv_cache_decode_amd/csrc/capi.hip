// C ABI of libcsa2: argument validation, workspace layout, launch order.
// The operations and their sources are documented in include/csa2.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "csa2_device.h"
#include "csa2_internal.h"

namespace {

using csa2::BLOCK;

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// scales are positive normal floats (their reciprocals are finite too)
bool good_scale(float s) { return isnormal(s) && s > 0.0f; }

// Block-maxima row stride (floats) for contexts up to max_ctx.
int64_t m_stride(int64_t max_ctx) {
    int64_t nb = (max_ctx + BLOCK - 1) / BLOCK;
    return (nb + 63) / 64 * 64;
}

// Workspace of the top-k stages for rows of up to max_n entries.
size_t select_bytes(int32_t B, int64_t max_n) {
    return align_up(csa2::topk_workspace_bytes(B, max_n));
}

struct FullLayout {
    size_t m_off, pool_off, s_off, sel_off, total;
};

FullLayout full_layout(int32_t B, int64_t max_ctx, int32_t n_blocks) {
    FullLayout L;
    L.m_off = 0;
    L.pool_off = align_up(L.m_off + (size_t)B * (size_t)m_stride(max_ctx) * sizeof(float));
    L.s_off = align_up(L.pool_off + (size_t)B * (size_t)n_blocks * sizeof(int32_t));
    L.sel_off = align_up(L.s_off + (size_t)B * (size_t)n_blocks * BLOCK * sizeof(float));
    const size_t sel_blocks = select_bytes(B, (max_ctx + BLOCK - 1) / BLOCK);
    const size_t sel_pool = select_bytes(B, (int64_t)n_blocks * BLOCK);
    L.total = L.sel_off + (sel_blocks > sel_pool ? sel_blocks : sel_pool);
    return L;
}

size_t reindex_bytes(int32_t B, int32_t n_blocks) {
    return align_up((size_t)B * (size_t)n_blocks * BLOCK * sizeof(float)) +
           select_bytes(B, (int64_t)n_blocks * BLOCK);
}

// Fused Reindex layer: barrier words, pool scores, the tiles' partial records.
struct LayerLayout {
    size_t s_off, part_off, total;
};

int32_t layer_tiles(int32_t topk) { return (topk + 63) / 64 + CSA2_WINDOW / 64; }

LayerLayout layer_layout(int32_t B, int32_t n_blocks, int32_t topk) {
    LayerLayout L;
    L.s_off = align_up(sizeof(csa2::LayerSync));
    L.part_off = align_up(L.s_off + (size_t)B * (size_t)n_blocks * BLOCK * sizeof(float));
    L.total = L.part_off + align_up((size_t)B * (size_t)layer_tiles(topk) *
                                    csa2::ATTN_PART_FLOATS * sizeof(float));
    return L;
}

size_t attn_bytes(int32_t B, int32_t topk) {
    return align_up((size_t)csa2::attn_partials(B, topk, csa2::ATTN_NO_CAP) *
                    csa2::ATTN_PART_FLOATS * sizeof(float));
}

csa2_status check_cache(const csa2_cache* c, bool need_kv, bool need_idxk) {
    if (!c) return CSA2_ERR_INVALID_ARG;
    if ((need_kv && !c->kv) || (need_idxk && !c->idxk)) return CSA2_ERR_INVALID_ARG;
    if (c->n_seq <= 0 || c->cap <= 0) return CSA2_ERR_INVALID_ARG;
    if (need_idxk && !good_scale(c->idxk_scale)) return CSA2_ERR_INVALID_ARG;
    if (c->page_table) {
        const int32_t p = c->page_tokens;
        if (p < 64 || p > 65536 || (p & (p - 1))) return CSA2_ERR_UNSUPPORTED;
        if (c->n_pages <= 0 || c->cap % p) return CSA2_ERR_INVALID_ARG;
    }
    return CSA2_OK;
}

csa2_status check_window(const csa2_window* w, const csa2_cache* c) {
    if (!w || !w->k || !w->v) return CSA2_ERR_INVALID_ARG;
    if (w->n_layers <= 0 || w->n_seq != c->n_seq) return CSA2_ERR_INVALID_ARG;
    if (w->w_cap < CSA2_WINDOW) return CSA2_ERR_UNSUPPORTED;
    if (!good_scale(w->k_scale) || !good_scale(w->v_scale)) return CSA2_ERR_INVALID_ARG;
    return CSA2_OK;
}

csa2_status check_select(int32_t B, int32_t n_blocks, int32_t block, int32_t topk) {
    if (B < 0) return CSA2_ERR_INVALID_ARG;
    if (B > 65535) return CSA2_ERR_UNSUPPORTED;
    if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
    if (n_blocks < 1 || n_blocks > CSA2_MAX_POOL) return CSA2_ERR_UNSUPPORTED;
    if (topk < 1 || topk > CSA2_MAX_TOPK) return CSA2_ERR_UNSUPPORTED;
    if ((int64_t)topk > (int64_t)n_blocks * block) return CSA2_ERR_INVALID_ARG;
    return CSA2_OK;
}

csa2_status launched(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH; }

// ---------------------------------------------------------------------------
// Fixed scratch of csa2_decode_attn_noalloc: the split queries' partial records
// live in a file-scope device array instead of a caller workspace.  Every GPU
// the library runs on holds its own copy until the process ends.  In host code
// the array's name is only a host-side stand-in, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is handed to kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = CSA2_NOALLOC_SCRATCH_BYTES;
constexpr int64_t NOALLOC_MAX_PARTS =
    (int64_t)(NOALLOC_SCRATCH_BYTES / (csa2::ATTN_PART_FLOATS * sizeof(float)));
static_assert(NOALLOC_MAX_PARTS >= csa2::ATTN_MIN_CAP, "the tile kernel's partials must fit");
constexpr int MAX_DEVICES = 64;

std::mutex scratch_mu;
float* scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device id, once looked up

}  // namespace

static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

// Device address of this device's scratch array (null on failure).
float* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_ptr[dev] = static_cast<float*>(p);
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* csa2_status_string(csa2_status s) {
    // A C caller may pass any int; reading it as the enum type would be
    // undefined for values outside the enumerators' range, so read its bits.
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_INVALID_ARG: return "invalid argument";
        case CSA2_ERR_UNSUPPORTED: return "unsupported size";
        case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
        case CSA2_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

size_t csa2_workspace_bytes(int32_t op, int32_t B, int64_t max_ctx, int32_t n_blocks,
                            int32_t block, int32_t topk) {
    if (B < 0) return 0;
    switch (op) {
        case CSA2_OP_INDEX_FULL:
            if (max_ctx < 0 || check_select(B, n_blocks, block, topk) != CSA2_OK) return 0;
            return full_layout(B, max_ctx, n_blocks).total;
        case CSA2_OP_INDEX_REINDEX:
            if (check_select(B, n_blocks, block, topk) != CSA2_OK) return 0;
            return reindex_bytes(B, n_blocks);
        case CSA2_OP_DECODE_ATTN:
            if (topk < 1 || topk > CSA2_MAX_TOPK) return 0;
            return attn_bytes(B, topk);
        case CSA2_OP_SELECT_POOL:
            if (max_ctx < 0 || n_blocks < 1 || n_blocks > CSA2_MAX_POOL) return 0;
            return select_bytes(B, (max_ctx + BLOCK - 1) / BLOCK);
        case CSA2_OP_REINDEX_LAYER_FUSED:
            if (check_select(B, n_blocks, block, topk) != CSA2_OK) return 0;
            return layer_layout(B, n_blocks, topk).total;
    }
    return 0;
}

csa2_status csa2_compress_kv(const csa2_cache* cache, const csa2_window* win, const float* k,
                             const float* v, const float* idx_k, const float* win_k,
                             const float* win_v, const int32_t* seq, const int64_t* pos,
                             int64_t n, int32_t m, hipStream_t stream) {
    csa2_status st = check_cache(cache, true, idx_k != nullptr);
    if (st != CSA2_OK) return st;
    if (!seq || !pos || n < 0) return CSA2_ERR_INVALID_ARG;
    if (m != 1 && m != 2) return CSA2_ERR_UNSUPPORTED;
    if ((k == nullptr) != (v == nullptr)) return CSA2_ERR_INVALID_ARG;
    if (!k && (idx_k || !win_k)) return CSA2_ERR_INVALID_ARG;   // window only
    if (k && n % m != 0) return CSA2_ERR_INVALID_ARG;
    if ((win_k == nullptr) != (win_v == nullptr)) return CSA2_ERR_INVALID_ARG;
    if (win_k) {
        st = check_window(win, cache);
        if (st != CSA2_OK) return st;
        if (win->n_layers > 65533) return CSA2_ERR_UNSUPPORTED;
    }
    if (n > ((int64_t)1 << 34)) return CSA2_ERR_UNSUPPORTED;
    if (n == 0) return CSA2_OK;
    return launched(csa2::launch_quantize(*cache, win, k, v, idx_k, win_k, win_v, seq, pos, n,
                                          m, stream));
}

csa2_status csa2_quantize_kv(const csa2_cache* cache, const csa2_window* win, const float* k,
                             const float* v, const float* idx_k, const float* win_k,
                             const float* win_v, const int32_t* seq, const int64_t* pos,
                             int64_t n, hipStream_t stream) {
    if (!k || !v) return CSA2_ERR_INVALID_ARG;
    return csa2_compress_kv(cache, win, k, v, idx_k, win_k, win_v, seq, pos, n, 1, stream);
}

csa2_status csa2_index_full(const csa2_cache* cache, const float* q_idx, const float* w,
                            const int32_t* seq, const int64_t* ctx, int32_t B,
                            int64_t max_ctx, int32_t n_blocks, int32_t block, int32_t topk,
                            int32_t* pool, int32_t* idx, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    csa2_status st = check_cache(cache, false, true);
    if (st != CSA2_OK) return st;
    if (!q_idx || !w || !seq || !ctx || !idx) return CSA2_ERR_INVALID_ARG;
    st = check_select(B, n_blocks, block, topk);
    if (st != CSA2_OK) return st;
    if (max_ctx < 0 || max_ctx > cache->cap) return CSA2_ERR_INVALID_ARG;
    if (B == 0) return CSA2_OK;
    const FullLayout L = full_layout(B, max_ctx, n_blocks);
    if (!ws || ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws);
    float* M = reinterpret_cast<float*>(base + L.m_off);
    int32_t* pool_out = pool ? pool : reinterpret_cast<int32_t*>(base + L.pool_off);
    float* S = reinterpret_cast<float*>(base + L.s_off);
    void* sel = base + L.sel_off;

    hipError_t e = csa2::launch_score_blocks(*cache, q_idx, w, seq, ctx, B, max_ctx,
                                             m_stride(max_ctx), M,
                                             stream);
    if (e != hipSuccess) return CSA2_ERR_LAUNCH;
    e = csa2::launch_topk(M, m_stride(max_ctx), ctx, max_ctx, 0, nullptr, 0, B, n_blocks,
                          pool_out, sel, stream);
    if (e != hipSuccess) return CSA2_ERR_LAUNCH;
    e = csa2::launch_score_pool(*cache, q_idx, w, seq, ctx, B, pool_out, n_blocks, S, stream);
    if (e != hipSuccess) return CSA2_ERR_LAUNCH;
    return launched(csa2::launch_topk(S, (int64_t)n_blocks * BLOCK, nullptr, 0,
                                      n_blocks * BLOCK, pool_out, n_blocks, B, topk, idx, sel,
                                      stream));
}

csa2_status csa2_index_block_scores(const csa2_cache* cache, const float* q_idx, const float* w,
                                    const int32_t* seq, const int64_t* ctx, int32_t B,
                                    int64_t max_ctx, float* M, int64_t m_stride_,
                                    hipStream_t stream) {
    csa2_status st = check_cache(cache, false, true);
    if (st != CSA2_OK) return st;
    if (!q_idx || !w || !seq || !ctx || !M || B < 0) return CSA2_ERR_INVALID_ARG;
    if (B > 65535) return CSA2_ERR_UNSUPPORTED;
    if (max_ctx < 0 || max_ctx > cache->cap) return CSA2_ERR_INVALID_ARG;
    if (m_stride_ < (max_ctx + BLOCK - 1) / BLOCK) return CSA2_ERR_INVALID_ARG;
    if (B == 0 || max_ctx == 0) return CSA2_OK;
    return launched(csa2::launch_score_blocks(*cache, q_idx, w, seq, ctx, B, max_ctx, m_stride_,
                                              M, stream));
}

csa2_status csa2_index_select_pool(const float* M, int64_t m_stride_, const int64_t* ctx,
                                   int32_t B, int64_t max_ctx, int32_t n_blocks, int32_t* pool,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!M || !ctx || !pool || B < 0 || max_ctx < 0) return CSA2_ERR_INVALID_ARG;
    if (B > 65535 || n_blocks < 1 || n_blocks > CSA2_MAX_POOL) return CSA2_ERR_UNSUPPORTED;
    if (m_stride_ < (max_ctx + BLOCK - 1) / BLOCK) return CSA2_ERR_INVALID_ARG;
    // rows are read as float4: 16-byte aligned rows
    if ((reinterpret_cast<uintptr_t>(M) & 15) || (m_stride_ & 3)) return CSA2_ERR_INVALID_ARG;
    if (B == 0) return CSA2_OK;
    const size_t need = select_bytes(B, (max_ctx + BLOCK - 1) / BLOCK);
    if (need && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
    return launched(csa2::launch_topk(M, m_stride_, ctx, max_ctx, 0, nullptr, 0, B, n_blocks,
                                      pool, ws, stream));
}

csa2_status csa2_index_reindex(const csa2_cache* cache, const float* q_idx, const float* w,
                               const int32_t* seq, const int64_t* ctx, int32_t B,
                               const int32_t* pool, int32_t n_blocks, int32_t block,
                               int32_t topk, int32_t* idx, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
    csa2_status st = check_cache(cache, false, true);
    if (st != CSA2_OK) return st;
    if (!q_idx || !w || !seq || !ctx || !pool || !idx) return CSA2_ERR_INVALID_ARG;
    st = check_select(B, n_blocks, block, topk);
    if (st != CSA2_OK) return st;
    if (B == 0) return CSA2_OK;
    if (!ws || ws_bytes < reindex_bytes(B, n_blocks)) return CSA2_ERR_WORKSPACE;
    float* S = static_cast<float*>(ws);
    void* sel = static_cast<char*>(ws) +
                align_up((size_t)B * (size_t)n_blocks * BLOCK * sizeof(float));
    hipError_t e = csa2::launch_score_pool(*cache, q_idx, w, seq, ctx, B, pool, n_blocks, S,
                                           stream);
    if (e != hipSuccess) return CSA2_ERR_LAUNCH;
    return launched(csa2::launch_topk(S, (int64_t)n_blocks * BLOCK, nullptr, 0,
                                      n_blocks * BLOCK, pool, n_blocks, B, topk, idx, sel,
                                      stream));
}

csa2_status csa2_decode_attn_ex(const csa2_cache* cache, const csa2_window* win, int32_t layer,
                                const float* q, const int32_t* idx, const int32_t* seq,
                                const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                                const uint8_t* kvg_in, uint8_t* kvg_out, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    csa2_status st = check_cache(cache, true, false);
    if (st != CSA2_OK) return st;
    st = check_window(win, cache);
    if (st != CSA2_OK) return st;
    if (!q || !idx || !seq || !ctx || !out) return CSA2_ERR_INVALID_ARG;
    if (kvg_in && kvg_out) return CSA2_ERR_INVALID_ARG;
    if (layer < 0 || layer >= win->n_layers || B < 0 || !isfinite(sm_scale))
        return CSA2_ERR_INVALID_ARG;
    if (topk < 1 || topk > CSA2_MAX_TOPK || B > 65535) return CSA2_ERR_UNSUPPORTED;
    if (B == 0) return CSA2_OK;
    const size_t need = attn_bytes(B, topk);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
    return launched(csa2::launch_attn(*cache, *win, layer, q, idx, seq, ctx, B, topk, sm_scale,
                                      kvg_in, kvg_out, out, static_cast<float*>(ws),
                                      csa2::ATTN_NO_CAP, stream));
}

csa2_status csa2_decode_attn_noalloc(const csa2_cache* cache, const csa2_window* win,
                                     int32_t layer, const float* q, const int32_t* idx,
                                     const int32_t* seq, const int64_t* ctx, int32_t B,
                                     int32_t topk, float sm_scale, const uint8_t* kvg_in,
                                     uint8_t* kvg_out, float* out, hipStream_t stream) {
    csa2_status st = check_cache(cache, true, false);
    if (st != CSA2_OK) return st;
    st = check_window(win, cache);
    if (st != CSA2_OK) return st;
    if (!q || !idx || !seq || !ctx || !out) return CSA2_ERR_INVALID_ARG;
    if (kvg_in && kvg_out) return CSA2_ERR_INVALID_ARG;
    if (layer < 0 || layer >= win->n_layers || B < 0 || !isfinite(sm_scale))
        return CSA2_ERR_INVALID_ARG;
    if (topk < 1 || topk > CSA2_MAX_TOPK || B > 65535) return CSA2_ERR_UNSUPPORTED;
    if (B == 0) return CSA2_OK;
    // the launch plan is capped to the scratch; a plan past it is refused
    const int64_t parts = csa2::attn_partials(B, topk, NOALLOC_MAX_PARTS);
    if (parts > NOALLOC_MAX_PARTS) return CSA2_ERR_WORKSPACE;
    float* part = nullptr;
    if (parts > 0) {
        part = device_scratch();
        if (!part) return CSA2_ERR_LAUNCH;
    }
    return launched(csa2::launch_attn(*cache, *win, layer, q, idx, seq, ctx, B, topk, sm_scale,
                                      kvg_in, kvg_out, out, part, NOALLOC_MAX_PARTS, stream));
}

csa2_status csa2_reindex_layer_fused(const csa2_cache* cache, const csa2_window* win,
                                     int32_t layer, const float* q_idx, const float* w,
                                     const float* q, const int32_t* seq, const int64_t* ctx,
                                     int32_t B, const int32_t* pool, int32_t n_blocks,
                                     int32_t block, int32_t topk, float sm_scale, int32_t* idx,
                                     uint8_t* kvg_out, float* out, int32_t max_polls,
                                     int32_t* status, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    csa2_status st = check_cache(cache, true, true);
    if (st != CSA2_OK) return st;
    st = check_window(win, cache);
    if (st != CSA2_OK) return st;
    if (!q_idx || !w || !q || !seq || !ctx || !pool || !idx || !out || !status)
        return CSA2_ERR_INVALID_ARG;
    if (layer < 0 || layer >= win->n_layers || !isfinite(sm_scale)) return CSA2_ERR_INVALID_ARG;
    st = check_select(B, n_blocks, block, topk);
    if (st != CSA2_OK) return st;
    if ((int64_t)B * layer_tiles(topk) > csa2::ATTN_MIN_CAP) return CSA2_ERR_UNSUPPORTED;
    if (B == 0) return CSA2_OK;
    const LayerLayout L = layer_layout(B, n_blocks, topk);
    if (!ws || ws_bytes < L.total) return CSA2_ERR_WORKSPACE;
    // every workgroup of the launch must be resident at once
    if (!csa2::reindex_layer_fits(*cache, B, n_blocks, topk)) return CSA2_ERR_UNSUPPORTED;
    char* base = static_cast<char*>(ws);
    return launched(csa2::launch_reindex_layer(
        *cache, *win, layer, q_idx, w, q, seq, ctx, B, pool, n_blocks, topk, sm_scale, idx,
        kvg_out, out, max_polls, status, reinterpret_cast<csa2::LayerSync*>(base),
        reinterpret_cast<float*>(base + L.s_off), reinterpret_cast<float*>(base + L.part_off),
        stream));
}

csa2_status csa2_decode_attn(const csa2_cache* cache, const csa2_window* win, int32_t layer,
                             const float* q, const int32_t* idx, const int32_t* seq,
                             const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                             float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    return csa2_decode_attn_ex(cache, win, layer, q, idx, seq, ctx, B, topk, sm_scale, nullptr,
                               nullptr, out, ws, ws_bytes, stream);
}

}  // extern "C"
