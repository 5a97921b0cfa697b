// Host-side launchers behind the C ABI (internal to libcsa2).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa2.h"
#include "csa2_device.h"

namespace csa2 {

// Device-side view of a cache descriptor's page table (unused when the cache
// is contiguous; the descriptor has been validated by the caller).
inline PageMap page_map(const csa2_cache& c) {
    PageMap m{};
    if (c.page_table) {
        m.table = c.page_table;
        m.shift = 0;
        while ((1 << m.shift) < c.page_tokens) ++m.shift;
        m.per_seq = c.cap >> m.shift;
        m.n_pages = c.n_pages;
    }
    return m;
}

// Quantise-on-write of n rows into the cache (and window stores); with m = 2
// each pair of rows becomes one global entry from their fp32 mean (n even).
hipError_t launch_quantize(const csa2_cache& c, const csa2_window* w, const float* k,
                           const float* v, const float* idx_k, const float* win_k,
                           const float* win_v, const int32_t* seq, const int64_t* pos,
                           int64_t n, int32_t m, hipStream_t stream);

// Full-context scoring: block maxima M[b][j] for blocks j < ceil(ctx[b]/8).
hipError_t launch_score_blocks(const csa2_cache& c, const float* q_idx, const float* w,
                               const int32_t* seq, const int64_t* ctx, int32_t B,
                               int64_t max_ctx, int64_t m_stride, float* M,
                               hipStream_t stream);

// Pool scoring: S[b][i] = score of position pool[b][i/8]*8 + i%8, or -inf when
// the pool slot is -1 or the position is >= ctx[b].
hipError_t launch_score_pool(const csa2_cache& c, const float* q_idx, const float* w,
                             const int32_t* seq, const int64_t* ctx, int32_t B,
                             const int32_t* pool, int32_t n_blocks, float* S,
                             hipStream_t stream);

// Top-k select per row, ties to the lower index, output ascending, -1 padded.
// Row b has n = ceil(ctx[b]/8) entries (ctx != null, block mode) or n_fixed
// entries (pool mode); -inf entries are absent.  With pool != null an entry i
// is reported as pool[b][i/8]*8 + i%8, else as i.  ws must hold
// topk_workspace_bytes(B, longest row) bytes (may be null when that is 0).
hipError_t launch_topk(const float* vals, int64_t stride, const int64_t* ctx,
                       int64_t max_ctx, int32_t n_fixed, const int32_t* pool,
                       int32_t n_blocks, int32_t B, int32_t k, int32_t* out, void* ws,
                       hipStream_t stream);
size_t topk_workspace_bytes(int32_t B, int64_t max_n);

// Split-K gather/dequant attention for one layer plus the cross-split merge.
// kvg_in (optional): main records read from [B][topk][RECORD] instead of the
// cache; kvg_out (optional): the main records read are also stored there.
// The launch plan writes at most max_parts partial records (ATTN_NO_CAP: the
// plan's own choice; a cap must be at least ATTN_MIN_CAP).
hipError_t launch_attn(const csa2_cache& c, const csa2_window& w, int32_t layer,
                       const float* q, const int32_t* idx, const int32_t* seq,
                       const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                       const uint8_t* kvg_in, uint8_t* kvg_out, float* out, float* partials,
                       int64_t max_parts, hipStream_t stream);

// Partial records an attention call writes (0 when no query is split).
int64_t attn_partials(int32_t B, int32_t topk, int64_t max_parts);
constexpr size_t ATTN_PART_FLOATS = 16 + 16 + 16 * 128;
constexpr int64_t ATTN_NO_CAP = INT64_MAX;
constexpr int64_t ATTN_MIN_CAP = 768;   // the tile kernel's largest grid

// Barrier words of the fused Reindex layer (zero-filled once before first use),
// each on a 128-byte line of its own: arrivals at the current grid barrier (0
// between barriers) and the barriers completed.
struct LayerSync {
    struct alignas(128) Word {
        uint32_t v;
    };
    Word count;
    Word gen;
};

// One Reindex layer (pool scores, top-k, attention tiles, merge) in one
// cooperative launch; scores holds [B][n_blocks * 8] floats, partials
// [B][tiles][ATTN_PART_FLOATS].  Bit-identical to launch_score_pool +
// launch_topk + launch_attn whenever launch_attn takes its tile path.
hipError_t launch_reindex_layer(const csa2_cache& c, const csa2_window& w, int32_t layer,
                                const float* q_idx, const float* wts, const float* q,
                                const int32_t* seq, const int64_t* ctx, int32_t B,
                                const int32_t* pool, int32_t n_blocks, int32_t topk,
                                float sm_scale, int32_t* idx, uint8_t* kvg_out, float* out,
                                int32_t max_polls, int32_t* status, LayerSync* sync,
                                float* scores, float* partials, hipStream_t stream);
// Whether that launch's grid (one round of every stage) can be resident on the
// current device.
bool reindex_layer_fits(const csa2_cache& c, int32_t B, int32_t n_blocks, int32_t topk);

}  // namespace csa2
