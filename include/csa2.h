/*
 * csa2.h - C ABI of libcsa2, CSA2 decode attention over a compressed global
 * KV cache on AMD MI355X (gfx950).
 *
 * What the calls compute comes from these pages (news summaries of the
 * DeepSeek-V4.1-Flash technical report):
 *  [P1] trawling.dev, "DeepSeek-V4.1-Flash released - a 552B multimodal MoE that
 *       cuts the KV cache to 890 bytes per token", section "CSA2 and FP4 KV caching".
 *  [P3] cursorai.co.kr, "DeepSeek-V4.1-Flash: how an 890-byte KV cache changes
 *       agent infrastructure", section 3, step 3 "FP4 KV cache quantisation".
 *  [P4] origotech.dev, "Inside DeepSeek V4.1-Flash: KV cache, the 1017 update and
 *       the Harness stack", section "How the architecture shrinks the KV cache"
 *       and its sub-section "FP4 and SWA Bounded Replay".
 *  [P5] ttj.kr, "DeepSeek-V4.1-Flash compresses the KV cache to 890 bytes per
 *       token", section "CSA2 and the attention redesign".
 *
 * Conventions shared by every call
 *  - Every array argument is a DEVICE pointer allocated by the caller; the
 *    descriptor structs themselves are host memory read during the call.
 *  - The library allocates nothing, frees nothing, never synchronises and keeps
 *    no global state (except the fixed per-GPU scratch array of
 *    csa2_decode_attn_noalloc, below): each call validates its arguments on the
 *    host, enqueues kernels on `stream` and returns.  Calls are reentrant; calls on different
 *    streams must not share a workspace.
 *  - Argument errors are reported synchronously through the return value and
 *    enqueue nothing.  Launch errors return CSA2_ERR_LAUNCH.  Device-side
 *    faults surface at the caller's next synchronisation.
 *  - Per-query arrays seq[] and ctx[] live on the device.  seq[b] names the
 *    cache sequence query b reads; ctx[b] = N is the number of visible
 *    positions 0..N-1 (the current token included).  Kernels clamp values
 *    outside [0, n_seq) / [0, max_ctx] so that no access leaves the buffers;
 *    results for such queries are unspecified.
 *  - Inputs must be finite.  Index outputs are ascending and padded with -1.
 *
 * Data layout in HBM (the cache descriptor)
 *  - kv   [n_seq][cap][144] bytes (paged: [n_pages][page_tokens][144], below),
 *         one record per token:
 *         [0,64)   K codes, FP4 E2M1, channel 2j in the low nibble of byte j,
 *                  channel 2j+1 in the high nibble;
 *         [64,128) V codes, same packing;
 *         [128,136) 8 K scales, E4M3FN, scale g covers channels 16g..16g+15;
 *         [136,144) 8 V scales.
 *    (FP4 E2M1 main KV with one E4M3 scale per 16 channels, quantised after
 *    RoPE: [P1] "CSA2 and FP4 KV caching", [P4] "FP4 and SWA Bounded Replay";
 *    0.5 byte per element: [P3] section 3 step 3.)
 *  - idxk [n_seq][cap][64] bytes (paged: [n_pages][page_tokens][64]), E4M3FN
 *    indexer keys; key value = code value times idxk_scale.  Main KV and
 *    indexer keys are shared by every layer of the decoder ([P1] "CSA2 and FP4
 *    KV caching"; [P4] mode list).
 *  - Paged caches.  The global store is the long-lived part of the cache: it is
 *    kept while the sliding-window KV is not persisted and is rebuilt by
 *    replaying the last 128 tokens ([P4] "FP4 and SWA Bounded Replay").  A
 *    serving layer therefore allocates it in pages.  With a page table, the
 *    record and indexer key of position t of sequence s live in row
 *    t % page_tokens of physical page page_table[s][t / page_tokens] of kv and
 *    idxk.  page_tokens is a power of two in [64, 65536] (a 64-key scan step
 *    never straddles two pages), cap is a multiple of it, and the table is
 *    [n_seq][cap / page_tokens] int32 on the device.  Entries of pages that
 *    hold no visible position are never used for data and may be -1; any entry
 *    outside [0, n_pages) is clamped into it, so that no access leaves kv/idxk.
 *    Results are bit-identical to a contiguous cache holding the same bytes.
 *  - window k/v [n_layers][n_seq][w_cap][128] bytes, E4M3FN, one store per
 *    layer; position u lives in slot u % w_cap; value = code times k_scale /
 *    v_scale.  (FP8 sliding-window KV: [P4] "FP4 and SWA Bounded Replay";
 *    size 128: [P4], [P5] "CSA2 and the attention redesign".)
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed shapes. */
#define CSA2_D 128          /* K / V channels of the single shared KV head */
#define CSA2_HEADS 16       /* attention query heads */
#define CSA2_IDX_HEADS 4    /* indexer heads */
#define CSA2_IDX_DIM 64     /* indexer dims */
#define CSA2_WINDOW 128     /* sliding-window tokens ([P4], [P5]) */
#define CSA2_RECORD 144     /* bytes per FP4 K+V record */
#define CSA2_BLOCK 8        /* positions per indexer block ([P4]) */
#define CSA2_MAX_TOPK 2048  /* largest supported topk */
#define CSA2_MAX_POOL 4096  /* largest supported n_blocks */

typedef enum csa2_status {
    CSA2_OK = 0,
    CSA2_ERR_INVALID_ARG = 1,  /* null pointer, negative size, out-of-range value,
                                  cap not a multiple of page_tokens */
    CSA2_ERR_UNSUPPORTED = 2,  /* a size the library does not implement
                                  (including page_tokens) */
    CSA2_ERR_WORKSPACE = 3,    /* ws null or ws_bytes below csa2_workspace_bytes */
    CSA2_ERR_LAUNCH = 4        /* a kernel launch failed (hipGetLastError) */
} csa2_status;

/* The shared compressed store: main-KV records and indexer keys.  A zeroed
 * tail (page_table NULL) describes a contiguous cache. */
typedef struct csa2_cache {
    uint8_t* kv;        /* device [n_seq][cap][144], or [n_pages][page_tokens][144] */
    uint8_t* idxk;      /* device [n_seq][cap][64],  or [n_pages][page_tokens][64]  */
    float idxk_scale;   /* per-tensor scale of the indexer keys (positive, normal) */
    int32_t n_seq;
    int64_t cap;        /* positions per sequence */
    const int32_t* page_table;  /* NULL, or device [n_seq][cap / page_tokens] page ids */
    int32_t page_tokens;        /* paged only: tokens per page, power of two in [64, 65536] */
    int32_t n_pages;            /* paged only: physical pages behind kv and idxk (> 0) */
} csa2_cache;

/* Per-layer FP8 sliding-window stores, all layers in one allocation. */
typedef struct csa2_window {
    uint8_t* k;         /* device [n_layers][n_seq][w_cap][128] */
    uint8_t* v;         /* device, same shape */
    float k_scale;      /* per-tensor scales (positive, normal floats) */
    float v_scale;
    int32_t n_layers;
    int32_t n_seq;      /* must equal the cache's n_seq */
    int32_t w_cap;      /* slots per sequence, >= 128 */
} csa2_window;

/* Operation ids for csa2_workspace_bytes. */
enum {
    CSA2_OP_INDEX_FULL = 1,
    CSA2_OP_INDEX_REINDEX = 2,
    CSA2_OP_DECODE_ATTN = 3,
    CSA2_OP_SELECT_POOL = 4,
    CSA2_OP_REINDEX_LAYER_FUSED = 5
};

/*
 * csa2_quantize_kv - quantise-on-write of n new tokens.
 * Passage: main KV stored as FP4 E2M1 with one E4M3 scale per 16 channels,
 * quantised after RoPE; sliding-window KV kept in FP8 ([P4] "FP4 and SWA
 * Bounded Replay"; [P1] "CSA2 and FP4 KV caching").
 *   k, v      [n][128] fp32, post-RoPE main K and V rows -> record at
 *             kv[seq[i]][pos[i]] (for a paged cache, the row the page table
 *             gives for that position).  Per 16-channel group: scale code =
 *             E4M3(fp32(amax)/6) rounded to nearest even and saturated at 448;
 *             each nibble = nearest E2M1 value of x/scale (ties to even,
 *             saturating at 6, sign of x kept); a zero scale gives zero codes.
 *   idx_k     [n][64] fp32 or NULL -> idxk[seq[i]][pos[i]] = E4M3(x/idxk_scale).
 *   win_k/v   [win->n_layers][n][128] fp32 or NULL (both or neither) -> slot
 *             pos[i] % w_cap of every layer's window store, E4M3(x/scale).
 *   win       may be NULL when win_k/win_v are NULL.
 *   seq, pos  [n] device; pos must lie in [0, cap).  Rows with seq or pos out of
 *             range are skipped.  A paged cache must own a page for every pos
 *             written (an entry outside [0, n_pages) is clamped, so the row
 *             lands in some other page).  Rows are written in parallel: duplicate
 *             (seq, pos) pairs, or window rows of one call that share a slot
 *             (same seq, equal pos % w_cap), race.
 */
csa2_status csa2_quantize_kv(const csa2_cache* cache, const csa2_window* win,
                             const float* k, const float* v, const float* idx_k,
                             const float* win_k, const float* win_v, const int32_t* seq,
                             const int64_t* pos, int64_t n, hipStream_t stream);

/*
 * csa2_compress_kv - quantise-on-write at global-KV compression m.
 * Passage: the encoder's CSA2 layers run at compression m = 2, the decoder's at
 * m = 1 ([P4] "How the architecture shrinks the KV cache").  The pages give the
 * ratio, not the operator; this library's reading: global entry e of a
 * sequence stands for its m tokens at positions m*e .. m*e + m - 1, and its K,
 * V and indexer-key rows are those tokens' rows averaged in fp32 ((r0 + r1) *
 * 0.5 for m = 2: one rounding of the sum, an exact halving), then quantised as
 * csa2_quantize_kv quantises a token row.  The window keeps every token.  A
 * query with N tokens of context then sees entries [0, N / m) (complete groups)
 * and window rows [N - 128, N): pass ctx / m to the indexer calls and ctx to
 * csa2_decode_attn.
 *   m         1 or 2 (else CSA2_ERR_UNSUPPORTED); with k given, n must be a
 *             multiple of m (else CSA2_ERR_INVALID_ARG).  m = 1 is exactly
 *             csa2_quantize_kv.
 *   k, v, idx_k  [n][128] / [n][64] fp32 token rows; rows i*m .. i*m + m - 1
 *             form group i, written as entry pos[i*m] / m of sequence seq[i*m]
 *             (record and indexer key; the cache's cap counts entries).  The
 *             caller passes each group's tokens in position order, the first at
 *             a multiple of m; a group whose first position is not a multiple
 *             of m is skipped, and the other rows' seq and pos are not read.
 *             k and v both NULL (idx_k NULL, win_k given): window rows only, n
 *             any -- for tokens whose group is not complete yet.
 *   win_k/v   as for csa2_quantize_kv, one row per token at slot pos[i] % w_cap;
 *             token positions lie in [0, m * cap).
 *   Other arguments, errors and races as for csa2_quantize_kv.
 */
csa2_status csa2_compress_kv(const csa2_cache* cache, const csa2_window* win,
                             const float* k, const float* v, const float* idx_k,
                             const float* win_k, const float* win_v, const int32_t* seq,
                             const int64_t* pos, int64_t n, int32_t m, hipStream_t stream);

/*
 * csa2_index_full - Full-mode indexer: score, block pool, top-k.
 * Passage: a Full layer computes its own indexer query and a fresh top-k; the
 * first Full layer selects 2,048 blocks of 8 positions (a 16,384-position pool)
 * and top-k is 512 ([P4] "How the architecture shrinks the KV cache"; [P1]
 * "CSA2 and FP4 KV caching").  Score function and block score are this
 * library's reading: score_t = sum_h w_h * max(0, q_h . khat_t), khat = key
 * code value * idxk_scale; block score = max over the block's positions < N.
 *   q_idx     [B][4][64] fp32, w [B][4] fp32.
 *   max_ctx   host bound with ctx[b] <= max_ctx <= cap for all b (sizes grids).
 *   n_blocks  pool size in blocks, 1..4096 (2048 in the pages); block must be 8.
 *             The top-k positions always lie in the topk best blocks, so a Full
 *             layer whose pool no Reindex layer reads may pass n_blocks = topk
 *             and get the same idx for a quarter of the pool scoring.
 *   topk      1..2048 and <= n_blocks*8 (512 in the pages).
 *   pool      [B][n_blocks] int32 out, or NULL: the n_blocks largest block
 *             scores (ties to the lower block), ascending, -1 padded.
 *   idx       [B][topk] int32 out: the topk largest scores among the pool's
 *             positions < N (ties to the lower position), ascending, -1 padded.
 *   ws        device workspace of at least
 *             csa2_workspace_bytes(CSA2_OP_INDEX_FULL, B, max_ctx, n_blocks, 8, topk).
 */
csa2_status csa2_index_full(const csa2_cache* cache, const float* q_idx, const float* w,
                            const int32_t* seq, const int64_t* ctx, int32_t B,
                            int64_t max_ctx, int32_t n_blocks, int32_t block, int32_t topk,
                            int32_t* pool, int32_t* idx, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * csa2_index_reindex - Reindex-mode indexer over a given pool.
 * Passage: a Reindex layer reuses the previous layer's main KV and indexer keys,
 * has its own indexer query and recomputes top-k; only Reindex layers score the
 * first Full layer's pool ([P4] "How the architecture shrinks the KV cache";
 * [P1] "CSA2 and FP4 KV caching").
 *   pool      [B][n_blocks] int32 (as written by csa2_index_full), ascending,
 *             -1 entries ignored.  Positions >= ctx[b] are ignored.
 *   idx       [B][topk] int32 out, same ranking and padding rules as above.
 *   ws        at least csa2_workspace_bytes(CSA2_OP_INDEX_REINDEX, B, 0, n_blocks, 8, topk).
 */
csa2_status csa2_index_reindex(const csa2_cache* cache, const float* q_idx, const float* w,
                               const int32_t* seq, const int64_t* ctx, int32_t B,
                               const int32_t* pool, int32_t n_blocks, int32_t block,
                               int32_t topk, int32_t* idx, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * Stages of csa2_index_full, for callers that schedule (or time) them apart.
 * csa2_index_full(q, w) is exactly csa2_index_block_scores, then
 * csa2_index_select_pool, then csa2_index_reindex with the same q and w.
 *
 * csa2_index_block_scores - M[b][j] = max of score_t over block j's positions
 * t < N, for j < ceil(N/8); entries j >= ceil(N/8) are left untouched.
 *   M         [B][m_stride] fp32 out, m_stride >= ceil(max_ctx/8).
 */
csa2_status csa2_index_block_scores(const csa2_cache* cache, const float* q_idx, const float* w,
                                    const int32_t* seq, const int64_t* ctx, int32_t B,
                                    int64_t max_ctx, float* M, int64_t m_stride,
                                    hipStream_t stream);

/*
 * csa2_index_select_pool - pool[b] = the n_blocks largest of M[b][0..ceil(N/8))
 * (ties to the lower block), ascending, -1 padded.  n_blocks in 1..4096.  M must
 * be 16-byte aligned with m_stride a multiple of 4; -inf entries count as absent.
 *   ws        csa2_workspace_bytes(CSA2_OP_SELECT_POOL, B, max_ctx, n_blocks, 8, 1)
 *             bytes (zero for rows of up to 32,768 blocks; ws may then be NULL).
 */
csa2_status csa2_index_select_pool(const float* M, int64_t m_stride, const int64_t* ctx,
                                   int32_t B, int64_t max_ctx, int32_t n_blocks, int32_t* pool,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_decode_attn - gather, dequantise and attend for one layer.
 * Passage: attention reads the top-k selected global positions plus a local
 * 128-token sliding window ([P4] "How the architecture shrinks the KV cache";
 * [P5] "CSA2 and the attention redesign"); Reuse layers reuse main KV and top-k
 * indices (pass the same idx again).  Reading: one softmax per head over the
 * valid main rows idx[b][j] >= 0 and the window rows of positions
 * [max(0, N-128), N); logits (q_h . k) * sm_scale; no sink, no bias.
 *   layer     window layer in [0, win->n_layers).
 *   ctx       tokens of context N per query (the window rows are those of
 *             positions [N-128, N)); a main entry is valid below min(N, cap).
 *             For a store compressed m-fold (csa2_compress_kv) N is still the
 *             token count and the entries are at most N / m.
 *   q         [B][16][128] fp32, |q| < 65504.
 *   idx       [B][topk] int32 positions (< ctx[b]) or -1.
 *   out       [B][16][128] fp32.  A query with no valid entry gets zeros.
 *   ws        at least csa2_workspace_bytes(CSA2_OP_DECODE_ATTN, B, 0, 0, 0, topk)
 *             bytes: the split queries' partial results.  That is zero when no
 *             query is split (B >= 1024); ws may then be NULL.
 */
csa2_status csa2_decode_attn(const csa2_cache* cache, const csa2_window* win, int32_t layer,
                             const float* q, const int32_t* idx, const int32_t* seq,
                             const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                             float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_decode_attn_ex - csa2_decode_attn that keeps the gathered main KV for
 * the layers that reuse it.
 * Passage: Reuse layers take both the KV and the top-k indices of their group's
 * Full or Reindex layer ([P4] mode list; [P5] "CSA2 and the attention
 * redesign").  The main KV is shared by every layer, so the records gathered
 * for one layer of a group are the records of all its layers.
 *   kvg_out   NULL, or a [B][topk][144] device buffer: the call also stores the
 *             record it reads for entry j of query b (valid entries only) at
 *             kvg_out[b][j].  Other bytes are left untouched.
 *   kvg_in    NULL, or a buffer that a kvg_out call with the same cache, idx,
 *             seq, ctx, B and topk filled: main rows are read from kvg_in[b][j]
 *             (contiguous, at addresses that do not wait for idx) instead of
 *             the cache.  idx still decides which entries are valid.
 *   At most one of kvg_in / kvg_out may be non-NULL (else CSA2_ERR_INVALID_ARG);
 *   with both NULL this is csa2_decode_attn.  The other arguments and the
 *   results are those of csa2_decode_attn, bit for bit.
 */
csa2_status csa2_decode_attn_ex(const csa2_cache* cache, const csa2_window* win, int32_t layer,
                                const float* q, const int32_t* idx, const int32_t* seq,
                                const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                                const uint8_t* kvg_in, uint8_t* kvg_out, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * csa2_decode_attn_noalloc - csa2_decode_attn_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace and allocates
 * nothing: the split queries' partial records go to a fixed scratch array of
 * CSA2_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from
 * the first call on that GPU until the process ends (its device address is
 * looked up on that first call).  The launch plan is that of
 * csa2_decode_attn_ex, except that a large batch on the split streaming path
 * uses fewer splits when its partial records would not fit the scratch (down
 * to one workgroup per query, which writes none), so results agree with
 * csa2_decode_attn_ex within the attention tolerance and are bit-identical
 * whenever the plans agree.  Arguments, results and status codes are those of
 * csa2_decode_attn_ex without ws / ws_bytes; CSA2_ERR_WORKSPACE if a plan ever
 * needed more than the scratch, CSA2_ERR_LAUNCH if the scratch's address
 * cannot be obtained.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  Nothing in the scratch needs clearing between
 * calls (each call writes every partial record it reads).
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (8u << 20)
csa2_status csa2_decode_attn_noalloc(const csa2_cache* cache, const csa2_window* win,
                                     int32_t layer, const float* q, const int32_t* idx,
                                     const int32_t* seq, const int64_t* ctx, int32_t B,
                                     int32_t topk, float sm_scale, const uint8_t* kvg_in,
                                     uint8_t* kvg_out, float* out, hipStream_t stream);

/*
 * csa2_reindex_layer_fused - one Reindex layer in a single cooperative launch:
 * csa2_index_reindex(q_idx, w, pool -> idx) followed by
 * csa2_decode_attn_ex(q, idx, kvg_out -> out), with the layer's four stages
 * (pool scores, top-k, attention tiles, merge) separated by grid-wide barriers
 * inside one kernel instead of kernel boundaries.
 * Passage: a Reindex layer re-scores only its group's candidate pool with its
 * own indexer query over the shared indexer keys, re-selects the top-k
 * positions and attends over them plus its sliding window ([P4] "How the
 * architecture shrinks the KV cache"; [P5] "CSA2 and the attention redesign").
 *   Arguments as in csa2_index_reindex and csa2_decode_attn_ex (block must be
 *   8; kvg_out may be NULL).  idx, out and kvg_out are bit-identical to those
 *   two calls.  One ctx serves both stages, so the store is uncompressed
 *   (m = 1: Reindex layers are decoder layers).  B * (ceil(topk / 64) + 2) must not exceed 768 (the batches the
 *   separate attention call runs as 64-entry tiles; else CSA2_ERR_UNSUPPORTED).
 *   status    device int32: nothing is written when every barrier completes;
 *             a workgroup that polled a barrier max_polls times without seeing
 *             it complete ORs 1 into *status and goes on, and the results of
 *             that call are undefined.  The caller clears it.
 *   max_polls polls per barrier wait before giving up; <= 0 selects a default
 *             of about a second.
 *   ws        csa2_workspace_bytes(CSA2_OP_REINDEX_LAYER_FUSED, B, 0, n_blocks, 8,
 *             topk) bytes.  Its first 256 bytes hold the barrier words: they must
 *             be zero before the first call with this workspace (zero-fill it
 *             once) and every call leaves its count at zero, except a call that
 *             gave up, after which they must be zero-filled again.
 *   The kernel's workgroups must all be resident at once; the grid is capped at
 *   the device's resident limit (CSA2_ERR_LAUNCH if the cooperative launch is
 *   refused).  Calls sharing a workspace must not overlap.
 */
csa2_status csa2_reindex_layer_fused(const csa2_cache* cache, const csa2_window* win,
                                     int32_t layer, const float* q_idx, const float* w,
                                     const float* q, const int32_t* seq, const int64_t* ctx,
                                     int32_t B, const int32_t* pool, int32_t n_blocks,
                                     int32_t block, int32_t topk, float sm_scale, int32_t* idx,
                                     uint8_t* kvg_out, float* out, int32_t max_polls,
                                     int32_t* status, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* Workspace bytes an operation needs (0 for unknown op or invalid sizes). */
size_t csa2_workspace_bytes(int32_t op, int32_t B, int64_t max_ctx, int32_t n_blocks,
                            int32_t block, int32_t topk);

/* Static description of a status code. */
const char* csa2_status_string(csa2_status s);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
