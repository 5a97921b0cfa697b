/* Host-side argument validation of every libcsa2 entry point, for the host
 * sanitizer build: each call below is rejected (or has no work) before any
 * kernel launch, so no GPU is needed.  Exit status 0 and no sanitizer report
 * are the pass condition; a wrong status exits with the failing line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "csa2.h"

#define EXPECT(call, want)                                                          \
    do {                                                                            \
        csa2_status got_ = (call);                                                  \
        if (got_ != (want)) {                                                       \
            printf("line %d: status %d, expected %d\n", __LINE__, (int)got_, (int)(want)); \
            return 1;                                                               \
        }                                                                           \
    } while (0)

int main(void) {
    /* never dereferenced on these paths: stand-in device addresses */
    uint8_t* fake = (uint8_t*)(uintptr_t)0x1000;
    float* ff = (float*)(uintptr_t)0x2000;
    int32_t* fi = (int32_t*)(uintptr_t)0x3000;
    int64_t* fl = (int64_t*)(uintptr_t)0x4000;
    char ws_host[64];
    void* ws = ws_host;
    csa2_cache c;
    memset(&c, 0, sizeof c);
    c.kv = fake; c.idxk = fake; c.idxk_scale = 1.0f; c.n_seq = 4; c.cap = 1 << 20;
    csa2_window w;
    memset(&w, 0, sizeof w);
    w.k = fake; w.v = fake; w.k_scale = 1.0f; w.v_scale = 1.0f; w.n_layers = 20; w.n_seq = 4;
    w.w_cap = 128;

    /* quantize */
    EXPECT(csa2_quantize_kv(NULL, NULL, ff, ff, NULL, NULL, NULL, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_quantize_kv(&c, NULL, NULL, ff, NULL, NULL, NULL, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_quantize_kv(&c, NULL, ff, ff, NULL, ff, NULL, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_quantize_kv(&c, NULL, ff, ff, NULL, ff, ff, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_quantize_kv(&c, NULL, ff, ff, NULL, NULL, NULL, fi, fl, -1, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_quantize_kv(&c, NULL, ff, ff, NULL, NULL, NULL, fi, fl, 0, NULL), CSA2_OK);
    EXPECT(csa2_quantize_kv(&c, &w, ff, ff, ff, ff, ff, fi, fl, 0, NULL), CSA2_OK);
    /* compression: m in {1, 2}, n a multiple of m, window-only calls */
    EXPECT(csa2_compress_kv(&c, NULL, ff, ff, NULL, NULL, NULL, fi, fl, 4, 3, NULL), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_compress_kv(&c, NULL, ff, ff, NULL, NULL, NULL, fi, fl, 5, 2, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_compress_kv(&c, NULL, NULL, ff, NULL, NULL, NULL, fi, fl, 4, 2, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_compress_kv(&c, NULL, NULL, NULL, NULL, NULL, NULL, fi, fl, 4, 2, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_compress_kv(&c, &w, NULL, NULL, ff, ff, ff, fi, fl, 4, 2, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_compress_kv(&c, &w, NULL, NULL, NULL, ff, ff, fi, fl, 0, 2, NULL), CSA2_OK);
    EXPECT(csa2_compress_kv(&c, NULL, ff, ff, ff, NULL, NULL, fi, fl, 0, 1, NULL), CSA2_OK);
    {
        csa2_cache bad = c;
        bad.idxk_scale = 0.0f;
        EXPECT(csa2_quantize_kv(&bad, NULL, ff, ff, ff, NULL, NULL, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
        bad = c;
        bad.page_table = fi; bad.page_tokens = 100; bad.n_pages = 4;
        EXPECT(csa2_quantize_kv(&bad, NULL, ff, ff, NULL, NULL, NULL, fi, fl, 1, NULL), CSA2_ERR_UNSUPPORTED);
        bad.page_tokens = 256; bad.cap = 1000;
        EXPECT(csa2_quantize_kv(&bad, NULL, ff, ff, NULL, NULL, NULL, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
        csa2_window bw = w;
        bw.w_cap = 64;
        EXPECT(csa2_quantize_kv(&c, &bw, ff, ff, NULL, ff, ff, fi, fl, 1, NULL), CSA2_ERR_UNSUPPORTED);
        bw = w; bw.n_seq = 3;
        EXPECT(csa2_quantize_kv(&c, &bw, ff, ff, NULL, ff, ff, fi, fl, 1, NULL), CSA2_ERR_INVALID_ARG);
    }

    /* Full indexer */
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, 4, 1 << 20, 2048, 8, 512, fi, fi, ws, 64, NULL), CSA2_ERR_WORKSPACE);
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, 4, 1 << 20, 2048, 4, 512, fi, fi, ws, 64, NULL), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, 4, 1 << 20, 5000, 8, 512, fi, fi, ws, 64, NULL), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, 4, 1 << 20, 16, 8, 512, fi, fi, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, 4, (1 << 20) + 1, 2048, 8, 512, fi, fi, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_full(&c, NULL, ff, fi, fl, 4, 1 << 20, 2048, 8, 512, fi, fi, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, -1, 1 << 20, 2048, 8, 512, fi, fi, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_full(&c, ff, ff, fi, fl, 0, 1 << 20, 2048, 8, 512, fi, fi, NULL, 0, NULL), CSA2_OK);
    EXPECT(csa2_index_block_scores(&c, ff, ff, fi, fl, 4, 1 << 20, ff, 10, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_block_scores(&c, ff, ff, fi, fl, 4, 0, ff, 0, NULL), CSA2_OK);
    EXPECT(csa2_index_select_pool(ff, 131072, fl, 4, 1 << 20, 2048, fi, NULL, 0, NULL), CSA2_ERR_WORKSPACE);
    EXPECT(csa2_index_select_pool((float*)(uintptr_t)0x2004, 131072, fl, 4, 1 << 20, 2048, fi, ws, 1u << 30, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_select_pool(ff, 131072, fl, 0, 1 << 20, 2048, fi, NULL, 0, NULL), CSA2_OK);

    /* Reindex */
    EXPECT(csa2_index_reindex(&c, ff, ff, fi, fl, 4, fi, 2048, 8, 512, fi, ws, 64, NULL), CSA2_ERR_WORKSPACE);
    EXPECT(csa2_index_reindex(&c, ff, ff, fi, fl, 4, NULL, 2048, 8, 512, fi, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_index_reindex(&c, ff, ff, fi, fl, 4, fi, 2048, 8, 0, fi, ws, 64, NULL), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_index_reindex(&c, ff, ff, fi, fl, 0, fi, 2048, 8, 512, fi, NULL, 0, NULL), CSA2_OK);

    /* attention */
    EXPECT(csa2_decode_attn(&c, &w, 0, ff, fi, fi, fl, 4, 512, 0.088f, ff, ws, 64, NULL), CSA2_ERR_WORKSPACE);
    EXPECT(csa2_decode_attn(&c, &w, 20, ff, fi, fi, fl, 4, 512, 0.088f, ff, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_decode_attn(&c, &w, -1, ff, fi, fi, fl, 4, 512, 0.088f, ff, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_decode_attn(&c, &w, 0, ff, fi, fi, fl, 4, 4096, 0.088f, ff, ws, 64, NULL), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_decode_attn(&c, NULL, 0, ff, fi, fi, fl, 4, 512, 0.088f, ff, ws, 64, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_decode_attn(&c, &w, 0, ff, fi, fi, fl, 0, 512, 0.088f, ff, NULL, 0, NULL), CSA2_OK);
    EXPECT(csa2_decode_attn_ex(&c, &w, 0, ff, fi, fi, fl, 4, 512, 0.088f, fake, fake, ff, ws, 1u << 30, NULL), CSA2_ERR_INVALID_ARG);
    {
        csa2_window bw = w;
        bw.v_scale = -1.0f;
        EXPECT(csa2_decode_attn(&c, &bw, 0, ff, fi, fi, fl, 4, 512, 0.088f, ff, ws, 1u << 30, NULL), CSA2_ERR_INVALID_ARG);
    }

    /* the no-allocation attention call: argument errors and an empty batch
       (none of them touches the library's scratch) */
    EXPECT(csa2_decode_attn_noalloc(&c, &w, 0, ff, fi, fi, fl, 0, 512, 0.088f, NULL, NULL, ff, NULL), CSA2_OK);
    EXPECT(csa2_decode_attn_noalloc(&c, &w, 0, ff, fi, fi, fl, 4, 512, 0.088f, fake, fake, ff, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_decode_attn_noalloc(&c, &w, 0, ff, fi, fi, fl, 4, 4096, 0.088f, NULL, NULL, ff, NULL), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_decode_attn_noalloc(&c, &w, 20, ff, fi, fi, fl, 4, 512, 0.088f, NULL, NULL, ff, NULL), CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_decode_attn_noalloc(&c, NULL, 0, ff, fi, fi, fl, 4, 512, 0.088f, NULL, NULL, ff, NULL), CSA2_ERR_INVALID_ARG);

    /* sizes and strings over a range of shapes */
    size_t total = 0;
    for (int32_t op = 0; op <= 5; ++op)
        for (int32_t b = -1; b < 70000; b = b < 8 ? b + 1 : b * 3)
            for (int64_t ctx = -1; ctx < ((int64_t)1 << 34); ctx = ctx < 2 ? ctx + 1 : ctx * 7)
                for (int32_t topk = 0; topk <= 5000; topk += 1250)
                    total += csa2_workspace_bytes(op, b, ctx, topk < 4100 ? 2048 : 4097, 8,
                                                  topk);
    for (int s = -1; s < 8; ++s) total += strlen(csa2_status_string((csa2_status)s));
    printf("abi driver ok %zu\n", total);
    return 0;
}
