/* Runs every oracle function once on small seeded inputs, for the host
 * sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer).  Inputs come
 * from a 64-bit LCG; nothing here computes what the method computes.  Exit
 * status 0 and no sanitizer report are the pass condition. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e2m1_value(uint8_t nib);
double oracle_e4m3_value(uint8_t c);
uint8_t oracle_e4m3_encode(float y);
void oracle_fp4_group(const float* x, uint8_t* nibbles, uint8_t* scale_code);
int oracle_record_bytes(void);
void oracle_quantize_kv(uint8_t* kv, uint8_t* idxk, float idxk_scale, int64_t cap,
                        int32_t n_seq, uint8_t* wk, uint8_t* wv, float wk_scale,
                        float wv_scale, int32_t w_cap, int32_t n_layers, const float* k,
                        const float* v, const float* idx_k, const float* win_k,
                        const float* win_v, const int32_t* seq, const int64_t* pos, int64_t n);
void oracle_compress_kv(uint8_t* kv, uint8_t* idxk, float idxk_scale, int64_t cap,
                        int32_t n_seq, uint8_t* wk, uint8_t* wv, float wk_scale,
                        float wv_scale, int32_t w_cap, int32_t n_layers, const float* k,
                        const float* v, const float* idx_k, const float* win_k,
                        const float* win_v, const int32_t* seq, const int64_t* pos, int64_t n,
                        int32_t m);
double oracle_index_score(const uint8_t* key, float scale, const float* q, const float* w);
int32_t oracle_topk(const double* val, const int64_t* ids, int64_t n, int32_t k, int32_t* out,
                    double* kth);
void oracle_score_range(const uint8_t* keys, float scale, const float* q, const float* w,
                        int64_t N, double* scores);
void oracle_index_full(const uint8_t* idxk, float scale, int64_t cap, const float* q_idx,
                       const float* w, const int32_t* seq, const int64_t* ctx, int32_t B,
                       int32_t n_blocks, int32_t block, int32_t topk, int32_t* pool,
                       int32_t* idx, double* kth_block, double* kth_pos);
void oracle_index_reindex(const uint8_t* idxk, float scale, int64_t cap, const float* q_idx,
                          const float* w, const int32_t* seq, const int64_t* ctx, int32_t B,
                          const int32_t* pool, int32_t n_blocks, int32_t block, int32_t topk,
                          int32_t* idx, double* kth_pos);
void oracle_decode_attn(const uint8_t* kv, int64_t cap, const uint8_t* wk, const uint8_t* wv,
                        float wk_scale, float wv_scale, int32_t w_cap, int32_t n_seq,
                        int32_t layer, const float* q, const int32_t* idx, const int32_t* seq,
                        const int64_t* ctx, int32_t B, int32_t topk, float sm_scale, float* out);

static uint64_t st = 0x9e3779b97f4a7c15ull;
static double unif(void) {   /* [0, 1) */
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(st >> 11) * (1.0 / 9007199254740992.0);
}
static float sym(double scale) { return (float)((2.0 * unif() - 1.0) * scale); }

static void* xcalloc(size_t n, size_t sz) {
    void* p = calloc(n ? n : 1, sz);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

int main(void) {
    enum { S = 2, CAP = 3000, L = 2, WCAP = 130, D = 128, DI = 64, B = 3 };
    int i, c;
    double acc = 0.0;
    for (c = 0; c < 16; ++c) acc += oracle_e2m1_value((uint8_t)c);
    for (c = 0; c < 256; ++c) {
        double v = oracle_e4m3_value((uint8_t)c);
        if (!isnan(v)) acc += v;
    }
    const float specials[] = {0.0f, -0.0f, 1e-30f, 448.0f, 464.0f, 1e30f, -1e30f, 0.001953125f};
    for (i = 0; i < 8; ++i) acc += oracle_e4m3_encode(specials[i]);
    for (i = 0; i < 1000; ++i) acc += oracle_e4m3_encode(sym(500.0));
    {
        float g[16];
        uint8_t nib[16], sc;
        for (i = 0; i < 200; ++i) {
            for (c = 0; c < 16; ++c) g[c] = sym(i % 7 == 0 ? 1e-6 : 30.0);
            oracle_fp4_group(g, nib, &sc);
            acc += sc + nib[i % 16];
        }
    }
    acc += oracle_record_bytes();

    /* quantise every position of two sequences, window rows for the last 200 */
    uint8_t* kv = xcalloc((size_t)S * CAP * 144, 1);
    uint8_t* idxk = xcalloc((size_t)S * CAP * DI, 1);
    uint8_t* wk = xcalloc((size_t)L * S * WCAP * D, 1);
    uint8_t* wv = xcalloc((size_t)L * S * WCAP * D, 1);
    const int64_t n = (int64_t)S * CAP;
    float* k = xcalloc((size_t)n * D, sizeof(float));
    float* v = xcalloc((size_t)n * D, sizeof(float));
    float* ik = xcalloc((size_t)n * DI, sizeof(float));
    int32_t* seq = xcalloc((size_t)n, sizeof(int32_t));
    int64_t* pos = xcalloc((size_t)n, sizeof(int64_t));
    for (i = 0; i < n; ++i) {
        seq[i] = (int32_t)(i / CAP);
        pos[i] = i % CAP;
        for (c = 0; c < D; ++c) { k[(size_t)i * D + c] = sym(3.0); v[(size_t)i * D + c] = sym(3.0); }
        for (c = 0; c < DI; ++c) ik[(size_t)i * DI + c] = sym(2.0);
    }
    oracle_quantize_kv(kv, idxk, 0.5f, CAP, S, NULL, NULL, 1.0f, 1.0f, WCAP, L, k, v, ik, NULL,
                       NULL, seq, pos, n);
    {
        const int64_t nw = 200;
        float* wkf = xcalloc((size_t)L * nw * D, sizeof(float));
        float* wvf = xcalloc((size_t)L * nw * D, sizeof(float));
        int32_t* ws = xcalloc((size_t)nw, sizeof(int32_t));
        int64_t* wp = xcalloc((size_t)nw, sizeof(int64_t));
        for (i = 0; i < L * nw * D; ++i) { wkf[i] = sym(4.0); wvf[i] = sym(4.0); }
        for (i = 0; i < nw; ++i) { ws[i] = (int32_t)(i % S); wp[i] = CAP - 1 - i / S; }
        oracle_quantize_kv(kv, NULL, 1.0f, CAP, S, wk, wv, 1.5f, 0.75f, WCAP, L, k, v, NULL,
                           wkf, wvf, ws, wp, nw);
        free(wkf); free(wvf); free(ws); free(wp);
    }
    {
        /* compression 2 into a store of CAP / 2 entries per sequence: the first
         * half of each sequence's tokens, a misaligned group, and window-only rows */
        const int64_t nc = CAP;                 /* tokens of sequence 0 and 1, CAP / 2 each */
        uint8_t* kv2 = xcalloc((size_t)S * (CAP / 2) * 144, 1);
        uint8_t* ik2 = xcalloc((size_t)S * (CAP / 2) * DI, 1);
        float* wkf = xcalloc((size_t)L * nc * D, sizeof(float));
        float* wvf = xcalloc((size_t)L * nc * D, sizeof(float));
        int32_t* cs = xcalloc((size_t)nc, sizeof(int32_t));
        int64_t* cp = xcalloc((size_t)nc, sizeof(int64_t));
        for (i = 0; i < L * nc * D; ++i) { wkf[i] = sym(4.0); wvf[i] = sym(4.0); }
        for (i = 0; i < nc; ++i) { cs[i] = (int32_t)(i / (nc / 2)); cp[i] = i % (nc / 2); }
        cp[2] = 3;                              /* group 1 starts at an odd position: skipped */
        oracle_compress_kv(kv2, ik2, 0.5f, CAP / 2, S, wk, wv, 1.5f, 0.75f, WCAP, L, k, v, ik,
                           wkf, wvf, cs, cp, nc, 2);
        oracle_compress_kv(kv2, NULL, 1.0f, CAP / 2, S, wk, wv, 1.5f, 0.75f, WCAP, L, NULL, NULL,
                           NULL, wkf, wvf, cs, cp, 7, 2);
        oracle_compress_kv(kv2, ik2, 0.5f, CAP / 2, S, NULL, NULL, 1.0f, 1.0f, WCAP, L, k, v, ik,
                           NULL, NULL, cs, cp, nc, 1);
        for (i = 0; i < S * (CAP / 2) * 144; ++i) acc += kv2[i];
        free(kv2); free(ik2); free(wkf); free(wvf); free(cs); free(cp);
    }

    /* indexer: scores, top-k, Full and Reindex with ragged contexts */
    float q[B * 4 * DI], w[B * 4];
    for (i = 0; i < B * 4 * DI; ++i) q[i] = sym(1.0);
    for (i = 0; i < B * 4; ++i) w[i] = (float)unif();
    acc += oracle_index_score(idxk, 0.5f, q, w);
    double* sc = xcalloc(CAP, sizeof(double));
    oracle_score_range(idxk, 0.5f, q, w, CAP, sc);
    int32_t tk[600];
    double kth;
    acc += oracle_topk(sc, NULL, CAP, 512, tk, &kth);
    acc += oracle_topk(sc, NULL, 7, 512, tk, &kth);
    acc += oracle_topk(sc, NULL, 0, 5, tk, &kth);
    const int32_t qs[B] = {1, 0, 1};
    const int64_t ctx[B] = {CAP, 1, 777};
    const int32_t NB = 64, TOPK = 100;
    int32_t* pool = xcalloc((size_t)B * NB, sizeof(int32_t));
    int32_t* idx = xcalloc((size_t)B * TOPK, sizeof(int32_t));
    double kb[B], kp[B];
    oracle_index_full(idxk, 0.5f, CAP, q, w, qs, ctx, B, NB, 8, TOPK, pool, idx, kb, kp);
    oracle_index_reindex(idxk, 0.5f, CAP, q, w, qs, ctx, B, pool, NB, 8, TOPK, idx, kp);

    /* attention over the Reindex selection, both layers */
    float* qa = xcalloc((size_t)B * 16 * D, sizeof(float));
    float* out = xcalloc((size_t)B * 16 * D, sizeof(float));
    for (i = 0; i < B * 16 * D; ++i) qa[i] = sym(1.0);
    for (i = 0; i < L; ++i)
        oracle_decode_attn(kv, CAP, wk, wv, 1.5f, 0.75f, WCAP, S, i, qa, idx, qs, ctx, B, TOPK,
                           0.08838834764831845f, out);
    for (i = 0; i < B * 16 * D; ++i) acc += out[i];
    printf("oracle driver ok %.6g\n", acc);
    free(kv); free(idxk); free(wk); free(wv); free(k); free(v); free(ik); free(seq); free(pos);
    free(sc); free(pool); free(idx); free(qa); free(out);
    return 0;
}
