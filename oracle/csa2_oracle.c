/*
 * CSA2 decode oracle: a plain, slow, scalar CPU definition of what the decode
 * path computes.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the
 * smoke check and by the benchmark's CPU-baseline leg, never by the product
 * path.  It shares no code with the HIP library.
 *
 * Sources (the pages are news summaries of the model's technical report):
 *  [P1] trawling.dev, "DeepSeek-V4.1-Flash released - a 552B multimodal MoE that
 *       cuts the KV cache to 890 bytes per token", section "CSA2 and FP4 KV
 *       caching": per-layer static modes Full/Reindex/Reuse sharing main KV and
 *       indexer K and reusing top-k indices; hierarchical indexer confined to
 *       the first Full layer's candidate pool; FP4 main KV in E2M1 with one
 *       E4M3 scale per 16 channels.
 *  [P3] cursorai.co.kr, "DeepSeek-V4.1-Flash: how an 890-byte KV cache changes
 *       agent infrastructure", section 3 "The secret of the 890-byte KV cache",
 *       step 3 "FP4 KV cache quantisation": 4 bits = 0.5 byte per element vs
 *       2 bytes for FP16, E2M1 format.
 *  [P4] origotech.dev, "Inside DeepSeek V4.1-Flash: KV cache, the 1017 update and
 *       the Harness stack", section "How the architecture shrinks the KV cache":
 *       the three modes; decoder = [Full + 3 Reuse] + 4 x [Reindex + 3 Reuse];
 *       top-k 512; 128-token sliding window; the first Full layer picks 2,048
 *       blocks of 8 positions (a 16,384-position pool) that only Reindex layers
 *       score; sub-section "FP4 and SWA Bounded Replay": main KV quantised to
 *       FP4 after RoPE, sliding-window KV kept in FP8.
 *  [P5] ttj.kr, "DeepSeek-V4.1-Flash compresses the KV cache to 890 bytes per
 *       token", section "CSA2 and the attention redesign": a size-128 local
 *       window + global sparse retrieval + cross-layer KV reuse.
 *
 * The pages leave open the indexer score, the block score, rounding rules and
 * layouts.  Readings taken here (each also listed in the design notes):
 *  - indexer score = sum_h w_h * ReLU(q_h . k), 4 heads x 64 dims, FP8 E4M3
 *    keys times one per-tensor fp32 scale;
 *  - block score = max over the block's visible positions;
 *  - E4M3 is OCP E4M3FN (bias 7, max 448, 0x7F/0xFF NaN), round to nearest
 *    even, saturating at 448, sign copied (so -0 encodes as 0x80);
 *  - FP4 group scale = E4M3(fp32(amax)/6), codes = nearest E2M1 value of x/s
 *    with ties to the even code, saturating at 6, sign of x kept; s = 0 gives
 *    magnitude 0;
 *  - 144-byte record: K codes [0,64), V codes [64,128), 8 K scales [128,136),
 *    8 V scales [136,144); channel 2j in the low nibble, 2j+1 in the high;
 *  - top-k ranks by value descending, ties to the lower index, output in
 *    ascending index order padded with -1;
 *  - attention: one softmax over the selected main rows and the window rows
 *    [max(0, N-128), N), logits q.k * sm_scale, no sink, no bias;
 *  - global-KV compression m (the encoder's m = 2): an entry is the fp32 mean
 *    of its m tokens' rows, quantised as a token row; the window keeps every
 *    token (oracle_compress_kv).
 *
 * Arithmetic: fp64 everywhere except where a step is defined in fp32 (the
 * amax/6 division and x/scale before FP8 rounding).  Build with -O2
 * -ffp-contract=off and without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_D 128       /* K and V channels */
#define OR_H 16        /* attention heads */
#define OR_HI 4        /* indexer heads */
#define OR_DI 64       /* indexer dims */
#define OR_W 128       /* sliding window */
#define OR_GROUP 16    /* channels per E4M3 scale */
#define OR_REC 144     /* bytes per FP4 K+V record */

/* ------------------------------------------------------------------ codecs */

/* E2M1 magnitudes for codes 0..7: {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Derived from
 * the format: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
 * subnormal (value m * 0.5). */
double oracle_e2m1_value(uint8_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN value of a byte: exponent 0 is subnormal m/8 * 2^-6, else
 * (1 + m/8) * 2^(e-7); 0x7F and 0xFF are NaN. */
double oracle_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Round |y| to the nearest E4M3FN value (ties to even mantissa), saturating at
 * 448; the sign bit of y is copied.  In a binade [2^e, 2^(e+1)) the grid step is
 * 2^(e-3); below 2^-6 it is the subnormal step 2^-9.  Anything >= 448 maps to
 * 448 (the band [448, 464) rounds there anyway). */
uint8_t oracle_e4m3_encode(float y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y), step, r;
    int e, code;
    if (!(a < 448.0)) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        step = ldexp(1.0, -9);
        r = nearbyint(a / step);               /* exact quotient, RNE rounding */
        return sign | (uint8_t)r;              /* r = 8 is 2^-6 = code 0x08 */
    }
    e = ilogb(a);
    step = ldexp(1.0, e - 3);
    r = nearbyint(a / step);                   /* 8..16 */
    if (r == 16.0) { r = 8.0; e += 1; }
    code = ((e + 7) << 3) | ((int)r - 8);
    return sign | (uint8_t)code;
}

/* Nearest E2M1 magnitude code of a >= 0 on the grid s * {0,.5,1,1.5,2,3,4,6},
 * ties to the even code, saturating at code 7.  s and the grid products have
 * few significant bits, so every distance that can decide the winner is
 * computed exactly in fp64. */
static int e2m1_nearest(double a, double s) {
    int c, best = 0;
    double bd = INFINITY;
    if (s == 0.0) return 0;
    if (a >= 6.0 * s) return 7;
    for (c = 0; c < 8; ++c) {
        double d = fabs(a - s * oracle_e2m1_value((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    return best;
}

/* Quantise one group of 16 channels: scale code and 16 nibbles (sign | mag). */
void oracle_fp4_group(const float* x, uint8_t* nibbles, uint8_t* scale_code) {
    float amax = 0.0f, s_real;
    double s;
    int i;
    for (i = 0; i < OR_GROUP; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    s_real = amax / 6.0f;                      /* IEEE fp32 division */
    *scale_code = oracle_e4m3_encode(s_real);
    s = oracle_e4m3_value(*scale_code);
    for (i = 0; i < OR_GROUP; ++i)
        nibbles[i] = (uint8_t)((signbit(x[i]) ? 8 : 0) | e2m1_nearest(fabs((double)x[i]), s));
}

/* Quantise a D-channel vector into D/2 code bytes and D/16 scale bytes. */
static void fp4_vector(const float* x, int dim, uint8_t* codes, uint8_t* scales) {
    uint8_t nib[OR_GROUP];
    int g, j;
    for (g = 0; g < dim / OR_GROUP; ++g) {
        oracle_fp4_group(x + g * OR_GROUP, nib, &scales[g]);
        for (j = 0; j < OR_GROUP / 2; ++j)
            codes[g * (OR_GROUP / 2) + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
    }
}

/* Dequantised channel c of an FP4 vector. */
static double fp4_channel(const uint8_t* codes, const uint8_t* scales, int c) {
    uint8_t byte = codes[c / 2];
    uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
    return oracle_e2m1_value(nib) * oracle_e4m3_value(scales[c / OR_GROUP]);
}

int oracle_record_bytes(void) { return OR_D / 2 * 2 + OR_D / OR_GROUP * 2; }

/* --------------------------------------------------------- quantise-on-write */

/* Write n new tokens.  Row i goes to sequence seq[i], position pos[i]:
 *   kv record      kv   + (seq*cap + pos) * 144     (k[i], v[i], FP4)
 *   indexer key    idxk + (seq*cap + pos) * 64      (E4M3 of idx_k[i]/idxk_scale)
 *   window rows    wk/wv + ((l*n_seq + seq)*w_cap + pos % w_cap) * 128 for each
 *                  layer l < n_layers (E4M3 of win_k/win_v [l][i] / scale).
 * idx_k and win_* may be NULL. */
void oracle_quantize_kv(uint8_t* kv, uint8_t* idxk, float idxk_scale, int64_t cap,
                        int32_t n_seq, uint8_t* wk, uint8_t* wv, float wk_scale,
                        float wv_scale, int32_t w_cap, int32_t n_layers,
                        const float* k, const float* v, const float* idx_k,
                        const float* win_k, const float* win_v, const int32_t* seq,
                        const int64_t* pos, int64_t n) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        int64_t row = (int64_t)seq[i] * cap + pos[i];
        uint8_t* rec = kv + row * OR_REC;
        int c, l;
        fp4_vector(k + i * OR_D, OR_D, rec, rec + 128);
        fp4_vector(v + i * OR_D, OR_D, rec + 64, rec + 136);
        if (idx_k && idxk)
            for (c = 0; c < OR_DI; ++c)
                idxk[row * OR_DI + c] = oracle_e4m3_encode(idx_k[i * OR_DI + c] / idxk_scale);
        if (win_k && wk)
            for (l = 0; l < n_layers; ++l) {
                int64_t slot = (((int64_t)l * n_seq + seq[i]) * w_cap + pos[i] % w_cap) * OR_D;
                const float* xk = win_k + ((int64_t)l * n + i) * OR_D;
                const float* xv = win_v + ((int64_t)l * n + i) * OR_D;
                for (c = 0; c < OR_D; ++c) {
                    wk[slot + c] = oracle_e4m3_encode(xk[c] / wk_scale);
                    wv[slot + c] = oracle_e4m3_encode(xv[c] / wv_scale);
                }
            }
    }
    (void)n_seq;
}

/* Global-KV compression m (origotech.dev deep dive, section "How the
 * architecture shrinks the KV cache": the encoder's CSA2 layers run at
 * compression m = 2, the decoder's at m = 1).  The pages give the ratio, not
 * the operator.  Reading taken here: global entry e of a sequence stands for
 * its m tokens at positions m*e .. m*e + m - 1, and its K, V and indexer-key
 * rows are those tokens' rows averaged in fp32 (the sum in position order,
 * then times 1/m; for m = 2 that is one rounding of the sum and an exact
 * halving), then quantised exactly as a token row is.  The window keeps every
 * token.
 *
 * Input rows i*m .. i*m + m - 1 form group i (n must be a multiple of m); the
 * group's entry is pos[i*m] / m of sequence seq[i*m], and a group whose first
 * position is not a multiple of m is skipped.  Window rows are written for
 * every token at its own position, as in oracle_quantize_kv.  m = 1 writes the
 * same bytes as oracle_quantize_kv.  With k and v NULL only window rows are
 * written (tokens whose group is not complete yet). */
static void mean_rows(const float* x, int32_t m, int dim, float* out) {
    int c, j;
    for (c = 0; c < dim; ++c) {
        float acc = x[c];
        for (j = 1; j < m; ++j) acc = acc + x[(int64_t)j * dim + c];
        out[c] = acc * (1.0f / (float)m);
    }
}

void oracle_compress_kv(uint8_t* kv, uint8_t* idxk, float idxk_scale, int64_t cap,
                        int32_t n_seq, uint8_t* wk, uint8_t* wv, float wk_scale,
                        float wv_scale, int32_t w_cap, int32_t n_layers,
                        const float* k, const float* v, const float* idx_k,
                        const float* win_k, const float* win_v, const int32_t* seq,
                        const int64_t* pos, int64_t n, int32_t m) {
    int64_t g, i;
    const int64_t n_groups = (k && v) ? n / m : 0;
#pragma omp parallel for schedule(static)
    for (g = 0; g < n_groups; ++g) {
        const int64_t i0 = g * m;
        float xk[OR_D], xv[OR_D], xi[OR_DI];
        int64_t row;
        uint8_t* rec;
        int c;
        if (pos[i0] % m != 0) continue;
        row = (int64_t)seq[i0] * cap + pos[i0] / m;
        rec = kv + row * OR_REC;
        mean_rows(k + i0 * OR_D, m, OR_D, xk);
        mean_rows(v + i0 * OR_D, m, OR_D, xv);
        fp4_vector(xk, OR_D, rec, rec + 128);
        fp4_vector(xv, OR_D, rec + 64, rec + 136);
        if (idx_k && idxk) {
            mean_rows(idx_k + i0 * OR_DI, m, OR_DI, xi);
            for (c = 0; c < OR_DI; ++c)
                idxk[row * OR_DI + c] = oracle_e4m3_encode(xi[c] / idxk_scale);
        }
    }
    if (!(win_k && wk)) return;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        int c, l;
        for (l = 0; l < n_layers; ++l) {
            int64_t slot = (((int64_t)l * n_seq + seq[i]) * w_cap + pos[i] % w_cap) * OR_D;
            const float* xk = win_k + ((int64_t)l * n + i) * OR_D;
            const float* xv = win_v + ((int64_t)l * n + i) * OR_D;
            for (c = 0; c < OR_D; ++c) {
                wk[slot + c] = oracle_e4m3_encode(xk[c] / wk_scale);
                wv[slot + c] = oracle_e4m3_encode(xv[c] / wv_scale);
            }
        }
    }
}

/* ------------------------------------------------------------------ indexer */

/* score_t = sum_h w_h * max(0, q_h . khat_t), khat = E4M3(code) * scale, fp64. */
double oracle_index_score(const uint8_t* key, float scale, const float* q, const float* w) {
    double score = 0.0;
    int h, c;
    for (h = 0; h < OR_HI; ++h) {
        double dot = 0.0;
        for (c = 0; c < OR_DI; ++c)
            dot += (double)q[h * OR_DI + c] * (oracle_e4m3_value(key[c]) * (double)scale);
        if (dot > 0.0) score += (double)w[h] * dot;
    }
    return score + 0.0;   /* canonical +0 */
}

typedef struct { double v; int64_t i; } vi_t;

static int by_value_desc_index_asc(const void* a, const void* b) {
    const vi_t* x = (const vi_t*)a;
    const vi_t* y = (const vi_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int by_int_asc(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* The k largest of n (value, index) pairs, ties to the lower index; their
 * indices in ascending order, padded with -1 up to k.  Returns how many were
 * selected; *kth receives the value of the last selected pair (or -inf). */
int32_t oracle_topk(const double* val, const int64_t* ids, int64_t n, int32_t k,
                    int32_t* out, double* kth) {
    vi_t* a = (vi_t*)malloc(sizeof(vi_t) * (size_t)(n > 0 ? n : 1));
    int64_t i, m = n < k ? n : k;
    for (i = 0; i < n; ++i) { a[i].v = val[i]; a[i].i = ids ? ids[i] : i; }
    qsort(a, (size_t)n, sizeof(vi_t), by_value_desc_index_asc);
    for (i = 0; i < m; ++i) out[i] = (int32_t)a[i].i;
    qsort(out, (size_t)m, sizeof(int32_t), by_int_asc);
    for (i = m; i < k; ++i) out[i] = -1;
    if (kth) *kth = m > 0 ? a[m - 1].v : -INFINITY;
    free(a);
    return (int32_t)m;
}

/* Scores of positions [0, N) of one sequence's indexer keys. */
void oracle_score_range(const uint8_t* keys, float scale, const float* q, const float* w,
                        int64_t N, double* scores) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < N; ++t)
        scores[t] = oracle_index_score(keys + t * OR_DI, scale, q, w);
}

/* Scores of the visible positions in the pool's blocks; returns the count. */
static int64_t pool_positions(const int32_t* pool, int32_t n_blocks, int32_t block,
                              int64_t N, int64_t* pos) {
    int64_t cnt = 0;
    int32_t j, o;
    for (j = 0; j < n_blocks; ++j) {
        if (pool[j] < 0) continue;
        for (o = 0; o < block; ++o) {
            int64_t t = (int64_t)pool[j] * block + o;
            if (t < N) pos[cnt++] = t;
        }
    }
    return cnt;
}

/* Full mode for B queries.  For query b over sequence seq[b] with N = ctx[b]:
 *   1. score every position t < N;
 *   2. block maxima M_j over [8j, 8j+8) intersect [0, N);
 *   3. pool = the n_blocks largest M_j (ties to the lower block), ascending, -1 pad;
 *   4. idx  = the topk largest scores among the pool's positions < N (ties to the
 *      lower position), ascending, -1 pad.
 * Optional diagnostics: kth_block[b], kth_pos[b] = the last selected values. */
void oracle_index_full(const uint8_t* idxk, float scale, int64_t cap, const float* q_idx,
                       const float* w, const int32_t* seq, const int64_t* ctx, int32_t B,
                       int32_t n_blocks, int32_t block, int32_t topk, int32_t* pool,
                       int32_t* idx, double* kth_block, double* kth_pos) {
    int32_t b;
    for (b = 0; b < B; ++b) {
        int64_t N = ctx[b], nb = (N + block - 1) / block, j, t, cnt;
        const uint8_t* keys = idxk + (int64_t)seq[b] * cap * OR_DI;
        double* sc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* M = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
        int64_t* pp = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_blocks * block);
        double* ps = (double*)malloc(sizeof(double) * (size_t)n_blocks * block);
        int32_t* pl = pool + (int64_t)b * n_blocks;
        double kb, kp;
        oracle_score_range(keys, scale, q_idx + (int64_t)b * OR_HI * OR_DI,
                           w + (int64_t)b * OR_HI, N, sc);
        for (j = 0; j < nb; ++j) {
            M[j] = -INFINITY;
            for (t = j * block; t < (j + 1) * block && t < N; ++t)
                if (sc[t] > M[j]) M[j] = sc[t];
        }
        oracle_topk(M, NULL, nb, n_blocks, pl, &kb);
        cnt = pool_positions(pl, n_blocks, block, N, pp);
        for (t = 0; t < cnt; ++t) ps[t] = sc[pp[t]];
        oracle_topk(ps, pp, cnt, topk, idx + (int64_t)b * topk, &kp);
        if (kth_block) kth_block[b] = kb;
        if (kth_pos) kth_pos[b] = kp;
        free(sc); free(M); free(pp); free(ps);
    }
}

/* Reindex mode: own q_idx / w, shared keys; score only the pool's positions
 * < N and take the topk largest (ties to the lower position). */
void oracle_index_reindex(const uint8_t* idxk, float scale, int64_t cap,
                          const float* q_idx, const float* w, const int32_t* seq,
                          const int64_t* ctx, int32_t B, const int32_t* pool,
                          int32_t n_blocks, int32_t block, int32_t topk, int32_t* idx,
                          double* kth_pos) {
    int32_t b;
    for (b = 0; b < B; ++b) {
        int64_t N = ctx[b], t, cnt;
        const uint8_t* keys = idxk + (int64_t)seq[b] * cap * OR_DI;
        int64_t* pp = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_blocks * block);
        double* ps = (double*)malloc(sizeof(double) * (size_t)n_blocks * block);
        double kp;
        cnt = pool_positions(pool + (int64_t)b * n_blocks, n_blocks, block, N, pp);
        for (t = 0; t < cnt; ++t)
            ps[t] = oracle_index_score(keys + pp[t] * OR_DI, scale,
                                       q_idx + (int64_t)b * OR_HI * OR_DI,
                                       w + (int64_t)b * OR_HI);
        oracle_topk(ps, pp, cnt, topk, idx + (int64_t)b * topk, &kp);
        if (kth_pos) kth_pos[b] = kp;
        free(pp); free(ps);
    }
}

/* --------------------------------------------------------------- attention */

/* Decode attention for one layer.  Entry set per query b: the FP4 main rows at
 * idx[b][*] >= 0 (dequantised K and V), then the layer's FP8 window rows for
 * positions u in [max(0, N-128), N) at slot u % w_cap.  Per head h:
 *   z_e = (q_h . k_e) * sm_scale;  p = softmax(z);  out_h = sum_e p_e v_e.
 * fp64 throughout, rounded to fp32 at the end. */
void oracle_decode_attn(const uint8_t* kv, int64_t cap, const uint8_t* wk,
                        const uint8_t* wv, float wk_scale, float wv_scale, int32_t w_cap,
                        int32_t n_seq, int32_t layer, const float* q, const int32_t* idx,
                        const int32_t* seq, const int64_t* ctx, int32_t B, int32_t topk,
                        float sm_scale, float* out) {
    int32_t b;
#pragma omp parallel for schedule(dynamic, 1)
    for (b = 0; b < B; ++b) {
        int64_t N = ctx[b], u0 = N - OR_W > 0 ? N - OR_W : 0, u;
        int32_t ne = 0, e, j, h, c;
        double* K = (double*)malloc(sizeof(double) * (size_t)(topk + OR_W) * OR_D);
        double* V = (double*)malloc(sizeof(double) * (size_t)(topk + OR_W) * OR_D);
        double* z = (double*)malloc(sizeof(double) * (size_t)(topk + OR_W));
        for (j = 0; j < topk; ++j) {
            int32_t t = idx[(int64_t)b * topk + j];
            const uint8_t* rec;
            if (t < 0) continue;
            rec = kv + ((int64_t)seq[b] * cap + t) * OR_REC;
            for (c = 0; c < OR_D; ++c) {
                K[(int64_t)ne * OR_D + c] = fp4_channel(rec, rec + 128, c);
                V[(int64_t)ne * OR_D + c] = fp4_channel(rec + 64, rec + 136, c);
            }
            ++ne;
        }
        for (u = u0; u < N; ++u) {
            int64_t slot = (((int64_t)layer * n_seq + seq[b]) * w_cap + u % w_cap) * OR_D;
            for (c = 0; c < OR_D; ++c) {
                K[(int64_t)ne * OR_D + c] = oracle_e4m3_value(wk[slot + c]) * (double)wk_scale;
                V[(int64_t)ne * OR_D + c] = oracle_e4m3_value(wv[slot + c]) * (double)wv_scale;
            }
            ++ne;
        }
        for (h = 0; h < OR_H; ++h) {
            const float* qh = q + ((int64_t)b * OR_H + h) * OR_D;
            double zmax = -INFINITY, denom = 0.0;
            for (e = 0; e < ne; ++e) {
                double dot = 0.0;
                for (c = 0; c < OR_D; ++c) dot += (double)qh[c] * K[(int64_t)e * OR_D + c];
                z[e] = dot * (double)sm_scale;
                if (z[e] > zmax) zmax = z[e];
            }
            for (e = 0; e < ne; ++e) { z[e] = exp(z[e] - zmax); denom += z[e]; }
            for (c = 0; c < OR_D; ++c) {
                double acc = 0.0;
                for (e = 0; e < ne; ++e) acc += z[e] * V[(int64_t)e * OR_D + c];
                out[((int64_t)b * OR_H + h) * OR_D + c] = ne > 0 ? (float)(acc / denom) : 0.0f;
            }
        }
        free(K); free(V); free(z);
    }
}
