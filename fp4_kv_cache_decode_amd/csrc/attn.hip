// Gather, dequantise and attend: one layer of CSA2 decode attention.
//
// What is computed: each query attends to its top-k selected global positions
// plus a local sliding window of 128 tokens (origotech.dev deep dive "Inside
// DeepSeek V4.1-Flash", section "How the architecture shrinks the KV cache";
// ttj.kr "CSA2 and the attention redesign").  Main KV is FP4 E2M1 with one E4M3
// scale per 16 channels and the window KV is FP8 (origotech.dev "FP4 and SWA
// Bounded Replay").  Reading taken here: one softmax per head over the valid
// main rows and the window rows [max(0,N-128), N), logits (q.k)*sm_scale.
//
// Design: split-K over 64-entry tiles.  Workgroup (tile, b) gathers its 64
// entries (144-byte records, or 256-byte window rows), dequantises them into
// LDS as f16 (exact: an E2M1 value times an E4M3 scale has at most 5
// significant bits, an E4M3 value has 4), and runs the 16-head x 64-entry x
// 128-dim contraction on MFMA (v_mfma_f32_16x16x16_f16).  The fp32 query and
// the fp32 softmax weights are each split into f16 hi + lo parts and issued as
// two MFMAs, so products are exact and accumulation is fp32: the result is
// fp32-accurate, far inside the 2e-3 output budget.  Each tile writes its
// running max m, sum l and unnormalised output o; a merge kernel rescales and
// combines the tiles (the same algebra an unsplit online softmax uses).
//
// FP4 dequantisation: the f16 encodings of the E2M1 magnitudes {0, .5, 1, 1.5,
// 2, 3, 4, 6} differ only in their high byte, so v_perm_b32 with an 8-byte table
// turns four code nibbles into four f16 high bytes in one instruction; a packed
// f16 multiply by the group's E4M3 scale is exact (at most 6 significant bits).
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int AT_THREADS = 256;
constexpr int TILE = 64;
constexpr int KROW = 136;    // f16 per K row in LDS (128 + 8 pad)
constexpr int VROW = 72;     // f16 per transposed V row (64 + 8 pad)
constexpr int PROW = 72;     // f16 per P row
constexpr float NEG_INF = -__builtin_huge_valf();

struct AttnArgs {
    const uint8_t* kv;
    const uint8_t* wk;
    const uint8_t* wv;
    const float* q;
    const int32_t* idx;
    const int32_t* seq;
    const int64_t* ctx;
    float* part;
    int64_t cap;
    int32_t n_seq;
    int32_t w_cap;
    int32_t layer;
    int32_t topk;
    int32_t n_main;          // main tiles
    int32_t n_tiles;
    float wk_scale;
    float wv_scale;
    float sm_scale;
};

struct AttnShared {
    _Float16 K[TILE * KROW];
    _Float16 Vt[D * VROW];
    _Float16 Phi[HEADS * PROW];
    _Float16 Plo[HEADS * PROW];
    float red[4][HEADS];
    float lsum[4][HEADS];
    int valid[TILE];
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// f16 high bytes of the E2M1 magnitudes 0..3 and 4..7 (a v_perm_b32 table).
constexpr uint32_t E2M1_HB_LO = 0x3E3C3800u;
constexpr uint32_t E2M1_HB_HI = 0x46444240u;

// f16 value of a signed E4M3 scale code (exact).
__device__ __forceinline__ half2_t scale_h2(uint32_t code) {
    const float s = e4m3_value_pos(code & 0x7f) * ((code & 0x80) ? -1.0f : 1.0f);
    const _Float16 h = (_Float16)s;
    return half2_t{h, h};
}

// 8 FP4 codes (one dword; channel 2j in the low nibble of byte j) -> 4 f16x2
// words (channels 2j, 2j+1 in word j), times the group scale.
__device__ __forceinline__ void fp4x8_to_f16x2(uint32_t w, half2_t scale, uint32_t* o) {
    // high bytes of channels 0,2,4,6 and 1,3,5,7; sign bit = nibble bit 3
    const uint32_t he = __builtin_amdgcn_perm(E2M1_HB_HI, E2M1_HB_LO, w & 0x07070707u) |
                        ((w << 4) & 0x80808080u);
    const uint32_t ho = __builtin_amdgcn_perm(E2M1_HB_HI, E2M1_HB_LO, (w >> 4) & 0x07070707u) |
                        (w & 0x80808080u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // bytes: 0x00, even high byte j, 0x00, odd high byte j (selector 12 = 0x00)
        const uint32_t sel = 0x0Cu | ((uint32_t)j << 8) | (0x0Cu << 16) | ((uint32_t)(4 + j) << 24);
        const uint32_t x = __builtin_amdgcn_perm(ho, he, sel);
        const half2_t v = __builtin_bit_cast(half2_t, x) * scale;
        o[j] = __builtin_bit_cast(uint32_t, v);
    }
}

__global__ void __launch_bounds__(AT_THREADS) attn_kernel(AttnArgs a) {
    __shared__ AttnShared sh;
    const int tile = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int32_t s = a.seq[b];
    const int64_t N = clamp64(a.ctx[b], 0, a.cap);
    const bool seq_ok = s >= 0 && s < a.n_seq;
    const bool is_main = tile < a.n_main;
    float* part = a.part + ((int64_t)b * a.n_tiles + tile) * ATTN_PART_FLOATS;

    // ---- query fragments first, independent of the gather chain (A operand,
    // hi/lo f16): Q[h = lane%16][16ks + 4(lane/16) + 0..3]
    half4_t qhi[8], qlo[8];
    {
        const int h = lane & 15, g = lane >> 4;
        const float* qrow = a.q + ((int64_t)b * HEADS + h) * D + 4 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const float4 v = *reinterpret_cast<const float4*>(qrow + 16 * ks);
            const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                _Float16 hi = (_Float16)x[i];
                qhi[ks][i] = hi;
                qlo[ks][i] = (_Float16)(x[i] - (float)hi);
            }
        }
    }
    // ---- gather + dequantise: 4 threads per entry, 32 channels each
    {
        const int e = t >> 2, q4 = t & 3;
        bool ok = false;
        uint32_t kw[16], vw[16];      // f16x2 words: channels 32*q4 + 2j, 2j+1
        if (is_main) {
            const int j = tile * TILE + e;
            const int32_t pos = (j < a.topk) ? a.idx[(int64_t)b * a.topk + j] : -1;
            ok = seq_ok && pos >= 0 && pos < N;
            if (ok) {
                const uint8_t* rec = a.kv + ((int64_t)s * a.cap + pos) * RECORD;
                const uint4 kc = *reinterpret_cast<const uint4*>(rec + 16 * q4);
                const uint4 vc = *reinterpret_cast<const uint4*>(rec + 64 + 16 * q4);
                const uint4 sc = *reinterpret_cast<const uint4*>(rec + 128);
                // K scales are bytes 0..7 of sc, V scales bytes 8..15; this
                // thread's 32 channels are groups 2*q4 and 2*q4 + 1
                const uint32_t ks = (q4 < 2 ? sc.x : sc.y) >> (16 * (q4 & 1));
                const uint32_t vs = (q4 < 2 ? sc.z : sc.w) >> (16 * (q4 & 1));
                const half2_t k0 = scale_h2(ks & 0xff), k1 = scale_h2((ks >> 8) & 0xff);
                const half2_t v0 = scale_h2(vs & 0xff), v1 = scale_h2((vs >> 8) & 0xff);
                fp4x8_to_f16x2(kc.x, k0, kw + 0);
                fp4x8_to_f16x2(kc.y, k0, kw + 4);
                fp4x8_to_f16x2(kc.z, k1, kw + 8);
                fp4x8_to_f16x2(kc.w, k1, kw + 12);
                fp4x8_to_f16x2(vc.x, v0, vw + 0);
                fp4x8_to_f16x2(vc.y, v0, vw + 4);
                fp4x8_to_f16x2(vc.z, v1, vw + 8);
                fp4x8_to_f16x2(vc.w, v1, vw + 12);
            }
        } else {
            const int64_t u0 = N > WINDOW ? N - WINDOW : 0;
            const int64_t u = u0 + (int64_t)(tile - a.n_main) * TILE + e;
            ok = seq_ok && u < N;
            if (ok) {
                const int64_t slot =
                    (((int64_t)a.layer * a.n_seq + s) * a.w_cap + u % a.w_cap) * D + 32 * q4;
                const uint4* kp = reinterpret_cast<const uint4*>(a.wk + slot);
                const uint4* vp = reinterpret_cast<const uint4*>(a.wv + slot);
                const uint4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
                const uint32_t kr[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                const uint32_t vr[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float2 a0 = e4m3x2_to_f32<false>(kr[i]), a1 = e4m3x2_to_f32<true>(kr[i]);
                    const float2 b0 = e4m3x2_to_f32<false>(vr[i]), b1 = e4m3x2_to_f32<true>(vr[i]);
                    kw[2 * i] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)a0.x, (_Float16)a0.y});
                    kw[2 * i + 1] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)a1.x, (_Float16)a1.y});
                    vw[2 * i] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)b0.x, (_Float16)b0.y});
                    vw[2 * i + 1] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)b1.x, (_Float16)b1.y});
                }
            }
        }
        if (!ok) {
#pragma unroll
            for (int i = 0; i < 16; ++i) kw[i] = vw[i] = 0u;
        }
        uint4* krow = reinterpret_cast<uint4*>(&sh.K[e * KROW + 32 * q4]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            krow[i] = make_uint4(kw[4 * i], kw[4 * i + 1], kw[4 * i + 2], kw[4 * i + 3]);
        unsigned short* vt = reinterpret_cast<unsigned short*>(sh.Vt);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            vt[(32 * q4 + 2 * i) * VROW + e] = (unsigned short)(vw[i] & 0xffffu);
            vt[(32 * q4 + 2 * i + 1) * VROW + e] = (unsigned short)(vw[i] >> 16);
        }
        if (q4 == 0) sh.valid[e] = ok;
    }

    __syncthreads();

    // ---- S = Q K^T for entries 16*wave .. +15
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
    {
        const int ent = 16 * wave + (lane & 15), g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const half4_t kf = *reinterpret_cast<const half4_t*>(&sh.K[ent * KROW + 16 * ks + 4 * g]);
            sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(qhi[ks], kf, sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(qlo[ks], kf, sacc, 0, 0, 0);
        }
    }
    // lane holds S[head 4*(lane/16) + r][entry 16*wave + lane%16]
    const float lscale = a.sm_scale * (is_main ? 1.0f : a.wk_scale);
    const bool ent_ok = sh.valid[16 * wave + (lane & 15)];
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = ent_ok ? sacc[r] * lscale : NEG_INF;

    // ---- tile max per head: 16 lanes of a row, then the 4 waves
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = sv[r];
        v = fmaxf(v, dpp_f32<DPP_XOR1>(v));
        v = fmaxf(v, dpp_f32<DPP_XOR2>(v));
        v = fmaxf(v, dpp_f32<DPP_ROR4>(v));
        v = fmaxf(v, dpp_f32<DPP_ROR8>(v));
        mx[r] = v;
    }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sh.red[wave][4 * (lane >> 4) + r] = mx[r];
    }
    __syncthreads();
    float m_tile[4], p[4], lsum[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * (lane >> 4) + r;
        m_tile[r] = fmaxf(fmaxf(sh.red[0][h], sh.red[1][h]), fmaxf(sh.red[2][h], sh.red[3][h]));
        p[r] = (m_tile[r] == NEG_INF || sv[r] == NEG_INF) ? 0.0f : expf(sv[r] - m_tile[r]);
        float v = p[r];
        v += dpp_f32<DPP_XOR1>(v);
        v += dpp_f32<DPP_XOR2>(v);
        v += dpp_f32<DPP_ROR4>(v);
        v += dpp_f32<DPP_ROR8>(v);
        lsum[r] = v;
        const int ent = 16 * wave + (lane & 15);
        _Float16 ph = (_Float16)p[r];
        sh.Phi[h * PROW + ent] = ph;
        sh.Plo[h * PROW + ent] = (_Float16)(p[r] - (float)ph);
    }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sh.lsum[wave][4 * (lane >> 4) + r] = lsum[r];
    }
    __syncthreads();   // P and the per-wave sums written
    if (t < HEADS) {
        part[HEADS + t] = sh.lsum[0][t] + sh.lsum[1][t] + sh.lsum[2][t] + sh.lsum[3][t];
    }

    // ---- O = P V for dims 32*wave .. +31 (two 16-dim tiles)
    float4_t oacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    {
        const int h = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half4_t ph = *reinterpret_cast<const half4_t*>(&sh.Phi[h * PROW + 16 * ks + 4 * g]);
            const half4_t pl = *reinterpret_cast<const half4_t*>(&sh.Plo[h * PROW + 16 * ks + 4 * g]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int d = 32 * wave + 16 * nt + (lane & 15);
                const half4_t vf = *reinterpret_cast<const half4_t*>(&sh.Vt[d * VROW + 16 * ks + 4 * g]);
                oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vf, oacc[nt], 0, 0, 0);
                oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vf, oacc[nt], 0, 0, 0);
            }
        }
    }
    // lane holds O[head 4*(lane/16) + r][dim 32*wave + 16*nt + lane%16]
    const float vscale = is_main ? 1.0f : a.wv_scale;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * (lane >> 4) + r;
            const int d = 32 * wave + 16 * nt + (lane & 15);
            part[2 * HEADS + h * D + d] = oacc[nt][r] * vscale;
        }
    }
    if (wave == 0 && (lane & 15) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) part[4 * (lane >> 4) + r] = m_tile[r];
    }
}

// Combine the tiles of each query: out = sum_t e^(m_t - M) o_t / sum_t e^(m_t - M) l_t.
// Each thread owns 8 output dims of one head; it loads the partials of up to
// MERGE_BATCH tiles at once (one memory round trip for the default 10 tiles).
constexpr int MERGE_BATCH = 12;     // tiles whose loads are in flight together

__global__ void __launch_bounds__(AT_THREADS) attn_merge_kernel(const float* part, int32_t n_tiles,
                                                                 float* out) {
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int h = t >> 4;                 // 16 threads per head
    const int d0 = (t & 15) * 8;          // 8 dims each
    const float* pb = part + (int64_t)b * n_tiles * ATTN_PART_FLOATS;
    float M = NEG_INF, L = 0.0f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // groups of MERGE_BATCH tiles: every load of a group is issued before use,
    // and M / L / acc are rescaled online when a group raises the max
    for (int i0 = 0; i0 < n_tiles; i0 += MERGE_BATCH) {
        float m[MERGE_BATCH], l[MERGE_BATCH];
        float4 o[MERGE_BATCH][2];
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            const int i = i0 + u < n_tiles ? i0 + u : n_tiles - 1;
            const float* pt = pb + (int64_t)i * ATTN_PART_FLOATS;
            m[u] = i0 + u < n_tiles ? pt[h] : NEG_INF;
            l[u] = pt[HEADS + h];
            const float4* po = reinterpret_cast<const float4*>(pt + 2 * HEADS + h * D + d0);
            o[u][0] = po[0];
            o[u][1] = po[1];
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) Mn = fmaxf(Mn, m[u]);
        if (Mn == NEG_INF) continue;
        const float c = M == NEG_INF ? 0.0f : expf(M - Mn);
        L *= c;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= c;
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            const float wgt = m[u] == NEG_INF ? 0.0f : expf(m[u] - Mn);
            L += wgt * l[u];
            acc[0] += wgt * o[u][0].x;
            acc[1] += wgt * o[u][0].y;
            acc[2] += wgt * o[u][0].z;
            acc[3] += wgt * o[u][0].w;
            acc[4] += wgt * o[u][1].x;
            acc[5] += wgt * o[u][1].y;
            acc[6] += wgt * o[u][1].z;
            acc[7] += wgt * o[u][1].w;
        }
        M = Mn;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float4* o = reinterpret_cast<float4*>(out + ((int64_t)b * HEADS + h) * D + d0);
    o[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    o[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
}

}  // namespace

hipError_t launch_attn(const csa2_cache& c, const csa2_window& w, int32_t layer,
                       const float* q, const int32_t* idx, const int32_t* seq,
                       const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                       float* out, float* partials, hipStream_t stream) {
    AttnArgs a{};
    a.kv = c.kv;
    a.wk = w.k;
    a.wv = w.v;
    a.q = q;
    a.idx = idx;
    a.seq = seq;
    a.ctx = ctx;
    a.part = partials;
    a.cap = c.cap;
    a.n_seq = c.n_seq;
    a.w_cap = w.w_cap;
    a.layer = layer;
    a.topk = topk;
    a.n_main = (topk + TILE - 1) / TILE;
    a.n_tiles = attn_tiles(topk);
    a.wk_scale = w.k_scale;
    a.wv_scale = w.v_scale;
    a.sm_scale = sm_scale;
    hipLaunchKernelGGL(attn_kernel, dim3(a.n_tiles, B), dim3(AT_THREADS), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(B), dim3(AT_THREADS), 0, stream, partials,
                       a.n_tiles, out);
    return hipGetLastError();
}

}  // namespace csa2
