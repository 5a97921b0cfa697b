// Gather, dequantise and attend: device code shared by the attention kernels
// and the fused Reindex layer.  What is computed and the kernels' design are
// described at the top of attn.hip: one softmax per head over a query's
// selected FP4 main rows and its 128-token FP8 window (origotech.dev deep dive
// "Inside DeepSeek V4.1-Flash", section "How the architecture shrinks the KV
// cache"; origotech.dev "FP4 and SWA Bounded Replay").
#pragma once

#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {
namespace attn_dev {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int AT_THREADS = 256;
constexpr int AT_WAVES = AT_THREADS / 64;
constexpr int SUB = 16;                   // entries per wave step
constexpr float NEG_INF = -__builtin_huge_valf();
// floats per head row of the waves' O in LDS when they are combined: the 16
// lanes that write one 16-byte piece of 16 heads' rows at once land on 16
// distinct bank groups (a 128-float row would put all 16 on the same one)
constexpr int OROW = D + 4;
// tile kernel (small batches): used while B x tiles fits one wave of workgroups
constexpr int64_t TILE_KERNEL_MAX_WG = 768;
constexpr int TILE = 64;
// largest context length (tokens) an attention call takes from ctx[]
constexpr int64_t CTX_TOKENS_MAX = (int64_t)1 << 40;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Stream kernel V^T tile of one wave, in dwords.  Row d = 16m + t (channel d,
// m = d / 16) holds the step's 16 entries as 8 f16 pairs (dword j: entries 2j,
// 2j+1) and starts at vt_block(m) + VT_ROW * t.  Writes go out as one row per
// instruction from each of 8 lanes per group m; reads are the PV A operand,
// rows 16mt + i and dwords 2kb, 2kb + 1 for lane (i, kb).  With 32 four-byte
// banks served per half wave (4-byte accesses) or quarter wave (8-byte):
//  * a write instruction's half wave covers groups m with equal bit 1, whose
//    blocks start in distinct quarters of the banks (vt_block(m) mod 32), so
//    its 4 rows x 8 dwords hit 32 distinct banks;
//  * a read's quarter wave covers 16 rows of one block at stride 10 dwords,
//    whose 2-dword pieces fall on 16 distinct even banks.
// Over 64 banks the 8 block starts are distinct too.  Blocks are 192 dwords
// apart plus that offset, so they do not overlap (a block spans 158 dwords).
constexpr int VT_ROW = 10;
__host__ __device__ constexpr int vt_block(int m) {
    return 192 * m + 8 * ((m & 1) | (((m >> 2) & 1) << 1) | (((m >> 1) & 1) << 2));
}
constexpr int VT_DWORDS = vt_block(7) + VT_ROW * 15 + 8 + 2;   // 8-byte multiple

// Lane slot holding query slice ks for lane L: L with its low three bits
// flipped by ks and bit 4 of L.  Reads by 8-lane groups stay a permutation of
// the group; the prologue's 16-lane stores of one head (varying ks and g)
// land on 8 distinct slots mod 8.
__host__ __device__ constexpr int q_slot(int ks, int L) {
    return L ^ (ks | (((L >> 4) & 1) << 2));
}

struct AttnShared {
    union {
        struct {
            uint32_t vt[AT_WAVES][VT_DWORDS];      // per-wave V^T of one step
            half8_t q[2][4][64];                   // query slices (hi, lo), by q_slot
        } st;
        struct {
            float o[AT_WAVES][HEADS * OROW];
            float m[AT_WAVES][HEADS];
            float l[AT_WAVES][HEADS];
        } mg;                                      // the waves' softmax states
    };
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// The gfx950 scaled converters.  Their fp32 scale operand applies only its
// power of two (E8M0 semantics), so it is 1 here and the E4M3 group scale is
// applied by a packed f16 multiply (exact: at most 6 significant bits).
// FP4: byte `sel` of w -> (low nibble, high nibble) as exact E2M1 values.
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_h2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// FP8: word HI of w -> two exact E4M3 values.
template <bool HI>
__device__ __forceinline__ half2_t fp8x2_h2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
// 8 FP4 codes (channel 2j in the low nibble of byte j) times a group scale ->
// 4 f16x2 words (channels 2j, 2j+1 in word j).
__device__ __forceinline__ void fp4x8_scaled(uint32_t w, half2_t scale, uint32_t* o) {
    o[0] = __builtin_bit_cast(uint32_t, fp4x2_h2<0>(w) * scale);
    o[1] = __builtin_bit_cast(uint32_t, fp4x2_h2<1>(w) * scale);
    o[2] = __builtin_bit_cast(uint32_t, fp4x2_h2<2>(w) * scale);
    o[3] = __builtin_bit_cast(uint32_t, fp4x2_h2<3>(w) * scale);
}

constexpr float LOG2E = 1.4426950408889634f;
// stream kernel softmax: the running reference max lags the true max by at most
// 2^8 in weight, so every weight stays far inside f16 for the hi/lo split
constexpr float RESCALE_SLACK = 8.0f;
constexpr float LN2 = 0.6931471805599453f;


// ---------------------------------------------------------------------------
// Tile kernel (small batches, latency): one workgroup per (query, 64-entry
// tile), each of its 4 waves owning 16 entries.  The work of a wave is one
// step of the stream kernel's loop (attn.hip), with the same lane roles: lane
// (c, g) gathers K channels 32g..32g+31 of entry c and V channel group
// 4(c mod 2) + g of the entry pair containing c; S^T = K Q^T comes out of
// v_mfma_f32_16x16x32_f16 with K straight from the gathering lane's
// registers, the softmax weights stay where S^T left them as the B operand of
// O^T = V^T P^T, and only V is transposed, through the wave's own LDS tile.
// The 4 waves' (m, l, O) are combined in LDS and the tile writes one partial
// record.  The index load is issued first and the query's loads right after
// it, so the query's staging overlaps the record loads.

struct TileArgs {
    const uint8_t* kv;
    const uint8_t* kvg_in;   // [B][topk][RECORD] gathered main records, or null
    uint8_t* kvg_out;        // where to store the gathered main records, or null
    const uint8_t* wk;
    const uint8_t* wv;
    const float* q;
    const int32_t* idx;
    const int32_t* seq;
    const int64_t* ctx;
    float* part;
    int64_t cap;
    PageMap pm;              // page table of a paged cache (table null otherwise)
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

// Address modes of the main records: 32-bit offsets from the sequence's base
// (every contiguous cache whose sequences span at most 4 GiB), 64-bit offsets,
// or a page table.
enum { AM_OFF32 = 0, AM_FLAT64 = 1, AM_PAGED = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Buffer resource word 3 on gfx9-family targets (32-bit data format, no
// swizzle); loads past num_records return zeros.
constexpr int BUF_DWORD3 = 0x00020000;

// The query's f16 hi + lo slices in LDS (B operand of S^T = K Q^T on
// 16x16x32 MFMA): lane (c, g) takes Q[h = c][32g + 8ks .. +7] for slice ks.
// The workgroup loads the query once, coalesced (two float4 per thread), and
// stores each half4 in the lane slot q_slot(ks, lane) that reads it.
__device__ __forceinline__ void stage_query(AttnShared& sh, const float* q, int t) {
    float4 qv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
        qv[k] = *reinterpret_cast<const float4*>(q + 4 * (t + AT_THREADS * k));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int f = t + AT_THREADS * k;                    // float4 index: h * 32 + d / 4
        const int h = f >> 5, d = 4 * (f & 31);
        const int gq = d >> 5, ks = (d >> 3) & 3, half = (d >> 2) & 1;
        const float x[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
        half4_t hi4, lo4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const _Float16 hi = (_Float16)x[i];
            hi4[i] = hi;
            lo4[i] = (_Float16)(x[i] - (float)hi);
        }
        const int sl = q_slot(ks, 16 * gq + h);
        reinterpret_cast<half4_t*>(&sh.st.q[0][ks][sl])[half] = hi4;
        reinterpret_cast<half4_t*>(&sh.st.q[1][ks][sl])[half] = lo4;
    }
}

// Dequantisation of one 16-entry step held by the lane (c, g):
//  main:   r[0..3] K codes of entry c, channels 32g..32g+31; r[4..7] that
//          record's 16 scale bytes; r[8..9] and r[10..11] V codes of channel
//          group m of entries 2j and 2j+1
//  window: r[0..7] K bytes of entry c, channels 32g..32g+31; r[8..11] and
//          r[12..15] V bytes of channels 16m..16m+15 of entries 2j and 2j+1
// K becomes the four A-operand slices of S^T = K Q^T, V the 16 f16 pairs
// (V[2j][16m + u], V[2j+1][16m + u]) of the transposed V tile.
__device__ __forceinline__ void dequant_main(const uint32_t* r, int g, int o, uint32_t vsel,
                                             half8_t* kf, uint32_t* vw) {
    // K scales of groups 2g, 2g+1 (adjacent bytes of the K scale block)
    const half2_t ks2 = fp8x2_h2<false>(((g >> 1) ? r[5] : r[4]) >> (16 * (g & 1)));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint32_t w4[4];
        fp4x8_scaled(r[ks], ks < 2 ? half2_t{ks2.x, ks2.x} : half2_t{ks2.y, ks2.y}, w4);
        kf[ks] = __builtin_bit_cast(half8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    }
    // V scales of group m of entries 2j, 2j+1: byte g of V scale dword o of
    // each record; the partner lane c ^ 1 holds the other record
    const uint32_t send = o ? r[6] : r[7];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, DPP_XOR1, 0xf, 0xf, false);
    const half2_t vs = fp8x2_h2<false>(__builtin_amdgcn_perm(o ? r[7] : r[6], recv, vsel));
    // interleave the two entries' nibbles so that one conversion gives a
    // (2j, 2j+1) pair: byte k of x holds channel 2k of both, of y channel 2k+1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint32_t A = r[8 + u], Bv = r[10 + u];
        const uint32_t x = (A & 0x0f0f0f0fu) | ((Bv << 4) & 0xf0f0f0f0u);
        const uint32_t y = ((A >> 4) & 0x0f0f0f0fu) | (Bv & 0xf0f0f0f0u);
        vw[8 * u + 0] = __builtin_bit_cast(uint32_t, fp4x2_h2<0>(x) * vs);
        vw[8 * u + 1] = __builtin_bit_cast(uint32_t, fp4x2_h2<0>(y) * vs);
        vw[8 * u + 2] = __builtin_bit_cast(uint32_t, fp4x2_h2<1>(x) * vs);
        vw[8 * u + 3] = __builtin_bit_cast(uint32_t, fp4x2_h2<1>(y) * vs);
        vw[8 * u + 4] = __builtin_bit_cast(uint32_t, fp4x2_h2<2>(x) * vs);
        vw[8 * u + 5] = __builtin_bit_cast(uint32_t, fp4x2_h2<2>(y) * vs);
        vw[8 * u + 6] = __builtin_bit_cast(uint32_t, fp4x2_h2<3>(x) * vs);
        vw[8 * u + 7] = __builtin_bit_cast(uint32_t, fp4x2_h2<3>(y) * vs);
    }
}
__device__ __forceinline__ void dequant_window(const uint32_t* r, half8_t* kf, uint32_t* vw) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        kf[ks] = __builtin_bit_cast(
            half8_t, make_uint4(__builtin_bit_cast(uint32_t, fp8x2_h2<false>(r[2 * ks])),
                                __builtin_bit_cast(uint32_t, fp8x2_h2<true>(r[2 * ks])),
                                __builtin_bit_cast(uint32_t, fp8x2_h2<false>(r[2 * ks + 1])),
                                __builtin_bit_cast(uint32_t, fp8x2_h2<true>(r[2 * ks + 1]))));
    // bytes of the two entries interleaved: (A0 B0 A1 B1), (A2 B2 A3 B3)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t A = r[8 + u], Bv = r[12 + u];
        const uint32_t p0 = __builtin_amdgcn_perm(Bv, A, 0x05010400u);
        const uint32_t p1 = __builtin_amdgcn_perm(Bv, A, 0x07030602u);
        vw[4 * u + 0] = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(p0));
        vw[4 * u + 1] = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(p0));
        vw[4 * u + 2] = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(p1));
        vw[4 * u + 3] = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(p1));
    }
}

// v_perm selector putting the V scale bytes of entries 2j, 2j+1 (byte g of the
// lane's own dword and of the one received from lane c ^ 1) in order
__device__ __forceinline__ uint32_t vscale_sel(int o, int g) {
    return o ? ((uint32_t)g | ((4u + g) << 8) | 0x0c0c0000u)
             : ((4u + g) | ((uint32_t)g << 8) | 0x0c0c0000u);
}

// Window slot of position u0 (u0 mod w_cap); 32-bit division whenever u0 fits.
__device__ __forceinline__ int32_t window_slot(int64_t u0, int32_t w_cap) {
    return u0 <= (int64_t)0xffffffffll ? (int32_t)((uint32_t)u0 % (uint32_t)w_cap)
                                       : (int32_t)(u0 % w_cap);
}

// Body of tile `tile` of query b (both uniform), AT_THREADS threads, t the
// thread's index among them.  It has exactly TILE_BARRIERS workgroup barriers,
// none under a condition, so several tiles can run side by side in one larger
// workgroup (each with its own AttnShared).
constexpr int TILE_BARRIERS = 3;
template <int AM>
__device__ __forceinline__ void tile_body(const TileArgs& a, AttnShared& sh, int tile, int b,
                                          int t) {
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int jp = c >> 1, o = c & 1, m = 4 * o + g;    // V: entries 2jp, 2jp+1, group m
    const bool is_main = tile < a.n_main;
    // the wave's 16 entries: list indices e0.. (main) or window offsets off0..
    const int e0 = tile * TILE + 16 * wave;
    const int off0 = (tile - a.n_main) * TILE + 16 * wave;   // window tiles: < 128 <= w_cap

    // ---- loads in order of need: the index (and the query's sequence and
    // length), the query, then the records
    int32_t pos = -1;
    if (is_main && e0 + c < a.topk) pos = a.idx[(int64_t)b * a.topk + e0 + c];
    const int32_t s = a.seq[b];
    // N counts tokens (the window is [N - 128, N)); main entries are valid below
    // min(N, cap), which also keeps every record load inside the store (with a
    // compressed store N exceeds the entries, and the indices stay below N / m)
    const int64_t N = clamp64(a.ctx[b], 0, CTX_TOKENS_MAX);
    const int64_t n_main = N < a.cap ? N : a.cap;
    const bool seq_ok = s >= 0 && s < a.n_seq;
    const uint32_t n_ok = seq_ok ? (uint32_t)(n_main < INT32_MAX ? n_main : INT32_MAX) : 0u;

    // ---- per kind of tile: the record (or window row) loads, the query's
    // staging while they are in flight, then the dequantisation.  Each branch
    // consumes everything it loads, so no load is pending where the branches
    // join (a pending load there would make the compiler wait for all of them
    // before the first record load).
    half8_t kf[4];
    uint32_t vw[16];
    uint32_t okb3;                          // validity of entries c, 2jp, 2jp+1 (bits 0..2)
    if (is_main) {
        const int32_t pos_p = __builtin_amdgcn_mov_dpp(pos, DPP_XOR1, 0xf, 0xf, false);
        const int32_t pa = o ? pos_p : pos, pb = o ? pos : pos_p;
        const bool oka = (uint32_t)pa < n_ok, okb = (uint32_t)pb < n_ok;
        const int ea = e0 + 2 * jp;
        uint32_t r[12];
        u32x4 kc, sc;
        u32x2 va, vb;
        const bool main_buf = a.kvg_in != nullptr || AM == AM_OFF32;
        if (main_buf) {
            const uint8_t* base = a.kvg_in ? a.kvg_in + (int64_t)b * a.topk * RECORD
                                           : a.kv + (seq_ok ? (int64_t)s * a.cap * RECORD : 0);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)base, 0,
                (int)(a.kvg_in ? (uint32_t)a.topk * (uint32_t)RECORD
                               : (uint32_t)(AM == AM_OFF32 ? a.cap * RECORD : 0)),
                BUF_DWORD3);
            const uint32_t oa = a.kvg_in ? (uint32_t)(ea < a.topk ? ea : 0) * RECORD
                                         : (oka ? (uint32_t)pa * RECORD : 0u);
            const uint32_t ob = a.kvg_in ? (uint32_t)(ea + 1 < a.topk ? ea + 1 : 0) * RECORD
                                         : (okb ? (uint32_t)pb * RECORD : 0u);
            const uint32_t oc = o ? ob : oa;
            kc = __builtin_amdgcn_raw_buffer_load_b128(rs, oc + 16 * g, 0, 0);
            sc = __builtin_amdgcn_raw_buffer_load_b128(rs, oc + 128, 0, 0);
            va = __builtin_amdgcn_raw_buffer_load_b64(rs, oa + 8 * m + 64, 0, 0);
            vb = __builtin_amdgcn_raw_buffer_load_b64(rs, ob + 8 * m + 64, 0, 0);
        } else {
            auto rec = [&](int32_t p, bool ok) -> const uint8_t* {
                if constexpr (AM == AM_PAGED)
                    return a.kv + (ok ? cache_row<true>(a.pm, a.cap, s, p) * RECORD : 0);
                else
                    return a.kv + (ok ? ((int64_t)s * a.cap + p) * RECORD : 0);
            };
            const uint8_t* ra = rec(pa, oka);
            const uint8_t* rb = rec(pb, okb);
            const uint8_t* rc = o ? rb : ra;
            kc = *reinterpret_cast<const u32x4*>(rc + 16 * g);
            sc = *reinterpret_cast<const u32x4*>(rc + 128);
            va = *reinterpret_cast<const u32x2*>(ra + 64 + 8 * m);
            vb = *reinterpret_cast<const u32x2*>(rb + 64 + 8 * m);
        }
        stage_query(sh, a.q + (int64_t)b * HEADS * D, t);
        r[0] = kc[0]; r[1] = kc[1]; r[2] = kc[2]; r[3] = kc[3];
        r[4] = sc[0]; r[5] = sc[1]; r[6] = sc[2]; r[7] = sc[3];
        r[8] = va[0]; r[9] = va[1]; r[10] = vb[0]; r[11] = vb[1];
        const bool okc = o ? okb : oka;
        okb3 = (uint32_t)okc | ((uint32_t)oka << 1) | ((uint32_t)okb << 2);
        if (a.kvg_out) {
            // this lane's share of the records: entry c's K bytes 16g.. and
            // (g = 0) scale bytes; V group m of entries 2jp and 2jp+1
            uint8_t* da = a.kvg_out + ((int64_t)b * a.topk + ea) * RECORD;
            uint8_t* dc = da + o * RECORD;
            if (okc) {
                *reinterpret_cast<uint4*>(dc + 16 * g) = make_uint4(r[0], r[1], r[2], r[3]);
                if (g == 0)
                    *reinterpret_cast<uint4*>(dc + 128) = make_uint4(r[4], r[5], r[6], r[7]);
            }
            if (oka) *reinterpret_cast<uint2*>(da + 64 + 8 * m) = make_uint2(r[8], r[9]);
            if (okb) *reinterpret_cast<uint2*>(da + RECORD + 64 + 8 * m) = make_uint2(r[10], r[11]);
        }
        dequant_main(r, g, o, vscale_sel(o, g), kf, vw);
    } else {
        const int64_t u0 = N > WINDOW ? N - WINDOW : 0;
        const int w_ok = seq_ok ? (int)(N - u0) : 0;
        const bool oka = off0 + 2 * jp < w_ok, okb = off0 + 2 * jp + 1 < w_ok;
        const int64_t win_base = ((int64_t)a.layer * a.n_seq + (seq_ok ? s : 0)) * a.w_cap;
        const int32_t slot0 = window_slot(u0, a.w_cap);
        auto wrow = [&](int e) -> uint32_t {                 // (u0 + e) mod w_cap, times D
            int32_t sl = slot0 + e;
            sl = sl >= a.w_cap ? sl - a.w_cap : sl;
            return (uint32_t)sl * (uint32_t)D;
        };
        const uint32_t ra = oka ? wrow(off0 + 2 * jp) : 0u, rb = okb ? wrow(off0 + 2 * jp + 1) : 0u;
        const uint32_t rc = o ? rb : ra;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.wk + win_base * D), 0, a.w_cap * D, BUF_DWORD3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.wv + win_base * D), 0, a.w_cap * D, BUF_DWORD3);
        const u32x4 k0 = __builtin_amdgcn_raw_buffer_load_b128(rk, rc + 32 * g, 0, 0);
        const u32x4 k1 = __builtin_amdgcn_raw_buffer_load_b128(rk, rc + 32 * g + 16, 0, 0);
        const u32x4 va = __builtin_amdgcn_raw_buffer_load_b128(rv, ra + 16 * m, 0, 0);
        const u32x4 vb = __builtin_amdgcn_raw_buffer_load_b128(rv, rb + 16 * m, 0, 0);
        stage_query(sh, a.q + (int64_t)b * HEADS * D, t);
        uint32_t r[16];
        r[0] = k0[0]; r[1] = k0[1]; r[2] = k0[2]; r[3] = k0[3];
        r[4] = k1[0]; r[5] = k1[1]; r[6] = k1[2]; r[7] = k1[3];
        r[8] = va[0]; r[9] = va[1]; r[10] = va[2]; r[11] = va[3];
        r[12] = vb[0]; r[13] = vb[1]; r[14] = vb[2]; r[15] = vb[3];
        okb3 = (uint32_t)(o ? okb : oka) | ((uint32_t)oka << 1) | ((uint32_t)okb << 2);
        dequant_window(r, kf, vw);
    }
    const bool ok_c = okb3 & 1u;
    const uint64_t vmask = __ballot(ok_c);      // bit e (e < 16): entry e of the wave valid
    const bool all_valid = (vmask & 0xffffu) == 0xffffu;
    if (!all_valid) {
        // absent entries contribute exact zeros whatever their bytes hold
        if (!ok_c) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kf[ks] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
        const uint32_t keep = ((okb3 & 2u) ? 0x0000ffffu : 0u) | ((okb3 & 4u) ? 0xffff0000u : 0u);
#pragma unroll
        for (int u = 0; u < 16; ++u) vw[u] &= keep;
    }

    // ---- V^T into the wave's LDS tile: row 16m + u, dword jp
    uint32_t* vt = sh.st.vt[wave];
    {
        uint32_t* const vt_wr = vt + vt_block(m) + jp;
#pragma unroll
        for (int u = 0; u < 16; ++u) vt_wr[VT_ROW * u] = vw[u];
    }
    // the tile is private to this wave and LDS executes a wave's operations in
    // order; this only keeps the compiler from moving its reads above the writes
    asm volatile("" ::: "memory");

    __syncthreads();                            // the query slices are in LDS

    // ---- S^T = K Q^T: lane (c, g) gets S[head c][entry 4g + r]; hi and lo
    // parts of q in two independent accumulator chains
    float4_t sacc;
    {
        float4_t shi = {0.f, 0.f, 0.f, 0.f}, slo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int qs = q_slot(ks, lane);
            shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], sh.st.q[0][ks][qs], shi, 0, 0, 0);
            slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], sh.st.q[1][ks][qs], slo, 0, 0, 0);
        }
        sacc = shi + slo;
    }
    // logits in log2 units (log2(e) folded into the scale): exp2 is one v_exp_f32
    const float lscale = a.sm_scale * LOG2E * (is_main ? 1.0f : a.wk_scale);
    float sv[4];
    float mx = NEG_INF;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const bool v_ok = (vmask >> (4 * g + q4)) & 1u;
        sv[q4] = v_ok ? sacc[q4] * lscale : NEG_INF;
        mx = fmaxf(mx, sv[q4]);
    }
    mx = max_xor32(max_xor16(mx));              // the wave's max for head c
    half4_t phi, plo;
    float lsum = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float p = sv[q4] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(sv[q4] - mx);
        lsum += p;
        const _Float16 h = (_Float16)p;
        phi[q4] = h;
        plo[q4] = (_Float16)(p - (float)h);
    }
    lsum = add_xor32(add_xor16(lsum));

    // ---- O^T = V^T P^T over the wave's 16 entries: O^T[d = 16 mt + 4g + r][h = c]
    float4_t o_acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const half4_t vf =
            *reinterpret_cast<const half4_t*>(vt + vt_block(mt) + VT_ROW * c + 2 * g);
        float4_t acc = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, phi, float4_t{0.f, 0.f, 0.f, 0.f},
                                                             0, 0, 0);
        o_acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, plo, acc, 0, 0, 0);
    }

    // ---- combine the 4 waves in LDS and write the tile's partial record
    __syncthreads();                            // every wave is done with its V^T tile
    if (g == 0) {
        sh.mg.m[wave][c] = mx;
        sh.mg.l[wave][c] = lsum;
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<float4_t*>(&sh.mg.o[wave][c * OROW + 16 * mt + 4 * g]) = o_acc[mt];
    __syncthreads();
    {
        const int h = t >> 4, d0 = (t & 15) * 8;
        float mw[AT_WAVES], M = NEG_INF;
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) {
            mw[w] = sh.mg.m[w][h];
            M = fmaxf(M, mw[w]);
        }
        float L = 0.0f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (M != NEG_INF) {
#pragma unroll
            for (int w = 0; w < AT_WAVES; ++w) {
                const float wt = mw[w] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - M);
                L += wt * sh.mg.l[w][h];
                const float4* src = reinterpret_cast<const float4*>(&sh.mg.o[w][h * OROW + d0]);
                const float4 x0 = src[0], x1 = src[1];
                acc[0] += wt * x0.x; acc[1] += wt * x0.y; acc[2] += wt * x0.z; acc[3] += wt * x0.w;
                acc[4] += wt * x1.x; acc[5] += wt * x1.y; acc[6] += wt * x1.z; acc[7] += wt * x1.w;
            }
        }
        // the window's per-tensor V scale multiplies its PV products
        const float vscale = is_main ? 1.0f : a.wv_scale;
        float* part = a.part + ((int64_t)b * a.n_tiles + tile) * ATTN_PART_FLOATS;
        if ((t & 15) == 0) {
            part[h] = M * LN2;                  // partials carry natural-log maxima
            part[HEADS + h] = L;
        }
        float4* dst = reinterpret_cast<float4*>(part + 2 * HEADS + h * D + d0);
        dst[0] = make_float4(acc[0] * vscale, acc[1] * vscale, acc[2] * vscale, acc[3] * vscale);
        dst[1] = make_float4(acc[4] * vscale, acc[5] * vscale, acc[6] * vscale, acc[7] * vscale);
    }
}

// Combine the partials of each query: out = sum_t e^(m_t - M) o_t / sum_t e^(m_t - M) l_t.
// One workgroup per (head, query) and one thread per output dim, so the partial
// loads spread over B x 16 compute units; each thread loads its dim of up to
// MERGE_BATCH partials at once (one memory round trip for the 10 tiles of top-512).
constexpr int MERGE_BATCH = 12;

// Body of the merge of head h of query b (uniform), D threads, d the thread's
// output dim.  No barrier.
__device__ __forceinline__ void merge_body(const float* part, int32_t n_parts, float* out, int h,
                                           int b, int d) {
    const float* pb = part + (int64_t)b * n_parts * ATTN_PART_FLOATS;
    float M = NEG_INF, L = 0.0f, acc = 0.0f;
    // groups of MERGE_BATCH partials: every load of a group is issued before
    // use, and M / L / acc are rescaled online when a group raises the max
    for (int i0 = 0; i0 < n_parts; i0 += MERGE_BATCH) {
        float m[MERGE_BATCH], l[MERGE_BATCH], o[MERGE_BATCH];
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            const int i = i0 + u < n_parts ? i0 + u : n_parts - 1;
            const float* pt = pb + (int64_t)i * ATTN_PART_FLOATS;
            m[u] = i0 + u < n_parts ? pt[h] : NEG_INF;
            l[u] = pt[HEADS + h];
            o[u] = pt[2 * HEADS + h * D + d];
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) Mn = fmaxf(Mn, m[u]);
        if (Mn == NEG_INF) continue;
        const float c = M == NEG_INF ? 0.0f : expf(M - Mn);
        L *= c;
        acc *= c;
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            const float wgt = m[u] == NEG_INF ? 0.0f : expf(m[u] - Mn);
            L += wgt * l[u];
            acc += wgt * o[u];
        }
        M = Mn;
    }
    out[((int64_t)b * HEADS + h) * D + d] = L > 0.0f ? acc * (1.0f / L) : 0.0f;
}

}  // namespace attn_dev
}  // namespace csa2
