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
// Two kernels share the partial format and the merge kernel.  For few queries
// (the decode batches of long contexts) the tile kernel runs one workgroup per
// (query, 64-entry tile) so that every tile's gather starts at once.  For many
// queries the stream kernel below keeps fewer, longer-lived workgroups busy.
//
// Stream kernel (gfx950, wave64): each wave streams 16-entry steps of one query with
// its own online softmax (flash-decoding).  For a step, lane (c, g) (c = lane
// mod 16, g = lane / 16) gathers entry c: 32 K channels 32g..32g+31 and 32 V
// channels {8g + 32k + i}.  Scores are computed transposed, S^T = K Q^T, on
// v_mfma_f32_16x16x16_f16 with K as the A operand straight from the gathering
// lane's registers: the contraction over channels is taken in the order
// d = 32g + 4ks + j, which is the order the lane holds them in, and the query
// fragments are loaded in the same order.  The result leaves lane (c, g) with
// the scores of head c for entries 4g..4g+3, which is exactly the B-operand
// layout of O^T = V^T P^T, so the softmax weights never move between lanes.
// Only V is transposed, through a per-wave LDS tile; no barrier is needed
// inside the loop because every wave touches only its own tile.  The next
// step's records are in flight while a step is computed.
//
// Precision: dequantised values are exact in f16 (an E2M1 value times an E4M3
// scale has at most 6 significant bits, an E4M3 value has 4).  The fp32 query
// and the fp32 softmax weights are split into f16 hi + lo parts and issued as
// two MFMAs, so products are exact and accumulation is fp32.
//
// A workgroup (4 waves) owns a range of a query's steps; the waves' (m, l, O)
// are combined in LDS.  With one workgroup per query (large batches) it writes
// the output directly; otherwise each split writes (m, l, O) partials and the
// merge kernel combines them (the same algebra an unsplit softmax uses), one
// workgroup per (head, query).
//
// Gathered records: a Reuse layer attends over the main rows its group's first
// layer gathered (the main KV is shared by every layer).  With kvg_out a call
// also stores each valid main record it read at [b][j] of a compact buffer;
// with kvg_in a call reads record [b][j] from that buffer, at an address that
// does not wait for the index load, and the index only decides validity.  The
// bytes are the same, so the results are bit-identical.
//
// Dequantisation (both kernels): gfx950's v_cvt_scalef32_pk_f16_fp4 / _fp8 turn
// two codes into two exact f16 values per instruction; the E4M3 group scale is
// then one packed f16 multiply, exact (at most 6 significant bits).
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int AT_THREADS = 256;
constexpr int AT_WAVES = AT_THREADS / 64;
constexpr int SUB = 16;                   // entries per wave step
constexpr int32_t STREAM_WG_TARGET = 1024;  // stream workgroups to aim for per launch
constexpr int VT_STRIDE = 24;             // f16 per transposed V row (16 entries + 8 pad):
                                          // conflict-free packed writes and operand reads
constexpr float NEG_INF = -__builtin_huge_valf();
// floats per head row of the waves' O in LDS when they are combined: the 16
// lanes that write one 16-byte piece of 16 heads' rows at once land on 16
// distinct bank groups (a 128-float row would put all 16 on the same one)
constexpr int OROW = D + 4;
// tile kernel (small batches): used while B x tiles fits one wave of workgroups
constexpr int64_t TILE_KERNEL_MAX_WG = 768;
constexpr int TILE = 64;

struct StreamArgs {
    const uint8_t* kv;
    const uint8_t* kvg_in;   // [B][topk][RECORD] gathered main records, or null
    uint8_t* kvg_out;        // where to store the gathered main records, or null
    const uint8_t* wk;
    const uint8_t* wv;
    const float* q;
    const int32_t* idx;
    const int32_t* seq;
    const int64_t* ctx;
    float* part;             // [B][n_split][ATTN_PART_FLOATS] when n_split > 1
    float* out;              // [B][16][128] when n_split == 1
    int64_t cap;
    PageMap pm;              // page table of a paged cache (table null otherwise)
    int32_t n_seq;
    int32_t w_cap;
    int32_t layer;
    int32_t topk;
    int32_t n_sub_main;      // steps over the index list
    int32_t n_sub;           // plus the window's steps
    int32_t n_split;         // workgroups per query
    float wk_scale;
    float wv_scale;
    float sm_scale;
};

struct StreamShared {
    union {
        struct {
            _Float16 vt[AT_WAVES][D * VT_STRIDE];  // per-wave V^T of one step
            half4_t q[2][8][64];                   // query fragments (hi, lo) per ks, per lane
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
// step of the stream kernel's loop (below): lane (c, g) gathers its entry's K
// channels 32g..32g+31 and V channels {8g + 32k + i}, S^T = K Q^T comes out of
// MFMA with K straight from the gathering lane's registers (here as
// v_mfma_f32_16x16x32_f16, four K = 32 slices of the contraction), the
// softmax weights stay where S^T left them as the B operand of O^T = V^T P^T,
// and only V is transposed, through the wave's own LDS tile.  The 4 waves'
// (m, l, O) are combined in LDS and the tile writes one partial record.
// The index load is issued first and the query's loads right after it, so
// the query's conversion overlaps the record loads.

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

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

struct TileShared {
    union {
        struct {
            _Float16 vt[AT_WAVES][D * VT_STRIDE];  // per-wave V^T of its 16 entries
            half8_t q[2][4][64];                   // query slices (hi, lo) per lane
        } st;
        struct {
            float o[AT_WAVES][HEADS * OROW];
            float m[AT_WAVES][HEADS];
            float l[AT_WAVES][HEADS];
        } mg;                                      // the waves' softmax states
    };
};

template <bool PAGED>
__global__ void __launch_bounds__(AT_THREADS) attn_tile_kernel(TileArgs a) {
    __shared__ TileShared sh;
    const int tile = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int c = lane & 15, g = lane >> 4;
    const bool is_main = tile < a.n_main;
    // this lane's entry: index j of the list (main) or offset `off` in the window
    const int j = tile * TILE + 16 * wave + c;
    const int off = (tile - a.n_main) * TILE + 16 * wave + c;   // window tiles: < 128 <= w_cap

    // ---- loads in order of need: the index (and the query's sequence and
    // length), the query, then the records
    int32_t pos = -1;
    if (is_main && j < a.topk) pos = a.idx[(int64_t)b * a.topk + j];
    const int32_t s = a.seq[b];
    const int64_t N = clamp64(a.ctx[b], 0, a.cap);
    const bool seq_ok = s >= 0 && s < a.n_seq;
    // the query, once per workgroup and coalesced: two float4 per thread
    float4 qv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
        qv[k] = *reinterpret_cast<const float4*>(a.q + (int64_t)b * HEADS * D +
                                                  4 * (t + AT_THREADS * k));

    // ---- per kind of tile: the record (or window row) loads, the query's
    // conversion while they are in flight, then the dequantisation.  Each
    // branch consumes everything it loads, so no load is pending where the
    // branches join (a pending load there would make the compiler wait for all
    // of them before the first record load).
    half8_t kf[4];                        // K: A-operand slices of S^T = K Q^T
    uint32_t vv[16];                      // V f16x2: channels 8g+32k+2i, +1 in vv[4k+i]
    // q as f16 hi + lo in the B-operand slices of S^T = K Q^T: slice sl of
    // lane (c, g) takes channels 32g + 8 sl .. +7 of head c; each float4 goes
    // to the lane, slice and half that take it (read back after a barrier)
    auto convert_q = [&]() {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = 4 * (t + AT_THREADS * k);          // h * 128 + d, d % 4 == 0
            const int h = e >> 7, d = e & (D - 1);
            const float x[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
            half4_t hi4, lo4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16 hi = (_Float16)x[i];
                hi4[i] = hi;
                lo4[i] = (_Float16)(x[i] - (float)hi);
            }
            const int fl = 16 * (d >> 5) + h, sl = (d >> 3) & 3;
            _Float16* qh = reinterpret_cast<_Float16*>(&sh.st.q[0][sl][fl]) + (d & 4);
            _Float16* ql = reinterpret_cast<_Float16*>(&sh.st.q[1][sl][fl]) + (d & 4);
            *reinterpret_cast<half4_t*>(qh) = hi4;
            *reinterpret_cast<half4_t*>(ql) = lo4;
        }
    };
    bool ok;
    if (is_main) {
        // r[0..3] K codes of channels 32g.., r[4..7] V codes of channels
        // 8g+32k..+7, r[8..11] the record's 16 scale bytes
        ok = seq_ok && pos >= 0 && pos < N;
        const uint8_t* rec =
            a.kvg_in ? a.kvg_in + ((int64_t)b * a.topk + (j < a.topk ? j : 0)) * RECORD
                     : a.kv + (ok ? cache_row<PAGED>(a.pm, a.cap, s, pos) * RECORD : 0);
        uint32_t r[12];
        const uint4 kc = *reinterpret_cast<const uint4*>(rec + 16 * g);
        const uint4 sc = *reinterpret_cast<const uint4*>(rec + 128);
        r[0] = kc.x; r[1] = kc.y; r[2] = kc.z; r[3] = kc.w;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r[4 + k] = *reinterpret_cast<const uint32_t*>(rec + 64 + 4 * g + 16 * k);
        r[8] = sc.x; r[9] = sc.y; r[10] = sc.z; r[11] = sc.w;
        convert_q();
        if (a.kvg_out && ok) {
            // this lane's share of the record: K bytes 16g.., V dwords 64 + 4g +
            // 16k, and (g = 0) the 16 scale bytes
            uint8_t* dst = a.kvg_out + ((int64_t)b * a.topk + j) * RECORD;
            *reinterpret_cast<uint4*>(dst + 16 * g) = make_uint4(r[0], r[1], r[2], r[3]);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<uint32_t*>(dst + 64 + 4 * g + 16 * k) = r[4 + k];
            if (g == 0)
                *reinterpret_cast<uint4*>(dst + 128) = make_uint4(r[8], r[9], r[10], r[11]);
        }
        // K scales of groups 2g, 2g+1 (adjacent bytes); V scales of groups
        // 2k + g/2, k = 0..3 (bytes g/2, g/2 + 2, ... of the V scale block)
        const half2_t ks2 = fp8x2_h2<false>(((g >> 1) ? r[9] : r[8]) >> (16 * (g & 1)));
        const uint32_t gh = (uint32_t)(g >> 1);
        const uint32_t vsel = gh | ((2u + gh) << 8) | ((4u + gh) << 16) | ((6u + gh) << 24);
        const uint32_t vsb = __builtin_amdgcn_perm(r[11], r[10], vsel);
        const half2_t vs01 = fp8x2_h2<false>(vsb), vs23 = fp8x2_h2<true>(vsb);
        const half2_t k0 = half2_t{ks2.x, ks2.x}, k1 = half2_t{ks2.y, ks2.y};
        const half2_t vsc[4] = {half2_t{vs01.x, vs01.x}, half2_t{vs01.y, vs01.y},
                                half2_t{vs23.x, vs23.x}, half2_t{vs23.y, vs23.y}};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w4[4];
            fp4x8_scaled(r[i], i < 2 ? k0 : k1, w4);
            kf[i] = __builtin_bit_cast(half8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) fp4x8_scaled(r[4 + k], vsc[k], vv + 4 * k);
    } else {
        // r[0..7] K bytes of channels 32g.., r[8..15] V bytes of channels 8g+32k..+7
        const int64_t u0 = N > WINDOW ? N - WINDOW : 0;
        ok = seq_ok && u0 + off < N;
        // (u0 + off) mod w_cap from the uniform u0 mod w_cap: one subtract
        int32_t w = (int32_t)(u0 % a.w_cap) + off;
        w = w >= a.w_cap ? w - a.w_cap : w;
        const int64_t row = ok ? (((int64_t)a.layer * a.n_seq + s) * a.w_cap + w) * D : 0;
        uint32_t r[16];
        const uint4 k0 = *reinterpret_cast<const uint4*>(a.wk + row + 32 * g);
        const uint4 k1 = *reinterpret_cast<const uint4*>(a.wk + row + 32 * g + 16);
        r[0] = k0.x; r[1] = k0.y; r[2] = k0.z; r[3] = k0.w;
        r[4] = k1.x; r[5] = k1.y; r[6] = k1.z; r[7] = k1.w;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint2 v = *reinterpret_cast<const uint2*>(a.wv + row + 8 * g + 32 * k);
            r[8 + 2 * k] = v.x;
            r[9 + 2 * k] = v.y;
        }
        convert_q();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a0 = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(r[2 * i]));
            const uint32_t a1 = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(r[2 * i]));
            const uint32_t a2 = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(r[2 * i + 1]));
            const uint32_t a3 = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(r[2 * i + 1]));
            kf[i] = __builtin_bit_cast(half8_t, make_uint4(a0, a1, a2, a3));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            vv[4 * k] = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(r[8 + 2 * k]));
            vv[4 * k + 1] = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(r[8 + 2 * k]));
            vv[4 * k + 2] = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(r[9 + 2 * k]));
            vv[4 * k + 3] = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(r[9 + 2 * k]));
        }
    }
    if (!ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) vv[i] = 0u;
    }
    const uint64_t vmask = __ballot(ok);        // bit e (e < 16): entry e of the wave valid

    // ---- V^T into the wave's LDS tile: lanes c and c^1 swap halves so that
    // each writes one dword of two entries (row stride VT_STRIDE: conflict free)
    _Float16* vt = sh.st.vt[wave];
    {
        const uint32_t pair_sel = (c & 1) ? 0x03020706u : 0x05040100u;
        const int vt_w = (c & 1) ? VT_STRIDE + (c - 1) : c;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = vv[4 * k + i];
                const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, DPP_XOR1, 0xf, 0xf,
                                                                      false);
                const int d = 8 * g + 32 * k + 2 * i;
                *reinterpret_cast<uint32_t*>(vt + vt_w + d * VT_STRIDE) =
                    __builtin_amdgcn_perm(y, x, pair_sel);
            }
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
        for (int sl = 0; sl < 4; ++sl) {
            shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[sl], sh.st.q[0][sl][lane], shi, 0, 0,
                                                         0);
            slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[sl], sh.st.q[1][sl][lane], slo, 0, 0,
                                                         0);
        }
        sacc = shi + slo;
    }
    // logits in log2 units (log2(e) folded into the scale): exp2 is one v_exp_f32
    const float lscale = a.sm_scale * LOG2E * (is_main ? 1.0f : a.wk_scale);
    float sv[4];
    float m = NEG_INF;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const bool v_ok = (vmask >> (4 * g + q4)) & 1u;
        sv[q4] = v_ok ? sacc[q4] * lscale : NEG_INF;
        m = fmaxf(m, sv[q4]);
    }
    m = max_xor32(max_xor16(m));                // the wave's max for head c
    half4_t phi, plo;
    float lsum = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float p = sv[q4] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(sv[q4] - m);
        lsum += p;
        const _Float16 h = (_Float16)p;
        phi[q4] = h;
        plo[q4] = (_Float16)(p - (float)h);
    }
    lsum = add_xor32(add_xor16(lsum));

    // ---- O^T = V^T P^T over the wave's 16 entries: O^T[d = 16 mt + 4g + r][h = c]
    float4_t o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const half4_t vf = *reinterpret_cast<const half4_t*>(&vt[(16 * mt + c) * VT_STRIDE + 4 * g]);
        float4_t acc = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, phi, float4_t{0.f, 0.f, 0.f, 0.f},
                                                             0, 0, 0);
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, plo, acc, 0, 0, 0);
    }

    // ---- combine the 4 waves in LDS and write the tile's partial record
    __syncthreads();                            // every wave is done with its V^T tile
    if (g == 0) {
        sh.mg.m[wave][c] = m;
        sh.mg.l[wave][c] = lsum;
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<float4_t*>(&sh.mg.o[wave][c * OROW + 16 * mt + 4 * g]) = o[mt];
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

// ---------------------------------------------------------------------------
// Stream kernel (large batches, bandwidth): see the file header.

// Raw bytes of one step's entry for this lane, loaded ahead of use.
//  main:   r[0..3] K codes of channels 32g..32g+31, r[4..7] V codes of channels
//          8g+32k..8g+32k+7 (k = 0..3), r[8..11] the record's 16 scale bytes
//  window: r[0..7] K bytes of channels 32g..32g+31, r[8..15] V bytes of
//          channels 8g+32k..+7 (two dwords per k)
struct Raw {
    uint32_t r[16];
};

// 4 workgroups (16 waves) per CU: at most 128 VGPRs
template <bool PAGED>
__global__ void __launch_bounds__(AT_THREADS, 4) attn_stream_kernel(StreamArgs a) {
    __shared__ StreamShared sh;
    const int split = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int32_t s = a.seq[b];
    const int64_t N = clamp64(a.ctx[b], 0, a.cap);
    const bool seq_ok = s >= 0 && s < a.n_seq;
    const int64_t u0 = N > WINDOW ? N - WINDOW : 0;
    const int32_t slot0 = (int32_t)(u0 % a.w_cap);         // window slot of position u0
    const int64_t win_base = ((int64_t)a.layer * a.n_seq + (seq_ok ? s : 0)) * a.w_cap;
    // this workgroup's steps [t_begin, t_end); wave w takes t_begin + w, + 4, ...
    const int t_begin = (int)((int64_t)split * a.n_sub / a.n_split);
    const int t_end = (int)((int64_t)(split + 1) * a.n_sub / a.n_split);
    const int main_end = t_end < a.n_sub_main ? t_end : a.n_sub_main;
    const int32_t* idx_row = a.idx + (int64_t)b * a.topk;


    auto load_idx = [&](int st) -> int32_t {
        const int j = SUB * st + c;
        return (st < main_end && j < a.topk) ? idx_row[j] : -1;
    };
    // issue the loads of step st for this lane; returns whether the entry is valid
    auto fetch = [&](int st, int32_t pos, Raw& w) -> bool {
#pragma unroll
        for (int i = 0; i < 16; ++i) w.r[i] = 0u;
        if (st < a.n_sub_main) {
            const bool ok = seq_ok && pos >= 0 && pos < N;
            const int j = SUB * st + c;
            const uint8_t* rec =
                a.kvg_in ? a.kvg_in + ((int64_t)b * a.topk + (j < a.topk ? j : 0)) * RECORD
                         : a.kv + (ok ? cache_row<PAGED>(a.pm, a.cap, s, pos) * RECORD : 0);
            const uint4 kc = *reinterpret_cast<const uint4*>(rec + 16 * g);
            const uint4 sc = *reinterpret_cast<const uint4*>(rec + 128);
            w.r[0] = kc.x; w.r[1] = kc.y; w.r[2] = kc.z; w.r[3] = kc.w;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w.r[4 + k] = *reinterpret_cast<const uint32_t*>(rec + 64 + 4 * g + 16 * k);
            w.r[8] = sc.x; w.r[9] = sc.y; w.r[10] = sc.z; w.r[11] = sc.w;
            return ok;
        }
        const int off = (st - a.n_sub_main) * SUB + c;      // < 128 <= w_cap
        const bool ok = seq_ok && u0 + off < N;
        int32_t slot = slot0 + off;                          // (u0 + off) mod w_cap
        slot = slot >= a.w_cap ? slot - a.w_cap : slot;
        const int64_t row = ok ? (win_base + slot) * D : 0;
        const uint4 k0 = *reinterpret_cast<const uint4*>(a.wk + row + 32 * g);
        const uint4 k1 = *reinterpret_cast<const uint4*>(a.wk + row + 32 * g + 16);
        w.r[0] = k0.x; w.r[1] = k0.y; w.r[2] = k0.z; w.r[3] = k0.w;
        w.r[4] = k1.x; w.r[5] = k1.y; w.r[6] = k1.z; w.r[7] = k1.w;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint2 v = *reinterpret_cast<const uint2*>(a.wv + row + 8 * g + 32 * k);
            w.r[8 + 2 * k] = v.x;
            w.r[9 + 2 * k] = v.y;
        }
        return ok;
    };

    // softmax state of head c (lanes c, c+16, c+32, c+48 hold the same m; l is
    // this lane's partial sum) and O^T[d = 16 mt + 4g + r][h = c]
    float m_run = NEG_INF, l_run = 0.0f;
    float4_t o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    _Float16* vt = sh.st.vt[wave];

    // packed V^T writes: byte selector (even lane: own low half, then the
    // neighbour's low half; odd lane: the neighbour's high half, then its own)
    // and the lane's offset inside the tile
    const uint32_t pair_sel = (c & 1) ? 0x03020706u : 0x05040100u;
    const int vt_w = (c & 1) ? VT_STRIDE + (c - 1) : c;
    // v_perm selector gathering V scale bytes g/2, g/2 + 2, g/2 + 4, g/2 + 6 of
    // the record's 8-byte V scale block (dwords r[10], r[11])
    const uint32_t gh = (uint32_t)(g >> 1);
    const uint32_t vsel = gh | ((2u + gh) << 8) | ((4u + gh) << 16) | ((6u + gh) << 24);
    int st = t_begin + wave;
    // two steps in flight: while step i is computed, step i+1 is arriving and
    // step i+2 is issued (its index list entries were loaded one step earlier)
    Raw cur, nxt;
    bool ok_cur = false, ok_nxt = false;
    int32_t idx_next = -1;
    if (st < t_end) {
        ok_cur = fetch(st, load_idx(st), cur);
        idx_next = load_idx(st + AT_WAVES);
    }
    // ---- query fragments (B operand of S^T = K Q^T): Q[h = c][32g + 4ks + j],
    // split into f16 hi + lo; built after the first steps' loads were issued,
    // so the two latencies overlap.  Every wave uses the same fragments: the
    // workgroup loads the query once, coalesced (two float4 per thread), and
    // stores each float4 as the half4 of the lane and ks that take it (in lane
    // order, so the per-step reads are conflict free).
    {
        float4 qv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
            qv[k] = *reinterpret_cast<const float4*>(a.q + (int64_t)b * HEADS * D +
                                                      4 * (t + AT_THREADS * k));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = 4 * (t + AT_THREADS * k);          // h * 128 + d, d % 4 == 0
            const int h = e >> 7, d = e & (D - 1);
            const float x[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
            half4_t hi4, lo4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16 hi = (_Float16)x[i];
                hi4[i] = hi;
                lo4[i] = (_Float16)(x[i] - (float)hi);
            }
            const int fl = 16 * (d >> 5) + h, ks = (d >> 2) & 7;
            sh.st.q[0][ks][fl] = hi4;
            sh.st.q[1][ks][fl] = lo4;
        }
    }
    __syncthreads();
    // The window's per-tensor V scale multiplies the PV products of window
    // steps only.  A wave takes its main steps before its window steps, so O is
    // divided by the scale before its first window step and multiplied back
    // after the loop: the softmax weights enter the f16 split unscaled, which
    // keeps them inside f16 whatever the scale.
    bool in_window = false;
    for (; st < t_end; st += AT_WAVES) {
        const bool is_main = st < a.n_sub_main;
        if (!is_main && !in_window) {
            in_window = true;
            const float inv = 1.0f / a.wv_scale;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt] *= inv;
        }
        // ---- dequantise this step: K into A-operand fragments, V into LDS (V^T)
        half4_t kf[8];
        uint32_t vv[16];                      // f16x2: channels 8g+32k+2i, +1 in vv[4k+i]
        if (is_main && a.kvg_out && ok_cur) {
            // this lane's share of the record: K bytes 16g.., V dwords
            // 64 + 4g + 16k, and (g = 0) the 16 scale bytes
            uint8_t* dst = a.kvg_out + ((int64_t)b * a.topk + SUB * st + c) * RECORD;
            *reinterpret_cast<uint4*>(dst + 16 * g) =
                make_uint4(cur.r[0], cur.r[1], cur.r[2], cur.r[3]);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<uint32_t*>(dst + 64 + 4 * g + 16 * k) = cur.r[4 + k];
            if (g == 0)
                *reinterpret_cast<uint4*>(dst + 128) =
                    make_uint4(cur.r[8], cur.r[9], cur.r[10], cur.r[11]);
        }
        if (is_main) {
            // K scales of groups 2g, 2g+1 (adjacent bytes); V scales of groups
            // 2k + g/2, k = 0..3 (bytes g/2, g/2 + 2, ... of the V scale block)
            const half2_t ks2 =
                fp8x2_h2<false>(((g >> 1) ? cur.r[9] : cur.r[8]) >> (16 * (g & 1)));
            const uint32_t vsb = __builtin_amdgcn_perm(cur.r[11], cur.r[10], vsel);
            const half2_t vs01 = fp8x2_h2<false>(vsb), vs23 = fp8x2_h2<true>(vsb);
            const half2_t k0 = half2_t{ks2.x, ks2.x}, k1 = half2_t{ks2.y, ks2.y};
            const half2_t vsc[4] = {half2_t{vs01.x, vs01.x}, half2_t{vs01.y, vs01.y},
                                    half2_t{vs23.x, vs23.x}, half2_t{vs23.y, vs23.y}};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t w4[4];
                fp4x8_scaled(cur.r[i], i < 2 ? k0 : k1, w4);
                kf[2 * i] = __builtin_bit_cast(half4_t, make_uint2(w4[0], w4[1]));
                kf[2 * i + 1] = __builtin_bit_cast(half4_t, make_uint2(w4[2], w4[3]));
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) fp4x8_scaled(cur.r[4 + k], vsc[k], vv + 4 * k);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kf[i] = __builtin_bit_cast(
                    half4_t, make_uint2(__builtin_bit_cast(uint32_t, fp8x2_h2<false>(cur.r[i])),
                                        __builtin_bit_cast(uint32_t, fp8x2_h2<true>(cur.r[i]))));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vv[4 * k] = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(cur.r[8 + 2 * k]));
                vv[4 * k + 1] = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(cur.r[8 + 2 * k]));
                vv[4 * k + 2] = __builtin_bit_cast(uint32_t, fp8x2_h2<false>(cur.r[9 + 2 * k]));
                vv[4 * k + 3] = __builtin_bit_cast(uint32_t, fp8x2_h2<true>(cur.r[9 + 2 * k]));
            }
        }
        if (!ok_cur) {
#pragma unroll
            for (int i = 0; i < 8; ++i) kf[i] = half4_t{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 16; ++i) vv[i] = 0u;
        }
        const uint64_t vmask = __ballot(ok_cur);     // bit e (e < 16): entry e valid
        {
            // lanes c and c^1 swap halves so that each writes one dword of two
            // entries: the even lane (V[c][d], V[c+1][d]) into row d, the odd
            // lane (V[c-1][d+1], V[c][d+1]) into row d+1
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = vv[4 * k + i];
                    const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, DPP_XOR1, 0xf, 0xf,
                                                                          false);
                    const int d = 8 * g + 32 * k + 2 * i;
                    *reinterpret_cast<uint32_t*>(vt + vt_w + d * VT_STRIDE) =
                        __builtin_amdgcn_perm(y, x, pair_sel);
                }
        }
        // the V^T tile is private to this wave and LDS executes a wave's
        // operations in order; this only keeps the compiler from moving the
        // tile's reads above its writes
        asm volatile("" ::: "memory");
        // ---- step i+2's loads go out now and overlap the MFMA work below
        const int sn = st + AT_WAVES;
        if (sn < t_end) {
            ok_nxt = fetch(sn, idx_next, nxt);
            idx_next = load_idx(sn + AT_WAVES);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- S^T = K Q^T: lane (c, g) gets S[head c][entry 4g + r]
        float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(kf[ks], sh.st.q[0][ks][lane], sacc, 0,
                                                         0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(kf[ks], sh.st.q[1][ks][lane], sacc, 0,
                                                         0, 0);
        }
        // logits in log2 units (log2(e) folded into the scale): exp2 is one
        // v_exp_f32; m_run is kept in the same units
        const float lscale = a.sm_scale * LOG2E * (is_main ? 1.0f : a.wk_scale);
        float sv[4];
        float tmax = NEG_INF;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = (vmask >> (4 * g + r)) & 1u;
            sv[r] = ok ? sacc[r] * lscale : NEG_INF;
            tmax = fmaxf(tmax, sv[r]);
        }
        tmax = max_xor32(max_xor16(tmax));
        // The reference max moves only when a logit exceeds it by more than
        // RESCALE_SLACK (log2 units), so O is rescaled rarely.  Any reference
        // gives the same softmax; weights stay below 2^RESCALE_SLACK.
        const bool grew = tmax > m_run + RESCALE_SLACK;
        const float m_new = grew ? tmax : m_run;
        const float alpha = m_run == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        half4_t phi, plo;
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = sv[r] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(sv[r] - m_new);
            psum += p;
            const _Float16 h = (_Float16)p;
            phi[r] = h;
            plo[r] = (_Float16)(p - (float)h);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // ---- O^T = O^T * alpha + V^T P^T; alpha is exactly 1 for a head whose
        // running max did not move, so the rescale is skipped when none moved
        if (__ballot(grew)) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const half4_t vf =
                *reinterpret_cast<const half4_t*>(&vt[(16 * mt + c) * VT_STRIDE + 4 * g]);
            o[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, phi, o[mt], 0, 0, 0);
            o[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, plo, o[mt], 0, 0, 0);
        }
        cur = nxt;
        ok_cur = ok_nxt;
        asm volatile("" ::: "memory");     // next step's tile writes after these reads
    }

    if (in_window) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[mt] *= a.wv_scale;
    }

    // ---- combine the 4 waves: l over the 4 lanes of a head, then LDS
    l_run = add_xor32(add_xor16(l_run));
    __syncthreads();                       // every wave is done with its V^T tile
    if (g == 0) {
        sh.mg.m[wave][c] = m_run;
        sh.mg.l[wave][c] = l_run;
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<float4_t*>(&sh.mg.o[wave][c * OROW + 16 * mt + 4 * g]) = o[mt];
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
        if (a.n_split == 1) {
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            float4* dst = reinterpret_cast<float4*>(a.out + ((int64_t)b * HEADS + h) * D + d0);
            dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
            dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
        } else {
            float* part = a.part + ((int64_t)b * a.n_split + split) * ATTN_PART_FLOATS;
            if ((t & 15) == 0) {
                part[h] = M * LN2;           // partials carry natural-log maxima
                part[HEADS + h] = L;
            }
            float4* dst = reinterpret_cast<float4*>(part + 2 * HEADS + h * D + d0);
            dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

// Combine the partials of each query: out = sum_t e^(m_t - M) o_t / sum_t e^(m_t - M) l_t.
// One workgroup per (head, query) and one thread per output dim, so the partial
// loads spread over B x 16 compute units; each thread loads its dim of up to
// MERGE_BATCH partials at once (one memory round trip for the 10 tiles of top-512).
constexpr int MERGE_BATCH = 12;

__global__ void __launch_bounds__(D) attn_merge_kernel(const float* part, int32_t n_parts,
                                                       float* out) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
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

}  // namespace

namespace {

// Launch shape of one call: the tile kernel while B x tiles fits one wave of
// workgroups, else the stream kernel with about one workgroup per resident slot
// (256 CUs x 4) and at least one step per wave.
struct AttnPlan {
    bool tile;
    int32_t n_split;         // workgroups (partial records) per query
};

// max_parts caps the partial records (a fixed scratch): the stream kernel's
// split is lowered until B x split fits, down to one workgroup per query,
// which writes no partials.  The tile kernel's B x tiles <= 768 records must
// fit the cap (callers pass at least that many).
AttnPlan attn_plan(int32_t B, int32_t topk, int64_t max_parts) {
    const int32_t n_tiles = (topk + TILE - 1) / TILE + WINDOW / TILE;
    if ((int64_t)B * n_tiles <= TILE_KERNEL_MAX_WG) return {true, n_tiles};
    const int32_t n_sub = (topk + SUB - 1) / SUB + WINDOW / SUB;
    const int32_t max_split = (n_sub + AT_WAVES - 1) / AT_WAVES;
    int32_t split = (STREAM_WG_TARGET + B - 1) / B;
    split = split < 1 ? 1 : (split > max_split ? max_split : split);
    if (split > 1 && (int64_t)B * split > max_parts) {
        const int64_t fit = max_parts / B;
        split = fit < 2 ? 1 : (int32_t)fit;
    }
    return {false, split};
}

}  // namespace

int64_t attn_partials(int32_t B, int32_t topk, int64_t max_parts) {
    const AttnPlan p = attn_plan(B, topk, max_parts);
    return p.n_split > 1 ? (int64_t)B * p.n_split : 0;
}

hipError_t launch_attn(const csa2_cache& c, const csa2_window& w, int32_t layer,
                       const float* q, const int32_t* idx, const int32_t* seq,
                       const int64_t* ctx, int32_t B, int32_t topk, float sm_scale,
                       const uint8_t* kvg_in, uint8_t* kvg_out, float* out, float* partials,
                       int64_t max_parts, hipStream_t stream) {
    const AttnPlan p = attn_plan(B, topk, max_parts);
    if (p.tile) {
        // few queries: one workgroup per 64-entry tile, the shortest dependency chain
        TileArgs a{};
        a.kv = c.kv;
        a.kvg_in = kvg_in;
        a.kvg_out = kvg_out;
        a.wk = w.k;
        a.wv = w.v;
        a.q = q;
        a.idx = idx;
        a.seq = seq;
        a.ctx = ctx;
        a.part = partials;
        a.cap = c.cap;
        a.pm = page_map(c);
        a.n_seq = c.n_seq;
        a.w_cap = w.w_cap;
        a.layer = layer;
        a.topk = topk;
        a.n_main = (topk + TILE - 1) / TILE;
        a.n_tiles = p.n_split;
        a.wk_scale = w.k_scale;
        a.wv_scale = w.v_scale;
        a.sm_scale = sm_scale;
        if (c.page_table)
            hipLaunchKernelGGL(attn_tile_kernel<true>, dim3(a.n_tiles, B), dim3(AT_THREADS), 0,
                               stream, a);
        else
            hipLaunchKernelGGL(attn_tile_kernel<false>, dim3(a.n_tiles, B), dim3(AT_THREADS), 0,
                               stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_merge_kernel, dim3(HEADS, B), dim3(D), 0, stream, partials,
                           a.n_tiles, out);
        return hipGetLastError();
    }
    StreamArgs a{};
    a.kv = c.kv;
    a.kvg_in = kvg_in;
    a.kvg_out = kvg_out;
    a.wk = w.k;
    a.wv = w.v;
    a.q = q;
    a.idx = idx;
    a.seq = seq;
    a.ctx = ctx;
    a.part = partials;
    a.out = out;
    a.cap = c.cap;
    a.pm = page_map(c);
    a.n_seq = c.n_seq;
    a.w_cap = w.w_cap;
    a.layer = layer;
    a.topk = topk;
    a.wk_scale = w.k_scale;
    a.wv_scale = w.v_scale;
    a.sm_scale = sm_scale;
    a.n_sub_main = (topk + SUB - 1) / SUB;
    a.n_sub = a.n_sub_main + WINDOW / SUB;
    a.n_split = p.n_split;
    if (c.page_table)
        hipLaunchKernelGGL(attn_stream_kernel<true>, dim3(a.n_split, B), dim3(AT_THREADS), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(attn_stream_kernel<false>, dim3(a.n_split, B), dim3(AT_THREADS), 0,
                           stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(HEADS, B), dim3(D), 0, stream, partials,
                       a.n_split, out);
    return hipGetLastError();
}

}  // namespace csa2
