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
// mod 16, g = lane / 16) gathers K channels 32g..32g+31 of entry c and the V
// channel group m = 4(c mod 2) + g (channels 16m..16m+15) of the entry pair
// 2j, 2j+1 (j = c / 2), so each V conversion yields one f16 pair of two
// entries, which is one dword of the transposed V tile.  Scores are computed
// transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_f16 with K as the A operand
// straight from the gathering lane's registers: slice ks of the contraction
// takes channels 32g + 8ks .. +7, the order the lane holds them in, and the
// query slices are staged in LDS in the same order.  The result leaves lane
// (c, g) with the scores of head c for entries 4g..4g+3, which is exactly the
// B-operand layout of O^T = V^T P^T (v_mfma_f32_16x16x16_f16), so the softmax
// weights never move between lanes.  Only V is transposed, through a per-wave
// LDS tile; no barrier is needed inside the loop because every wave touches
// only its own tile.  The next step's records are in flight while a step is
// computed.  Records are read with buffer loads: 32-bit offsets from the
// sequence's base, the constant parts in the instruction.
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
#include "attn_dev.h"

namespace csa2 {

namespace {

using namespace attn_dev;

constexpr int32_t STREAM_WG_TARGET = 1024;  // stream workgroups to aim for per launch

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

// The dispatcher deals workgroups round-robin over the 8 XCDs (workgroup id mod 8),
// each with its own L2.  xcd_work maps a 1-D grid of 8 * ceil(W / 8) workgroups onto
// W query-major work items so that each XCD runs one contiguous range of them: a
// query's tiles, and then its merges, sit on the same XCD or two.  -1 marks the
// padding workgroups.
__device__ __forceinline__ int xcd_work(int id, int W) {
    const int per = (W + 7) >> 3;
    const int work = (id & 7) * per + (id >> 3);
    return work < W ? work : -1;
}

dim3 xcd_grid(int64_t W) { return dim3((unsigned)(8 * ((W + 7) / 8))); }

// One workgroup per (64-entry tile, query), placed by xcd_work.
template <int AM>
__global__ void __launch_bounds__(AT_THREADS) attn_tile_kernel(TileArgs a, int32_t B) {
    __shared__ AttnShared sh;
    const int work = xcd_work(blockIdx.x, B * a.n_tiles);
    if (work < 0) return;
    tile_body<AM>(a, sh, work % a.n_tiles, work / a.n_tiles, threadIdx.x);
}

// ---------------------------------------------------------------------------
// Stream kernel (large batches, bandwidth): see the file header.

// Raw bytes of one step for this lane, loaded ahead of use.
//  main:   r[0..3] K codes of entry c, channels 32g..32g+31; r[4..7] that
//          record's 16 scale bytes; r[8..9] and r[10..11] V codes of channel
//          group m of entries 2j and 2j+1
//  window: r[0..7] K bytes of entry c, channels 32g..32g+31; r[8..11] and
//          r[12..15] V bytes of channels 16m..16m+15 of entries 2j and 2j+1
struct Raw {
    uint32_t r[16];
};



// 4 workgroups (16 waves) per CU: at most 128 VGPRs
template <int AM>
__global__ void __launch_bounds__(AT_THREADS, 4) attn_stream_kernel(StreamArgs a) {
    __shared__ AttnShared sh;
    const int split = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int j = c >> 1, o = c & 1, m = 4 * o + g;    // V: entries 2j, 2j+1, channel group m
    const int32_t s = a.seq[b];
    // tokens of context (window [N - 128, N)); main entries below min(N, cap)
    const int64_t N = clamp64(a.ctx[b], 0, CTX_TOKENS_MAX);
    const int64_t n_main = N < a.cap ? N : a.cap;
    const bool seq_ok = s >= 0 && s < a.n_seq;
    const int64_t u0 = N > WINDOW ? N - WINDOW : 0;
    const int32_t slot0 = window_slot(u0, a.w_cap);         // window slot of position u0
    const int64_t win_base = ((int64_t)a.layer * a.n_seq + (seq_ok ? s : 0)) * a.w_cap;
    // this workgroup's steps [t_begin, t_end); wave w takes t_begin + w, + 4, ...
    // (split x n_sub stays far below 2^32: n_sub <= 264, split < n_sub)
    const int t_begin = (int)((uint32_t)(split * a.n_sub) / (uint32_t)a.n_split);
    const int t_end = (int)((uint32_t)((split + 1) * a.n_sub) / (uint32_t)a.n_split);
    const int main_end = t_end < a.n_sub_main ? t_end : a.n_sub_main;
    const int32_t* idx_row = a.idx + (int64_t)b * a.topk;
    // valid main positions are [0, n_ok) and valid window entries [0, w_ok)
    const uint32_t n_ok = seq_ok ? (uint32_t)(n_main < INT32_MAX ? n_main : INT32_MAX) : 0u;
    const int w_ok = seq_ok ? (int)(N - u0) : 0;
    // uniform bases: the sequence's first record, the query's gathered records
    // and its window rows
    const uint8_t* kv_s = a.kv + (AM != AM_PAGED && seq_ok ? (int64_t)s * a.cap * RECORD : 0);
    const uint8_t* kvg_b = a.kvg_in ? a.kvg_in + (int64_t)b * a.topk * RECORD : nullptr;
    const uint8_t* wk_q = a.wk + win_base * D;
    const uint8_t* wv_q = a.wv + win_base * D;

    // Buffer resources (uniform) for 32-bit-offset loads with the constant
    // parts in the instruction's offset field: the sequence's records (or the
    // query's gathered records), the query's window rows and index list.
    const bool main_buf = kvg_b != nullptr || AM == AM_OFF32;
    const __amdgpu_buffer_rsrc_t rs_main = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kvg_b ? kvg_b : kv_s), 0,
        (int)(kvg_b ? (uint32_t)a.topk * (uint32_t)RECORD
                    : (uint32_t)(AM == AM_OFF32 ? a.cap * RECORD : 0)),
        BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rs_wk =
        __builtin_amdgcn_make_buffer_rsrc((void*)wk_q, 0, a.w_cap * D, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rs_wv =
        __builtin_amdgcn_make_buffer_rsrc((void*)wv_q, 0, a.w_cap * D, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rs_idx =
        __builtin_amdgcn_make_buffer_rsrc((void*)idx_row, 0, a.topk * 4, BUF_DWORD3);

    // index list entry c of step st, loaded one step ahead of its fetch (past
    // the list the load returns 0; fetch discards it)
    auto load_idx = [&](int st) -> int32_t {
        return __builtin_amdgcn_raw_buffer_load_b32(rs_idx, 4 * (SUB * st + c), 0, 0);
    };
    // issue the loads of step st; raw is this lane's index list load (entry c).
    // Returns the validity of entry c and of its partner c ^ 1 (the pair 2j,
    // 2j+1 is (c, partner) for even c, (partner, c) for odd c).
    struct Valid {
        bool c, p;
    };
    auto fetch = [&](int st, int32_t raw, Raw& w) -> Valid {
        if (st < a.n_sub_main) {
            const int32_t pos = (st < main_end && SUB * st + c < a.topk) ? raw : -1;
            const int32_t pos_p = __builtin_amdgcn_mov_dpp(pos, DPP_XOR1, 0xf, 0xf, false);
            const bool okc = (uint32_t)pos < n_ok, okp = (uint32_t)pos_p < n_ok;
            const int32_t pa = o ? pos_p : pos, pb = o ? pos : pos_p;
            const int e = SUB * st + 2 * j;
            u32x4 kc, sc;
            u32x2 va, vb;
            if (main_buf) {
                // an absent entry's offset reads zeros past the buffer, or a
                // record in it that its validity discards
                const uint32_t oa = kvg_b ? (uint32_t)(e < a.topk ? e : 0) * RECORD
                                          : (uint32_t)pa * (uint32_t)RECORD;
                const uint32_t ob = kvg_b ? (uint32_t)(e + 1 < a.topk ? e + 1 : 0) * RECORD
                                          : (uint32_t)pb * (uint32_t)RECORD;
                const uint32_t oc = o ? ob : oa;
                kc = __builtin_amdgcn_raw_buffer_load_b128(rs_main, oc + 16 * g, 0, 0);
                sc = __builtin_amdgcn_raw_buffer_load_b128(rs_main, oc + 128, 0, 0);
                va = __builtin_amdgcn_raw_buffer_load_b64(rs_main, oa + 8 * m + 64, 0, 0);
                vb = __builtin_amdgcn_raw_buffer_load_b64(rs_main, ob + 8 * m + 64, 0, 0);
            } else {
                const bool oka = o ? okp : okc, okb = o ? okc : okp;
                auto rec = [&](int32_t pp, bool ok) -> const uint8_t* {
                    if constexpr (AM == AM_PAGED)
                        return a.kv + (ok ? cache_row<true>(a.pm, a.cap, s, pp) * RECORD : 0);
                    else
                        return kv_s + (ok ? (int64_t)pp * RECORD : 0);
                };
                const uint8_t* ra = rec(pa, oka);
                const uint8_t* rb = rec(pb, okb);
                const uint8_t* rc = o ? rb : ra;
                kc = *reinterpret_cast<const u32x4*>(rc + 16 * g);
                sc = *reinterpret_cast<const u32x4*>(rc + 128);
                va = *reinterpret_cast<const u32x2*>(ra + 64 + 8 * m);
                vb = *reinterpret_cast<const u32x2*>(rb + 64 + 8 * m);
            }
            w.r[0] = kc[0]; w.r[1] = kc[1]; w.r[2] = kc[2]; w.r[3] = kc[3];
            w.r[4] = sc[0]; w.r[5] = sc[1]; w.r[6] = sc[2]; w.r[7] = sc[3];
            w.r[8] = va[0]; w.r[9] = va[1]; w.r[10] = vb[0]; w.r[11] = vb[1];
            w.r[12] = w.r[13] = w.r[14] = w.r[15] = 0u;     // unused by main steps
            return Valid{okc, okp};
        }
        const int off = (st - a.n_sub_main) * SUB;           // + entry < 128 <= w_cap
        // (u0 + off + e) mod w_cap for every entry of the step (absent ones
        // read a row in the window that their validity discards)
        auto wrow = [&](int e) -> uint32_t {
            int32_t sl = slot0 + off + e;
            sl = sl >= a.w_cap ? sl - a.w_cap : sl;
            return (uint32_t)sl * (uint32_t)D;
        };
        const uint32_t ra = wrow(2 * j), rb = wrow(2 * j + 1);
        const uint32_t rc = o ? rb : ra;
        const u32x4 k0 = __builtin_amdgcn_raw_buffer_load_b128(rs_wk, rc + 32 * g, 0, 0);
        const u32x4 k1 = __builtin_amdgcn_raw_buffer_load_b128(rs_wk, rc + 32 * g + 16, 0, 0);
        const u32x4 va = __builtin_amdgcn_raw_buffer_load_b128(rs_wv, ra + 16 * m, 0, 0);
        const u32x4 vb = __builtin_amdgcn_raw_buffer_load_b128(rs_wv, rb + 16 * m, 0, 0);
        w.r[0] = k0[0]; w.r[1] = k0[1]; w.r[2] = k0[2]; w.r[3] = k0[3];
        w.r[4] = k1[0]; w.r[5] = k1[1]; w.r[6] = k1[2]; w.r[7] = k1[3];
        w.r[8] = va[0]; w.r[9] = va[1]; w.r[10] = va[2]; w.r[11] = va[3];
        w.r[12] = vb[0]; w.r[13] = vb[1]; w.r[14] = vb[2]; w.r[15] = vb[3];
        return Valid{off + c < w_ok, off + (c ^ 1) < w_ok};
    };

    // softmax state of head c (lanes c, c+16, c+32, c+48 hold the same m; l is
    // this lane's partial sum) and O^T[d = 16 mt + 4g + r][h = c]
    float m_run = NEG_INF, l_run = 0.0f;
    float4_t o_acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o_acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    uint32_t* vt = sh.st.vt[wave];
    // V^T tile addresses: this lane writes row 16m + t, dword j (t = 0..15) and
    // reads, as the PV A operand, row 16mt + c, dwords 2g, 2g + 1 (mt = 0..7)
    uint32_t* const vt_wr = vt + vt_block(m) + j;
    const uint32_t* const vt_rd = vt + VT_ROW * c + 2 * g;
    // v_perm selector putting the V scale bytes of entries 2j, 2j+1 (byte g of
    // the lane's own dword and of the one received from lane c ^ 1) in order
    const uint32_t vsel = vscale_sel(o, g);
    int st = t_begin + wave;
    // one step in flight: while step i is computed, step i+1's records are
    // arriving (their index list entries were loaded one step earlier)
    Raw cur;
    Valid ok_cur{false, false};
    int32_t idx_next = -1;
    if (st < t_end) {
        ok_cur = fetch(st, load_idx(st), cur);
        idx_next = load_idx(st + AT_WAVES);
    }
    stage_query(sh, a.q + (int64_t)b * HEADS * D, t);
    int qs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qs[ks] = q_slot(ks, lane);
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
            for (int mt = 0; mt < 8; ++mt) o_acc[mt] *= inv;
        }
        const bool ok_c = ok_cur.c;
        const uint64_t vmask = __ballot(ok_c);        // bit e (e < 16): entry e valid
        const bool all_valid = (vmask & 0xffffu) == 0xffffu;
        // ---- dequantise this step: K into A-operand slices, V into f16 pairs
        half8_t kf[4];
        uint32_t vw[16];                      // (V[2j][16m + u], V[2j+1][16m + u]) in vw[u]
        if (is_main) {
            if (a.kvg_out) {
                // this lane's share of the records: entry c's K bytes 16g.. and
                // (g = 0) scale bytes; V group m of entries 2j and 2j+1
                const int e = SUB * st + 2 * j;
                uint8_t* da = a.kvg_out + ((int64_t)b * a.topk + e) * RECORD;
                uint8_t* dc = da + o * RECORD;
                if (ok_c) {
                    *reinterpret_cast<uint4*>(dc + 16 * g) =
                        make_uint4(cur.r[0], cur.r[1], cur.r[2], cur.r[3]);
                    if (g == 0)
                        *reinterpret_cast<uint4*>(dc + 128) =
                            make_uint4(cur.r[4], cur.r[5], cur.r[6], cur.r[7]);
                }
                if (o ? ok_cur.p : ok_cur.c)
                    *reinterpret_cast<uint2*>(da + 64 + 8 * m) = make_uint2(cur.r[8], cur.r[9]);
                if (o ? ok_cur.c : ok_cur.p)
                    *reinterpret_cast<uint2*>(da + RECORD + 64 + 8 * m) =
                        make_uint2(cur.r[10], cur.r[11]);
            }
            dequant_main(cur.r, g, o, vsel, kf, vw);
        } else {
            dequant_window(cur.r, kf, vw);
        }
        if (!all_valid) {
            // absent entries contribute exact zeros whatever their bytes hold
            if (!ok_c) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kf[ks] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
            }
            const bool oka = o ? ok_cur.p : ok_cur.c, okb = o ? ok_cur.c : ok_cur.p;
            const uint32_t keep = (oka ? 0x0000ffffu : 0u) | (okb ? 0xffff0000u : 0u);
#pragma unroll
            for (int u = 0; u < 16; ++u) vw[u] &= keep;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) vt_wr[VT_ROW * u] = vw[u];
        // the V^T tile is private to this wave and LDS executes a wave's
        // operations in order; this only keeps the compiler from moving the
        // tile's reads above its writes
        asm volatile("" ::: "memory");
        // ---- step i+1's loads go out now and overlap the MFMA work below
        const int sn = st + AT_WAVES;
        if (sn < t_end) {
            ok_cur = fetch(sn, idx_next, cur);
            idx_next = load_idx(sn + AT_WAVES);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- S^T = K Q^T: lane (c, g) gets S[head c][entry 4g + r]; the hi and
        // lo halves of the query accumulate in two independent chains
        float4_t shi = {0.f, 0.f, 0.f, 0.f}, slo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], sh.st.q[0][ks][qs[ks]], shi, 0, 0, 0);
            slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], sh.st.q[1][ks][qs[ks]], slo, 0, 0, 0);
        }
        // logits in log2 units (log2(e) folded into the scale): exp2 is one
        // v_exp_f32; m_run is kept in the same units
        const float lscale = a.sm_scale * LOG2E * (is_main ? 1.0f : a.wk_scale);
        float sv[4];
        float tmax = NEG_INF;
        if (all_valid) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sv[r] = (shi[r] + slo[r]) * lscale;
                tmax = fmaxf(tmax, sv[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = (vmask >> (4 * g + r)) & 1u;
                sv[r] = ok ? (shi[r] + slo[r]) * lscale : NEG_INF;
                tmax = fmaxf(tmax, sv[r]);
            }
        }
        tmax = max_xor32(max_xor16(tmax));
        // The reference max moves only when a logit exceeds it by more than
        // RESCALE_SLACK (log2 units), so O is rescaled rarely.  Any reference
        // gives the same softmax; weights stay below 2^RESCALE_SLACK.
        const bool grew = tmax > m_run + RESCALE_SLACK;
        const float m_new = grew ? tmax : m_run;
        half4_t phi, plo;
        float psum = 0.0f;
        float alpha;
        if (all_valid) {
            // m_new is finite here; exp2(-inf) is 0 on the first step
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(sv[r] - m_new);
                psum += p;
                const _Float16 h = (_Float16)p;
                phi[r] = h;
                plo[r] = (_Float16)(p - (float)h);
            }
        } else {
            alpha = m_run == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = sv[r] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(sv[r] - m_new);
                psum += p;
                const _Float16 h = (_Float16)p;
                phi[r] = h;
                plo[r] = (_Float16)(p - (float)h);
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // ---- O^T = O^T * alpha + V^T P^T; alpha is exactly 1 for a head whose
        // running max did not move, so the rescale is skipped when none moved
        if (__ballot(grew)) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o_acc[mt] *= alpha;
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const half4_t vf = *reinterpret_cast<const half4_t*>(vt_rd + vt_block(mt));
            o_acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, phi, o_acc[mt], 0, 0, 0);
            o_acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, plo, o_acc[mt], 0, 0, 0);
        }
        asm volatile("" ::: "memory");     // next step's tile writes after these reads
    }

    if (in_window) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o_acc[mt] *= a.wv_scale;
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

// One workgroup per (head, query), placed by xcd_work; one thread per output dim.
__global__ void __launch_bounds__(D) attn_merge_kernel(const float* part, int32_t n_parts,
                                                       float* out, int32_t B) {
    const int work = xcd_work(blockIdx.x, B * HEADS);
    if (work < 0) return;
    merge_body(part, n_parts, out, work % HEADS, work / HEADS, threadIdx.x);
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
    // 32-bit record offsets while one sequence's records span at most 4 GiB
    const bool off32 = (uint64_t)c.cap * RECORD <= 0xffffffffull;
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
            hipLaunchKernelGGL(attn_tile_kernel<AM_PAGED>, xcd_grid((int64_t)B * a.n_tiles),
                               dim3(AT_THREADS), 0, stream, a, B);
        else if (off32)
            hipLaunchKernelGGL(attn_tile_kernel<AM_OFF32>, xcd_grid((int64_t)B * a.n_tiles),
                               dim3(AT_THREADS), 0, stream, a, B);
        else
            hipLaunchKernelGGL(attn_tile_kernel<AM_FLAT64>, xcd_grid((int64_t)B * a.n_tiles),
                               dim3(AT_THREADS), 0, stream, a, B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_merge_kernel, xcd_grid((int64_t)B * HEADS), dim3(D), 0, stream,
                           partials, a.n_tiles, out, B);
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
        hipLaunchKernelGGL(attn_stream_kernel<AM_PAGED>, dim3(a.n_split, B), dim3(AT_THREADS), 0,
                           stream, a);
    else if (off32)
        hipLaunchKernelGGL(attn_stream_kernel<AM_OFF32>, dim3(a.n_split, B), dim3(AT_THREADS), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(attn_stream_kernel<AM_FLAT64>, dim3(a.n_split, B), dim3(AT_THREADS), 0,
                           stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, xcd_grid((int64_t)B * HEADS), dim3(D), 0, stream,
                       partials, a.n_split, out, B);
    return hipGetLastError();
}

}  // namespace csa2
