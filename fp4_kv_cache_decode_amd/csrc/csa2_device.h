// Device helpers shared by the libcsa2 kernels (gfx950 / CDNA4, wave64).
//
// Number formats (see include/csa2.h for the record layout):
//  * E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, max 448,
//    exponent 0 subnormal with step 2^-9, 0x7F/0xFF NaN.
//  * E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, values
//    {0, .5, 1, 1.5, 2, 3, 4, 6}.
// The pages fix the formats (FP4 E2M1 with one E4M3 scale per 16 channels,
// FP8 window): trawling.dev "CSA2 and FP4 KV caching"; origotech.dev deep dive,
// "FP4 and SWA Bounded Replay".  Rounding is round-to-nearest-even with
// saturation, the sign of the input kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int D = 128;
constexpr int HEADS = 16;
constexpr int IDX_HEADS = 4;
constexpr int IDX_DIM = 64;
constexpr int WINDOW = 128;
constexpr int RECORD = 144;
constexpr int BLOCK = 8;

// ---------------------------------------------------------------- E4M3 encode
// Round a finite fp32 to E4M3FN, nearest-even, saturating at 448, sign kept.
// Works on the fp32 bit pattern: in the normal range the 23-bit mantissa is
// rounded to 3 bits with the carry allowed to ripple into the exponent; below
// 2^-6 the value is scaled by 2^9 (exact) and rounded to an integer step count.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    uint32_t u = __float_as_uint(y);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x43e00000u) {                 // |y| >= 448
        code = 0x7eu;
    } else if (a < 0x3c800000u) {           // |y| < 2^-6: subnormal grid
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // 0..8
    } else {
        uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);                    // RNE at bit 20
        code = (r >> 20) - (120u << 3);                                  // rebias 127 -> 7
    }
    return sign | code;
}

// Exact fp32 value of a non-negative E4M3 code (used for the FP4 group scale).
__device__ __forceinline__ float e4m3_value_pos(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
}

// ---------------------------------------------------------------- E2M1 encode
// Magnitude code of |x| on the grid s*{0,.5,1,1.5,2,3,4,6}: count the rounding
// thresholds s*{.25,.75,1.25,1.75,2.5,3.5,5} that |x| passes.  At an exact
// threshold the even code wins, so odd-to-even boundaries use >= and
// even-to-odd ones use >.  The products have at most 7 significant bits and
// are exact in fp32, so this is exact round-to-nearest-even of x/s with no
// division.  Above 5*s everything maps to code 7 (saturation).
__device__ __forceinline__ uint32_t e2m1_mag(float a, float s) {
    uint32_t m = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) +
                 (a > 2.5f * s) + (a >= 3.5f * s) + (a > 5.0f * s);
    return s == 0.0f ? 0u : m;
}

// f16 bit pattern of an E2M1 nibble (sign kept).
__device__ __forceinline__ uint32_t e2m1_to_f16_bits(uint32_t nib) {
    uint32_t mag = nib & 7u;
    uint32_t bits = (mag >= 2u) ? ((mag << 9) + (14u << 10)) : (mag ? 0x3800u : 0u);
    return bits | ((nib & 8u) << 12);
}

// ---------------------------------------------------------------- E4M3 decode
// Two E4M3FN bytes of a dword (word_sel picks bytes 0-1 or 2-3) to fp32 with the
// gfx950 converter (OCP E4M3FN on this target).
template <bool HI>
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t dw) {
    auto r = __builtin_amdgcn_cvt_pk_f32_fp8((int)dw, HI);
    return make_float2(r[0], r[1]);
}

// ---------------------------------------------------------------- cross-lane
// DPP row operations (16-lane rows).  ctrl values: quad_perm = perm bits,
// row_ror:n = 0x120 + n.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROR2 = 0x122;     // row_ror:2
constexpr int DPP_ROR4 = 0x124;     // row_ror:4
constexpr int DPP_ROR8 = 0x128;     // row_ror:8

// Lanes l and l ^ 16 (or l ^ 32) combined without an LDS round trip: gfx950's
// v_permlane16_swap / v_permlane32_swap of v with itself leave v[l & ~16] in
// one result and v[l | 16] in the other (resp. 32), so their max or sum is the
// pair's.
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order-preserving map of a finite float to uint32 (larger float -> larger
// key); -0.0 is folded onto +0.0 so equal values tie.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// ---------------------------------------------------------------- cache rows
// Row of kv / idxk that holds position t of sequence s.  A contiguous cache
// keeps sequence s in rows s*cap .. s*cap + cap - 1.  A paged cache keeps t in
// row t mod 2^shift of the physical page its table names for page t >> shift;
// table entries outside [0, n_pages) are clamped into it, so a bad or unused
// entry cannot move an access outside the buffers.
struct PageMap {
    const int32_t* table;   // [n_seq][per_seq] physical page ids (paged caches)
    int64_t per_seq;        // pages per sequence: cap >> shift
    int32_t shift;          // log2 of the tokens per page
    int32_t n_pages;
};

template <bool PAGED>
__device__ __forceinline__ int64_t cache_row(const PageMap& m, int64_t cap, int32_t s,
                                             int64_t t) {
    if (!PAGED) return (int64_t)s * cap + t;
    int32_t pg = m.table[(int64_t)s * m.per_seq + (t >> m.shift)];
    pg = pg < 0 ? 0 : (pg >= m.n_pages ? m.n_pages - 1 : pg);
    return ((int64_t)pg << m.shift) + (t & (((int64_t)1 << m.shift) - 1));
}

// ---------------------------------------------------------------- LDS copies
// 64-byte rows (an indexer key, or 16 floats of a top-k row) staged in LDS by
// global_load_lds_dwordx4: one instruction copies a contiguous 1 KB (lane l's
// 16 bytes land at lds + 16 l), so the global side is fully coalesced and no
// VGPR holds data in flight.  Reading 16 consecutive rows' same 16-byte chunk
// would hit only four 16-byte bank groups, so the chunks of row j (j mod 16)
// are stored rotated by chunk_rot(j): chunk m sits at position
// (m + chunk_rot(j)) mod 4 of the row's 64 bytes.  The rotation is applied on
// the load side (each lane fetches the chunk that belongs at its LDS position,
// the same contiguous 1 KB per instruction) and undone by per-lane read
// addresses.  chunk_rot is a permutation within every group of 4 rows with
// equal j mod 4 (16-lane passes over 64 banks) and within every group of 4
// rows of equal parity in an aligned run of 8 (8-lane passes over 32 banks).
__device__ __forceinline__ int chunk_rot(int j) { return ((j >> 1) ^ (j >> 3)) & 3; }

// One 1 KB copy: lane l's 16 bytes from sbase + voff to LDS address
// lds_addr + 16 l.  m0 is named as clobbered: it carries the LDS address, and
// no code of these kernels keeps a value in m0.  NT marks the load
// non-temporal (data read once).  Written as inline asm so that the compiler
// neither reorders the copies nor drains vmcnt before every LDS read; callers
// wait explicitly with wait_vm (loads complete in order).  The memory clobber
// keeps LDS reads after their wait and before the next refill of the slot.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void dma_1k(uint32_t voff, const uint8_t* sbase, uint32_t lds_addr) {
    if (NT)
        asm volatile(
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1 nt"
            :
            : "v"(voff), "s"(sbase), "s"(lds_addr)
            : "memory", "m0");
    else
        asm volatile(
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1"
            :
            : "v"(voff), "s"(sbase), "s"(lds_addr)
            : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace csa2
