// The per-(token, module) inner loop shared by the gather kernels: read 24
// FP8 rows and their scales, dequantise, sum in fp32 in ascending q.
//
// Rows are 256 FP8 E4M3 codes [How to Run DeepSeek-V4.1-Flash: 510 GB, and
// 203 GB of It Is a Lookup Table, section "Engram: the table that is never
// multiplied"]; a wave reads one row as 64 lanes x 4 B, lane l holding
// elements 4l..4l+3.  Two scale formats, both read with scalar loads (the
// tables are read-only while a kernel runs, so the scalar cache may hold
// them):
//   ENGRAM_SCALE_F32_ROW       one fp32 per row;
//   ENGRAM_SCALE_E8M0_BLOCK32  eight E8M0 exponents per row, one per 32
//                              elements (the row's 8 bytes of scales, one
//                              8-byte load; lane l uses byte l/8).  An E8M0
//                              byte e is 2^(e-127), and 255 is NaN.
#pragma once

#include "engram_internal.h"

namespace engram {

typedef float f32x4 __attribute__((ext_vector_type(4)));
// A pointer into device global memory (address space 1): loads through it
// are global_load instructions, not flat ones.
typedef const __attribute__((address_space(1))) uint32_t* global_u32_ptr;

// Wave-uniform copy of lane k's 64-bit value given as two 32-bit halves.
__device__ __forceinline__ uint64_t readlane64(uint32_t lo, uint32_t hi, int k) {
    return static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, k))) |
           (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, k))) << 32);
}

// fp32 value of an E8M0 scale byte: the bits e << 23 for 1 <= e <= 254,
// the subnormal 2^-127 for e = 0, NaN for e = 255.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    uint32_t bits = e == 0u ? 0x00400000u : (e << 23);
    bits = e == 255u ? 0x7FC00000u : bits;
    return __builtin_bit_cast(float, bits);
}

// Dequantised element pair of a row word: bytes 0..3 of `v` times `sc`.
__device__ __forceinline__ f32x4 decode_word(uint32_t v, float sc) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), true);
    f32x4 r = {lo[0] * sc, lo[1] * sc, hi[0] * sc, hi[1] * sc};
    return r;
}

// Lane-addressed loads.  Lane q < 24 of the wave owns row q of the module:
// it holds that row's address and forms the row's base and its scale's
// address, so no wave-uniform register holds more than one row pointer at a
// time (8 waves per SIMD fit).  Lanes 24..63 repeat row 0.  Row k is then
// read by the whole wave (64 lanes x 4 B, lane l holding elements 4l..4l+3)
// from the base broadcast out of lane k, and its scale by one scalar load
// from the broadcast scale address.  Scalar scale loads measured ~10% faster
// per launch than one vector load that gathers the 24 scales across lanes.
__device__ __forceinline__ uint32_t owned_row(uint32_t lane) { return lane < kRowsPerModule ? lane : 0u; }

typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
typedef const __attribute__((address_space(4))) uint64_t* const_u64_ptr;

struct RowSet {
    uint32_t v[kRowsPerModule];     // this lane's 4 codes of each row
    uint32_t s_lo[kRowsPerModule];  // scale of each row (wave-uniform): fp32 bits, or E8M0 bytes 0..3
    uint32_t s_hi[kRowsPerModule];  //   E8M0 bytes 4..7
};

// Table and scale base pointers of the sub-table whose row this lane owns
// (s0 + owned_row(lane)): lane-indexed loads from the plan's pointer arrays,
// which a kernel can request early, before the row address is known.
struct RowBases {
    uint64_t tab, sc;
};
__device__ __forceinline__ RowBases row_bases(const GatherParams& P, uint32_t s0, uint32_t lane) {
    const uint32_t q = owned_row(lane);
    return RowBases{reinterpret_cast<uint64_t>(P.tab[s0 + q]), reinterpret_cast<uint64_t>(P.sc[s0 + q])};
}

// `a`: this lane's address, the row of its sub-table (bases from row_bases).
template <int FMT>
__device__ __forceinline__ void load_rows_at(const RowBases& rb, uint32_t a, uint32_t lane, RowSet& r) {
    constexpr uint64_t kScaleBytes = FMT == ENGRAM_SCALE_F32_ROW ? 4u : 8u;
    const uint64_t base = rb.tab + static_cast<uint64_t>(a) * kRowBytes;
    const uint64_t sadr = rb.sc + static_cast<uint64_t>(a) * kScaleBytes;
    const uint32_t base_lo = static_cast<uint32_t>(base), base_hi = static_cast<uint32_t>(base >> 32);
    const uint32_t sadr_lo = static_cast<uint32_t>(sadr), sadr_hi = static_cast<uint32_t>(sadr >> 32);
#pragma unroll
    for (int k = 0; k < kRowsPerModule; ++k) {
        const global_u32_ptr row = reinterpret_cast<global_u32_ptr>(readlane64(base_lo, base_hi, k));
        // Cache policy by n-gram order.  The 8 order-2 rows (k < 8) are the
        // ones a token stream repeats (bigrams of frequent tokens: 28-37% of
        // a Zipf prompt's order-2 reads hit a row read earlier in the same
        // launch, against 5-9% for order 3 and ~1% for order 4), so they are
        // plain loads that L2 may keep; the rest are non-temporal.
        if (k < ENGRAM_N_HEADS)
            r.v[k] = row[lane];
        else
            r.v[k] = __builtin_nontemporal_load(row + lane);
        const uint64_t sk = readlane64(sadr_lo, sadr_hi, k);
        if (FMT == ENGRAM_SCALE_F32_ROW) {
            r.s_lo[k] = *reinterpret_cast<const_u32_ptr>(sk);
        } else {
            const uint64_t g = *reinterpret_cast<const_u64_ptr>(sk);
            r.s_lo[k] = static_cast<uint32_t>(g);
            r.s_hi[k] = static_cast<uint32_t>(g >> 32);
        }
        // row k's broadcasts are used up here: no more than one row's
        // pointers are live in scalar registers
        __builtin_amdgcn_sched_barrier(0);
    }
}

// `a`: this lane's address, the row of sub-table s0 + owned_row(lane).
template <int FMT>
__device__ __forceinline__ void load_rows(const GatherParams& P, uint32_t s0, uint32_t a, uint32_t lane, RowSet& r) {
    load_rows_at<FMT>(row_bases(P, s0, lane), a, lane, r);
}

// Scale of row k for this lane's 4 elements.
template <int FMT>
__device__ __forceinline__ float row_scale(const RowSet& r, int k, uint32_t lane) {
    if (FMT == ENGRAM_SCALE_F32_ROW) return __builtin_bit_cast(float, r.s_lo[k]);
    const uint32_t blk = lane >> 3;  // 32-element block of elements 4*lane .. 4*lane+3
    const uint32_t word = blk < 4u ? r.s_lo[k] : r.s_hi[k];
    return e8m0_to_f32((word >> ((blk & 3u) * 8u)) & 0xFFu);
}

// Per-module sum: fused multiply-add of the dequantised rows into 4 fp32
// accumulators per lane, in ascending k, from +0.
template <int FMT>
__device__ __forceinline__ f32x4 sum_rows(const RowSet& r, uint32_t lane) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kRowsPerModule; ++k) {
        const float sc = row_scale<FMT>(r, k, lane);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.v[k]), false);  // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.v[k]), true);   // bytes 2, 3
        acc.x = __builtin_fmaf(lo[0], sc, acc.x);
        acc.y = __builtin_fmaf(lo[1], sc, acc.y);
        acc.z = __builtin_fmaf(hi[0], sc, acc.z);
        acc.w = __builtin_fmaf(hi[1], sc, acc.w);
    }
    return acc;
}

// Weighted sum: the scale of row k is first multiplied by the caller's
// weight for that row (`w` is this lane's weight, of its owned row, in fp32),
// then enters the same fused multiply-add sequence as sum_rows; with every
// weight 1 the result is bitwise that of sum_rows.
template <int FMT>
__device__ __forceinline__ f32x4 weighted_sum_rows(const RowSet& r, float w, uint32_t lane) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t wbits = __builtin_bit_cast(uint32_t, w);
#pragma unroll
    for (int k = 0; k < kRowsPerModule; ++k) {
        const float wk = __builtin_bit_cast(float, static_cast<uint32_t>(__builtin_amdgcn_readlane(wbits, k)));
        const float s = row_scale<FMT>(r, k, lane) * wk;
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.v[k]), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.v[k]), true);
        acc.x = __builtin_fmaf(lo[0], s, acc.x);
        acc.y = __builtin_fmaf(lo[1], s, acc.y);
        acc.z = __builtin_fmaf(hi[0], s, acc.z);
        acc.w = __builtin_fmaf(hi[1], s, acc.w);
    }
    return acc;
}

}  // namespace engram
