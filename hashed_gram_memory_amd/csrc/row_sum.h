// The per-(token, module) inner loop shared by the gather kernels: read 24
// FP8 rows and their scales, dequantise, sum in fp32 in ascending q.
//
// Rows are 256 FP8 E4M3 codes [How to Run DeepSeek-V4.1-Flash: 510 GB, and
// 203 GB of It Is a Lookup Table, section "Engram: the table that is never
// multiplied"]; a wave reads one row as 64 lanes x 4 B, lane l holding
// elements 4l..4l+3.  Two scale formats:
//   ENGRAM_SCALE_F32_ROW       one fp32 per row (wave-uniform scalar load);
//   ENGRAM_SCALE_E8M0_BLOCK32  eight E8M0 exponents per row, one per 32
//                              elements (the row's 8 bytes of scales; lane l
//                              loads byte l/8).  An E8M0 byte e is
//                              2^(e-127), and 255 is NaN.
#pragma once

#include "engram_internal.h"

namespace engram {

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Loads of the 24 rows of a module and of their scales (per lane: the scale
// of this lane's 4 elements), all issued before any is used.
template <int FMT, bool VSCALE>
__device__ __forceinline__ void load_rows(const GatherParams& P, uint32_t s0, const uint32_t (&a)[kRowsPerModule],
                                          uint32_t lane, uint32_t (&v)[kRowsPerModule],
                                          float (&sc)[kRowsPerModule]) {
    uint32_t e8[kRowsPerModule];
    const uint32_t blk = lane >> 3;  // 32-element block of elements 4*lane .. 4*lane+3
    uint32_t vzero = 0;
    if (VSCALE) asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
#pragma unroll
    for (int q = 0; q < kRowsPerModule; ++q) {
        const uint32_t* row =
            reinterpret_cast<const uint32_t*>(P.tab[s0 + q] + static_cast<uint64_t>(a[q]) * kRowBytes);
        v[q] = __builtin_nontemporal_load(row + lane);
        if (FMT == ENGRAM_SCALE_F32_ROW)
            sc[q] = static_cast<const float*>(P.sc[s0 + q])[a[q] + vzero];
        else
            e8[q] = static_cast<const uint8_t*>(P.sc[s0 + q])[static_cast<uint64_t>(a[q]) * 8u + blk];
    }
    if (FMT == ENGRAM_SCALE_E8M0_BLOCK32) {
#pragma unroll
        for (int q = 0; q < kRowsPerModule; ++q) sc[q] = e8m0_to_f32(e8[q]);
    }
}

template <int FMT, bool VSCALE = false>
__device__ __forceinline__ f32x4 sum_rows(const GatherParams& P, uint32_t s0, const uint32_t (&a)[kRowsPerModule],
                                          uint32_t lane) {
    uint32_t v[kRowsPerModule];
    float sc[kRowsPerModule];
    load_rows<FMT, VSCALE>(P, s0, a, lane, v, sc);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < kRowsPerModule; ++q) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[q]), false);  // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[q]), true);   // bytes 2, 3
        acc.x = __builtin_fmaf(lo[0], sc[q], acc.x);
        acc.y = __builtin_fmaf(lo[1], sc[q], acc.y);
        acc.z = __builtin_fmaf(hi[0], sc[q], acc.z);
        acc.w = __builtin_fmaf(hi[1], sc[q], acc.w);
    }
    return acc;
}


// Weighted sum of the 24 rows: the scale of row q is first multiplied by the
// caller's weight w[q] (rounded to fp32), then enters the same fused
// multiply-add sequence as sum_rows; with every weight 1 the result is
// bitwise that of sum_rows.
template <int FMT>
__device__ __forceinline__ f32x4 weighted_sum_rows(const GatherParams& P, uint32_t s0,
                                                   const uint32_t (&a)[kRowsPerModule],
                                                   const float (&w)[kRowsPerModule], uint32_t lane) {
    uint32_t v[kRowsPerModule];
    float sc[kRowsPerModule];
    load_rows<FMT, false>(P, s0, a, lane, v, sc);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < kRowsPerModule; ++q) {
        const float s = sc[q] * w[q];
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[q]), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[q]), true);
        acc.x = __builtin_fmaf(lo[0], s, acc.x);
        acc.y = __builtin_fmaf(lo[1], s, acc.y);
        acc.z = __builtin_fmaf(hi[0], s, acc.z);
        acc.w = __builtin_fmaf(hi[1], s, acc.w);
    }
    return acc;
}

}  // namespace engram
