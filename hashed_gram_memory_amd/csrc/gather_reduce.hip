// Gather-reduce kernel: read 24 FP8 rows per (token, module), dequantise
// with the per-row scale and sum them into one fp32 vector of 256.
//
// The pages: every token reads 48 rows of 256 FP8 bytes (two modules of 24)
// [How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a Lookup
// Table, section "Engram: the table that is never multiplied"; DeepSeek V4.1
// Flash: The VRAM Killer, section "What makes up the 511 GB of weights?"];
// the rows come from FP8 tables and are combined [Running DeepSeek V4.1
// Flash locally: the numbers beyond 552B, section "Backbone, Engram, and
// active parameters describe different scales"].  It is a lookup, not a
// matrix product: HBM-bound random 256-byte reads, no MFMA.
//
// Mapping (gfx950, wave64):
//   * one wavefront per (token, module); a row is one coalesced
//     global_load_dword of 64 lanes x 4 B, lane l holding elements 4l..4l+3;
//   * the 24 addresses of a (token, module) are contiguous: lane q < 24
//     loads address q (one vector load for all 24) and forms row q's base
//     and its scale's address; the wave then broadcasts them one row at a
//     time, so few scalar registers are live and 8 waves per SIMD fit;
//   * each scale is a scalar load from its broadcast address (faster than
//     one vector load that gathers the 24 scale lines across lanes);
//   * all 24 row and scale loads are issued before the first is consumed, so
//     a wave keeps 24 x 256 B of rows in flight;
//   * cache policy by n-gram order: the order-2 rows, which a token stream
//     repeats, are plain loads that L2 may keep; the order-3 and order-4
//     rows, nearly all read once, are non-temporal (every 4-byte scale read
//     still fetches a 64-byte sector: scalar-cache misses leave L2 as
//     64-byte requests);
//   * decode with the gfx950 packed FP8 (OCP E4M3) -> fp32 conversion, then
//     fused multiply-add into 4 fp32 accumulators per lane in ascending q
//     (row_sum.h, shared with the fused lookup);
//   * the 1 KiB result is written with non-temporal stores so output
//     traffic does not evict table rows from L2 / MALL;
//   * block b serves module b % 2 for 4 consecutive tokens.  (A layout that
//     sent each module to its own half of the 8 XCDs, so each XCD's L2 saw
//     half of the sub-tables, measured 1% slower.)
#include "row_sum.h"

namespace engram {
namespace {

template <bool kDedup, int FMT>
__global__ __launch_bounds__(256) void gather_reduce_kernel(const GatherParams P, const uint32_t* __restrict__ addr,
                                                            uint32_t item_base, uint32_t item_end, uint32_t n_tok,
                                                            const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ n_unique,
                                                            float* __restrict__ out) {
    const uint32_t b = blockIdx.x;
    const uint32_t module = b & 1u;  // block b: module b % 2 of 4 consecutive items
    const uint32_t group = b >> 1;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t item = item_base + group * 4u + wave;

    uint32_t limit = item_end;
    if (kDedup) {
        const int32_t nu = *n_unique;  // negative: the dedup call failed, there are no groups
        limit = nu > 0 ? min(limit, static_cast<uint32_t>(nu)) : 0u;
    }
    if (item >= limit) return;

    uint32_t tok = item;
    if (kDedup) {
        const uint32_t first = static_cast<uint32_t>(offsets[item]);
        if (first >= n_tok) return;
        tok = static_cast<uint32_t>(perm[first]);
        if (tok >= n_tok) return;
    }
    const uint32_t s0 = module * kRowsPerModule;
    // lane q < 24 takes the address of the module's row q (one coalesced load)
    const uint32_t a = addr[static_cast<size_t>(tok) * kSub + s0 + owned_row(lane)];
    RowSet r;
    load_rows<FMT>(P, s0, a, lane, r);
    const f32x4 acc = sum_rows<FMT>(r, lane);

    const size_t col = static_cast<size_t>(module) * kRowBytes + lane * 4u;
    if (!kDedup) {
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(tok) * (2 * kRowBytes) + col));
    } else {
        // A group has at least one member (the token read above), so the
        // first store is unconditional; a loop that could run zero times
        // would let the compiler sink the loads below a branch that the
        // row-base broadcasts cannot follow, keeping all 24 live at once.
        // The members' indices are read 64 at a time, one per lane, and
        // broadcast one by one, so a group shared by many sequences costs one
        // load per 64 members instead of a dependent load before every store.
        uint32_t i = static_cast<uint32_t>(offsets[item]);
        const uint32_t end = min(static_cast<uint32_t>(offsets[item + 1]), n_tok);
        do {
            const uint32_t cnt = min(64u, end - i);
            const uint32_t mine = lane < cnt ? static_cast<uint32_t>(perm[i + lane]) : n_tok;
            uint32_t j = 0;
            do {
                const uint32_t t = static_cast<uint32_t>(__builtin_amdgcn_readlane(mine, j));
                if (t < n_tok)
                    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(t) * (2 * kRowBytes) + col));
            } while (++j < cnt);
            i += cnt;
        } while (i < end);
    }
}

template <bool kDedup, int FMT>
void launch_one(const GatherParams& p, dim3 grid, hipStream_t stream, const uint32_t* addr, uint32_t base, uint32_t end,
                uint32_t n_tok, const int32_t* perm, const int32_t* offsets, const int32_t* n_unique, float* out) {
    hipLaunchKernelGGL((gather_reduce_kernel<kDedup, FMT>), grid, dim3(256), 0, stream, p, addr, base, end, n_tok, perm,
                       offsets, n_unique, out);
}

}  // namespace

hipError_t launch_gather_reduce(const GatherParams& p, const uint32_t* addr, uint32_t n_tok, const int32_t* perm,
                                const int32_t* offsets, const int32_t* n_unique, float* out, hipStream_t stream) {
    // 4 items (one per wave) per block and module; groups rounded up to a
    // multiple of 4 so that every (group, module) maps to exactly one block.
    // Launches cover at most 2^24 items so the grid stays far below 2^32
    // threads.
    constexpr uint32_t kChunk = 1u << 24;
    const bool mx = p.scale_format == ENGRAM_SCALE_E8M0_BLOCK32;
    for (uint32_t base = 0; base < n_tok; base += kChunk) {
        const uint32_t n = min(kChunk, n_tok - base);
        const uint32_t groups = ((n + 3u) / 4u + 3u) & ~3u;
        const dim3 grid(2u * groups);
        if (perm && mx)
            launch_one<true, ENGRAM_SCALE_E8M0_BLOCK32>(p, grid, stream, addr, base, base + n, n_tok, perm, offsets, n_unique, out);
        else if (perm)
            launch_one<true, ENGRAM_SCALE_F32_ROW>(p, grid, stream, addr, base, base + n, n_tok, perm, offsets, n_unique, out);
        else if (mx)
            launch_one<false, ENGRAM_SCALE_E8M0_BLOCK32>(p, grid, stream, addr, base, base + n, n_tok, perm, offsets, n_unique, out);
        else
            launch_one<false, ENGRAM_SCALE_F32_ROW>(p, grid, stream, addr, base, base + n, n_tok, perm, offsets, n_unique, out);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace engram
