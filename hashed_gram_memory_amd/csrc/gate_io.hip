// Outputs for the learned gate that follows the lookup.
//
// The pages: each retrieved row is compared with the hidden state by a
// learned gate that can suppress it before the module's rows join the
// residual stream [How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It
// Is a Lookup Table, sections "The architecture" and "Engram: the table that
// is never multiplied"].  The gate's weights and form are not given, so the
// library provides the two inputs such a gate needs:
//   gather_rows_kernel      the 48 dequantised rows of each token, un-reduced;
//   gather_weighted_kernel  the per-module sum with one caller weight per row
//                           (a gate's output applied without a second pass).
// Mapping as gather_reduce_kernel: one wave per (token, module), block b
// serving module b % 2, rows read as 64 lanes x 4 B.
#include "row_sum.h"

namespace engram {
namespace {

template <int FMT>
__global__ __launch_bounds__(256) void gather_weighted_kernel(const GatherParams P, const uint32_t* __restrict__ addr,
                                                              const float* __restrict__ weights, uint32_t tok_base,
                                                              uint32_t n_tok, float* __restrict__ out) {
    const uint32_t b = blockIdx.x;
    const uint32_t module = b & 1u;  // block b: module b % 2 of 4 consecutive items
    const uint32_t group = b >> 1;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t tok = tok_base + group * 4u + wave;
    if (tok >= n_tok) return;
    const uint32_t s0 = module * kRowsPerModule;
    const size_t own = static_cast<size_t>(tok) * kSub + s0 + owned_row(lane);
    const uint32_t a = addr[own];
    const float w = weights[own];
    RowSet r;
    load_rows<FMT>(P, s0, a, lane, r);
    const f32x4 acc = weighted_sum_rows<FMT>(r, w, lane);
    __builtin_nontemporal_store(
        acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(tok) * (2 * kRowBytes) + module * kRowBytes + lane * 4u));
}

template <int FMT>
__global__ __launch_bounds__(256) void gather_rows_kernel(const GatherParams P, const uint32_t* __restrict__ addr,
                                                          uint32_t tok_base, uint32_t n_tok, float* __restrict__ rows) {
    const uint32_t b = blockIdx.x;
    const uint32_t module = b & 1u;  // block b: module b % 2 of 4 consecutive items
    const uint32_t group = b >> 1;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t tok = tok_base + group * 4u + wave;
    if (tok >= n_tok) return;
    const uint32_t s0 = module * kRowsPerModule;
    const uint32_t a = addr[static_cast<size_t>(tok) * kSub + s0 + owned_row(lane)];
    RowSet r;
    load_rows<FMT>(P, s0, a, lane, r);
    float* dst = rows + (static_cast<size_t>(tok) * kSub + s0) * kRowBytes + lane * 4u;
#pragma unroll
    for (int k = 0; k < kRowsPerModule; ++k)
        __builtin_nontemporal_store(decode_word(r.v[k], row_scale<FMT>(r, k, lane)),
                                    reinterpret_cast<f32x4*>(dst + k * kRowBytes));
}

template <int FMT>
hipError_t launch_chunked(bool weighted, const GatherParams& p, const uint32_t* addr, const float* weights,
                          uint32_t n_tok, float* out, hipStream_t stream) {
    constexpr uint32_t kChunk = 1u << 24;
    for (uint32_t base = 0; base < n_tok; base += kChunk) {
        const uint32_t n = min(kChunk, n_tok - base);
        const uint32_t groups = ((n + 3u) / 4u + 3u) & ~3u;
        const dim3 grid(2u * groups), block(256);
        if (weighted)
            hipLaunchKernelGGL((gather_weighted_kernel<FMT>), grid, block, 0, stream, p, addr, weights, base, base + n,
                               out);
        else
            hipLaunchKernelGGL((gather_rows_kernel<FMT>), grid, block, 0, stream, p, addr, base, base + n, out);
        // hipGetLastError also clears the error, so its value is what gets returned
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gate_io(const GatherParams& p, const uint32_t* addr, const float* weights, uint32_t n_tok,
                          float* out, hipStream_t stream) {
    const bool weighted = weights != nullptr;
    if (p.scale_format == ENGRAM_SCALE_E8M0_BLOCK32)
        return launch_chunked<ENGRAM_SCALE_E8M0_BLOCK32>(weighted, p, addr, weights, n_tok, out, stream);
    return launch_chunked<ENGRAM_SCALE_F32_ROW>(weighted, p, addr, weights, n_tok, out, stream);
}

}  // namespace engram
