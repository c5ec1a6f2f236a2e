// Batched gather: engram_gather_reduce (direct mode) for a batch of n_seq
// sequences whose addresses were hashed ahead of time, visiting the tokens in
// the batch order of batch_order.h instead of token order.  The pages compute
// every address from the ids before the lookup [DeepSeek V4.1 Flash: The VRAM
// Killer, section "What makes up the 511 GB of weights?"]; prompts that share
// a prefix then read the same rows in every sequence, and this order lets one
// XCD's L2 serve the repeats.  Per token the work, and so the result, is that
// of gather_reduce_kernel: the same loader and fused multiply-add sequence.
#include "batch_order.h"
#include "row_sum.h"

namespace engram {
namespace {

template <int FMT>
__global__ __launch_bounds__(256) void gather_batched_kernel(const GatherParams P, const uint32_t* __restrict__ addr,
                                                             uint32_t item_base, uint32_t item_end, BatchOrder batch,
                                                             float* __restrict__ out) {
    const uint32_t b = blockIdx.x;
    const uint32_t module = b & 1u;  // block b: module b % 2 of 4 consecutive items
    const uint32_t group = b >> 1;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t item = item_base + group * 4u + wave;
    if (item >= item_end) return;
    uint32_t seq, t;
    const uint32_t tok = batched_token(item, batch, &seq, &t);

    const uint32_t s0 = module * kRowsPerModule;
    const uint32_t a = addr[static_cast<size_t>(tok) * kSub + s0 + owned_row(lane)];
    RowSet r;
    load_rows<FMT>(P, s0, a, lane, r);
    const f32x4 acc = sum_rows<FMT>(r, lane);
    __builtin_nontemporal_store(
        acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(tok) * (2 * kRowBytes) + module * kRowBytes + lane * 4u));
}

}  // namespace

hipError_t launch_gather_batched(const GatherParams& p, const uint32_t* addr, uint32_t n_tok, uint32_t seq_len,
                                 float* out, hipStream_t stream) {
    // Launches cover at most 2^24 items so the grid stays far below 2^32 threads.
    constexpr uint32_t kChunk = 1u << 24;
    const BatchOrder batch = batch_order(n_tok, seq_len);
    for (uint32_t base = 0; base < n_tok; base += kChunk) {
        const uint32_t n = min(kChunk, n_tok - base);
        const uint32_t groups = ((n + 3u) / 4u + 3u) & ~3u;
        const dim3 grid(2u * groups), block(256);
        if (p.scale_format == ENGRAM_SCALE_E8M0_BLOCK32)
            hipLaunchKernelGGL((gather_batched_kernel<ENGRAM_SCALE_E8M0_BLOCK32>), grid, block, 0, stream, p, addr, base,
                               base + n, batch, out);
        else
            hipLaunchKernelGGL((gather_batched_kernel<ENGRAM_SCALE_F32_ROW>), grid, block, 0, stream, p, addr, base,
                               base + n, batch, out);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace engram
