// Batched gather: engram_gather_reduce (direct mode) for a batch of n_seq
// sequences whose addresses were hashed ahead of time, visiting the tokens in
// the batch order of batch_order.h instead of token order.  The pages compute
// every address from the ids before the lookup [DeepSeek V4.1 Flash: The VRAM
// Killer, section "What makes up the 511 GB of weights?"]; prompts that share
// a prefix then read the same rows in every sequence, and this order lets one
// XCD's L2 serve the repeats.  Per token the work, and so the result, is that
// of gather_reduce_kernel: the same loader and fused multiply-add sequence.
//
// With several sequences per block in a large batch (kShare), the waves of a
// block that share a position are that position of consecutive sequences.
// Each wave posts its 24 addresses and its token in LDS; after a barrier, a
// wave whose addresses equal an earlier wave's ends, and the first wave of
// each set of equal addresses gathers once and stores the sum to every token
// of the set, since equal addresses give the same rows and so the same sum.
// A prefix shared by the batch is then gathered once per block of sequences
// instead of once per sequence.
#include "batch_order.h"
#include "row_sum.h"

namespace engram {
namespace {

template <int FMT, uint32_t W, bool kShare>
__global__ __launch_bounds__(64 * W) void gather_batched_kernel(const GatherParams P,
                                                                const uint32_t* __restrict__ addr, uint32_t blk_base,
                                                                BatchOrder o, float* __restrict__ out) {
    const uint32_t module = blockIdx.x & 1u;  // block b: module b % 2 of batch-order block b / 2
    const uint32_t blk = blk_base + (blockIdx.x >> 1);
    if (blk >= o.n_blocks) return;  // the whole block
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t seq, t;
    bool valid;
    block_token(blk, wave, o, &seq, &t, &valid);
    // an idle wave reads token 0's addresses (in bounds) and stores nothing
    const size_t tok = valid ? static_cast<size_t>(seq) * o.seq_len + t : 0u;
    const uint32_t s0 = module * kRowsPerModule;
    const uint32_t a = addr[tok * kSub + s0 + owned_row(lane)];
    f32x4* dst = reinterpret_cast<f32x4*>(out + tok * (2 * kRowBytes) + module * kRowBytes + lane * 4u);
    if (!kShare) {
        if (!valid) return;
        RowSet r;
        load_rows<FMT>(P, s0, a, lane, r);
        __builtin_nontemporal_store(sum_rows<FMT>(r, lane), dst);
        return;
    }
    __shared__ uint32_t sa[W][kRowsPerModule];
    __shared__ uint32_t stok[W];  // token + 1; 0 for an idle wave
    const RowBases rb = row_bases(P, s0, lane);
    if (lane < kRowsPerModule) sa[wave][lane] = a;
    if (lane == 0) stok[wave] = valid ? static_cast<uint32_t>(tok) + 1u : 0u;
    __syncthreads();
    // The first wave of each set of equal addresses gathers and stores the sum
    // to every token of the set; the others have nothing left to do.
    if (!valid || first_equal_wave(sa, stok, wave, lane, a) != wave) return;
    RowSet r;
    load_rows_at<FMT>(rb, a, lane, r);
    const f32x4 acc = sum_rows<FMT>(r, lane);
    __builtin_nontemporal_store(acc, dst);
    store_to_equal_waves<W>(sa, stok, wave, lane, a, acc, out + module * kRowBytes + lane * 4u);
}

template <int FMT>
void launch_one(const GatherParams& p, const uint32_t* addr, uint32_t base, uint32_t nb, const BatchOrder& o,
                float* out, hipStream_t stream) {
    const dim3 grid(2u * nb);
    if (o.wshift == 3)
        hipLaunchKernelGGL((gather_batched_kernel<FMT, 8, true>), grid, dim3(512), 0, stream, p, addr, base, o, out);
    else if (o.share)
        hipLaunchKernelGGL((gather_batched_kernel<FMT, 4, true>), grid, dim3(256), 0, stream, p, addr, base, o, out);
    else
        hipLaunchKernelGGL((gather_batched_kernel<FMT, 4, false>), grid, dim3(256), 0, stream, p, addr, base, o, out);
}

}  // namespace

hipError_t launch_gather_batched(const GatherParams& p, const uint32_t* addr, uint32_t n_tok, uint32_t seq_len,
                                 float* out, hipStream_t stream) {
    // Launches cover at most 2^22 blocks per module, so the grid stays below 2^31 threads.
    constexpr uint32_t kChunkBlocks = 1u << 22;
    const BatchOrder o = batch_order(n_tok, seq_len);
    for (uint32_t base = 0; base < o.n_blocks; base += kChunkBlocks) {
        const uint32_t nb = min(kChunkBlocks, o.n_blocks - base);
        if (p.scale_format == ENGRAM_SCALE_E8M0_BLOCK32)
            launch_one<ENGRAM_SCALE_E8M0_BLOCK32>(p, addr, base, nb, o, out, stream);
        else
            launch_one<ENGRAM_SCALE_F32_ROW>(p, addr, base, nb, o, out, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace engram
