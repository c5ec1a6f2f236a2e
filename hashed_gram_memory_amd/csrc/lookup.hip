// Fused lookup: hash and gather-reduce in one kernel, no address buffer.
//
// The row addresses depend on the token ids alone [DeepSeek V4.1 Flash: The
// VRAM Killer, section "What makes up the 511 GB of weights?"; How to Run
// DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a Lookup Table, section
// "Engram: the table that is never multiplied"], so the wave that gathers a
// (token, module) can compute its own 24 addresses instead of reading them.
// This drops the 192-byte address write and read per token and one launch,
// which is what a decode step of a few tokens is made of.
//
// Mapping: one wave per (token, module), tokens visited in the batch order
// of batch_order.h (tiles of 64 positions, sequence by sequence within a
// tile; plain token order for one sequence).  The window ids are
// wave-uniform; lane q < 24
// hashes row q of the module in parallel with the others, with the same
// multiply-xor and modulus (a mask for power-of-two row counts) as
// hash_kernel, and then owns that row in the lane-addressed loads.  The
// accumulation is the fused multiply-add sequence of gather_reduce_kernel, so
// the result is bitwise identical to engram_hash followed by
// engram_gather_reduce.
#include "batch_order.h"
#include "row_sum.h"

namespace engram {
namespace {

struct LookupParams {
    HashParams h;
    GatherParams g;
};

__device__ __forceinline__ uint32_t mod_rows(uint64_t x, uint64_t R, uint64_t magic) {
    const uint64_t q = __umul64hi(x, magic);
    uint64_t r = x - q * R;
    if (r >= R) r -= R;
    return static_cast<uint32_t>(r);
}

template <bool POW2, int FMT>
__global__ __launch_bounds__(256) void lookup_kernel(const LookupParams P, const int32_t* __restrict__ ids,
                                                     const int32_t* __restrict__ history, uint32_t item_base,
                                                     uint32_t item_end, BatchOrder batch, float* __restrict__ out) {
    const uint32_t b = blockIdx.x;
    const uint32_t m = b & 1u;  // block b: module b % 2 of 4 consecutive items
    const uint32_t group = b >> 1;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t item = item_base + group * 4u + wave;
    if (item >= item_end) return;
    uint32_t seq, t;
    const uint32_t tok = batched_token(item, batch, &seq, &t);

    // Window of the token (wave-uniform): w[k] = id k positions back, else history, else 0.
    uint64_t w[ENGRAM_MAX_ORDER];
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_ORDER; ++k)
        w[k] = window_id(ids, history, P.h.vocab_map, tok, seq, static_cast<int32_t>(t), k);

    // Lane q < 24 hashes the module's row q = 8*(order-2) + head (lanes
    // 24..63 repeat row 0) and keeps the address for the lane-addressed loads.
    const uint32_t s0 = m * kRowsPerModule;
    const uint32_t mb = m * (kRowsPerModule * ENGRAM_MAX_ORDER);
    const uint32_t q = owned_row(lane);
    const uint32_t order = ENGRAM_MIN_ORDER + q / ENGRAM_N_HEADS;
    uint64_t x = 0;
#pragma unroll
    for (uint32_t k = 0; k < ENGRAM_MAX_ORDER; ++k)
        if (k < order) x ^= w[k] * P.h.mult[mb + q * ENGRAM_MAX_ORDER + k];
    const uint64_t R = P.h.rows[s0 + q];
    const uint32_t a = POW2 ? static_cast<uint32_t>(x & (R - 1u)) : mod_rows(x, R, P.h.magic[s0 + q]);

    RowSet r;
    load_rows<FMT>(P.g, s0, a, lane, r);
    const f32x4 acc = sum_rows<FMT>(r, lane);
    __builtin_nontemporal_store(
        acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(tok) * (2 * kRowBytes) + m * kRowBytes + lane * 4u));
}

}  // namespace

hipError_t launch_lookup(const HashParams& h, const GatherParams& g, const int32_t* ids, const int32_t* history,
                         uint32_t n_tok, uint32_t seq_len, float* out, hipStream_t stream) {
    LookupParams p;
    p.h = h;
    p.g = g;
    bool pow2 = true;
    for (int s = 0; s < kSub; ++s) pow2 = pow2 && (h.rows[s] & (h.rows[s] - 1u)) == 0;
    // Launches cover at most 2^24 items so the grid stays far below 2^32
    // threads.
    constexpr uint32_t kChunk = 1u << 24;
    const bool mx = g.scale_format == ENGRAM_SCALE_E8M0_BLOCK32;
    const BatchOrder batch = batch_order(n_tok, seq_len);
    for (uint32_t base = 0; base < n_tok; base += kChunk) {
        const uint32_t n = min(kChunk, n_tok - base);
        const uint32_t groups = ((n + 3u) / 4u + 3u) & ~3u;
        const dim3 grid(2u * groups), block(256);
        if (pow2 && mx)
            hipLaunchKernelGGL((lookup_kernel<true, ENGRAM_SCALE_E8M0_BLOCK32>), grid, block, 0, stream, p, ids, history,
                               base, base + n, batch, out);
        else if (pow2)
            hipLaunchKernelGGL((lookup_kernel<true, ENGRAM_SCALE_F32_ROW>), grid, block, 0, stream, p, ids, history, base,
                               base + n, batch, out);
        else if (mx)
            hipLaunchKernelGGL((lookup_kernel<false, ENGRAM_SCALE_E8M0_BLOCK32>), grid, block, 0, stream, p, ids,
                               history, base, base + n, batch, out);
        else
            hipLaunchKernelGGL((lookup_kernel<false, ENGRAM_SCALE_F32_ROW>), grid, block, 0, stream, p, ids, history,
                               base, base + n, batch, out);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace engram
