// Hash kernel: 48 row addresses per token.
//
// Per token, the suffix n-grams of order 2, 3 and 4 are hashed by 8 heads in
// each of 2 modules, one row per (module, order, head) [How to Run
// DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a Lookup Table, section
// "Engram: the table that is never multiplied"; DeepSeek V4.1 Flash: The VRAM
// Killer, section "What makes up the 511 GB of weights?"].  The hash itself
// (multiply-xor of the id window, then mod R_s) is this library's reading;
// the pages do not print one.
//
// Layout: a block covers 64 tokens with 6 waves, one per (module, order);
// lane l of every wave is token l of the block.  A wave's 8 heads share the
// (module, order), so its 32 multipliers and its 8 (R, magic) pairs are
// wave-uniform scalar loads from the kernel arguments.  The block first
// stages the 67 ids its windows read in LDS; each thread reads its token's
// window from there and puts its 8 addresses into an LDS tile of the block's
// 64 x 48 addresses, which the block then writes as one contiguous 12 KiB run
// with 16-byte stores.  The
// kernel is store-bound and small next to the gather (196 B per token
// against ~14.7 KB).
#include "engram_internal.h"

namespace engram {
namespace {

// Exact x mod R for 1 <= R <= 2^32 with magic = floor((2^64-1)/R):
// q = floor(x*magic / 2^64) is floor(x/R) or one less, so one correction.
__device__ __forceinline__ uint32_t mod_rows(uint64_t x, uint64_t R, uint64_t magic) {
    const uint64_t q = __umul64hi(x, magic);
    uint64_t r = x - q * R;
    if (r >= R) r -= R;
    return static_cast<uint32_t>(r);
}

// The 8 addresses of one (module, order) for a window; ORDER and the
// power-of-two case are compile-time so the loops and the modulus are
// straight-line code.
template <int ORDER, bool POW2>
__device__ __forceinline__ void hash_heads(const HashParams& P, const uint64_t (&w)[ENGRAM_MAX_ORDER], uint32_t mbase,
                                           uint32_t s0, uint32_t (&a)[ENGRAM_N_HEADS]) {
#pragma unroll
    for (int h = 0; h < ENGRAM_N_HEADS; ++h) {
        uint64_t x = 0;
#pragma unroll
        for (int k = 0; k < ORDER; ++k) x ^= w[k] * P.mult[mbase + h * ENGRAM_MAX_ORDER + k];
        if (POW2)
            a[h] = static_cast<uint32_t>(x & (P.rows[s0 + h] - 1u));  // R = 2^k: x mod R is the low k bits
        else
            a[h] = mod_rows(x, P.rows[s0 + h], P.magic[s0 + h]);
    }
}

template <bool POW2>
__global__ __launch_bounds__(384) void hash_kernel(const HashParams P, const int32_t* __restrict__ ids,
                                                   const int32_t* __restrict__ history, uint32_t n_tok,
                                                   uint32_t seq_len, uint32_t* __restrict__ addr) {
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (module, order) = (wave/3, 2+wave%3)
    // Tokens past the end compute a clamped duplicate and are not stored, so
    // every thread reaches the barrier below.
    const uint32_t tok = min(blockIdx.x * 64u + (threadIdx.x & 63u), n_tok - 1u);
    const uint32_t m = wave / 3u;
    const uint32_t oi = wave % 3u;  // order - 2
    const uint32_t seq = tok / seq_len;
    const int32_t t = static_cast<int32_t>(tok - seq * seq_len);

    // Stage the ids the block's windows read, flat positions first-3 ..
    // first+63, once in LDS (with the vocabulary map already applied), so the
    // 6 waves read their windows from LDS instead of 24 global loads per token.
    const uint32_t first = blockIdx.x * 64u;
    __shared__ uint32_t win_ids[64 + ENGRAM_MAX_ORDER - 1];
    if (threadIdx.x < 64u + ENGRAM_MAX_ORDER - 1) {
        const int64_t flat = static_cast<int64_t>(first) - (ENGRAM_MAX_ORDER - 1) + threadIdx.x;
        uint32_t v = 0;
        if (flat >= 0 && flat < static_cast<int64_t>(n_tok)) {
            v = static_cast<uint32_t>(ids[flat]);
            if (P.vocab_map) v = P.vocab_map[v];
        }
        win_ids[threadIdx.x] = v;
    }
    __syncthreads();

    // Window: w[k] = id at position t-k; before the sequence start, the
    // caller's history (history[seq][2] is position -1) or id 0, each through
    // the vocabulary map.
    uint64_t w[ENGRAM_MAX_ORDER];
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_ORDER; ++k) {
        if (t - k >= 0)
            w[k] = win_ids[tok - k - first + (ENGRAM_MAX_ORDER - 1)];
        else
            w[k] = window_id(ids, history, P.vocab_map, tok, seq, t, k);
    }

    const uint32_t mbase = wave * (ENGRAM_N_HEADS * ENGRAM_MAX_ORDER);  // multipliers of (m, order, head 0, k 0)
    const uint32_t s0 = m * kRowsPerModule + oi * ENGRAM_N_HEADS;
    uint32_t a[ENGRAM_N_HEADS];
    if (oi == 0)
        hash_heads<2, POW2>(P, w, mbase, s0, a);
    else if (oi == 1)
        hash_heads<3, POW2>(P, w, mbase, s0, a);
    else
        hash_heads<4, POW2>(P, w, mbase, s0, a);

    // Stage the block's 64 x 48 addresses in LDS, then write them out as
    // one contiguous 12 KiB run with coalesced 16-byte stores.
    __shared__ uint4 stage[64 * kSub / 4];
    uint4* my = stage + (threadIdx.x & 63u) * (kSub / 4) + s0 / 4;
    my[0] = make_uint4(a[0], a[1], a[2], a[3]);
    my[1] = make_uint4(a[4], a[5], a[6], a[7]);
    __syncthreads();
    const uint32_t n_vec = (min(64u, n_tok - first) * kSub) / 4u;  // 16-byte words this block owns
    uint4* dst = reinterpret_cast<uint4*>(addr + static_cast<size_t>(first) * kSub);
    for (uint32_t i = threadIdx.x; i < n_vec; i += blockDim.x) dst[i] = stage[i];
}

}  // namespace

hipError_t launch_hash(const HashParams& p, const int32_t* ids, const int32_t* history, uint32_t n_tok,
                       uint32_t seq_len, uint32_t* addr, hipStream_t stream) {
    const uint32_t blocks = (n_tok + 63u) / 64u;
    bool pow2 = true;
    for (int s = 0; s < kSub; ++s) pow2 = pow2 && (p.rows[s] & (p.rows[s] - 1u)) == 0;
    if (pow2)
        hipLaunchKernelGGL(hash_kernel<true>, dim3(blocks), dim3(384), 0, stream, p, ids, history, n_tok, seq_len, addr);
    else
        hipLaunchKernelGGL(hash_kernel<false>, dim3(blocks), dim3(384), 0, stream, p, ids, history, n_tok, seq_len,
                           addr);
    return hipGetLastError();
}

}  // namespace engram
