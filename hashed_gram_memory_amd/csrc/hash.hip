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
// Layout: one thread per token.  The 192 multipliers and the 48 (R, magic)
// pairs are kernel arguments indexed by compile-time constants, so they are
// wave-uniform scalar loads; only the four window ids live in vector
// registers.  Each thread writes its 48 addresses as 12 dwordx4 stores
// (192 contiguous bytes per token).  The kernel is store-bound and tiny
// next to the gather (196 B per token vs ~14.7 KB).
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

__global__ __launch_bounds__(256) void hash_kernel(const HashParams P, const int32_t* __restrict__ ids,
                                                   const int32_t* __restrict__ history, uint32_t n_tok,
                                                   uint32_t seq_len, uint32_t* __restrict__ addr) {
    const uint32_t tok = blockIdx.x * 256u + threadIdx.x;
    if (tok >= n_tok) return;
    const uint32_t seq = tok / seq_len;
    const int32_t t = static_cast<int32_t>(tok - seq * seq_len);

    // Window: w[k] = id at position t-k; before the sequence start, the
    // caller's history (history[seq][2] is position -1) or id 0.
    uint64_t w[ENGRAM_MAX_ORDER];
#pragma unroll
    for (int k = 0; k < ENGRAM_MAX_ORDER; ++k) {
        int32_t v = 0;
        if (t - k >= 0)
            v = ids[tok - k];
        else if (history)
            v = history[seq * 3u + static_cast<uint32_t>(3 + t - k)];
        w[k] = static_cast<uint32_t>(v);
    }

    uint32_t a[kSub];
#pragma unroll
    for (int m = 0; m < ENGRAM_N_MODULES; ++m) {
#pragma unroll
        for (int n = ENGRAM_MIN_ORDER; n <= ENGRAM_MAX_ORDER; ++n) {
#pragma unroll
            for (int h = 0; h < ENGRAM_N_HEADS; ++h) {
                const int base = ((m * 3 + (n - ENGRAM_MIN_ORDER)) * ENGRAM_N_HEADS + h) * ENGRAM_MAX_ORDER;
                uint64_t x = 0;
#pragma unroll
                for (int k = 0; k < n; ++k) x ^= w[k] * P.mult[base + k];
                const int s = m * kRowsPerModule + (n - ENGRAM_MIN_ORDER) * ENGRAM_N_HEADS + h;
                a[s] = mod_rows(x, P.rows[s], P.magic[s]);
            }
        }
    }

    uint4* dst = reinterpret_cast<uint4*>(addr + static_cast<size_t>(tok) * kSub);
#pragma unroll
    for (int i = 0; i < kSub / 4; ++i) dst[i] = make_uint4(a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]);
}

}  // namespace

hipError_t launch_hash(const HashParams& p, const int32_t* ids, const int32_t* history, uint32_t n_tok,
                       uint32_t seq_len, uint32_t* addr, hipStream_t stream) {
    const uint32_t blocks = (n_tok + 255u) / 256u;
    hipLaunchKernelGGL(hash_kernel, dim3(blocks), dim3(256), 0, stream, p, ids, history, n_tok, seq_len, addr);
    return hipGetLastError();
}

}  // namespace engram
