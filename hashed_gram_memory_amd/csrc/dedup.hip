// Deduplication of equal id windows for batched prefill with shared prefixes.
//
// The row addresses of a token depend on its id window alone [DeepSeek V4.1
// Flash: The VRAM Killer, section "What makes up the 511 GB of weights?";
// How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a Lookup
// Table, section "Engram: the table that is never multiplied"], so tokens
// with equal windows read the same 48 rows and one lookup can serve them
// all.  Prompts that share a prefix (the pages' agent workloads served
// largely from a prefix cache) repeat whole windows across sequences.
//
// Method: a stable least-significant-digit radix sort of the token indices
// by the key (w_0, w_1, w_2, w_3), 8-bit digits, w_3's low byte first and
// w_0's high byte last (16 passes); then a group flag where the key changes,
// an exclusive scan of the flags, and the group start offsets.
//
// Each pass is three kernels:
//   hist:    per-block digit histogram of the block's tile   -> counts[d][b]
//   scan:    one block, exclusive scan of counts (digit-major) -> offsets
//   scatter: per 256-element sub-tile, a stable rank among equal digits
//            (wave ballots match lanes with the same digit; per-wave counts
//            in LDS order the waves), written to out[offset[d][b] + rank].
// Keys are not materialised: the digit of token `tok` is re-read from the
// id stream (2 MiB for 524,288 tokens, L2-resident) in every pass.
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kMaxBlocks = 1024;
constexpr int kPasses = 16;

struct Ids {
    const int32_t* ids;
    const int32_t* history;
    uint32_t seq_len;
};

// w_k of token tok: the id k positions back, else history, else 0 (zero-extended).
__device__ __forceinline__ uint32_t window_word(const Ids& s, uint32_t tok, int k) {
    const uint32_t seq = tok / s.seq_len;
    const int32_t t = static_cast<int32_t>(tok - seq * s.seq_len);
    if (t - k >= 0) return static_cast<uint32_t>(s.ids[tok - k]);
    if (s.history) return static_cast<uint32_t>(s.history[seq * 3u + static_cast<uint32_t>(3 + t - k)]);
    return 0u;
}

// Pass p sorts by byte (p % 4) of word w_{3 - p/4}.
__device__ __forceinline__ uint32_t digit_of(const Ids& s, uint32_t tok, int pass) {
    const int k = 3 - pass / 4;
    return (window_word(s, tok, k) >> (8 * (pass % 4))) & 0xFFu;
}

__global__ __launch_bounds__(kThreads) void hist_kernel(Ids s, const int32_t* __restrict__ perm_in, uint32_t n,
                                                        uint32_t tile, int pass, uint32_t* __restrict__ counts) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t b = blockIdx.x;
    const uint32_t begin = b * tile;
    const uint32_t end = min(n, begin + tile);
    for (uint32_t i = begin + threadIdx.x; i < end; i += kThreads) {
        const uint32_t tok = perm_in ? static_cast<uint32_t>(perm_in[i]) : i;
        atomicAdd(&h[digit_of(s, tok, pass)], 1u);
    }
    __syncthreads();
    counts[threadIdx.x * gridDim.x + b] = h[threadIdx.x];
}

// Exclusive scan of `len` values in one block of 1024 threads; total to *total.
__global__ __launch_bounds__(1024) void scan_kernel(uint32_t* __restrict__ v, uint32_t len,
                                                    uint32_t* __restrict__ total) {
    __shared__ uint32_t part[1024];
    const uint32_t per = (len + 1023u) / 1024u;
    const uint32_t begin = min(len, threadIdx.x * per);
    const uint32_t end = min(len, begin + per);
    uint32_t sum = 0;
    for (uint32_t i = begin; i < end; ++i) sum += v[i];
    part[threadIdx.x] = sum;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 partial sums.
    for (uint32_t off = 1; off < 1024u; off <<= 1) {
        const uint32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0u;
        __syncthreads();
        part[threadIdx.x] += add;
        __syncthreads();
    }
    uint32_t run = threadIdx.x ? part[threadIdx.x - 1] : 0u;
    for (uint32_t i = begin; i < end; ++i) {
        const uint32_t x = v[i];
        v[i] = run;
        run += x;
    }
    if (threadIdx.x == 1023 && total) *total = part[1023];
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(Ids s, const int32_t* __restrict__ perm_in, uint32_t n,
                                                           uint32_t tile, int pass,
                                                           const uint32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm_out) {
    __shared__ uint32_t base[256];          // next free slot of each digit for this block
    __shared__ uint32_t wave_cnt[kWaves][256];
    const uint32_t b = blockIdx.x;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    base[threadIdx.x] = offsets[threadIdx.x * gridDim.x + b];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wave_cnt[w][threadIdx.x] = 0;
    __syncthreads();

    const uint32_t begin = b * tile;
    const uint32_t end = min(n, begin + tile);
    const uint64_t lt = (uint64_t(1) << lane) - 1u;
    for (uint32_t i0 = begin; i0 < end; i0 += kThreads) {
        const uint32_t i = i0 + threadIdx.x;
        const bool valid = i < end;
        uint32_t tok = 0, d = 0;
        if (valid) {
            tok = perm_in ? static_cast<uint32_t>(perm_in[i]) : i;
            d = digit_of(s, tok, pass);
        }
        // Lanes of this wave holding the same digit.
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool set = (d >> bit) & 1u;
            const uint64_t m = __ballot(set);
            peers &= set ? m : ~m;
        }
        const uint32_t rank_in_wave = __popcll(peers & lt);
        if (valid && rank_in_wave == 0) wave_cnt[wave][d] = __popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t rank = base[d] + rank_in_wave;
            for (uint32_t w = 0; w < wave; ++w) rank += wave_cnt[w][d];
            perm_out[rank] = static_cast<int32_t>(tok);
        }
        __syncthreads();
        uint32_t add = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            add += wave_cnt[w][threadIdx.x];
            wave_cnt[w][threadIdx.x] = 0;
        }
        base[threadIdx.x] += add;
        __syncthreads();
    }
}

__device__ __forceinline__ bool same_window(const Ids& s, uint32_t a, uint32_t b) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (window_word(s, a, k) != window_word(s, b, k)) return false;
    return true;
}

__device__ __forceinline__ uint32_t group_flag(const Ids& s, const int32_t* __restrict__ perm, uint32_t i) {
    return i == 0 ? 1u : (same_window(s, static_cast<uint32_t>(perm[i - 1]), static_cast<uint32_t>(perm[i])) ? 0u : 1u);
}

__global__ __launch_bounds__(kThreads) void flag_count_kernel(Ids s, const int32_t* __restrict__ perm, uint32_t n,
                                                              uint32_t tile, uint32_t* __restrict__ bsum) {
    __shared__ uint32_t c;
    if (threadIdx.x == 0) c = 0;
    __syncthreads();
    const uint32_t begin = blockIdx.x * tile;
    const uint32_t end = min(n, begin + tile);
    uint32_t local = 0;
    for (uint32_t i = begin + threadIdx.x; i < end; i += kThreads) local += group_flag(s, perm, i);
    atomicAdd(&c, local);
    __syncthreads();
    if (threadIdx.x == 0) bsum[blockIdx.x] = c;
}

__global__ __launch_bounds__(kThreads) void group_offsets_kernel(Ids s, const int32_t* __restrict__ perm, uint32_t n,
                                                                 uint32_t tile, const uint32_t* __restrict__ bsum,
                                                                 const uint32_t* __restrict__ total,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ n_unique) {
    __shared__ uint32_t wave_sum[kWaves];
    __shared__ uint32_t run;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t lt = (uint64_t(1) << lane) - 1u;
    if (threadIdx.x == 0) run = bsum[blockIdx.x];
    __syncthreads();
    const uint32_t begin = blockIdx.x * tile;
    const uint32_t end = min(n, begin + tile);
    for (uint32_t i0 = begin; i0 < end; i0 += kThreads) {
        const uint32_t i = i0 + threadIdx.x;
        const uint32_t f = i < end ? group_flag(s, perm, i) : 0u;
        const uint64_t m = __ballot(f);
        if (lane == 0) wave_sum[wave] = __popcll(m);
        __syncthreads();
        uint32_t pos = run + __popcll(m & lt);
        for (uint32_t w = 0; w < wave; ++w) pos += wave_sum[w];
        if (f) offsets[pos] = static_cast<int32_t>(i);
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t add = 0;
            for (int w = 0; w < kWaves; ++w) add += wave_sum[w];
            run += add;
        }
        __syncthreads();
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
        offsets[*total] = static_cast<int32_t>(n);
        *n_unique = static_cast<int32_t>(*total);
    }
}

__global__ void empty_kernel(int32_t* __restrict__ offsets, int32_t* __restrict__ n_unique) {
    offsets[0] = 0;
    *n_unique = 0;
}

uint32_t tile_for(uint32_t n) {
    const uint32_t need = (n + kMaxBlocks - 1u) / kMaxBlocks;
    const uint32_t t = ((need + kThreads - 1u) / kThreads) * kThreads;
    return t < 2048u ? 2048u : t;
}

size_t align_up(size_t x) { return (x + 255u) & ~size_t(255u); }

struct Workspace {
    int32_t* tmp;      // [n] ping-pong permutation
    uint32_t* counts;  // [256 * blocks] digit counts -> offsets
    uint32_t* bsum;    // [blocks] group flags per block -> offsets
    uint32_t* total;   // [1]
};

Workspace carve(void* ws, uint32_t n) {
    char* p = static_cast<char*>(ws);
    Workspace w;
    w.tmp = reinterpret_cast<int32_t*>(p);
    p += align_up(size_t(n) * 4u);
    w.counts = reinterpret_cast<uint32_t*>(p);
    p += align_up(size_t(256) * kMaxBlocks * 4u);
    w.bsum = reinterpret_cast<uint32_t*>(p);
    p += align_up(size_t(kMaxBlocks) * 4u);
    w.total = reinterpret_cast<uint32_t*>(p);
    return w;
}

}  // namespace

size_t dedup_workspace_bytes(uint32_t n) {
    if (n == 0) return 0;
    return align_up(size_t(n) * 4u) + align_up(size_t(256) * kMaxBlocks * 4u) + align_up(size_t(kMaxBlocks) * 4u) +
           256u;
}

hipError_t launch_dedup(const int32_t* ids, const int32_t* history, uint32_t n, uint32_t seq_len, int32_t* perm,
                        int32_t* offsets, int32_t* n_unique, void* ws, hipStream_t stream) {
    if (n == 0) {
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(1), 0, stream, offsets, n_unique);
        return hipGetLastError();
    }
    const Ids s{ids, history, seq_len};
    const Workspace w = carve(ws, n);
    const uint32_t tile = tile_for(n);
    const uint32_t blocks = (n + tile - 1u) / tile;
    // Even passes write the workspace copy, odd passes the caller's perm, so
    // the 16th pass leaves the sorted order in perm.
    const int32_t* src = nullptr;  // identity before the first pass
    for (int pass = 0; pass < kPasses; ++pass) {
        int32_t* dst = (pass & 1) ? perm : w.tmp;
        hipLaunchKernelGGL(hist_kernel, dim3(blocks), dim3(kThreads), 0, stream, s, src, n, tile, pass, w.counts);
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, w.counts, 256u * blocks,
                           static_cast<uint32_t*>(nullptr));
        hipLaunchKernelGGL(scatter_kernel, dim3(blocks), dim3(kThreads), 0, stream, s, src, n, tile, pass, w.counts,
                           dst);
        src = dst;
    }
    hipLaunchKernelGGL(flag_count_kernel, dim3(blocks), dim3(kThreads), 0, stream, s, perm, n, tile, w.bsum);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, w.bsum, blocks, w.total);
    hipLaunchKernelGGL(group_offsets_kernel, dim3(blocks), dim3(kThreads), 0, stream, s, perm, n, tile, w.bsum,
                       w.total, offsets, n_unique);
    return hipGetLastError();
}

}  // namespace engram
