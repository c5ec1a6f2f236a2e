// Deduplication of equal id windows for batched prefill with shared prefixes.
//
// The row addresses of a token depend on its id window alone [DeepSeek V4.1
// Flash: The VRAM Killer, section "What makes up the 511 GB of weights?";
// How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a Lookup
// Table, section "Engram: the table that is never multiplied"], so tokens
// with equal windows read the same 48 rows and one lookup serves them all.
// Prompts that share a prefix repeat whole windows across sequences.
//
// Method: a stable least-significant-digit radix sort of (key, token) pairs
// with 8-bit digits, then a group flag where the key changes, a scan of the
// flags and the group start offsets.
//
// Key: with every id below 2^B (B from the plan's vocabulary bound, 31 when
// none is given), the window packs exactly into 4B bits,
//     key = w_0 * 2^(3B) + w_1 * 2^(2B) + w_2 * 2^B + w_3,
// whose numeric order is the lexicographic order of (w_0, w_1, w_2, w_3).  A
// 129,280-id vocabulary gives B = 17, a 68-bit key and 9 passes.
//
// A pass is three kernels, all with many blocks:
//   hist:     per-block digit histogram (wave ballots group equal digits so a
//             wave adds each distinct digit once)        -> cnt[digit][block]
//   colscan:  one block per digit: exclusive scan over blocks -> cnt, and the
//             digit's total                               -> tot[digit]
//   scatter:  every block scans the 256 totals in LDS, then ranks its elements
//             stably (per 256-element sub-tile: ballot match within a wave,
//             per-wave counts in LDS across waves) and moves (key, token).
#include "engram_internal.h"

namespace engram {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kTile = 1024;          // elements per block per pass (4 sub-tiles)

struct Ids {
    const int32_t* ids;
    const int32_t* history;
    uint32_t seq_len;
};

// w_k of token tok: the id k positions back, else history, else 0.
__device__ __forceinline__ uint32_t window_word(const Ids& s, uint32_t tok, int k) {
    const uint32_t seq = tok / s.seq_len;
    const int32_t t = static_cast<int32_t>(tok - seq * s.seq_len);
    if (t - k >= 0) return static_cast<uint32_t>(s.ids[tok - k]);
    if (s.history) return static_cast<uint32_t>(s.history[seq * 3u + static_cast<uint32_t>(3 + t - k)]);
    return 0u;
}

__global__ __launch_bounds__(kThreads) void build_keys_kernel(Ids s, uint32_t n, uint32_t bits,
                                                              uint64_t* __restrict__ klo, uint64_t* __restrict__ khi,
                                                              int32_t* __restrict__ val) {
    const uint32_t tok = blockIdx.x * kThreads + threadIdx.x;
    if (tok >= n) return;
    uint64_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // w_0 most significant
        hi = (hi << bits) | (lo >> (64 - bits));
        lo = (lo << bits) | window_word(s, tok, k);
    }
    klo[tok] = lo;
    khi[tok] = hi;
    val[tok] = static_cast<int32_t>(tok);
}

// Lanes of this wave whose `valid` digit equals this lane's.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid) {
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool set = (d >> bit) & 1u;
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
    }
    return peers;
}

__global__ __launch_bounds__(kThreads) void hist_kernel(const uint64_t* __restrict__ klo,
                                                        const uint64_t* __restrict__ khi, uint32_t n, int pass,
                                                        uint32_t* __restrict__ cnt) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t lt = (uint64_t(1) << lane) - 1u;
    const uint64_t* key = pass < 8 ? klo : khi;
    const int sh = 8 * (pass & 7);
    const uint32_t begin = blockIdx.x * kTile;
#pragma unroll
    for (uint32_t j = 0; j < kTile / kThreads; ++j) {
        const uint32_t i = begin + j * kThreads + threadIdx.x;
        const bool valid = i < n;
        const uint32_t d = valid ? static_cast<uint32_t>(key[i] >> sh) & 0xFFu : 0u;
        const uint64_t peers = match_digit(d, valid);
        if (valid && (peers & lt) == 0) atomicAdd(&h[d], static_cast<uint32_t>(__popcll(peers)));
    }
    __syncthreads();
    cnt[static_cast<size_t>(threadIdx.x) * gridDim.x + blockIdx.x] = h[threadIdx.x];
}

// Block-wide exclusive scan of one value per thread (blockDim.x = 1024).
__device__ __forceinline__ uint32_t block_exclusive_scan_1024(uint32_t x, uint32_t* part, uint32_t* total) {
    part[threadIdx.x] = x;
    __syncthreads();
    for (uint32_t off = 1; off < 1024u; off <<= 1) {
        const uint32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0u;
        __syncthreads();
        part[threadIdx.x] += add;
        __syncthreads();
    }
    const uint32_t incl = part[threadIdx.x];
    if (total) *total = part[1023];
    return incl - x;
}

// One block (1024 threads) per digit: exclusive scan of cnt[digit][0..blocks).
__global__ __launch_bounds__(1024) void colscan_kernel(uint32_t* __restrict__ cnt, uint32_t blocks,
                                                       uint32_t* __restrict__ tot) {
    __shared__ uint32_t part[1024];
    __shared__ uint32_t total;
    uint32_t* row = cnt + static_cast<size_t>(blockIdx.x) * blocks;
    const uint32_t per = (blocks + 1023u) / 1024u;
    const uint32_t b0 = min(blocks, threadIdx.x * per), b1 = min(blocks, b0 + per);
    uint32_t sum = 0;
    for (uint32_t b = b0; b < b1; ++b) sum += row[b];
    uint32_t run = block_exclusive_scan_1024(sum, part, &total);
    for (uint32_t b = b0; b < b1; ++b) {
        const uint32_t x = row[b];
        row[b] = run;
        run += x;
    }
    if (threadIdx.x == 0) tot[blockIdx.x] = total;
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(const uint64_t* __restrict__ klo,
                                                           const uint64_t* __restrict__ khi,
                                                           const int32_t* __restrict__ val, uint32_t n, int pass,
                                                           const uint32_t* __restrict__ cnt,
                                                           const uint32_t* __restrict__ tot,
                                                           uint64_t* __restrict__ klo_out,
                                                           uint64_t* __restrict__ khi_out,
                                                           int32_t* __restrict__ val_out) {
    __shared__ uint32_t base[256];  // next output slot of each digit for this block
    __shared__ uint32_t wave_cnt[kWaves][256];
    __shared__ uint32_t wsum[kWaves];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t lt = (uint64_t(1) << lane) - 1u;

    // Exclusive scan of the 256 digit totals (4 waves x 64 lanes).
    {
        const uint32_t t = tot[threadIdx.x];
        uint32_t x = t;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= static_cast<uint32_t>(off)) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        uint32_t pre = 0;
        for (uint32_t w = 0; w < wave; ++w) pre += wsum[w];
        base[threadIdx.x] = pre + x - t + cnt[static_cast<size_t>(threadIdx.x) * gridDim.x + blockIdx.x];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) wave_cnt[w][threadIdx.x] = 0;
        __syncthreads();
    }

    const uint32_t begin = blockIdx.x * kTile;
    const int sh = 8 * (pass & 7);
    for (uint32_t j = 0; j < kTile / kThreads; ++j) {
        const uint32_t i = begin + j * kThreads + threadIdx.x;
        const bool valid = i < n;
        uint64_t lo = 0, hi = 0;
        int32_t v = 0;
        if (valid) {
            lo = klo[i];
            hi = khi[i];
            v = val[i];
        }
        const uint32_t d = static_cast<uint32_t>((pass < 8 ? lo : hi) >> sh) & 0xFFu;
        const uint64_t peers = match_digit(d, valid);
        const uint32_t rank_in_wave = __popcll(peers & lt);
        if (valid && rank_in_wave == 0) wave_cnt[wave][d] = __popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pos = base[d] + rank_in_wave;
            for (uint32_t w = 0; w < wave; ++w) pos += wave_cnt[w][d];
            klo_out[pos] = lo;
            khi_out[pos] = hi;
            val_out[pos] = v;
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

__device__ __forceinline__ uint32_t group_flag(const uint64_t* __restrict__ klo, const uint64_t* __restrict__ khi,
                                               uint32_t i) {
    return (i == 0 || klo[i] != klo[i - 1] || khi[i] != khi[i - 1]) ? 1u : 0u;
}

__global__ __launch_bounds__(kThreads) void flag_count_kernel(const uint64_t* __restrict__ klo,
                                                              const uint64_t* __restrict__ khi, uint32_t n,
                                                              uint32_t* __restrict__ bsum) {
    const uint32_t begin = blockIdx.x * kTile;
    uint32_t local = 0;
    for (uint32_t i = begin + threadIdx.x; i < min(n, begin + kTile); i += kThreads) local += group_flag(klo, khi, i);
    __shared__ uint32_t c[kWaves];
    // wave reduction
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    if ((threadIdx.x & 63u) == 0) c[threadIdx.x >> 6] = local;
    __syncthreads();
    if (threadIdx.x == 0) bsum[blockIdx.x] = c[0] + c[1] + c[2] + c[3];
}

// Exclusive scan of len values with one block of 1024 threads; total to *total.
__global__ __launch_bounds__(1024) void scan_kernel(uint32_t* __restrict__ v, uint32_t len,
                                                    uint32_t* __restrict__ total) {
    __shared__ uint32_t part[1024];
    const uint32_t per = (len + 1023u) / 1024u;
    const uint32_t b0 = min(len, threadIdx.x * per), b1 = min(len, b0 + per);
    uint32_t sum = 0;
    for (uint32_t i = b0; i < b1; ++i) sum += v[i];
    uint32_t run = block_exclusive_scan_1024(sum, part, total);
    for (uint32_t i = b0; i < b1; ++i) {
        const uint32_t x = v[i];
        v[i] = run;
        run += x;
    }
}

__global__ __launch_bounds__(kThreads) void group_offsets_kernel(const uint64_t* __restrict__ klo,
                                                                 const uint64_t* __restrict__ khi, uint32_t n,
                                                                 const uint32_t* __restrict__ bsum,
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
    const uint32_t begin = blockIdx.x * kTile;
    for (uint32_t j = 0; j < kTile / kThreads; ++j) {
        const uint32_t i = begin + j * kThreads + threadIdx.x;
        const uint32_t f = i < n ? group_flag(klo, khi, i) : 0u;
        const uint64_t m = __ballot(f);
        if (lane == 0) wave_sum[wave] = __popcll(m);
        __syncthreads();
        uint32_t pos = run + __popcll(m & lt);
        for (uint32_t w = 0; w < wave; ++w) pos += wave_sum[w];
        if (f) offsets[pos] = static_cast<int32_t>(i);
        __syncthreads();
        if (threadIdx.x == 0) run += wave_sum[0] + wave_sum[1] + wave_sum[2] + wave_sum[3];
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

size_t align_up(size_t x) { return (x + 255u) & ~size_t(255u); }

struct Workspace {
    uint64_t* klo[2];
    uint64_t* khi[2];
    int32_t* val;      // second value buffer (the first is the caller's perm)
    uint32_t* cnt;     // [256][blocks]
    uint32_t* tot;     // [256]
    uint32_t* bsum;    // [blocks]
    uint32_t* total;   // [1]
};

size_t layout(uint32_t n, char* base, Workspace* w) {
    const uint32_t blocks = (n + kTile - 1u) / kTile;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += align_up(bytes);
        return p;
    };
    Workspace t;
    t.klo[0] = reinterpret_cast<uint64_t*>(take(size_t(n) * 8));
    t.klo[1] = reinterpret_cast<uint64_t*>(take(size_t(n) * 8));
    t.khi[0] = reinterpret_cast<uint64_t*>(take(size_t(n) * 8));
    t.khi[1] = reinterpret_cast<uint64_t*>(take(size_t(n) * 8));
    t.val = reinterpret_cast<int32_t*>(take(size_t(n) * 4));
    t.cnt = reinterpret_cast<uint32_t*>(take(size_t(256) * blocks * 4));
    t.tot = reinterpret_cast<uint32_t*>(take(256 * 4));
    t.bsum = reinterpret_cast<uint32_t*>(take(size_t(blocks) * 4));
    t.total = reinterpret_cast<uint32_t*>(take(4));
    if (w) *w = t;
    return off;
}

}  // namespace

uint32_t dedup_key_bits(uint32_t vocab_size) {
    if (vocab_size == 0) return 31;
    uint32_t b = 1;
    while (b < 31 && (uint64_t(1) << b) < vocab_size) ++b;
    return b;
}

size_t dedup_workspace_bytes(uint32_t n) { return n == 0 ? 0 : layout(n, nullptr, nullptr); }

hipError_t launch_dedup(const int32_t* ids, const int32_t* history, uint32_t n, uint32_t seq_len, uint32_t vocab_size,
                        int32_t* perm, int32_t* offsets, int32_t* n_unique, void* ws, hipStream_t stream) {
    if (n == 0) {
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(1), 0, stream, offsets, n_unique);
        return hipGetLastError();
    }
    const Ids s{ids, history, seq_len};
    Workspace w;
    layout(n, static_cast<char*>(ws), &w);
    const uint32_t bits = dedup_key_bits(vocab_size);
    const int passes = static_cast<int>((4 * bits + 7) / 8);
    const uint32_t blocks = (n + kTile - 1u) / kTile;
    // Value buffers alternate so that the last pass writes the caller's perm.
    int32_t* vbuf[2] = {perm, w.val};
    int cur = (passes & 1) ? 1 : 0;  // buffer holding the current values
    hipLaunchKernelGGL(build_keys_kernel, dim3((n + kThreads - 1u) / kThreads), dim3(kThreads), 0, stream, s, n, bits,
                       w.klo[0], w.khi[0], vbuf[cur]);
    int kc = 0;
    for (int pass = 0; pass < passes; ++pass) {
        hipLaunchKernelGGL(hist_kernel, dim3(blocks), dim3(kThreads), 0, stream, w.klo[kc], w.khi[kc], n, pass, w.cnt);
        hipLaunchKernelGGL(colscan_kernel, dim3(256), dim3(1024), 0, stream, w.cnt, blocks, w.tot);
        hipLaunchKernelGGL(scatter_kernel, dim3(blocks), dim3(kThreads), 0, stream, w.klo[kc], w.khi[kc], vbuf[cur], n,
                           pass, w.cnt, w.tot, w.klo[kc ^ 1], w.khi[kc ^ 1], vbuf[cur ^ 1]);
        kc ^= 1;
        cur ^= 1;
    }
    hipLaunchKernelGGL(flag_count_kernel, dim3(blocks), dim3(kThreads), 0, stream, w.klo[kc], w.khi[kc], n, w.bsum);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, w.bsum, blocks, w.total);
    hipLaunchKernelGGL(group_offsets_kernel, dim3(blocks), dim3(kThreads), 0, stream, w.klo[kc], w.khi[kc], n, w.bsum,
                       w.total, offsets, n_unique);
    return hipGetLastError();
}

}  // namespace engram
