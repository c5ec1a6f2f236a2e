// Input-range check: counts, without reading a table or the vocabulary map,
// the contract violations the lookup kernels do not check for themselves --
// negative ids, ids at or above the plan's vocabulary bound, and row
// addresses at or above their sub-table's row count.  The lookup reads the
// rows an address names [How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB
// of It Is a Lookup Table, section "Engram: the table that is never
// multiplied"], so an address out of range would read outside its table.
//
// One pass over the arrays: ballots count per wave, LDS per block, one
// atomic per block and counter.  A small kernel clears the three counters
// first (no memset, so the pair can be captured in a HIP graph).
#include <algorithm>

#include "engram_internal.h"

namespace engram {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kMaxBlocks = 4096;

struct CheckArgs {
    const int32_t* ids;       // [n_ids] or nullptr
    uint64_t n_ids;
    const int32_t* history;   // [n_hist] or nullptr
    uint64_t n_hist;
    uint32_t vocab;           // exclusive id bound, 0 = none beyond non-negative
    const uint4* addr;        // [n_addr_tok * 12] (48 words per token) or nullptr
    uint64_t n_quads;
    uint32_t last_row[kSub];  // R_s - 1 (R_s <= 2^32)
};

__global__ void clear_kernel(int32_t* __restrict__ counts) {
    if (threadIdx.x < 3) counts[threadIdx.x] = 0;
}

__device__ __forceinline__ uint32_t id_bad_negative(int32_t v) { return v < 0 ? 1u : 0u; }

__global__ __launch_bounds__(kThreads) void check_kernel(const CheckArgs a, int32_t* __restrict__ counts) {
    __shared__ uint32_t last_row[kSub];
    __shared__ uint32_t part[3][kThreads / 64];
    if (threadIdx.x < kSub) last_row[threadIdx.x] = a.last_row[threadIdx.x];
    __syncthreads();
    const uint64_t gtid = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
    const uint64_t stride = uint64_t(gridDim.x) * kThreads;
    uint32_t neg = 0, big = 0, bad_addr = 0;
    for (uint64_t i = gtid; i < a.n_ids + a.n_hist; i += stride) {
        const int32_t v = i < a.n_ids ? a.ids[i] : a.history[i - a.n_ids];
        neg += id_bad_negative(v);
        if (a.vocab != 0 && v >= 0 && static_cast<uint32_t>(v) >= a.vocab) ++big;
    }
    for (uint64_t q = gtid; q < a.n_quads; q += stride) {
        const uint4 x = a.addr[q];
        const uint32_t s0 = 4u * static_cast<uint32_t>(q % 12u);  // sub-tables of this quad of a token's 48 words
        bad_addr += (x.x > last_row[s0]) + (x.y > last_row[s0 + 1]) + (x.z > last_row[s0 + 2]) + (x.w > last_row[s0 + 3]);
    }
    // per-wave, then per-block sums; one atomic per block and counter
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        neg += __shfl_xor(neg, off);
        big += __shfl_xor(big, off);
        bad_addr += __shfl_xor(bad_addr, off);
    }
    const uint32_t wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63u) == 0) {
        part[0][wave] = neg;
        part[1][wave] = big;
        part[2][wave] = bad_addr;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        uint32_t c = 0;
#pragma unroll
        for (uint32_t k = 0; k < kThreads / 64; ++k) c += part[threadIdx.x][k];
        if (c) atomicAdd(&counts[threadIdx.x], static_cast<int32_t>(c));
    }
}

}  // namespace

hipError_t launch_check(const HashParams& h, uint32_t vocab, const int32_t* ids, uint64_t n_ids,
                        const int32_t* history, uint64_t n_hist, const uint32_t* addr, uint64_t n_addr_tok,
                        int32_t* counts, hipStream_t stream) {
    CheckArgs a;
    a.ids = ids;
    a.n_ids = ids ? n_ids : 0;
    a.history = history;
    a.n_hist = history ? n_hist : 0;
    a.vocab = vocab;
    a.addr = reinterpret_cast<const uint4*>(addr);
    a.n_quads = addr ? n_addr_tok * (kSub / 4) : 0;
    for (int s = 0; s < kSub; ++s) a.last_row[s] = static_cast<uint32_t>(h.rows[s] - 1u);
    hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(64), 0, stream, counts);
    const uint64_t work = std::max<uint64_t>(a.n_ids + a.n_hist, a.n_quads);
    const uint32_t blocks = static_cast<uint32_t>(std::min<uint64_t>(kMaxBlocks, std::max<uint64_t>(1, (work + kThreads - 1) / kThreads)));
    hipLaunchKernelGGL(check_kernel, dim3(blocks), dim3(kThreads), 0, stream, a, counts);
    return hipGetLastError();
}

}  // namespace engram
