// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

constexpr int kSub = ENGRAM_N_SUB;
constexpr int kRowsPerModule = ENGRAM_ROWS_PER_MODULE;
constexpr int kRowBytes = ENGRAM_ROW_BYTES;
constexpr int kMult = ENGRAM_N_MULT;
constexpr int64_t kMaxTokens = (int64_t(1) << 31) - 1;

// Everything the hash kernel needs, passed by value (lands in the kernel
// argument segment and is read with scalar loads).
struct HashParams {
    uint64_t mult[kMult];  // M[((m*3 + (n-2))*8 + h)*4 + k]
    uint64_t rows[kSub];   // R_s
    uint64_t magic[kSub];  // floor((2^64 - 1) / R_s): exact x mod R_s with one correction
    const uint32_t* vocab_map;  // id normalisation applied to window ids, or nullptr
};

// Window id k of a token: the id k positions back, else the caller's history
// (history[seq][2] is position -1), else id 0; then the plan's vocabulary map.
__device__ __forceinline__ uint32_t window_id(const int32_t* __restrict__ ids, const int32_t* __restrict__ history,
                                              const uint32_t* __restrict__ vocab_map, uint32_t tok, uint32_t seq,
                                              int32_t t, int k) {
    int32_t v = 0;
    if (t - k >= 0)
        v = ids[tok - k];
    else if (history)
        v = history[seq * 3u + static_cast<uint32_t>(3 + t - k)];
    const uint32_t u = static_cast<uint32_t>(v);
    return vocab_map ? vocab_map[u] : u;
}

// Row and scale base pointers of the 48 sub-tables, by value.  sc[s] points
// at fp32 [R_s] or at uint8 [R_s][8] (E8M0 per 32-element block), as
// scale_format says.
struct GatherParams {
    const uint8_t* tab[kSub];
    const void* sc[kSub];
    uint32_t scale_format;
};

}  // namespace engram

struct engram_plan_s {
    uint64_t hash_seed;
    uint32_t vocab_size;
    engram::HashParams hash;
    engram::GatherParams gather;
};

namespace engram {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipError_t launch_hash(const HashParams& p, const int32_t* ids, const int32_t* history,
                       uint32_t n_tok, uint32_t seq_len, uint32_t* addr, hipStream_t stream);

hipError_t launch_gather_reduce(const GatherParams& p, const uint32_t* addr, uint32_t n_tok,
                                const int32_t* perm, const int32_t* offsets, const int32_t* n_unique,
                                float* out, hipStream_t stream);

// perm == nullptr: direct mode; else dedup mode with engram_dedup's groups.
hipError_t launch_lookup(const HashParams& h, const GatherParams& g, const int32_t* ids, const int32_t* history,
                         uint32_t n_tok, uint32_t seq_len, const int32_t* perm, const int32_t* offsets,
                         const int32_t* n_unique, float* out, hipStream_t stream);

// weights != nullptr: weighted per-module sums into out [n_tok][2][256];
// weights == nullptr: un-reduced rows into out [n_tok][48][256].
hipError_t launch_gate_io(const GatherParams& p, const uint32_t* addr, const float* weights, uint32_t n_tok,
                          float* out, hipStream_t stream);

// Workspace bytes of launch_dedup for n_tok tokens under a vocabulary bound (0 = none).
size_t dedup_workspace_bytes(uint32_t n_tok, uint32_t vocab_size);

// Tokens per dedup call.  Each tile of the sort reads the published counts of
// all earlier tiles, a cost that grows with the square of the tile count.
constexpr int64_t kMaxDedupTokens = (int64_t(1) << 22);

hipError_t launch_dedup(const int32_t* ids, const int32_t* history, uint32_t n_tok, uint32_t seq_len,
                        uint32_t vocab_size, int32_t* perm, int32_t* offsets, int32_t* n_unique, void* ws,
                        hipStream_t stream);

// Counts into counts[3] (cleared first): negative ids, ids >= vocab (vocab > 0), addresses >= R_s.
hipError_t launch_check(const HashParams& h, uint32_t vocab, const int32_t* ids, uint64_t n_ids,
                        const int32_t* history, uint64_t n_hist, const uint32_t* addr, uint64_t n_addr_tok,
                        int32_t* counts, hipStream_t stream);

}  // namespace engram
