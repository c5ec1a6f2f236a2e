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
// of batch_order.h (tiles of 64 positions, several sequences at the same
// position per block; plain token order for one sequence).  In a large batch
// the waves of a block with equal addresses share one gather, as in the
// batched gather.  The window ids are wave-uniform; lane q < 24
// hashes row q of the module in parallel with the others, with the same
// multiply-xor and modulus (a mask for power-of-two row counts) as
// hash_kernel, and then owns that row in the lane-addressed loads.  The
// accumulation is the fused multiply-add sequence of gather_reduce_kernel, so
// the result is bitwise identical to engram_hash followed by
// engram_gather_reduce.
//
// Dedup mode (groups from engram_dedup): one wave per (group, module) takes
// the group's first token, hashes its window and gathers once, then stores
// the vector to every member, as gather_reduce_kernel does in dedup mode.
// Equal windows give equal addresses, so this is bitwise the direct result,
// with one hash and one gather per distinct window.
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

// Token ids and, in dedup mode, the groups that engram_dedup wrote.
struct Tokens {
    const int32_t* ids;
    const int32_t* history;
    uint32_t n_tok;
    const int32_t* perm;      // dedup mode only
    const int32_t* offsets;
    const int32_t* n_unique;
};

// How a launch maps blocks to tokens: the batch order of batch_order.h,
// each wave gathering for itself (kTokens) or the waves posting their
// addresses in LDS and the first of each set of equal ones gathering for all
// (kShared); or one wave per dedup group (kGroups).
enum { kTokens = 0, kShared = 1, kGroups = 2 };

template <bool POW2, int FMT, int MODE, uint32_t W = kBlockWaves>
__global__ __launch_bounds__(64 * W) void lookup_kernel(const LookupParams P, const Tokens T, uint32_t base,
                                                        uint32_t item_end, BatchOrder batch, float* __restrict__ out) {
    const int32_t* __restrict__ ids = T.ids;
    const int32_t* __restrict__ history = T.history;
    const uint32_t m = blockIdx.x & 1u;  // block b: module b % 2
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;

    uint32_t item = 0;  // kGroups: the group
    bool valid = true;  // kShared: an idle wave of a partial block still takes part in its barrier
    uint32_t seq = 0, t = 0;
    if (MODE == kGroups) {
        item = base + (blockIdx.x >> 1) * kBlockWaves + wave;
        const int32_t nu = *T.n_unique;  // negative: the dedup call failed, there are no groups
        const uint32_t limit = nu > 0 ? min(item_end, static_cast<uint32_t>(nu)) : 0u;
        if (item >= limit) return;
    } else {
        const uint32_t blk = base + (blockIdx.x >> 1);
        if (blk >= batch.n_blocks) return;  // the whole block
        block_token(blk, wave, batch, &seq, &t, &valid);
        if (MODE == kTokens && !valid) return;
        if (!valid) seq = t = 0;  // an idle wave works on token 0 and stores nothing
    }

    // Lane q < 24 hashes the module's row q = 8*(order-2) + head (lanes
    // 24..63 repeat row 0) and owns that row in the lane-addressed loads.  Its
    // lane-indexed parameters -- the 4 multipliers of its (order, head), its
    // row count (and reciprocal), its table and scale bases -- are requested
    // here, before the window ids, so that they take one memory round trip
    // together while the wave-uniform id loads below are in flight.  A row of
    // order n multiplies w_k for k < n only: the multiplier for k >= n is
    // replaced by 0, with no branch between the loads.
    const uint32_t s0 = m * kRowsPerModule;
    const uint32_t mb = m * (kRowsPerModule * ENGRAM_MAX_ORDER);
    const uint32_t q = owned_row(lane);
    const uint32_t order = ENGRAM_MIN_ORDER + q / ENGRAM_N_HEADS;
    uint64_t mk[ENGRAM_MAX_ORDER];
#pragma unroll
    for (uint32_t k = 0; k < ENGRAM_MAX_ORDER; ++k) mk[k] = P.h.mult[mb + q * ENGRAM_MAX_ORDER + k];
    const uint64_t R = P.h.rows[s0 + q];
    const uint64_t magic = POW2 ? 0u : P.h.magic[s0 + q];
    const RowBases rb = row_bases(P.g, s0, lane);

    uint32_t tok;
    if (MODE == kGroups) {
        // the group's first member; its position in its sequence gives the window
        const uint32_t first = static_cast<uint32_t>(T.offsets[item]);
        if (first >= T.n_tok) return;
        tok = static_cast<uint32_t>(T.perm[first]);
        if (tok >= T.n_tok) return;
        seq = tok / batch.seq_len;
        t = tok - seq * batch.seq_len;
    } else {
        tok = seq * batch.seq_len + t;
    }

    // Window of the token (wave-uniform): w[k] = id k positions back, else
    // history, else 0, each through the vocabulary map.  When the whole
    // window lies inside the sequence (every position but the first 3), the
    // 4 id loads, then the 4 map loads, are issued back to back.
    uint64_t w[ENGRAM_MAX_ORDER];
    if (t >= ENGRAM_MAX_ORDER - 1) {
        uint32_t v[ENGRAM_MAX_ORDER];
#pragma unroll
        for (int k = 0; k < ENGRAM_MAX_ORDER; ++k) v[k] = static_cast<uint32_t>(ids[tok - k]);
        const uint32_t* __restrict__ vmap = P.h.vocab_map;
        if (vmap) {
#pragma unroll
            for (int k = 0; k < ENGRAM_MAX_ORDER; ++k) v[k] = vmap[v[k]];
        }
#pragma unroll
        for (int k = 0; k < ENGRAM_MAX_ORDER; ++k) w[k] = v[k];
    } else {
#pragma unroll
        for (int k = 0; k < ENGRAM_MAX_ORDER; ++k)
            w[k] = window_id(ids, history, P.h.vocab_map, tok, seq, static_cast<int32_t>(t), k);
    }

    uint64_t x = 0;
#pragma unroll
    for (uint32_t k = 0; k < ENGRAM_MAX_ORDER; ++k) x ^= w[k] * (k < order ? mk[k] : 0u);
    const uint32_t a = POW2 ? static_cast<uint32_t>(x & (R - 1u)) : mod_rows(x, R, magic);

    const size_t col = static_cast<size_t>(m) * kRowBytes + lane * 4u;
    if (MODE == kShared) {
        // as gather_batched_kernel: the first wave of each set of equal
        // addresses in the block gathers once and stores to every token of
        // the set; the others end after the barrier
        __shared__ uint32_t sa[W][kRowsPerModule];
        __shared__ uint32_t stok[W];
        if (lane < kRowsPerModule) sa[wave][lane] = a;
        if (lane == 0) stok[wave] = valid ? tok + 1u : 0u;
        __syncthreads();
        if (!valid || first_equal_wave(sa, stok, wave, lane, a) != wave) return;
        RowSet r;
        load_rows_at<FMT>(rb, a, lane, r);
        const f32x4 acc = sum_rows<FMT>(r, lane);
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(tok) * (2 * kRowBytes) + col));
        store_to_equal_waves<W>(sa, stok, wave, lane, a, acc, out + col);
        return;
    }
    RowSet r;
    load_rows_at<FMT>(rb, a, lane, r);
    const f32x4 acc = sum_rows<FMT>(r, lane);
    if (MODE == kTokens) {
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(tok) * (2 * kRowBytes) + col));
    } else {
        // Every group has a member (the token above), so the first store is
        // unconditional, as in gather_reduce_kernel's dedup mode.  The
        // members' indices are read 64 at a time, one per lane, and broadcast
        // one by one: a group shared by many sequences costs one load per 64
        // members instead of a dependent load before every store.
        uint32_t i = static_cast<uint32_t>(T.offsets[item]);
        const uint32_t end = min(static_cast<uint32_t>(T.offsets[item + 1]), T.n_tok);
        do {
            const uint32_t cnt = min(64u, end - i);
            const uint32_t mine = lane < cnt ? static_cast<uint32_t>(T.perm[i + lane]) : T.n_tok;
            uint32_t j = 0;
            do {
                const uint32_t u = static_cast<uint32_t>(__builtin_amdgcn_readlane(mine, j));
                if (u < T.n_tok)
                    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(out + static_cast<size_t>(u) * (2 * kRowBytes) + col));
            } while (++j < cnt);
            i += cnt;
        } while (i < end);
    }
}

template <bool POW2, int FMT>
void launch_one(const LookupParams& p, const Tokens& tk, uint32_t grid, uint32_t base, uint32_t end,
                const BatchOrder& batch, float* out, hipStream_t stream) {
    if (tk.perm)
        hipLaunchKernelGGL((lookup_kernel<POW2, FMT, kGroups>), dim3(grid), dim3(256), 0, stream, p, tk, base, end,
                           batch, out);
    else if (batch.wshift == 3)
        hipLaunchKernelGGL((lookup_kernel<POW2, FMT, kShared, 8>), dim3(grid), dim3(512), 0, stream, p, tk, base, end,
                           batch, out);
    else if (batch.share)
        hipLaunchKernelGGL((lookup_kernel<POW2, FMT, kShared>), dim3(grid), dim3(256), 0, stream, p, tk, base, end,
                           batch, out);
    else
        hipLaunchKernelGGL((lookup_kernel<POW2, FMT, kTokens>), dim3(grid), dim3(256), 0, stream, p, tk, base, end,
                           batch, out);
}

}  // namespace

hipError_t launch_lookup(const HashParams& h, const GatherParams& g, const int32_t* ids, const int32_t* history,
                         uint32_t n_tok, uint32_t seq_len, const int32_t* perm, const int32_t* offsets,
                         const int32_t* n_unique, float* out, hipStream_t stream) {
    LookupParams p;
    p.h = h;
    p.g = g;
    const Tokens tk{ids, history, n_tok, perm, offsets, n_unique};
    bool pow2 = true;
    for (int s = 0; s < kSub; ++s) pow2 = pow2 && (h.rows[s] & (h.rows[s] - 1u)) == 0;
    // Dedup mode launches cover at most 2^24 groups, 4 per block; the batch
    // order at most 2^22 blocks (per module): either way the grid stays below
    // 2^31 threads.
    const bool mx = g.scale_format == ENGRAM_SCALE_E8M0_BLOCK32;
    const BatchOrder batch = batch_order(n_tok, seq_len);
    const uint32_t total = perm ? n_tok : batch.n_blocks;
    const uint32_t step = perm ? (1u << 24) : (1u << 22);
    for (uint32_t base = 0; base < total; base += step) {
        const uint32_t n = min(step, total - base);
        const uint32_t grid = perm ? 2u * (((n + 3u) / 4u + 3u) & ~3u) : 2u * n;
        if (pow2 && mx)
            launch_one<true, ENGRAM_SCALE_E8M0_BLOCK32>(p, tk, grid, base, base + n, batch, out, stream);
        else if (pow2)
            launch_one<true, ENGRAM_SCALE_F32_ROW>(p, tk, grid, base, base + n, batch, out, stream);
        else if (mx)
            launch_one<false, ENGRAM_SCALE_E8M0_BLOCK32>(p, tk, grid, base, base + n, batch, out, stream);
        else
            launch_one<false, ENGRAM_SCALE_F32_ROW>(p, tk, grid, base, base + n, batch, out, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace engram
