// Visiting order for a batch of sequences, shared by the fused lookup and
// the batched gather.
//
// A block of W waves (one module) takes G sequences at W / G consecutive
// positions, one wave per token: G = 8, 4, 2 or 1 (batch_order below picks it
// from the sequence count) and W = max(G, 4).  Blocks go in tiles of `tile`
// positions (64, or the whole sequence if shorter); within a tile, group of
// G sequences by group, and within a group by position.  The same positions
// of the next group come one group's blocks later, 64 / (W / G) blocks x 2
// modules for a 64-position tile, a multiple of 8, so the round-robin
// dispatcher (block b to XCD b % 8) sends them to the same XCD.  Sequences
// that share a prefix therefore find each prefix row in that XCD's L2 after
// its first fetch, and in a large batch the kernels go further (`share`):
// the waves of a block post their 24 addresses in LDS, and the first wave of
// each set of equal addresses gathers once and stores the sum for all of
// them.  With one sequence (G = 1) a block is 4 consecutive tokens and the
// order is plain token order.
#pragma once

#include "engram_internal.h"

namespace engram {

constexpr uint32_t kBatchTile = 64;
constexpr uint32_t kBlockWaves = 4;     // waves per block, unless G = 8
// Sharing sums within a block costs a barrier after the addresses are known,
// so a block's gathers start with its slowest address.  A launch of a few
// thousand tokens fits the chip at once (two waves per token; 256 CUs hold
// 8,192 waves) and is bound by that latency, so only batches of at least this
// many tokens share.
constexpr uint32_t kShareMinTokens = 8192;

struct BatchOrder {
    uint32_t n_seq, seq_len, tile;  // tile = min(kBatchTile, seq_len)
    uint32_t gshift;                // G = 1 << gshift sequences per block
    uint32_t wshift;                // W = 1 << wshift waves per block
    uint32_t share;                 // 1: equal-address waves share one gather
    uint32_t n_groups;              // ceil(n_seq / G)
    uint32_t full_tiles;            // tiles of `tile` positions
    uint32_t last;                  // positions in the partial last tile, 0 if none
    uint32_t tile_blocks;           // blocks per full tile (per module)
    uint32_t n_blocks;              // blocks per module in all
};

// Sequences per block: the largest power of two G <= 2^max_shift whose idle
// waves (G * groups - n_seq) are at most 1/8 of the sequences, else 1.
inline uint32_t batch_gshift(uint32_t n_seq, uint32_t max_shift) {
    for (uint32_t sh = max_shift; sh > 0; --sh) {
        const uint32_t g = 1u << sh;
        const uint64_t idle = uint64_t((n_seq + g - 1) / g) * g - n_seq;
        if (idle * 8u <= n_seq) return sh;
    }
    return 0;
}

// G = 8 (8-wave blocks) only where the waves share sums: it halves the
// gathers of a prefix shared by the batch, and without sharing it would only
// make the blocks larger.
inline BatchOrder batch_order(uint32_t n_tok, uint32_t seq_len) {
    BatchOrder o;
    o.n_seq = n_tok / seq_len;
    o.seq_len = seq_len;
    o.tile = seq_len < kBatchTile ? seq_len : kBatchTile;
    const bool large = n_tok >= kShareMinTokens;
    o.gshift = batch_gshift(o.n_seq, large ? 3u : 2u);
    o.wshift = o.gshift > 2u ? o.gshift : 2u;
    o.share = large && o.gshift > 0 ? 1u : 0u;
    const uint32_t per = 1u << (o.wshift - o.gshift);  // positions per block
    o.n_groups = (o.n_seq + (1u << o.gshift) - 1u) >> o.gshift;
    o.full_tiles = seq_len / o.tile;
    o.last = seq_len - o.full_tiles * o.tile;
    o.tile_blocks = o.n_groups * ((o.tile + per - 1u) / per);
    o.n_blocks = o.full_tiles * o.tile_blocks + o.n_groups * ((o.last + per - 1u) / per);
    return o;
}

// Sequence and position of wave `wave` of block `blk` (< o.n_blocks); *valid
// is false for the idle waves of a partial group or a narrow last tile.
// Host-callable too, so the mapping can be checked on the CPU.
__host__ __device__ __forceinline__ void block_token(uint32_t blk, uint32_t wave, const BatchOrder& o,
                                                     uint32_t* seq, uint32_t* t, bool* valid) {
    uint32_t tile_idx = o.full_tiles, rem, width = o.last;
    if (blk < o.full_tiles * o.tile_blocks) {
        tile_idx = blk / o.tile_blocks;
        width = o.tile;
    }
    rem = blk - tile_idx * o.tile_blocks;
    const uint32_t per = 1u << (o.wshift - o.gshift);
    const uint32_t bpg = (width + per - 1u) / per;  // blocks per group in this tile
    const uint32_t g = rem / bpg;
    const uint32_t q = rem - g * bpg;
    const uint32_t s = (g << o.gshift) + (wave & ((1u << o.gshift) - 1u));
    const uint32_t p = q * per + (wave >> o.gshift);
    *valid = s < o.n_seq && p < width;
    *seq = s;
    *t = tile_idx * o.tile + p;
}

// The first valid wave of the block, before this one, whose 24 addresses
// (lane q < 24 holds address q; lanes 24..63 repeat address 0) equal this
// wave's, or this wave itself.  sa holds every wave's addresses in LDS and
// stok[u] is nonzero for a valid wave u; call after the barrier that follows
// their writes.
__device__ __forceinline__ uint32_t first_equal_wave(const uint32_t (*sa)[kRowsPerModule], const uint32_t* stok,
                                                     uint32_t wave, uint32_t lane, uint32_t a) {
    const uint32_t q = lane < kRowsPerModule ? lane : 0u;
    for (uint32_t u = 0; u < wave; ++u)
        if (stok[u] && __ballot(lane < kRowsPerModule && sa[u][q] != a) == 0) return u;
    return wave;
}

// For the first wave of a set of equal addresses (first_equal_wave returned
// the wave itself): stores its sum `acc` to the token of every later valid
// wave with the same addresses, which end without gathering.  stok[u] holds
// wave u's token + 1; `col` is out advanced to this lane's columns of the
// module.  Equality is exact, so such a wave u finds this wave first too.
template <uint32_t W, class V>  // W waves per block; V: the lane's 4 floats
__device__ __forceinline__ void store_to_equal_waves(const uint32_t (*sa)[kRowsPerModule], const uint32_t* stok,
                                                     uint32_t wave, uint32_t lane, uint32_t a, V acc, float* col) {
    const uint32_t q = lane < kRowsPerModule ? lane : 0u;
    for (uint32_t u = wave + 1; u < W; ++u) {
        const uint32_t t = stok[u];
        if (t && __ballot(lane < kRowsPerModule && sa[u][q] != a) == 0)
            __builtin_nontemporal_store(acc, reinterpret_cast<V*>(col + static_cast<size_t>(t - 1u) * (2 * kRowBytes)));
    }
}

// The batched gather: engram_gather_reduce (direct mode) over n_seq x seq_len
// tokens, visited in the order above.
hipError_t launch_gather_batched(const GatherParams& p, const uint32_t* addr, uint32_t n_tok, uint32_t seq_len,
                                 float* out, hipStream_t stream);

}  // namespace engram
