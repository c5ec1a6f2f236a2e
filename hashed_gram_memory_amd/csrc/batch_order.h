// Visiting order for a batch of sequences, shared by the fused lookup and
// the batched gather.
//
// Items (one per token) are visited in tiles of `tile` positions (64, or the
// whole sequence if shorter); within a tile, sequence by sequence.
// Consecutive items are consecutive positions of one sequence, so a wave's
// neighbours write neighbouring outputs, and the same position of the next
// sequence comes `tile` items later: 32 blocks of 4 items x 2 modules for a
// 64-position tile, which the round-robin dispatcher (block b to XCD b % 8)
// sends to the same XCD.  Sequences that share a prefix therefore read each
// prefix row from that XCD's L2 after its first fetch.  With one sequence
// the order is plain token order.  Measured tile widths on 64 sequences
// sharing a 4,096-token prefix (fused lookup): 32 positions 1.02x, 128 1.04x,
// 256 1.12x the time of 64.
#pragma once

#include "engram_internal.h"

namespace engram {

constexpr uint32_t kBatchTile = 64;

struct BatchOrder {
    uint32_t n_seq, seq_len, tile;  // tile = min(kBatchTile, seq_len), so tile * n_seq <= n_tok
};

inline BatchOrder batch_order(uint32_t n_tok, uint32_t seq_len) {
    return BatchOrder{n_tok / seq_len, seq_len, seq_len < kBatchTile ? seq_len : kBatchTile};
}

// Token index of `item`; its sequence and position in *seq and *t.
__device__ __forceinline__ uint32_t batched_token(uint32_t item, const BatchOrder& o, uint32_t* seq, uint32_t* t) {
    const uint32_t span = o.tile * o.n_seq;  // items per tile of positions
    const uint32_t tile_idx = item / span;
    const uint32_t p0 = tile_idx * o.tile;
    const uint32_t width = min(o.tile, o.seq_len - p0);  // the last tile may be narrower
    const uint32_t rem = item - tile_idx * span;
    *seq = rem / width;
    *t = p0 + (rem - *seq * width);
    return *seq * o.seq_len + *t;
}

// The batched gather: engram_gather_reduce (direct mode) over n_seq x seq_len
// tokens, visited in the order above.
hipError_t launch_gather_batched(const GatherParams& p, const uint32_t* addr, uint32_t n_tok, uint32_t seq_len,
                                 float* out, hipStream_t stream);

}  // namespace engram
