// Host-side check of the batch order of hashed_gram_memory_amd/csrc/batch_order.h,
// the visiting order of the batched gather and the fused lookup: for each
// batch shape, every wave of every block maps to a token in bounds, every
// token is visited exactly once, and the block shape follows the rules the
// kernels assume (4 or 8 waves; 8 only with sharing; sharing only from
// kShareMinTokens tokens and with several sequences per block).  For full
// 64-position tiles it also checks that the blocks of the same positions of
// consecutive sequence groups are a multiple of 8 launch slots apart (two
// modules per block), i.e. on the same XCD under round-robin dispatch.
// Prints "ok <shapes>" and exits 0, or prints the first failure and exits 1.
#include <cstdio>
#include <vector>

#include "batch_order.h"

using engram::BatchOrder;

static int check(uint32_t n_seq, uint32_t seq_len) {
    const uint32_t n_tok = n_seq * seq_len;
    const BatchOrder o = engram::batch_order(n_tok, seq_len);
    const uint32_t G = 1u << o.gshift, W = 1u << o.wshift;
    if (o.n_seq != n_seq || (W != 4 && W != 8) || W < G || (W == 8 && !o.share) ||
        (o.share != 0) != (o.gshift > 0 && n_tok >= engram::kShareMinTokens)) {
        std::printf("shape %u x %u: bad block shape G=%u W=%u share=%u\n", n_seq, seq_len, G, W, o.share);
        return 1;
    }
    std::vector<unsigned char> seen(n_tok, 0);
    for (uint32_t blk = 0; blk < o.n_blocks; ++blk) {
        for (uint32_t wave = 0; wave < W; ++wave) {
            uint32_t seq = 0, t = 0;
            bool valid = false;
            engram::block_token(blk, wave, o, &seq, &t, &valid);
            if (!valid) continue;
            if (seq >= n_seq || t >= seq_len) {
                std::printf("shape %u x %u: block %u wave %u -> (%u, %u) out of bounds\n", n_seq, seq_len, blk,
                            wave, seq, t);
                return 1;
            }
            if (seen[size_t(seq) * seq_len + t]++) {
                std::printf("shape %u x %u: token (%u, %u) visited twice\n", n_seq, seq_len, seq, t);
                return 1;
            }
        }
    }
    for (uint32_t i = 0; i < n_tok; ++i)
        if (!seen[i]) {
            std::printf("shape %u x %u: token %u never visited\n", n_seq, seq_len, i);
            return 1;
        }
    if (o.tile == engram::kBatchTile && o.n_groups > 1 && (2u * (o.tile_blocks / o.n_groups)) % 8u != 0) {
        std::printf("shape %u x %u: group stride of %u blocks is not XCD-aligned\n", n_seq, seq_len,
                    o.tile_blocks / o.n_groups);
        return 1;
    }
    return 0;
}

int main() {
    const uint32_t lens[] = {1, 2, 3, 4, 5, 7, 63, 64, 65, 67, 127, 128, 129, 130, 150, 300, 1000, 4133};
    int shapes = 0;
    for (uint32_t n_seq = 1; n_seq <= 80; ++n_seq)
        for (uint32_t len : lens) {
            if (check(n_seq, len)) return 1;
            ++shapes;
        }
    const uint32_t big[][2] = {{64, 8192}, {57, 150}, {9, 1000}, {33, 260}, {128, 96}, {200, 41}, {1, 131072},
                               {8200, 1}, {4100, 2}, {2731, 3}};
    for (const auto& b : big) {
        if (check(b[0], b[1])) return 1;
        ++shapes;
    }
    std::printf("ok %d\n", shapes);
    return 0;
}
