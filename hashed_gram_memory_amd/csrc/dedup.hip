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
// with 8-bit digits, then group boundaries where the key changes.
//
// Key.  Each window id becomes a small integer m < 2^B and the window packs
// into 4B bits, key = m_0 * 2^(3B) + m_1 * 2^(2B) + m_2 * 2^B + m_3, whose
// numeric order is the lexicographic order of (w_0, w_1, w_2, w_3) as long
// as id -> m is strictly increasing.  Two mappings:
//   * compaction (vocabularies of 2^16 < V <= 2^18 ids): m is the rank of the
//     id among the ids this call uses.  A presence map over the vocabulary,
//     packed into a bitmap with prefix counts, gives the ranks, and B comes
//     from their count D on
//     the device: a 129,280-id vocabulary with 35,000 ids in use needs
//     B = 16, a 64-bit key and 8 passes, instead of B = 17 (68 bits, 9
//     passes).  The host launches the passes the vocabulary bound allows;
//     the ones the device does not need return at once.
//   * the id itself, B = ceil(log2 V) (31 when V is unknown), otherwise.
// An id at or above V (a contract violation) gets m = D, or is masked to B
// bits: its grouping is then unspecified, but nothing is read or written out
// of bounds.
//
// Presence map without clearing: an entry is "present" when it equals this
// call's stamp, a counter kept in the workspace and advanced once per call.
// A stale or uninitialised entry that happens to equal the stamp only adds a
// rank nobody uses: ranks stay strictly increasing over the ids in use.
//
// One kernel per pass: a tile of 4,096 elements ranks its elements by digit
// (wave ballots, stable), publishes its 256 digit counts (two 16-bit counts
// per status word, each with a ready bit), and sums the published counts of
// all earlier tiles, which with the pass's digit totals gives where each of
// its digits starts in the output.  The tile then scatters its elements.
// Tiles take their index from an atomic counter in start order, so every
// tile waited on has started and publishes before it waits on anyone: the
// waits end.  They are also bounded: past a spin limit a wait records an
// error and gives up, any other wait still pending gives up too, a tile
// whose wait gave up writes nothing, and the group count comes out as -1.
// Positions are checked against n before every store, so no outcome writes
// out of bounds.
//
// Kernels of one call, in stream order:
//   init    clear counters, histograms and statuses; mark the ids in use
//   bitmap  (compaction only) presence bitmap of the ids in use, with counts
//   keys    build every key (ranks from the bitmap staged in LDS); B and the
//           pass count; the histogram of the first pass's digit
//   pass p  p = 0 .. passes the bound allows - 1; also counts the next
//           pass's digit (the multiset of keys is the same in every pass);
//           the last one needed writes the token order into the caller's perm
//   groups  flags where the key changes, a look-back scan of their counts,
//           offsets and the group count
#include <stdlib.h>

#include <algorithm>

#include "engram_internal.h"

namespace engram {
namespace {

constexpr uint32_t kRadix = 256;
constexpr int kMaxPasses = 16;            // 4 x 31-bit ids = 124 key bits
constexpr uint32_t kPassThreads = 1024;   // 16 waves
constexpr uint32_t kPassWaves = kPassThreads / 64;
constexpr uint32_t kItems = 4;            // elements per thread and tile
constexpr uint32_t kTile = kPassThreads * kItems;  // 4,096 elements
constexpr uint32_t kWaveSpan = 64 * kItems;        // elements per wave and tile
constexpr uint32_t kKeyThreads = 512;
constexpr uint32_t kKeyItems = 8;         // tokens per thread in the key kernel
constexpr uint32_t kCompactMin = 1u << 16;  // compaction for vocabularies above this ...
constexpr uint32_t kCompactMax = 1u << 18;  // ... up to this
constexpr uint32_t kRankIds = 4096;        // ids per block of the presence bitmap (64 words)
constexpr uint32_t kMaxBitmapBlocks = kCompactMax / kRankIds;  // 64
constexpr uint32_t kSpinLimit = 1u << 18;  // default bound on a wait: about 2^18 x 128 clocks (~14 ms)

// Status words.  A pass tile publishes its 256 digit counts (each < 2^15)
// as 128 words of two 16-bit halves, each half with its top bit set; a
// group tile publishes one word, its count with the top bit set.  Zero means
// "not published yet".
constexpr uint32_t kPairReady = 0x80008000u;
constexpr uint32_t kWordReady = 0x80000000u;
constexpr uint32_t kStatusWords = kRadix / 2;  // words per pass tile
constexpr uint32_t kGroupsOfRows = kPassThreads / kStatusWords;  // earlier tiles read in parallel per thread column
constexpr uint32_t kLookAhead = 16;  // status loads in flight per thread in a pass's look-back

// Control block at the start of the workspace.
struct Ctl {
    // written by init or rank, read by the later kernels of the call
    uint32_t stamp;     // presence stamp of the last call (kept across calls)
    uint32_t npass;     // passes this call needs
    uint32_t has_hi;    // keys wider than 64 bits
    uint32_t bits;      // B
    uint32_t n_ids;     // D (compaction) or 0
    uint32_t spin_limit;  // bound on the polls of one wait (set by init each call)
    uint32_t pad0[58];
    // modified with atomics during the call
    uint32_t tile_ctr[kMaxPasses + 1];  // tile tickets of each pass, and of the group kernel
    uint32_t error;                     // a look-back gave up
    uint32_t pad1[46];
};
static_assert(sizeof(Ctl) == 512, "control block size");
// The group kernel's look-back reads one earlier tile per thread.
static_assert((kMaxDedupTokens + kTile - 1) / kTile <= kPassThreads, "tiles per call");

struct Ids {
    const int32_t* ids;
    const int32_t* history;
    uint32_t seq_len;
};

__device__ __forceinline__ uint32_t load_status(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_status(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan over the 64 lanes with DPP moves: row_shr 1, 2, 4, 8 within
// each row of 16 lanes, then row_bcast 15 and 31 across rows.  Plain VALU
// operations, with no LDS round trip (unlike a shuffle).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Sum over the 64 lanes, returned to every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    return __builtin_amdgcn_readlane(wave_inclusive_scan(x), 63);
}

__host__ __device__ inline uint32_t bits_for(uint64_t count) {  // smallest B >= 1 with 2^B >= count
    uint32_t b = 1;
    while (b < 31 && (uint64_t(1) << b) < count) ++b;
    return b;
}

// Wait until a published status word is ready; bounded.  Returns the word,
// or 0 after recording an error when the wait gives up.
__device__ __forceinline__ uint32_t wait_ready(const uint32_t* p, uint32_t word, uint32_t ready, uint32_t* error,
                                               uint32_t limit) {
    uint32_t spins = 0;
    while ((word & ready) != ready) {
        if (++spins > limit || load_status(error) != 0u) {
            store_status(error, 1u);
            return 0u;
        }
        __builtin_amdgcn_s_sleep(8);
        word = load_status(p);
    }
    return word;
}

// Lanes of this wave whose digit equals this lane's (valid lanes only).
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

__device__ __forceinline__ uint32_t key_digit(uint64_t lo, uint64_t hi, int pass) {
    return static_cast<uint32_t>((pass < 8 ? lo >> (8 * pass) : hi >> (8 * (pass - 8)))) & 0xFFu;
}

// Add a wave's digits (digit `pass` of each valid lane's key) to the wave's
// LDS histogram.  The lanes that share the first valid lane's digit are
// added with one atomic: ids are skewed, so one digit is often most of the
// wave (the high byte of a rank is mostly 0), and lane-by-lane atomics on one
// LDS word serialise.
__device__ __forceinline__ void count_digits(uint32_t* hist, uint64_t lo, uint64_t hi, int pass, bool valid,
                                             uint32_t lane) {
    const uint64_t live = __ballot(valid);
    if (live == 0) return;
    const uint32_t d = key_digit(lo, hi, pass);
    const uint32_t leader = static_cast<uint32_t>(__ffsll(static_cast<long long>(live))) - 1u;
    const uint32_t d0 = __builtin_amdgcn_readlane(d, leader);
    const uint64_t same = __ballot(valid && d == d0);
    if (lane == leader) atomicAdd(&hist[d0], static_cast<uint32_t>(__popcll(same)));
    if (valid && d != d0) atomicAdd(&hist[d], 1u);
}

struct Workspace {
    Ctl* ctl;
    uint32_t* hist;    // [kMaxPasses][256] digit totals
    uint32_t* status;  // [passes][tiles][128] digit counts of each pass tile, then [tiles] group counts
    uint32_t* flags;   // [V] presence stamps (compaction)
    uint64_t* bitmap;  // [64 * blocks] ids in use, one bit each (compaction)
    uint32_t* wpre;    // [64 * blocks] ids in use below each bitmap word, within its block of 4,096 ids
    uint32_t* bcount;  // [blocks] ids in use per block of 4,096 ids
    uint64_t* lo[2];   // [n] key bits 0..63
    uint64_t* hi[2];   // [n] key bits 64..127 (when the bound allows them)
    int32_t* val[2];   // [n] token indices between passes
};

// How a call keys its windows, from host-side facts alone.
struct KeyPlan {
    bool compact;
    uint32_t bits;     // B for id keys; the bound on B with compaction
    int max_passes;    // passes launched
    bool hi_possible;  // keys may exceed 64 bits
};

KeyPlan key_plan(uint32_t vocab) {
    KeyPlan k;
    k.compact = vocab > kCompactMin && vocab <= kCompactMax;
    if (k.compact) {
        // D <= V (a stale presence entry can count an id the call does not use); one more rank marks ids out
        // of range
        k.bits = bits_for(uint64_t(vocab) + 1u);
    } else {
        k.bits = vocab == 0 ? 31u : bits_for(vocab);
    }
    k.max_passes = static_cast<int>((4 * k.bits + 7) / 8);
    k.hi_possible = 4 * k.bits > 64;
    return k;
}

size_t align_up(size_t x) { return (x + 255u) & ~size_t(255u); }

size_t status_words(const KeyPlan& k, uint32_t tiles) { return (size_t(k.max_passes) * kStatusWords + 1) * tiles; }

size_t layout(uint32_t n, uint32_t vocab, char* base, Workspace* w) {
    const KeyPlan k = key_plan(vocab);
    const uint32_t tiles = (n + kTile - 1u) / kTile;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += align_up(bytes);
        return p;
    };
    Workspace t{};
    t.ctl = reinterpret_cast<Ctl*>(take(sizeof(Ctl)));
    t.hist = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * kMaxPasses * kRadix));
    t.status = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * status_words(k, tiles)));
    if (k.compact) {
        const uint32_t blocks = (vocab + kRankIds - 1u) / kRankIds;
        t.flags = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * vocab));
        t.bitmap = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * 64u * blocks));
        t.wpre = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 64u * blocks));
        t.bcount = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * blocks));
    }
    for (int i = 0; i < 2; ++i) t.lo[i] = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * n));
    if (k.hi_possible)
        for (int i = 0; i < 2; ++i) t.hi[i] = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * n));
    for (int i = 0; i < 2; ++i) t.val[i] = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * n));
    if (w) *w = t;
    return off;
}

// ---------------------------------------------------------------------------
// init: clear the per-call state; mark the ids in use (compaction)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void init_kernel(Ids s, uint32_t n, uint32_t vocab, uint32_t compact,
                                                   uint32_t zero_words, Workspace w, uint32_t id_bits,
                                                   uint32_t id_passes, uint32_t id_hi, uint32_t spin_limit) {
    const uint32_t gtid = blockIdx.x * 256u + threadIdx.x;
    const uint32_t stride = gridDim.x * 256u;
    if (gtid <= kMaxPasses) w.ctl->tile_ctr[gtid] = 0u;
    if (gtid == 0) {
        w.ctl->error = 0u;
        w.ctl->spin_limit = spin_limit;
    }
    for (uint32_t i = gtid; i < zero_words; i += stride) w.hist[i] = 0u;  // histograms and statuses
    if (gtid == 0 && !compact) {
        w.ctl->bits = id_bits;
        w.ctl->npass = id_passes;
        w.ctl->has_hi = id_hi;
        w.ctl->n_ids = 0;
    }
    if (!compact) return;
    const uint32_t stamp = w.ctl->stamp + 1u;
    for (uint32_t tok = gtid; tok < n; tok += stride) {
        const uint32_t id = static_cast<uint32_t>(s.ids[tok]);
        if (id < vocab) w.flags[id] = stamp;
        const uint32_t seq = tok / s.seq_len;
        if (tok == seq * s.seq_len) {  // first token of a sequence: the ids before it
            for (uint32_t k = 0; k < 3; ++k) {
                const uint32_t h = s.history ? static_cast<uint32_t>(s.history[seq * 3u + k]) : 0u;
                if (h < vocab) w.flags[h] = stamp;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bitmap (compaction): block b turns the presence stamps of ids
// [4096 b, 4096 (b+1)) into 64 bitmap words, the count of ids in use below
// each word within the block, and the block's count
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bitmap_kernel(uint32_t vocab, Workspace w) {
    __shared__ uint32_t wcnt[64];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t stamp = w.ctl->stamp + 1u;
    const uint32_t word0 = blockIdx.x * 64u + wave * 16u;  // this wave's 16 words
    // all 16 loads issued before the first is used (ids past the vocabulary
    // read its last entry and are masked below), so the wave waits once
    uint32_t f[16];
#pragma unroll
    for (uint32_t c = 0; c < 16; ++c) f[c] = w.flags[min(((word0 + c) << 6) + lane, vocab - 1u)];
    uint64_t word[16];
#pragma unroll
    for (uint32_t c = 0; c < 16; ++c) word[c] = __ballot(((word0 + c) << 6) + lane < vocab && f[c] == stamp);
    uint64_t mine = 0;
#pragma unroll
    for (uint32_t c = 0; c < 16; ++c)
        if (lane == c) mine = word[c];
    if (lane < 16) {
        w.bitmap[word0 + lane] = mine;
        wcnt[wave * 16u + lane] = static_cast<uint32_t>(__popcll(mine));
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t pre = 0;
        for (uint32_t c = 0; c < threadIdx.x; ++c) pre += wcnt[c];
        w.wpre[blockIdx.x * 64u + threadIdx.x] = pre;
        if (threadIdx.x == 63) w.bcount[blockIdx.x] = pre + wcnt[63];
    }
}

// ---------------------------------------------------------------------------
// keys: pack every window; the histogram of the first pass's digit.
// A block loads its 4,096 ids (and the 3 before them) and, with compaction,
// stages the whole presence bitmap with its prefix counts in LDS; it ranks
// each id once into LDS, so a key costs no dependent global loads:
// rank(id) = ids in use in earlier 4,096-id blocks + ids in use earlier in
// the block's words + set bits below id in its word.  With compaction the
// first block also records B, the pass count and the stamp for the rest of
// the call.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kKeyThreads) void keys_kernel(Ids s, uint32_t n, uint32_t vocab, uint32_t compact,
                                                           Workspace w) {
    constexpr uint32_t kKeyTile = kKeyThreads * kKeyItems;
    constexpr uint32_t kStage = (kKeyTile + 3u + kKeyThreads - 1u) / kKeyThreads;  // staged ids per thread
    constexpr uint32_t kWordsPerThread = 64u * kMaxBitmapBlocks / kKeyThreads;
    constexpr uint32_t kKeyWaves = kKeyThreads / 64;
    __shared__ uint32_t rank_s[kKeyTile + 3];  // m of the block's ids and the 3 before them
    __shared__ uint64_t bits_s[64 * kMaxBitmapBlocks];
    __shared__ uint32_t wpre_s[64 * kMaxBitmapBlocks];
    __shared__ uint32_t bpre_s[kMaxBitmapBlocks];
    __shared__ uint32_t h[kKeyWaves][kRadix];
    __shared__ uint32_t s_d;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t begin = blockIdx.x * kKeyTile;
    // Every global load of the staging -- the block's ids and the 3 before
    // them, and with compaction the bitmap, its word prefixes and the block
    // counts -- is issued before the first LDS store, so the block waits for
    // memory once.
    const uint32_t blocks = compact ? (vocab + kRankIds - 1u) / kRankIds : 0u;
    const uint32_t words = 64u * blocks;
    int32_t v[kStage];
#pragma unroll
    for (uint32_t c = 0; c < kStage; ++c) {
        const uint32_t i = c * kKeyThreads + threadIdx.x;
        const int64_t tok = int64_t(begin) + int64_t(i) - 3;
        v[c] = (i < kKeyTile + 3u && tok >= 0 && tok < int64_t(n)) ? s.ids[tok] : 0;
    }
    uint64_t bw[kWordsPerThread];
    uint32_t pw[kWordsPerThread];
#pragma unroll
    for (uint32_t c = 0; c < kWordsPerThread; ++c) {
        const uint32_t i = c * kKeyThreads + threadIdx.x;
        bw[c] = i < words ? w.bitmap[i] : 0u;
        pw[c] = i < words ? w.wpre[i] : 0u;
    }
    const uint32_t bc = threadIdx.x < blocks ? w.bcount[threadIdx.x] : 0u;
    for (uint32_t i = threadIdx.x; i < kKeyWaves * kRadix; i += kKeyThreads) (&h[0][0])[i] = 0u;
    uint32_t b, has_hi, n_ids = 0;
    if (compact) {
#pragma unroll
        for (uint32_t c = 0; c < kWordsPerThread; ++c) {
            const uint32_t i = c * kKeyThreads + threadIdx.x;
            if (i < words) {
                bits_s[i] = bw[c];
                wpre_s[i] = pw[c];
            }
        }
        if (threadIdx.x < kMaxBitmapBlocks) bpre_s[threadIdx.x] = bc;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t run = 0;
            for (uint32_t i = 0; i < blocks; ++i) {
                const uint32_t c = bpre_s[i];
                bpre_s[i] = run;
                run += c;
            }
            s_d = run;
        }
        __syncthreads();
        n_ids = s_d;
        b = bits_for(uint64_t(n_ids) + 1u);
        has_hi = 4u * b > 64u ? 1u : 0u;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            w.ctl->n_ids = n_ids;
            w.ctl->bits = b;
            w.ctl->npass = (4u * b + 7u) / 8u;
            w.ctl->has_hi = has_hi;
            w.ctl->stamp = w.ctl->stamp + 1u;  // the presence stamps of this call are consumed
        }
    } else {
        b = w.ctl->bits;
        has_hi = w.ctl->has_hi;
        __syncthreads();
    }
    // m of an id: its rank among the ids in use (compaction), else its low B bits
    const uint32_t mask = (1u << b) - 1u;
    auto rank_of = [&](uint32_t id) -> uint32_t {
        if (!compact) return id & mask;
        if (id >= vocab) return n_ids;  // ids out of range share the rank after the last
        const uint32_t wd = id >> 6;
        return bpre_s[id >> 12] + wpre_s[wd] +
               static_cast<uint32_t>(__popcll(bits_s[wd] & ((uint64_t(1) << (id & 63u)) - 1u)));
    };
    // Each staged id is ranked once (a window reads each of its ids' ranks
    // from LDS; ranking per window would look every id up four times).
#pragma unroll
    for (uint32_t c = 0; c < kStage; ++c) {
        const uint32_t i = c * kKeyThreads + threadIdx.x;
        if (i < kKeyTile + 3u) rank_s[i] = rank_of(static_cast<uint32_t>(v[c]));
    }
    __syncthreads();
    // All keys of the thread first, then their stores: a store between two
    // keys would make every later wait for memory (a history id) wait for it.
    uint64_t klo[kKeyItems], khi[kKeyItems];
#pragma unroll
    for (uint32_t j = 0; j < kKeyItems; ++j) {
        const uint32_t tok = begin + j * kKeyThreads + threadIdx.x;
        const bool valid = tok < n;
        uint64_t lo = 0, hi = 0;
        if (valid) {
            const uint32_t seq = tok / s.seq_len;
            const int32_t t = static_cast<int32_t>(tok - seq * s.seq_len);
#pragma unroll
            for (int k = 0; k < 4; ++k) {  // w_0 most significant
                uint32_t m;
                if (t - k >= 0)
                    m = rank_s[tok - begin + 3u - static_cast<uint32_t>(k)];
                else
                    m = rank_of(s.history ? static_cast<uint32_t>(s.history[seq * 3u + static_cast<uint32_t>(3 + t - k)]) : 0u);
                hi = (hi << b) | (lo >> (64u - b));
                lo = (lo << b) | m;
            }
            // histogram of the first pass's digit (each later pass counts its successor's)
            atomicAdd(&h[wave][static_cast<uint32_t>(lo) & 0xFFu], 1u);
        }
        klo[j] = lo;
        khi[j] = hi;
    }
#pragma unroll
    for (uint32_t j = 0; j < kKeyItems; ++j) {
        const uint32_t tok = begin + j * kKeyThreads + threadIdx.x;
        if (tok < n) {
            w.lo[0][tok] = klo[j];
            if (has_hi) w.hi[0][tok] = khi[j];
        }
    }
    __syncthreads();
    if (threadIdx.x < kRadix) {
        uint32_t c = 0;
#pragma unroll
        for (uint32_t k = 0; k < kKeyWaves; ++k) c += h[k][threadIdx.x];
        if (c) atomicAdd(&w.hist[threadIdx.x], c);
    }
}

// ---------------------------------------------------------------------------
// one pass of the radix sort: rank, look back, scatter
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPassThreads) void pass_kernel(uint32_t n, int pass, uint32_t tiles, Workspace w,
                                                            int32_t* __restrict__ perm) {
    Ctl* ctl = w.ctl;
    __shared__ uint32_t s_tile, s_failed;
    __shared__ uint32_t wave_hist[kPassWaves][kRadix];  // counts per wave, then exclusive prefixes across waves
    __shared__ uint32_t next_hist[kPassWaves][kRadix];  // this tile's counts of the next pass's digit, per wave
    __shared__ uint32_t tile_cnt[kRadix];
    __shared__ uint32_t tile_start[kRadix];  // where each digit's run starts within the tile's output order
    __shared__ uint32_t base[kRadix];  // where the tile's run of each digit starts in the output
    __shared__ uint32_t wsum[kRadix / 64], tsum[kRadix / 64];
    __shared__ uint32_t part[2][kGroupsOfRows][kStatusWords];  // earlier tiles' counts, per row group
    // the tile's elements in output order, so that each digit's run is written by consecutive threads
    __shared__ uint64_t stage_lo[kTile];
    __shared__ uint64_t stage_hi[kTile];
    __shared__ int32_t stage_val[kTile];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t lt = (uint64_t(1) << lane) - 1u;
    // The digit totals, the pass count and the ticket are read together (the
    // loads are issued before the atomic, whose result is waited for first);
    // a pass the call does not need returns after them (its ticket counter
    // is reset by the next call).
    uint32_t total = 0;  // this pass's total count of digit threadIdx.x (threads 0..255)
    if (threadIdx.x < kRadix) total = w.hist[pass * kRadix + threadIdx.x];
    const uint32_t npass = ctl->npass;
    const bool has_hi = ctl->has_hi != 0u;
    const uint32_t limit = ctl->spin_limit;
    uint32_t ticket = 0;
    if (threadIdx.x == 0) ticket = atomicAdd(&ctl->tile_ctr[pass], 1u);
    for (uint32_t i = threadIdx.x; i < kPassWaves * kRadix; i += kPassThreads) {
        (&wave_hist[0][0])[i] = 0u;
        (&next_hist[0][0])[i] = 0u;
    }
    if (threadIdx.x == 0) {
        s_tile = ticket;
        s_failed = 0u;
    }
    __syncthreads();
    if (static_cast<uint32_t>(pass) >= npass) return;  // this call's keys need fewer passes
    const bool last = static_cast<uint32_t>(pass) + 1u == npass;
    const uint32_t tile = s_tile;
    const int src = pass & 1, dst = src ^ 1;
    const uint64_t* __restrict__ lo_in = w.lo[src];
    const uint64_t* __restrict__ hi_in = w.hi[src];
    const int32_t* __restrict__ val_in = w.val[src];
    uint64_t* __restrict__ lo_out = w.lo[dst];
    uint64_t* __restrict__ hi_out = w.hi[dst];
    int32_t* __restrict__ val_out = last ? perm : w.val[dst];

    // this wave's 1,024 elements, 64 consecutive per step (steps in element order: the ranking is stable)
    const uint32_t first = tile * kTile + wave * kWaveSpan;
    uint64_t lo[kItems], hi[kItems];
    int32_t v[kItems];
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        const uint32_t i = first + j * 64u + lane;
        const bool valid = i < n;
        lo[j] = valid ? lo_in[i] : 0u;
        hi[j] = (valid && has_hi) ? hi_in[i] : 0u;
        v[j] = valid ? (pass == 0 ? static_cast<int32_t>(i) : val_in[i]) : 0;
    }
    uint32_t off[kItems];
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        const bool valid = first + j * 64u + lane < n;
        const uint32_t d = key_digit(lo[j], hi[j], pass);
        const uint64_t peers = match_digit(d, valid);
        const uint32_t before = wave_hist[wave][d];
        off[j] = before + static_cast<uint32_t>(__popcll(peers & lt));
        if (valid && (peers & lt) == 0) wave_hist[wave][d] = before + static_cast<uint32_t>(__popcll(peers));
    }
    __syncthreads();

    if (threadIdx.x < kRadix) {
        const uint32_t dd = threadIdx.x;
        uint32_t run = 0;
#pragma unroll
        for (uint32_t k = 0; k < kPassWaves; ++k) {
            const uint32_t c = wave_hist[k][dd];
            wave_hist[k][dd] = run;
            run += c;
        }
        tile_cnt[dd] = run;
        // exclusive scans of the pass's digit totals and of this tile's digit counts (threads 0..255 are waves
        // 0..3)
        const uint32_t x = wave_inclusive_scan(total);
        const uint32_t y = wave_inclusive_scan(run);
        if (lane == 63) {
            wsum[wave] = x;
            tsum[wave] = y;
        }
        base[dd] = x - total;
        tile_start[dd] = y - run;
    }
    __syncthreads();
    // publish this tile's counts: word i holds digits 2i (low half) and 2i + 1 (high half)
    const uint32_t* counts = w.status + size_t(pass) * tiles * kStatusWords;  // [tiles][128]
    if (threadIdx.x < kStatusWords) {
        const uint32_t i = threadIdx.x;
        store_status(w.status + (size_t(pass) * tiles + tile) * kStatusWords + i,
                     kPairReady | tile_cnt[2 * i] | (tile_cnt[2 * i + 1] << 16));
    }
    if (threadIdx.x < kRadix) {
        uint32_t pre = 0, tpre = 0;
        for (uint32_t k = 0; k < wave; ++k) {
            pre += wsum[k];
            tpre += tsum[k];
        }
        base[threadIdx.x] += pre;
        tile_start[threadIdx.x] += tpre;
    }
    {  // counts in the earlier tiles: thread (g, i) sums word i of tiles g, g + 8, g + 16, ... below this one,
       // kLookAhead loads in flight (one round for up to 8 x kLookAhead earlier tiles)
        const uint32_t g = threadIdx.x / kStatusWords, i = threadIdx.x % kStatusWords;
        uint32_t sum_lo = 0, sum_hi = 0;
        int failed = 0;  // a wait of this thread gave up
        bool counted = last;  // this thread's items are in the next digit's counts (none needed after the last pass)
        for (uint32_t t0 = g; t0 < tile; t0 += kLookAhead * kGroupsOfRows) {
            uint32_t word[kLookAhead];
#pragma unroll
            for (uint32_t j = 0; j < kLookAhead; ++j) {
                const uint32_t t = t0 + j * kGroupsOfRows;
                word[j] = t < tile ? load_status(counts + size_t(t) * kStatusWords + i) : kPairReady;
            }
            if (!counted) {  // while the first loads are in flight: this tile's counts of the next digit
#pragma unroll
                for (uint32_t j = 0; j < kItems; ++j)
                    count_digits(next_hist[wave], lo[j], hi[j], pass + 1, first + j * 64u + lane < n, lane);
                counted = true;
            }
#pragma unroll
            for (uint32_t j = 0; j < kLookAhead; ++j) {
                const uint32_t t = t0 + j * kGroupsOfRows;
                if (t < tile) {
                    const uint32_t c = wait_ready(counts + size_t(t) * kStatusWords + i, word[j], kPairReady, &ctl->error, limit);
                    failed |= c == 0u;
                    sum_lo += c & 0x7FFFu;
                    sum_hi += (c >> 16) & 0x7FFFu;
                }
            }
        }
        if (!counted) {  // no earlier tile for this thread to read
#pragma unroll
            for (uint32_t j = 0; j < kItems; ++j)
                count_digits(next_hist[wave], lo[j], hi[j], pass + 1, first + j * 64u + lane < n, lane);
        }
        part[0][g][i] = sum_lo;
        part[1][g][i] = sum_hi;
        if (failed) s_failed = 1u;
    }
    __syncthreads();
    if (threadIdx.x < kRadix) {
        const uint32_t dd = threadIdx.x;
        uint32_t e = 0;
#pragma unroll
        for (uint32_t g = 0; g < kGroupsOfRows; ++g) e += part[dd & 1u][g][dd >> 1];
        base[dd] += e;
        if (!last) {
            uint32_t c = 0;
#pragma unroll
            for (uint32_t k = 0; k < kPassWaves; ++k) c += next_hist[k][dd];
            if (c) atomicAdd(&w.hist[(pass + 1) * kRadix + dd], c);
        }
    }
    __syncthreads();
    // A wait of this tile gave up: its positions are unknown, so it writes
    // nothing.  (The error flag it set makes the call report n_unique = -1.
    // Other tiles still scatter to positions below n.)
    if (s_failed) return;

    // Stage the tile in output order: an element's place is where its digit's
    // run starts in the tile plus its stable rank among the tile's elements of
    // that digit.  Then thread i writes staged element i to the start of its
    // digit's run in the output plus its place in the run, so each run is
    // written by consecutive threads.
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        const uint32_t i = first + j * 64u + lane;
        if (i < n) {
            const uint32_t d = key_digit(lo[j], hi[j], pass);
            const uint32_t at = tile_start[d] + wave_hist[wave][d] + off[j];
            if (at < kTile) {
                stage_lo[at] = lo[j];
                if (has_hi) stage_hi[at] = hi[j];
                stage_val[at] = v[j];
            }
        }
    }
    __syncthreads();
    const uint32_t in_tile = min(kTile, n - tile * kTile);
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        const uint32_t i = j * kPassThreads + threadIdx.x;
        if (i < in_tile) {
            const uint64_t klo = stage_lo[i];
            const uint64_t khi = has_hi ? stage_hi[i] : 0u;
            const uint32_t d = key_digit(klo, khi, pass);
            const uint32_t pos = base[d] + (i - tile_start[d]);
            if (pos < n) {
                lo_out[pos] = klo;
                if (has_hi) hi_out[pos] = khi;
                val_out[pos] = stage_val[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// groups: boundaries where the sorted key changes -> offsets, n_unique
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPassThreads) void groups_kernel(uint32_t n, uint32_t tiles, uint32_t max_passes,
                                                              Workspace w, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ n_unique) {
    Ctl* ctl = w.ctl;
    __shared__ uint32_t s_tile, s_failed;
    __shared__ uint32_t wcount[kPassWaves];
    __shared__ uint32_t wexcl[kPassWaves];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t lt = (uint64_t(1) << lane) - 1u;
    // the control words are read before the ticket is taken, so both reads overlap
    const uint32_t q = ctl->npass & 1u;  // buffer the last pass wrote
    const uint32_t limit = ctl->spin_limit;
    const bool has_hi = ctl->has_hi != 0u;
    uint32_t ticket = 0;
    if (threadIdx.x == 0) ticket = atomicAdd(&ctl->tile_ctr[kMaxPasses], 1u);
    if (threadIdx.x == 0) {
        s_tile = ticket;
        s_failed = 0u;
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t* __restrict__ lo = w.lo[q];
    const uint64_t* __restrict__ hi = w.hi[q];
    uint32_t* st = w.status + size_t(max_passes) * kStatusWords * tiles;  // [tiles] group counts

    const uint32_t first = tile * kTile + wave * kWaveSpan;
    // Every key and its predecessor are loaded before the first comparison
    // (indices clamped to [0, n); n >= 1 here), so the wave waits once.
    // Without high key words the high loads read the low words again (cache
    // hits) and their comparison is masked: no load sits behind a branch.
    const uint64_t* __restrict__ hsrc = has_hi ? hi : lo;
    uint64_t cur[kItems], prev[kItems], cur_hi[kItems], prev_hi[kItems];
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        const uint32_t i = min(first + j * 64u + lane, n - 1u);
        const uint32_t ip = i == 0 ? 0u : i - 1u;
        cur[j] = lo[i];
        prev[j] = lo[ip];
        cur_hi[j] = hsrc[i];
        prev_hi[j] = hsrc[ip];
    }
    uint64_t m[kItems];
    uint32_t cnt = 0;
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        const uint32_t i = first + j * 64u + lane;
        const bool f = i < n && (i == 0 || cur[j] != prev[j] || (has_hi && cur_hi[j] != prev_hi[j]));
        m[j] = __ballot(f);
        cnt += static_cast<uint32_t>(__popcll(m[j]));
    }
    if (lane == 0) wcount[wave] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t total = 0;
        for (uint32_t k = 0; k < kPassWaves; ++k) total += wcount[k];
        store_status(st + tile, kWordReady | total);
    }
    {  // groups in the earlier tiles: wave k sums tiles 64k .. 64k + 63 below this one, all waves at once
        const uint32_t t = wave * 64u + lane;
        uint32_t c = 0;
        if (t < tile) {
            c = wait_ready(st + t, load_status(st + t), kWordReady, &ctl->error, limit);
            if (c == 0u) s_failed = 1u;
        }
        const uint32_t sum = wave_sum(c & ~kWordReady);
        if (lane == 0) wexcl[wave] = sum;
    }
    __syncthreads();
    // A wait of this tile gave up: its positions are unknown, so it writes no
    // offsets.  The tile that writes n_unique also reports a wait that gave
    // up anywhere in the call, in the sort or here, as -1.
    const bool last_tile = tile == tiles - 1u;
    if (s_failed || (last_tile && load_status(&ctl->error) != 0u)) {
        if (last_tile && threadIdx.x == 0) *n_unique = -1;
        return;
    }
    uint32_t excl = 0, total = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPassWaves; ++k) {
        excl += wexcl[k];
        total += wcount[k];
    }
    uint32_t pos = excl;
    for (uint32_t k = 0; k < wave; ++k) pos += wcount[k];
#pragma unroll
    for (uint32_t j = 0; j < kItems; ++j) {
        if ((m[j] >> lane) & 1u) {
            const uint32_t at = pos + static_cast<uint32_t>(__popcll(m[j] & lt));
            if (at < n) offsets[at] = static_cast<int32_t>(first + j * 64u + lane);
        }
        pos += static_cast<uint32_t>(__popcll(m[j]));
    }
    if (last_tile && threadIdx.x == 0) {
        total += excl;
        if (total <= n) offsets[total] = static_cast<int32_t>(n);
        *n_unique = static_cast<int32_t>(total);
    }
}

__global__ void empty_kernel(int32_t* __restrict__ offsets, int32_t* __restrict__ n_unique) {
    offsets[0] = 0;
    *n_unique = 0;
}

}  // namespace

// Bound on the polls of one device-side wait: ENGRAM_DEDUP_SPIN_LIMIT from the environment when set (a test forces
// the give-up path with a small value), else kSpinLimit.
static uint32_t dedup_spin_limit() {
    const char* v = getenv("ENGRAM_DEDUP_SPIN_LIMIT");
    if (!v || !*v) return kSpinLimit;
    char* end = nullptr;
    const unsigned long x = strtoul(v, &end, 10);
    return (end && *end == '\0' && x <= 0xFFFFFFFFul) ? static_cast<uint32_t>(x) : kSpinLimit;
}

size_t dedup_workspace_bytes(uint32_t n, uint32_t vocab_size) {
    return n == 0 ? 0 : layout(n, vocab_size, nullptr, nullptr);
}

hipError_t launch_dedup(const int32_t* ids, const int32_t* history, uint32_t n, uint32_t seq_len, uint32_t vocab_size,
                        int32_t* perm, int32_t* offsets, int32_t* n_unique, void* ws, hipStream_t stream) {
    if (n == 0) {
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(1), 0, stream, offsets, n_unique);
        return hipGetLastError();
    }
    const Ids s{ids, history, seq_len};
    const KeyPlan k = key_plan(vocab_size);
    Workspace w;
    layout(n, vocab_size, static_cast<char*>(ws), &w);
    const uint32_t tiles = (n + kTile - 1u) / kTile;
    const size_t zero_bytes =
        reinterpret_cast<char*>(w.status + status_words(k, tiles)) - reinterpret_cast<char*>(w.hist);
    const uint32_t zero_words = static_cast<uint32_t>(zero_bytes / sizeof(uint32_t));
    const uint32_t init_blocks = std::min<uint32_t>(2048u, (std::max<uint32_t>(n, zero_words) + 255u) / 256u);
    hipLaunchKernelGGL(init_kernel, dim3(init_blocks), dim3(256), 0, stream, s, n, vocab_size, uint32_t(k.compact),
                       zero_words, w, k.bits, uint32_t(k.max_passes), uint32_t(k.hi_possible), dedup_spin_limit());
    if (k.compact)
        hipLaunchKernelGGL(bitmap_kernel, dim3((vocab_size + kRankIds - 1u) / kRankIds), dim3(256), 0, stream,
                           vocab_size, w);
    hipLaunchKernelGGL(keys_kernel, dim3((n + kKeyThreads * kKeyItems - 1u) / (kKeyThreads * kKeyItems)),
                       dim3(kKeyThreads), 0, stream, s, n, vocab_size, uint32_t(k.compact), w);
    for (int pass = 0; pass < k.max_passes; ++pass)
        hipLaunchKernelGGL(pass_kernel, dim3(tiles), dim3(kPassThreads), 0, stream, n, pass, tiles, w, perm);
    hipLaunchKernelGGL(groups_kernel, dim3(tiles), dim3(kPassThreads), 0, stream, n, tiles, uint32_t(k.max_passes), w,
                       offsets, n_unique);
    return hipGetLastError();
}

}  // namespace engram
