// Host side of the C ABI: argument validation, plans, launches.
//
// Every entry point validates all of its arguments before it launches
// anything, so an error return leaves the outputs untouched.  Nothing here
// synchronises or allocates device memory.
#include <new>
#include <string.h>

#include "batch_order.h"
#include "engram_internal.h"

using namespace engram;

namespace {

// splitmix64 (Steele, Lea and Flood 2014): state advances by the golden
// gamma, output is the 30/27/31 xor-shift-multiply finaliser of the state.
struct SplitMix64 {
    uint64_t state;
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

bool valid_plan(engram_plan_t p) { return p != nullptr; }

int check_tokens(int64_t n_seq, int64_t seq_len, int64_t* n_tok) {
    if (n_seq < 0 || seq_len < 0) return ENGRAM_EINVAL;
    if (n_seq != 0 && seq_len > kMaxTokens / n_seq) return ENGRAM_ERANGE;
    *n_tok = n_seq * seq_len;
    return ENGRAM_OK;
}

}  // namespace

extern "C" {

int engram_plan_desc_init(engram_plan_desc* d) {
    if (!d) return ENGRAM_EINVAL;
    memset(d, 0, sizeof(*d));
    d->n_modules = ENGRAM_N_MODULES;
    d->min_order = ENGRAM_MIN_ORDER;
    d->max_order = ENGRAM_MAX_ORDER;
    d->n_heads = ENGRAM_N_HEADS;
    d->row_bytes = ENGRAM_ROW_BYTES;
    d->hash_seed = ENGRAM_DEFAULT_HASH_SEED;
    return ENGRAM_OK;
}

int engram_plan(const engram_plan_desc* d, engram_plan_t* out) {
    if (!d || !out) return ENGRAM_EINVAL;
    if (d->n_modules != ENGRAM_N_MODULES || d->min_order != ENGRAM_MIN_ORDER ||
        d->max_order != ENGRAM_MAX_ORDER || d->n_heads != ENGRAM_N_HEADS ||
        d->row_bytes != ENGRAM_ROW_BYTES)
        return ENGRAM_EUNSUPPORTED;
    if (!d->rows || !d->tables || !d->scales) return ENGRAM_EINVAL;
    if (d->scale_format != ENGRAM_SCALE_F32_ROW && d->scale_format != ENGRAM_SCALE_E8M0_BLOCK32)
        return ENGRAM_EUNSUPPORTED;
    if (d->reserved1 != 0) return ENGRAM_EINVAL;
    if (d->vocab_map && (d->vocab_size == 0 || !aligned(d->vocab_map, 4))) return ENGRAM_EINVAL;
    const uintptr_t scale_align = d->scale_format == ENGRAM_SCALE_F32_ROW ? 4 : 8;
    for (int s = 0; s < kSub; ++s) {
        const uint64_t r = d->rows[s];
        if (r == 0 || r > (uint64_t(1) << 32)) return ENGRAM_ERANGE;
        if (!d->tables[s] || !d->scales[s]) return ENGRAM_EINVAL;
        if (!aligned(d->tables[s], 16) || !aligned(d->scales[s], scale_align)) return ENGRAM_EINVAL;
    }
    engram_plan_s* p = new (std::nothrow) engram_plan_s;
    if (!p) return ENGRAM_EINVAL;
    memset(p, 0, sizeof(*p));
    p->hash_seed = d->hash_seed;
    p->vocab_size = d->vocab_size;
    SplitMix64 g{d->hash_seed};
    for (int i = 0; i < kMult; ++i) p->hash.mult[i] = g.next() | 1u;
    for (int s = 0; s < kSub; ++s) {
        p->hash.rows[s] = d->rows[s];
        p->hash.magic[s] = ~uint64_t(0) / d->rows[s];
        p->gather.tab[s] = d->tables[s];
        p->gather.sc[s] = d->scales[s];
    }
    p->gather.scale_format = d->scale_format;
    p->hash.vocab_map = d->vocab_map;
    *out = p;
    return ENGRAM_OK;
}

int engram_plan_destroy(engram_plan_t p) {
    delete p;
    return ENGRAM_OK;
}

int engram_plan_multipliers(engram_plan_t p, uint64_t* out) {
    if (!valid_plan(p) || !out) return ENGRAM_EINVAL;
    memcpy(out, p->hash.mult, sizeof(p->hash.mult));
    return ENGRAM_OK;
}

int engram_hash(engram_plan_t p, const int32_t* ids, const int32_t* history, int64_t n_seq,
                int64_t seq_len, uint32_t* addr, void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    int64_t n_tok = 0;
    int st = check_tokens(n_seq, seq_len, &n_tok);
    if (st != ENGRAM_OK) return st;
    if (n_tok == 0) return ENGRAM_OK;
    if (!ids || !addr || !aligned(ids, 4) || !aligned(addr, 16)) return ENGRAM_EINVAL;
    if (history && !aligned(history, 4)) return ENGRAM_EINVAL;
    hipError_t e = launch_hash(p->hash, ids, history, uint32_t(n_tok), uint32_t(seq_len), addr,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_gather_reduce(engram_plan_t p, const uint32_t* addr, int64_t n_tok, const int32_t* perm,
                         const int32_t* offsets, const int32_t* n_unique, float* out, void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    if (n_tok < 0 || n_tok > kMaxTokens) return ENGRAM_ERANGE;
    const int n_dedup = (perm != nullptr) + (offsets != nullptr) + (n_unique != nullptr);
    if (n_dedup != 0 && n_dedup != 3) return ENGRAM_EINVAL;
    if (n_tok == 0) return ENGRAM_OK;
    if (!addr || !out || !aligned(addr, 16) || !aligned(out, 16)) return ENGRAM_EINVAL;
    if (n_dedup == 3 && (!aligned(perm, 4) || !aligned(offsets, 4) || !aligned(n_unique, 4)))
        return ENGRAM_EINVAL;
    hipError_t e = launch_gather_reduce(p->gather, addr, uint32_t(n_tok), perm, offsets, n_unique, out,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_gather_reduce_batched(engram_plan_t p, const uint32_t* addr, int64_t n_seq, int64_t seq_len, float* out,
                                 void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    int64_t n_tok = 0;
    int st = check_tokens(n_seq, seq_len, &n_tok);
    if (st != ENGRAM_OK) return st;
    if (n_tok == 0) return ENGRAM_OK;
    if (!addr || !out || !aligned(addr, 16) || !aligned(out, 16)) return ENGRAM_EINVAL;
    hipError_t e = launch_gather_batched(p->gather, addr, uint32_t(n_tok), uint32_t(seq_len), out,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_lookup(engram_plan_t p, const int32_t* ids, const int32_t* history, int64_t n_seq, int64_t seq_len,
                  float* out, void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    int64_t n_tok = 0;
    int st = check_tokens(n_seq, seq_len, &n_tok);
    if (st != ENGRAM_OK) return st;
    if (n_tok == 0) return ENGRAM_OK;
    if (!ids || !out || !aligned(ids, 4) || !aligned(out, 16)) return ENGRAM_EINVAL;
    if (history && !aligned(history, 4)) return ENGRAM_EINVAL;
    hipError_t e = launch_lookup(p->hash, p->gather, ids, history, uint32_t(n_tok), uint32_t(seq_len), nullptr,
                                 nullptr, nullptr, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_lookup_dedup(engram_plan_t p, const int32_t* ids, const int32_t* history, int64_t n_seq, int64_t seq_len,
                        const int32_t* perm, const int32_t* offsets, const int32_t* n_unique, float* out,
                        void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    int64_t n_tok = 0;
    int st = check_tokens(n_seq, seq_len, &n_tok);
    if (st != ENGRAM_OK) return st;
    if (n_tok == 0) return ENGRAM_OK;
    if (!ids || !out || !aligned(ids, 4) || !aligned(out, 16)) return ENGRAM_EINVAL;
    if (history && !aligned(history, 4)) return ENGRAM_EINVAL;
    if (!perm || !offsets || !n_unique || !aligned(perm, 4) || !aligned(offsets, 4) || !aligned(n_unique, 4))
        return ENGRAM_EINVAL;
    hipError_t e = launch_lookup(p->hash, p->gather, ids, history, uint32_t(n_tok), uint32_t(seq_len), perm, offsets,
                                 n_unique, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_gather_weighted(engram_plan_t p, const uint32_t* addr, int64_t n_tok, const float* weights, float* out,
                           void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    if (n_tok < 0 || n_tok > kMaxTokens) return ENGRAM_ERANGE;
    if (n_tok == 0) return ENGRAM_OK;
    if (!addr || !weights || !out || !aligned(addr, 16) || !aligned(weights, 16) || !aligned(out, 16))
        return ENGRAM_EINVAL;
    hipError_t e = launch_gate_io(p->gather, addr, weights, uint32_t(n_tok), out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_gather_rows(engram_plan_t p, const uint32_t* addr, int64_t n_tok, float* rows, void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    if (n_tok < 0 || n_tok > kMaxTokens) return ENGRAM_ERANGE;
    if (n_tok == 0) return ENGRAM_OK;
    if (!addr || !rows || !aligned(addr, 16) || !aligned(rows, 16)) return ENGRAM_EINVAL;
    hipError_t e = launch_gate_io(p->gather, addr, nullptr, uint32_t(n_tok), rows, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_dedup_workspace(engram_plan_t p, int64_t n_tok, size_t* bytes) {
    if (!valid_plan(p) || !bytes) return ENGRAM_EINVAL;
    if (n_tok < 0 || n_tok > kMaxDedupTokens) return ENGRAM_ERANGE;
    *bytes = dedup_workspace_bytes(uint32_t(n_tok), p->vocab_size);
    return ENGRAM_OK;
}

int engram_dedup(engram_plan_t p, const int32_t* ids, const int32_t* history, int64_t n_seq,
                 int64_t seq_len, int32_t* perm, int32_t* offsets, int32_t* n_unique, void* ws,
                 size_t ws_bytes, void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    int64_t n_tok = 0;
    int st = check_tokens(n_seq, seq_len, &n_tok);
    if (st != ENGRAM_OK) return st;
    if (n_tok > kMaxDedupTokens) return ENGRAM_ERANGE;
    if (!offsets || !n_unique || !aligned(offsets, 4) || !aligned(n_unique, 4)) return ENGRAM_EINVAL;
    if (n_tok > 0) {
        if (!ids || !perm || !aligned(ids, 4) || !aligned(perm, 4)) return ENGRAM_EINVAL;
        if (history && !aligned(history, 4)) return ENGRAM_EINVAL;
    }
    const size_t need = dedup_workspace_bytes(uint32_t(n_tok), p->vocab_size);
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256))) return ENGRAM_EWORKSPACE;
    hipError_t e = launch_dedup(ids, history, uint32_t(n_tok), uint32_t(seq_len), p->vocab_size, perm, offsets,
                                n_unique, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

int engram_check_inputs(engram_plan_t p, const int32_t* ids, const int32_t* history, int64_t n_seq, int64_t seq_len,
                        const uint32_t* addr, int64_t n_addr_tok, int32_t* counts, void* stream) {
    if (!valid_plan(p)) return ENGRAM_EINVAL;
    int64_t n_tok = 0;
    int st = check_tokens(n_seq, seq_len, &n_tok);
    if (st != ENGRAM_OK) return st;
    if (n_addr_tok < 0 || n_addr_tok > kMaxTokens) return ENGRAM_ERANGE;
    if (!counts || !aligned(counts, 4)) return ENGRAM_EINVAL;
    if (ids && !aligned(ids, 4)) return ENGRAM_EINVAL;
    if (history && (!ids || !aligned(history, 4))) return ENGRAM_EINVAL;
    if (addr && !aligned(addr, 16)) return ENGRAM_EINVAL;
    hipError_t e = launch_check(p->hash, p->vocab_size, ids, uint64_t(n_tok), history, uint64_t(n_seq) * 3u, addr,
                                addr ? uint64_t(n_addr_tok) : 0u, counts, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}

const char* engram_status_string(int status) {
    switch (status) {
        case ENGRAM_OK: return "ENGRAM_OK";
        case ENGRAM_EINVAL: return "ENGRAM_EINVAL: null or misaligned pointer, or bad argument";
        case ENGRAM_ERANGE: return "ENGRAM_ERANGE: row or token count out of range";
        case ENGRAM_EWORKSPACE: return "ENGRAM_EWORKSPACE: workspace missing or too small";
        case ENGRAM_EHIP: return "ENGRAM_EHIP: the HIP runtime refused a launch";
        case ENGRAM_EUNSUPPORTED: return "ENGRAM_EUNSUPPORTED: unsupported geometry";
        default: return "unknown engram status";
    }
}

}  // extern "C"
