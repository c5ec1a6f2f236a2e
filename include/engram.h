/*
 * engram.h -- C ABI of the Engram n-gram memory lookup for AMD Instinct
 * MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [VRAM]  "DeepSeek V4.1 Flash: The VRAM Killer. Can You Run It Locally?",
 *           section "What makes up the 511 GB of weights?"
 *   [GUIDE] "How to Run DeepSeek-V4.1-Flash: 510 GB, and 203 GB of It Is a
 *           Lookup Table", sections "The architecture", "Where the 510 GB
 *           goes" and "Engram: the table that is never multiplied"
 *   [REQ]   "Running DeepSeek V4.1 Flash locally: the numbers beyond 552B",
 *           section "Backbone, Engram, and active parameters describe
 *           different scales"
 *   [X]     "How DeepSeek V4.1 Flash's 763B weights run on consumer GPUs"
 *   [BLOG]  stondo.github.io, "deepseek-v41-flash-552b-exl3-two-rtx-pro-6000",
 *           section "What eager-plus-NVMe actually delivers"
 *
 * The operation.  Two Engram modules each hash the suffix n-grams of order
 * 2, 3 and 4 of the token-id stream with 8 independent heads and read one
 * row per (order, head): 24 rows per module, 48 per token [GUIDE "Engram";
 * VRAM].  Rows are 256 bytes of FP8 [GUIDE "Engram"; REQ]; each carries one
 * fp32 scale, or 8 E8M0 exponents (one per 32 elements), as the plan says.
 * The row addresses depend on the token ids alone, so the
 * whole prompt is hashed before any row is read [VRAM; GUIDE "Engram"]: the
 * library exposes the hash and the gather as separate calls.  The 24
 * dequantised rows of a module are summed into one fp32 vector of 256
 * elements; the pages' learned gate that follows (row vs. hidden state,
 * [GUIDE "The architecture"]) is not part of this library.
 *
 * Conventions for every call:
 *   - Return value: ENGRAM_OK (0) or a negative engram_status.  No call
 *     throws, aborts or prints.
 *   - All arguments are validated on the host before anything is launched;
 *     on an error return nothing has been launched and no output was
 *     written.
 *   - Calls that take a stream are asynchronous on that stream (a
 *     hipStream_t passed as void*; NULL is the null stream).  They never
 *     synchronise and never allocate device memory.
 *   - Device pointers are owned by the caller and must stay valid until the
 *     work queued on the stream has finished.
 *   - Device-side faults (e.g. a table pointer that is not device memory)
 *     surface at the caller's next synchronisation, as usual in HIP.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Geometry of the lookup [GUIDE "Engram"; VRAM]. */
#define ENGRAM_N_MODULES 2        /* Engram modules (layers) per token           */
#define ENGRAM_MIN_ORDER 2        /* shortest suffix n-gram                      */
#define ENGRAM_MAX_ORDER 4        /* longest suffix n-gram, = id window length    */
#define ENGRAM_N_HEADS 8          /* hash heads per (module, order)              */
#define ENGRAM_ROWS_PER_MODULE 24 /* 3 orders x 8 heads                          */
#define ENGRAM_N_SUB 48           /* sub-tables = rows read per token            */
#define ENGRAM_ROW_BYTES 256      /* FP8 E4M3 codes per row = output width       */
#define ENGRAM_N_MULT 192         /* hash multipliers: 2 x 3 x 8 x 4             */

/* Row scale formats (engram_plan_desc.scale_format). */
#define ENGRAM_SCALE_F32_ROW 0       /* one fp32 scale per row                          */
#define ENGRAM_SCALE_E8M0_BLOCK32 1  /* 8 E8M0 bytes per row, one per 32 elements      */

/* Seed of the default hash multipliers: the bytes "ENGRAM" followed by 0x0001. */
#define ENGRAM_DEFAULT_HASH_SEED 0x454E4752414D0001ULL

typedef enum engram_status {
    ENGRAM_OK = 0,
    ENGRAM_EINVAL = -1,      /* NULL or misaligned pointer, bad shape or flag       */
    ENGRAM_ERANGE = -2,      /* row count 0 or > 2^32, token count out of range     */
    ENGRAM_EWORKSPACE = -3,  /* workspace NULL or smaller than required             */
    ENGRAM_EHIP = -4,        /* the HIP runtime refused a launch                    */
    ENGRAM_EUNSUPPORTED = -5 /* a geometry other than the one above                 */
} engram_status;

/*
 * Plan description.  Sub-table s = 24*m + 8*(n-2) + h holds module m, order
 * n, head h (module-major, then order, then head).
 *
 *   n_modules, min_order, max_order, n_heads, row_bytes
 *       Must equal 2, 2, 4, 8, 256 (else ENGRAM_EUNSUPPORTED).
 *   vocab_size
 *       Exclusive upper bound of the token ids (the vocabulary the ids are
 *       drawn from), or 0 when ids may take any value in [0, 2^31).  It is
 *       the length of vocab_map when there is one.  engram_dedup uses it to
 *       size its sort keys: 4*ceil(log2(vocab_size)) bits per window, or, for
 *       2^16 < vocab_size <= 2^18, 4*ceil(log2(D+1)) bits where D is the
 *       number of distinct ids the call uses.  Ids at or above vocab_size
 *       break the dedup grouping and, with a vocab_map, the hash (see
 *       engram_hash); engram_check_inputs counts them.
 *   hash_seed
 *       Seeds the 192 hash multipliers: M[i] is output i+1 of splitmix64
 *       (Steele, Lea and Flood 2014) seeded with hash_seed, with bit 0 set;
 *       i runs over (module, order, head, k) in that nesting, k = 0..3.
 *   rows[48]   (host array, copied)
 *       Rows R_s of sub-table s, 1 <= R_s <= 2^32.
 *   tables[48] (host array of device pointers, copied)
 *       Sub-table s as row-major uint8 [R_s][256] of FP8 E4M3 codes (OCP
 *       encoding: bias 7, no infinities, 0x7F/0xFF are NaN).  16-byte aligned.
 *   scales[48] (host array of device pointers, copied)
 *       ENGRAM_SCALE_F32_ROW: fp32 [R_s], the scale of each row; 4-byte
 *       aligned.
 *       ENGRAM_SCALE_E8M0_BLOCK32: uint8 [R_s][8], the 8 bytes of scales a
 *       row carries [GUIDE "Engram"], read as one E8M0 exponent per block of
 *       32 elements (element j uses byte j/32; e stands for 2^(e-127), 255
 *       is NaN), the microscaling form of FP8 named for these tables [X];
 *       8-byte aligned.
 *   scale_format
 *       ENGRAM_SCALE_F32_ROW (0, the default) or ENGRAM_SCALE_E8M0_BLOCK32
 *       (else ENGRAM_EUNSUPPORTED).
 *   reserved1
 *       Must be 0.
 *   vocab_map  (device pointer, not copied; NULL = none)
 *       uint32 [vocab_size]: the id normalisation applied before hashing.
 *       The pages' engines fold ids that differ only in case, accents or
 *       spacing into one id of a smaller vocabulary before hashing [GUIDE
 *       "Engram"]; the map is that table.  Every id of a window (history and
 *       the pad id 0 included) is replaced by vocab_map[id] before the
 *       multiply-xor.  Needs vocab_size > 0 (the map's length) and 4-byte
 *       alignment.  engram_dedup still groups raw windows: equal raw windows
 *       have equal mapped windows, so its groups stay valid.
 *
 * The plan copies the description; the tables themselves are not copied and
 * must outlive every call that uses the plan.
 */
typedef struct engram_plan_desc {
    uint32_t n_modules;
    uint32_t min_order;
    uint32_t max_order;
    uint32_t n_heads;
    uint32_t row_bytes;
    uint32_t vocab_size;           /* exclusive bound of token ids; 0 = any id in [0, 2^31) */
    uint64_t hash_seed;
    const uint64_t* rows;
    const uint8_t* const* tables;
    const void* const* scales;
    uint32_t scale_format;
    uint32_t reserved1;            /* must be 0 */
    const uint32_t* vocab_map;     /* device uint32 [vocab_size] or NULL */
} engram_plan_desc;

typedef struct engram_plan_s* engram_plan_t;

/* Fill a description with the default geometry and hash seed; the caller
 * still sets rows, tables and scales.  Returns ENGRAM_EINVAL on NULL. */
int engram_plan_desc_init(engram_plan_desc* desc);

/*
 * Validate a description and build an immutable plan: copies the row counts
 * and pointers, derives the multipliers and the exact division constants of
 * each R_s.  The geometry it accepts is the pages' one: two modules, orders
 * 2 to 4, 8 heads per order, 256-byte FP8 rows, 48 sub-tables [GUIDE
 * "Engram"; VRAM].  The pages print no hash constants; the multipliers are
 * this library's own (see hash_seed).  Host-only: touches no device and may
 * run before any device exists.  *out is set only on ENGRAM_OK.  A plan may
 * be used from several host threads and streams at once.  Errors: EINVAL
 * (NULL argument, pointer, misaligned pointer, reserved1 != 0, a vocab_map
 * without vocab_size), ERANGE (a row count of 0 or above 2^32),
 * EUNSUPPORTED (another geometry or scale format).
 */
int engram_plan(const engram_plan_desc* desc, engram_plan_t* out);

/* Release a plan (NULL is accepted).  No work using it may be in flight. */
int engram_plan_destroy(engram_plan_t plan);

/* Copy the 192 hash multipliers of a plan into host memory out[192], in
 * (module, order, head, k) order. */
int engram_plan_multipliers(engram_plan_t plan, uint64_t* out);

/*
 * Hash: 48 row addresses per token [GUIDE "Engram"; VRAM].
 *
 * Token tok = s*seq_len + t has the id window w_k = id at position t-k,
 * k = 0..3; positions before 0 read history[s][3 + (t-k)] (history[s][2] is
 * the id just before position 0) or, with history == NULL, id 0.  With a
 * vocab_map in the plan each w_k is then replaced by vocab_map[w_k].  For
 * module m, order n, head h, with u64 the zero-extension of the 32-bit id:
 *     x = XOR_{k<n} ( u64(w_k) * M[m][n][h][k] )   (mod 2^64)
 *     addr[tok][24*m + 8*(n-2) + h] = x mod R_s
 *
 *   ids      device int32 [n_seq][seq_len], ids in [0, 2^31), and below the
 *            plan's vocab_size when it has a vocab_map (the map is read at
 *            every window id, history and pad included, without a bounds
 *            check: a larger or negative id reads outside the map).  Not
 *            checked on the device; engram_check_inputs counts violations.
 *   history  device int32 [n_seq][3] or NULL; the same bounds as ids.
 *   addr     device uint32 [n_seq*seq_len][48], 16-byte aligned (output).
 *
 * n_seq*seq_len == 0 is a no-op.  Errors: EINVAL (NULL/misaligned pointer,
 * negative sizes), ERANGE (n_seq*seq_len >= 2^31).
 */
int engram_hash(engram_plan_t plan, const int32_t* ids, const int32_t* history,
                int64_t n_seq, int64_t seq_len, uint32_t* addr, void* stream);

/*
 * Gather, dequantise and sum [GUIDE "Engram"; REQ].
 *
 * For token tok, module m and element j:
 *     out[tok][m][j] = sum_{q=0..23} fp8(T_{24m+q}[a][j]) * scale_{24m+q}(a, j),
 *     a = addr[tok][24m+q],
 * scale(a, j) = scales[a] (fp32 per row) or 2^(scales[a][j/32] - 127) (E8M0
 * per 32-element block),
 * accumulated in fp32 in ascending q (fused multiply-add), starting at +0.
 *
 *   addr    device uint32 [n_tok][48] (as written by engram_hash); every
 *           address must be < R_s (not checked on the device).
 *   out     device fp32 [n_tok][2][256], 16-byte aligned (output).
 *
 * Direct mode: perm, offsets and n_unique all NULL.
 * Dedup mode: perm, offsets, n_unique as written by engram_dedup for the
 * same tokens; each group of tokens with equal windows is looked up once
 * and its vector stored to every member.  The result is bitwise identical
 * to direct mode.  In dedup mode the grid covers n_tok groups and exits
 * early past *n_unique, which stays on the device.
 *
 * n_tok == 0 is a no-op.  Errors: EINVAL (NULL/misaligned pointer, a partial
 * set of dedup pointers), ERANGE (n_tok < 0 or >= 2^31).
 */
int engram_gather_reduce(engram_plan_t plan, const uint32_t* addr, int64_t n_tok,
                         const int32_t* perm, const int32_t* offsets,
                         const int32_t* n_unique, float* out, void* stream);

/*
 * engram_gather_reduce in direct mode for a batch of n_seq sequences of
 * seq_len tokens whose addresses engram_hash wrote (addr[n_seq*seq_len][48],
 * token-major).  Same results, bitwise; the tokens are visited in tiles of 64
 * positions, up to 8 sequences at the same position per workgroup, so that
 * sequences sharing a prefix gather each prefix window once per workgroup
 * (in a batch of 8,192 tokens or more, tokens with equal addresses share one
 * gather) and read its rows from L2 after their first fetch (the pages hash
 * every address before the lookup [VRAM; GUIDE "Engram"], and batched prompts
 * often share a system prefix).
 *
 *   addr     device uint32 [n_seq*seq_len][48], 16-byte aligned.
 *   out      device fp32 [n_seq*seq_len][2][256], 16-byte aligned (output).
 *
 * n_seq*seq_len == 0 is a no-op.  Errors: EINVAL (NULL/misaligned pointer,
 * negative count), ERANGE (n_seq*seq_len above 2^31 - 1).
 */
int engram_gather_reduce_batched(engram_plan_t plan, const uint32_t* addr, int64_t n_seq, int64_t seq_len,
                                 float* out, void* stream);

/*
 * Inputs for the learned gate that follows the lookup: each retrieved row is
 * weighed against the hidden state before the module's rows are combined
 * [GUIDE "The architecture", "Engram"].  The gate itself (trained weights,
 * hidden states) is outside this library.
 *
 * engram_gather_weighted: as engram_gather_reduce (direct mode) with one
 * caller weight per row:
 *     out[tok][m][j] = sum_q fp8(T_{24m+q}[a][j]) * fp32(scale_{24m+q}(a, j) * w[tok][24m+q])
 * accumulated in fp32 in ascending q; with every weight 1 the result is
 * bitwise that of engram_gather_reduce.
 *   weights  device fp32 [n_tok][48] (same order as addr), 16-byte aligned.
 *   out      device fp32 [n_tok][2][256], 16-byte aligned (output).
 *
 * engram_gather_rows: the 48 dequantised rows of every token, un-reduced:
 *     rows[tok][s][j] = fp32(fp8(T_s[a][j]) * scale_s(a, j)),  a = addr[tok][s]
 *   rows     device fp32 [n_tok][48][256] (48 KiB per token), 16-byte aligned.
 *
 * n_tok == 0 is a no-op.  Errors: EINVAL (NULL/misaligned pointer), ERANGE.
 */
int engram_gather_weighted(engram_plan_t plan, const uint32_t* addr, int64_t n_tok,
                           const float* weights, float* out, void* stream);
int engram_gather_rows(engram_plan_t plan, const uint32_t* addr, int64_t n_tok, float* rows,
                       void* stream);

/*
 * Fused lookup: engram_hash followed by engram_gather_reduce (direct mode)
 * in one launch, without the address buffer.  The addresses depend on the
 * ids alone [VRAM; GUIDE "Engram"], so each (token, module) computes its own
 * 24 rows and gathers them.  Bitwise identical to the two calls.  A batch
 * of sequences is visited in the order of engram_gather_reduce_batched, so
 * sequences that share a prefix gather each prefix window once per workgroup
 * and read its rows from L2 after their first fetch: passing such sequences
 * in one call is cheaper than one call each.
 *
 *   ids, history, n_seq, seq_len   as for engram_hash.
 *   out       device fp32 [n_seq*seq_len][2][256], 16-byte aligned (output).
 *
 * n_seq*seq_len == 0 is a no-op.  Errors: EINVAL, ERANGE as engram_hash.
 */
int engram_lookup(engram_plan_t plan, const int32_t* ids, const int32_t* history,
                  int64_t n_seq, int64_t seq_len, float* out, void* stream);

/*
 * engram_lookup in dedup mode: one hash and one gather per group of tokens
 * with equal windows, the vector stored to every member of the group.  Equal
 * windows hash to equal rows [VRAM; GUIDE "Engram"], so the result is bitwise
 * that of engram_lookup (and of engram_hash + engram_gather_reduce in either
 * mode); the address buffer and the separate hash launch are gone, and a
 * window repeated across a batch (a shared prefix [BLOG]) is hashed once.
 *
 *   ids, history, n_seq, seq_len   as for engram_lookup, and the same tokens
 *             that engram_dedup grouped.
 *   perm, offsets, n_unique        as written by engram_dedup for those
 *             tokens (device int32, 4-byte aligned); *n_unique stays on the
 *             device.  *n_unique < 0 (a failed dedup call) writes nothing.
 *   out       device fp32 [n_seq*seq_len][2][256], 16-byte aligned (output).
 *
 * The grid covers n_seq*seq_len groups and exits early past *n_unique.  A
 * perm or offsets entry out of [0, n_tok) is skipped, never dereferenced.
 * n_seq*seq_len == 0 is a no-op.  Errors: EINVAL (NULL/misaligned pointer),
 * ERANGE as engram_hash.
 */
int engram_lookup_dedup(engram_plan_t plan, const int32_t* ids, const int32_t* history,
                        int64_t n_seq, int64_t seq_len, const int32_t* perm, const int32_t* offsets,
                        const int32_t* n_unique, float* out, void* stream);

/*
 * Workspace bytes engram_dedup needs for n_tok tokens under this plan
 * (host-only).  The size depends on the plan's vocab_size, which bounds the
 * width of the sort keys.  Errors: EINVAL (NULL plan or bytes), ERANGE
 * (n_tok < 0 or > 2^22).
 */
int engram_dedup_workspace(engram_plan_t plan, int64_t n_tok, size_t* bytes);

/*
 * Group the tokens whose id windows (w_0, w_1, w_2, w_3) are equal.
 *
 * The pages hash every row address from the token ids alone, before the
 * forward pass, so a whole batch's addresses are known up front and can be
 * fetched together [VRAM]; and in the serving setups they describe, most of
 * a prompt is a prefix other requests already sent [BLOG "What eager-plus-
 * NVMe actually delivers"].  Tokens with equal windows hash to the same 48
 * rows, so one lookup serves a whole group (engram_gather_reduce in dedup
 * mode).  Groups are ordered by ascending window (w_0 most significant, ids
 * compared as unsigned), tokens within a group by ascending index: the
 * result is unique.
 *
 *   ids, history, n_seq, seq_len   as for engram_hash.  Every id should be
 *             < the plan's vocab_size (when it is not 0); a larger or negative
 *             id is a contract violation: its grouping is then unspecified,
 *             but the call reads and writes nothing out of bounds.
 *   perm      device int32 [n_tok]: the tokens, group by group (output).
 *   offsets   device int32 [n_tok + 1]: offsets[u] is where group u starts
 *             in perm; offsets[n_unique] = n_tok; entries past n_unique are
 *             left unspecified (output).
 *   n_unique  device int32 [1]: the number of groups (output).  -1 reports
 *             that a bounded device-side wait of the sort gave up (the sort's
 *             tiles wait for the ones started before them; this does not
 *             happen unless the device stalls a running workgroup for
 *             milliseconds): perm and offsets are then invalid, and
 *             engram_gather_reduce in dedup mode treats the groups as empty.
 *             The bound is 262,144 polls per wait; the environment variable
 *             ENGRAM_DEDUP_SPIN_LIMIT, read at each call, overrides it (a
 *             test forces the give-up path with a small value).
 *   ws        device workspace of ws_bytes >= engram_dedup_workspace(plan,
 *             n_tok), 256-byte aligned, owned by the caller.  It keeps a
 *             small state between calls (no clearing needed, initial
 *             contents arbitrary); one call at a time may use it.
 *
 * n_tok == 0 writes offsets[0] = 0 and *n_unique = 0.  Errors: EINVAL,
 * ERANGE (n_tok > 2^22 = 4,194,304: split larger batches), EWORKSPACE.
 */
int engram_dedup(engram_plan_t plan, const int32_t* ids, const int32_t* history,
                 int64_t n_seq, int64_t seq_len, int32_t* perm, int32_t* offsets,
                 int32_t* n_unique, void* ws, size_t ws_bytes, void* stream);

/*
 * Opt-in input check: count, on the device and without faulting, the
 * contract violations the lookup calls do not check: the row addresses are
 * read as given [GUIDE "Engram"], and ids index the vocabulary map.  Reads
 * only ids, history and addr (never a table or the map), so it is safe on
 * any values.
 *
 *   ids, history, n_seq, seq_len   as for engram_hash, or ids == NULL (then
 *             history must be NULL too) to skip the id check.
 *   addr      device uint32 [n_addr_tok][48] as engram_hash writes it,
 *             16-byte aligned, or NULL to skip the address check.
 *   counts    device int32 [3], 4-byte aligned (output, overwritten):
 *             counts[0] = ids and history ids below 0,
 *             counts[1] = ids and history ids >= the plan's vocab_size
 *                         (always 0 when vocab_size is 0),
 *             counts[2] = addresses addr[t][s] >= R_s.
 *
 * Two launches on the stream (clear, count); no synchronisation.  Errors:
 * EINVAL (NULL plan or counts, misaligned pointer, history without ids),
 * ERANGE (a token count out of range).
 */
int engram_check_inputs(engram_plan_t plan, const int32_t* ids, const int32_t* history,
                        int64_t n_seq, int64_t seq_len, const uint32_t* addr, int64_t n_addr_tok,
                        int32_t* counts, void* stream);

/*
 * engram_dedup for callers that cannot allocate device memory (code under
 * HIP graph capture that forbids allocation, tight serving loops, harnesses
 * that disallow hipMalloc): the same kernels and results, with the workspace
 * in a fixed array of ENGRAM_DEDUP_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  The call itself allocates
 * nothing.  Arguments, outputs and errors are those of engram_dedup, without
 * ws and ws_bytes; a batch whose workspace (engram_dedup_workspace) exceeds
 * the fixed size returns ENGRAM_EWORKSPACE before anything is launched
 * (524,288 tokens fit under any plan).  All calls on one GPU share that
 * GPU's array: calls that overlap in time on one GPU (two streams, two host
 * threads) race and give wrong groups; serialise them.  The first call on a
 * device looks up the array's address there (hipGetSymbolAddress).
 */
#define ENGRAM_DEDUP_SCRATCH_BYTES (32u << 20)
int engram_dedup_noalloc(engram_plan_t plan, const int32_t* ids, const int32_t* history,
                         int64_t n_seq, int64_t seq_len, int32_t* perm, int32_t* offsets,
                         int32_t* n_unique, void* stream);

/* Static, human-readable name of a status code. */
const char* engram_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
