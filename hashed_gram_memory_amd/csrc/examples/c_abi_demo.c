/*
 * A C consumer of the Engram lookup ABI: no Python, no torch.
 *
 * Usage: c_abi_demo <out.bin> <n_tok> <rows> <table_seed>
 *
 * Allocates 48 sub-tables of <rows> rows with hipMalloc, fills them with the
 * seeded synthetic generator (engram_synth_fill), hashes the ids 0, 7, 14,
 * ... (one sequence of n_tok tokens, mod 129,280), gathers and sums, runs the
 * fused lookup too, and writes to <out.bin>:
 *     int32 ids[n_tok] | uint32 addr[n_tok][48] | float out[n_tok][2][256] | float fused[n_tok][2][256]
 * It also gathers the same addresses with engram_gather_reduce_batched and
 * checks that the result equals the flat gather's bit for bit.
 * Exit status 0 on success; any failing call or check prints why and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "engram.h"
#include "engram_synth.h"

#define CHECK_HIP(x)                                                        \
    do {                                                                    \
        hipError_t e_ = (x);                                                \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));   \
            return 1;                                                       \
        }                                                                   \
    } while (0)

#define CHECK_ENGRAM(x)                                                     \
    do {                                                                    \
        int s_ = (x);                                                       \
        if (s_ != ENGRAM_OK) {                                              \
            fprintf(stderr, "%s failed: %s\n", #x, engram_status_string(s_)); \
            return 1;                                                       \
        }                                                                   \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 5) {
        fprintf(stderr, "usage: %s out.bin n_tok rows table_seed\n", argv[0]);
        return 2;
    }
    const int64_t n_tok = atoll(argv[2]);
    const uint64_t rows = strtoull(argv[3], NULL, 10);
    const uint64_t seed = strtoull(argv[4], NULL, 10);
    if (n_tok <= 0 || rows == 0) return 2;

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    uint8_t* tab;
    float* sc;
    CHECK_HIP(hipMalloc((void**)&tab, ENGRAM_N_SUB * rows * ENGRAM_ROW_BYTES));
    CHECK_HIP(hipMalloc((void**)&sc, ENGRAM_N_SUB * rows * sizeof(float)));
    uint64_t rows_arr[ENGRAM_N_SUB];
    const uint8_t* tabs[ENGRAM_N_SUB];
    const void* scs[ENGRAM_N_SUB];
    for (int s = 0; s < ENGRAM_N_SUB; ++s) {
        rows_arr[s] = rows;
        tabs[s] = tab + (uint64_t)s * rows * ENGRAM_ROW_BYTES;
        scs[s] = sc + (uint64_t)s * rows;
        CHECK_ENGRAM(engram_synth_fill((uint8_t*)tabs[s], (float*)scs[s], rows, (uint32_t)s, seed, stream));
    }

    engram_plan_desc desc;
    CHECK_ENGRAM(engram_plan_desc_init(&desc));
    desc.rows = rows_arr;
    desc.tables = tabs;
    desc.scales = scs;
    engram_plan_t plan;
    CHECK_ENGRAM(engram_plan(&desc, &plan));

    int32_t* h_ids = (int32_t*)malloc(n_tok * sizeof(int32_t));
    for (int64_t i = 0; i < n_tok; ++i) h_ids[i] = (int32_t)((i * 7) % 129280);
    int32_t* ids;
    uint32_t* addr;
    float *out, *fused, *batched;
    const size_t out_bytes = (size_t)n_tok * 2 * ENGRAM_ROW_BYTES * sizeof(float);
    CHECK_HIP(hipMalloc((void**)&ids, n_tok * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&addr, n_tok * ENGRAM_N_SUB * sizeof(uint32_t)));
    CHECK_HIP(hipMalloc((void**)&out, out_bytes));
    CHECK_HIP(hipMalloc((void**)&fused, out_bytes));
    CHECK_HIP(hipMalloc((void**)&batched, out_bytes));
    CHECK_HIP(hipMemcpyAsync(ids, h_ids, n_tok * sizeof(int32_t), hipMemcpyHostToDevice, stream));

    CHECK_ENGRAM(engram_hash(plan, ids, NULL, 1, n_tok, addr, stream));
    CHECK_ENGRAM(engram_gather_reduce(plan, addr, n_tok, NULL, NULL, NULL, out, stream));
    CHECK_ENGRAM(engram_lookup(plan, ids, NULL, 1, n_tok, fused, stream));
    /* the same addresses gathered in the batch order, split into 7 equal sequences when the count allows:
       only the visiting order differs, so the result must be the flat gather's, bit for bit */
    const int64_t n_seq = n_tok % 7 == 0 ? 7 : 1;
    CHECK_ENGRAM(engram_gather_reduce_batched(plan, addr, n_seq, n_tok / n_seq, batched, stream));

    uint32_t* h_addr = (uint32_t*)malloc(n_tok * ENGRAM_N_SUB * sizeof(uint32_t));
    float* h_out = (float*)malloc(out_bytes);
    float* h_fused = (float*)malloc(out_bytes);
    float* h_batched = (float*)malloc(out_bytes);
    CHECK_HIP(hipMemcpyAsync(h_addr, addr, n_tok * ENGRAM_N_SUB * sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_out, out, out_bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_fused, fused, out_bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_batched, batched, out_bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    if (memcmp(h_batched, h_out, out_bytes) != 0) {
        fprintf(stderr, "engram_gather_reduce_batched differs from engram_gather_reduce\n");
        return 1;
    }

    /* dedup: ids with period 5, so most windows repeat; the tokens are grouped, then looked up once per group
       (engram_lookup_dedup) and once per group from the addresses (engram_gather_reduce in dedup mode): both must
       be the direct lookup's result, bit for bit */
    int32_t* h_rep = (int32_t*)malloc(n_tok * sizeof(int32_t));
    for (int64_t i = 0; i < n_tok; ++i) h_rep[i] = (int32_t)(i % 5);
    int32_t *rep, *perm, *offsets, *n_unique;
    uint32_t* rep_addr;
    float *rep_direct, *rep_dedup, *rep_gather;
    size_t ws_bytes = 0;
    void* ws;
    CHECK_ENGRAM(engram_dedup_workspace(plan, n_tok, &ws_bytes));
    CHECK_HIP(hipMalloc((void**)&rep, n_tok * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&perm, n_tok * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&offsets, (n_tok + 1) * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&n_unique, sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&rep_addr, n_tok * ENGRAM_N_SUB * sizeof(uint32_t)));
    CHECK_HIP(hipMalloc((void**)&rep_direct, out_bytes));
    CHECK_HIP(hipMalloc((void**)&rep_dedup, out_bytes));
    CHECK_HIP(hipMalloc((void**)&rep_gather, out_bytes));
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_HIP(hipMemcpyAsync(rep, h_rep, n_tok * sizeof(int32_t), hipMemcpyHostToDevice, stream));
    CHECK_ENGRAM(engram_dedup(plan, rep, NULL, 1, n_tok, perm, offsets, n_unique, ws, ws_bytes, stream));
    CHECK_ENGRAM(engram_lookup(plan, rep, NULL, 1, n_tok, rep_direct, stream));
    CHECK_ENGRAM(engram_lookup_dedup(plan, rep, NULL, 1, n_tok, perm, offsets, n_unique, rep_dedup, stream));
    CHECK_ENGRAM(engram_hash(plan, rep, NULL, 1, n_tok, rep_addr, stream));
    CHECK_ENGRAM(engram_gather_reduce(plan, rep_addr, n_tok, perm, offsets, n_unique, rep_gather, stream));
    float* h_rep_direct = (float*)malloc(out_bytes);
    float* h_rep_dedup = (float*)malloc(out_bytes);
    float* h_rep_gather = (float*)malloc(out_bytes);
    int32_t h_n_unique = -2;
    CHECK_HIP(hipMemcpyAsync(h_rep_direct, rep_direct, out_bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_rep_dedup, rep_dedup, out_bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_rep_gather, rep_gather, out_bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(&h_n_unique, n_unique, sizeof(int32_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    if (h_n_unique <= 0 || memcmp(h_rep_dedup, h_rep_direct, out_bytes) != 0 ||
        memcmp(h_rep_gather, h_rep_direct, out_bytes) != 0) {
        fprintf(stderr, "dedup-mode lookup or gather differs from the direct lookup (n_unique %d)\n", h_n_unique);
        return 1;
    }
    printf("dedup groups: %d\n", h_n_unique);

    FILE* f = fopen(argv[1], "wb");
    if (!f) return 1;
    fwrite(h_ids, sizeof(int32_t), n_tok, f);
    fwrite(h_addr, sizeof(uint32_t), n_tok * ENGRAM_N_SUB, f);
    fwrite(h_out, 1, out_bytes, f);
    fwrite(h_fused, 1, out_bytes, f);
    fclose(f);

    CHECK_ENGRAM(engram_plan_destroy(plan));
    CHECK_HIP(hipFree(ids));
    CHECK_HIP(hipFree(addr));
    CHECK_HIP(hipFree(out));
    CHECK_HIP(hipFree(fused));
    CHECK_HIP(hipFree(batched));
    CHECK_HIP(hipFree(tab));
    CHECK_HIP(hipFree(sc));
    CHECK_HIP(hipStreamDestroy(stream));
    free(h_ids);
    free(h_addr);
    free(h_out);
    free(h_fused);
    free(h_batched);
    CHECK_HIP(hipFree(rep));
    CHECK_HIP(hipFree(perm));
    CHECK_HIP(hipFree(offsets));
    CHECK_HIP(hipFree(n_unique));
    CHECK_HIP(hipFree(rep_addr));
    CHECK_HIP(hipFree(rep_direct));
    CHECK_HIP(hipFree(rep_dedup));
    CHECK_HIP(hipFree(rep_gather));
    CHECK_HIP(hipFree(ws));
    free(h_rep);
    free(h_rep_direct);
    free(h_rep_dedup);
    free(h_rep_gather);
    printf("c_abi_demo ok: %lld tokens\n", (long long)n_tok);
    return 0;
}
