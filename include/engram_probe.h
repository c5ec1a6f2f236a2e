/*
 * engram_probe.h -- memory-ceiling probes (measurement only; not part of the
 * lookup: these calls live in the measurement library, libengram_measure.so).
 *
 * The lookup's gather is bound by HBM.  These kernels measure, on the same
 * device and in the same process, what the memory system delivers for the
 * access patterns involved, so the gather's achieved bandwidth can be read
 * against a measured ceiling as well as against the 8 TB/s datasheet peak:
 *   - a streaming read and a streaming copy (16-byte vector accesses);
 *   - the gather itself with the row scales left out (rows only): the same
 *     wave layout and row loads as engram_gather_reduce, decoded rows summed
 *     without scaling, so its cost minus the full kernel's is the cost of the
 *     48 random 4-byte scale reads.
 *   - random reads of whole 256-, 512- or 1024-byte chunks: how efficiently
 *     DRAM serves accesses of the gather's size (a row is 256 bytes);
 *   - a random-row gather-sum with the row scales kept in different places:
 *     what DRAM charges for the scale of a row.
 * All return 0 or a negative engram_status; all are asynchronous on
 * `stream` and allocate nothing.
 */
#ifndef ENGRAM_PROBE_H
#define ENGRAM_PROBE_H

#include <stdint.h>

#include "engram.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) from device memory `src` (16-byte
 * aligned); `sink` is a device uint32 written only in a case that never
 * occurs in practice, to keep the reads alive. */
int engram_probe_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream);

/* Copy `bytes` (a multiple of 16) from `src` to `dst` (both 16-byte aligned,
 * not overlapping). */
int engram_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream);

/* Read about `read_bytes` in whole `chunk_bytes` chunks (256, 512 or 1024,
 * else ENGRAM_EUNSUPPORTED) at uniformly random chunk offsets of the device
 * buffer `buf` (`bytes` long, 256-byte aligned), 6 KiB per wavefront; offsets
 * come from splitmix64 of (seed, chunk counter).  `sink` as for
 * engram_probe_read. */
int engram_probe_random(const void* buf, uint64_t bytes, uint32_t chunk_bytes, uint64_t read_bytes, uint64_t seed,
                        uint32_t* sink, void* stream);

/* Gather-sum of 24 uniformly random rows per (token, module) of the device
 * buffer `buf` (`bytes` long, 256-byte aligned), writing fp32 [n_tok][2][256]
 * to `out` (16-byte aligned).  `layout` places the row scales:
 *   0  256-byte rows, no scales           (rows: bytes / 256)
 *   1  256-byte rows + fp32 scales in a separate array after all the rows
 *                                         (rows: bytes / 260)
 *   2  260-byte records, fp32 scale after the 256 codes (rows: bytes / 260)
 *   3  264-byte records, 8 E8M0 bytes after the codes   (rows: bytes / 264)
 * Any other layout is ENGRAM_EUNSUPPORTED.  The buffer's contents only need
 * to be readable; the output is for keeping the loads, not for checking. */
int engram_probe_records(const void* buf, uint64_t bytes, uint32_t layout, int64_t n_tok, uint64_t seed, float* out,
                         void* stream);

/* engram_gather_reduce in direct mode without the row scales: out[tok][m][j]
 * = sum over the module's 24 rows of the decoded code.  Same arguments and
 * checks as engram_gather_reduce. */
int engram_probe_rows(engram_plan_t plan, const uint32_t* addr, int64_t n_tok, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_PROBE_H */
