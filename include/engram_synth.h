/*
 * engram_synth.h -- seeded synthetic tables on the device (input data only).
 *
 * Not part of the lookup: these calls live in the measurement library,
 * libengram_measure.so, not in libengram.so.  Full-size Engram tables (48 x 2^24 rows x 256 B,
 * 192 GiB) cannot be shipped from the host in reasonable time, so the
 * synthetic workloads define every table byte and scale by a counter-based
 * generator and fill the tables on the device.  Host code regenerates any
 * row from the same definition to check results.
 *
 * Generator: splitmix64 (Steele, Lea and Flood 2014).  out(seed, idx) is
 * output idx+1 of the stream seeded with `seed`, i.e. the 30/27/31
 * xor-shift-multiply finaliser applied to seed + (idx+1)*0x9E3779B97F4A7C15.
 *   byte j of row r of sub-table s:
 *       z = out(seed, (s << 40) | (r << 6) | (j / 4));
 *       u = bits [16*(j%4), 16*(j%4)+16) of z;  v = (u * 254) >> 16;
 *       code = v < 127 ? v : v + 1      (uniform over the 254 non-NaN codes)
 *   scale of row r of sub-table s:
 *       z = out(seed, (1 << 63) | (s << 40) | r);
 *       scale = (2^22 + (((z >> 40) * 3) >> 2)) * 2^-23   (exact, in [0.5, 2))
 *   E8M0 block scales of row r of sub-table s (8 bytes, block b = byte b):
 *       z = out(seed, (3 << 62) | (s << 40) | r);
 *       e_b = 120 + ((((z >> 8b) & 255) * 15) >> 8)      (2^-7 .. 2^7)
 */
#ifndef ENGRAM_SYNTH_H
#define ENGRAM_SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Fill sub-table `sub_index` (0..47): table = device uint8 [rows][256]
 * (16-byte aligned), scales = device fp32 [rows]; either may be NULL to skip
 * it.  1 <= rows <= 2^32.  Asynchronous on `stream` (hipStream_t or NULL).
 * Returns 0 or a negative engram_status (see engram.h).
 */
int engram_synth_fill(uint8_t* table, float* scales, uint64_t rows, uint32_t sub_index,
                      uint64_t seed, void* stream);

/*
 * Fill the E8M0 block scales of sub-table `sub_index`: scales = device uint8
 * [rows][8] (8-byte aligned).  Same range checks as engram_synth_fill.
 */
int engram_synth_fill_e8m0(uint8_t* scales, uint64_t rows, uint32_t sub_index, uint64_t seed, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_SYNTH_H */
