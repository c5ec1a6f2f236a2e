/*
 * Host-side generator for the synthetic Engram tables (input data only).
 *
 * The tables in the workloads are random: uniform non-NaN FP8 E4M3 codes and
 * one fp32 scale per row in [0.5, 2).  Both sides of a parity check need the
 * same bytes, and the full-size tables (48 sub-tables x 2^24 rows x 256 B)
 * cannot be shipped from the host, so the data is defined by a counter-based
 * generator: every byte is a pure function of (table_seed, sub-table, row,
 * byte).  The device has its own implementation of the same definition; this
 * file holds the host one.  Nothing here is part of the lookup itself.
 *
 * Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Output number i (i >= 1)
 * of the stream seeded with `seed` is mix(seed + i * 0x9E3779B97F4A7C15),
 * where mix is the published 30/27/31 xor-shift-multiply finaliser.  The
 * table data uses output (idx + 1) for a counter idx:
 *
 *   codes:  idx = (s << 40) | (r << 6) | g,  g = byte / 4 (0..63);
 *           u   = 16-bit field (byte % 4) of that output;
 *           v   = (u * 254) >> 16             (0..253);
 *           code = v < 127 ? v : v + 1        (skips 0x7F and 0xFF, the NaNs)
 *   scales: idx = (1 << 63) | (s << 40) | r;
 *           k = 2^22 + (((out >> 40) * 3) >> 2);   scale = k * 2^-23
 *           (k < 2^24, so the scale is exact in fp32 and lies in [0.5, 2)).
 *   E8M0 block scales (8 bytes per row): idx = (3 << 62) | (s << 40) | r;
 *           byte b = 120 + (((out >> 8b) & 255) * 15 >> 8)   (2^-7 .. 2^7).
 */
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix_at(uint64_t seed, uint64_t idx)
{
    uint64_t z = seed + (idx + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline void row_codes(uint64_t seed, uint64_t s, uint64_t r, uint8_t *dst)
{
    for (uint64_t g = 0; g < 64; ++g) {
        uint64_t z = splitmix_at(seed, (s << 40) | (r << 6) | g);
        for (int b = 0; b < 4; ++b) {
            uint32_t u = (uint32_t)((z >> (16 * b)) & 0xFFFFu);
            uint32_t v = (u * 254u) >> 16;
            dst[4 * g + b] = (uint8_t)(v < 127u ? v : v + 1u);
        }
    }
}

static inline float row_scale(uint64_t seed, uint64_t s, uint64_t r)
{
    uint64_t z = splitmix_at(seed, (1ull << 63) | (s << 40) | r);
    uint32_t k = (1u << 22) + (uint32_t)(((z >> 40) * 3u) >> 2);
    return (float)k * (1.0f / 8388608.0f);
}

/* Rows rows[0..n) of sub-table s: codes to codes[i*256 ..], scales to scales[i]. */
void tablegen_rows(uint64_t seed, uint32_t s, const uint32_t *rows, int64_t n,
                   uint8_t *codes, float *scales)
{
    for (int64_t i = 0; i < n; ++i) {
        if (codes) row_codes(seed, s, rows[i], codes + i * 256);
        if (scales) scales[i] = row_scale(seed, s, rows[i]);
    }
}

/* Scatter form: write row rows[i] of sub-table s into a table laid out as
 * [R][256] (codes) and [R] (scales), i.e. into its own place. */
void tablegen_scatter(uint64_t seed, uint32_t s, const uint32_t *rows, int64_t n,
                      uint8_t *table, float *scales)
{
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = rows[i];
        if (table) row_codes(seed, s, r, table + r * 256u);
        if (scales) scales[r] = row_scale(seed, s, r);
    }
}

/* Contiguous range [r0, r0 + n) of sub-table s into codes[n*256], scales[n]. */
void tablegen_range(uint64_t seed, uint32_t s, uint64_t r0, uint64_t n,
                    uint8_t *codes, float *scales)
{
    for (uint64_t i = 0; i < n; ++i) {
        if (codes) row_codes(seed, s, r0 + i, codes + i * 256);
        if (scales) scales[i] = row_scale(seed, s, r0 + i);
    }
}

static inline void row_e8m0(uint64_t seed, uint64_t s, uint64_t r, uint8_t *dst)
{
    uint64_t z = splitmix_at(seed, (3ull << 62) | (s << 40) | r);
    for (int b = 0; b < 8; ++b) {
        uint32_t u = (uint32_t)((z >> (8 * b)) & 0xFFu);
        dst[b] = (uint8_t)(120u + ((u * 15u) >> 8));
    }
}

/* E8M0 block scales: rows[i] -> out[i*8 ..] */
void tablegen_e8m0_rows(uint64_t seed, uint32_t s, const uint32_t *rows, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) row_e8m0(seed, s, rows[i], out + i * 8);
}

/* Scatter form into a [R][8] array. */
void tablegen_e8m0_scatter(uint64_t seed, uint32_t s, const uint32_t *rows, int64_t n, uint8_t *scales)
{
    for (int64_t i = 0; i < n; ++i) row_e8m0(seed, s, rows[i], scales + (uint64_t)rows[i] * 8u);
}

/* Contiguous range [r0, r0 + n) into out[n*8]. */
void tablegen_e8m0_range(uint64_t seed, uint32_t s, uint64_t r0, uint64_t n, uint8_t *out)
{
    for (uint64_t i = 0; i < n; ++i) row_e8m0(seed, s, r0 + i, out + i * 8);
}
