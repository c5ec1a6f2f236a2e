// Seeded synthetic tables on the device (input data for tests and the
// benchmark; not part of the lookup).  Device implementation of the
// counter-based definition stated in engram_synth.h: splitmix64 output
// idx+1 for a counter idx built from (sub-table, row, byte group).
#include "engram_internal.h"
#include "engram_synth.h"

namespace engram {
namespace {

__device__ __forceinline__ uint64_t splitmix_at(uint64_t seed, uint64_t idx) {
    uint64_t z = seed + (idx + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Four codes from the four 16-bit fields of one generator output, packed
// little-endian (byte 4g+b of the row in bits 8b..8b+7).
__device__ __forceinline__ uint32_t codes4(uint64_t z) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t u = static_cast<uint32_t>(z >> (16 * b)) & 0xFFFFu;
        const uint32_t v = (u * 254u) >> 16;
        word |= (v < 127u ? v : v + 1u) << (8 * b);
    }
    return word;
}

// One thread per 16-byte chunk (4 generator outputs), grid-stride.
__global__ __launch_bounds__(256) void fill_codes_kernel(uint8_t* __restrict__ tab, uint64_t rows, uint64_t sub,
                                                         uint64_t seed) {
    const uint64_t n_chunks = rows * (kRowBytes / 16);
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t c = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
        const uint64_t r = c >> 4;
        const uint64_t g0 = (c & 15u) * 4u;
        const uint64_t base = (sub << 40) | (r << 6);
        uint4 w;
        w.x = codes4(splitmix_at(seed, base | (g0 + 0)));
        w.y = codes4(splitmix_at(seed, base | (g0 + 1)));
        w.z = codes4(splitmix_at(seed, base | (g0 + 2)));
        w.w = codes4(splitmix_at(seed, base | (g0 + 3)));
        reinterpret_cast<uint4*>(tab)[c] = w;
    }
}

__global__ __launch_bounds__(256) void fill_scales_kernel(float* __restrict__ sc, uint64_t rows, uint64_t sub,
                                                          uint64_t seed) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t r = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < rows; r += stride) {
        const uint64_t z = splitmix_at(seed, (uint64_t(1) << 63) | (sub << 40) | r);
        const uint32_t k = (1u << 22) + static_cast<uint32_t>(((z >> 40) * 3u) >> 2);
        sc[r] = static_cast<float>(k) * (1.0f / 8388608.0f);
    }
}

// Eight E8M0 exponents per row from the 8 bytes of one generator output.
__global__ __launch_bounds__(256) void fill_e8m0_kernel(uint2* __restrict__ sc, uint64_t rows, uint64_t sub,
                                                        uint64_t seed) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t r = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < rows; r += stride) {
        const uint64_t z = splitmix_at(seed, (uint64_t(3) << 62) | (sub << 40) | r);
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t u = static_cast<uint32_t>(z >> (8 * b)) & 0xFFu;
            w[b >> 2] |= (120u + ((u * 15u) >> 8)) << (8 * (b & 3));
        }
        sc[r] = make_uint2(w[0], w[1]);
    }
}

}  // namespace
}  // namespace engram

extern "C" int engram_synth_fill(uint8_t* table, float* scales, uint64_t rows, uint32_t sub_index, uint64_t seed,
                                 void* stream) {
    using namespace engram;
    if (rows == 0 || rows > (uint64_t(1) << 32)) return ENGRAM_ERANGE;
    if (sub_index >= static_cast<uint32_t>(kSub)) return ENGRAM_EINVAL;
    if (table && !aligned(table, 16)) return ENGRAM_EINVAL;
    if (scales && !aligned(scales, 4)) return ENGRAM_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // 256 CUs x 8 blocks of 256 threads, grid-stride over the table.
    const dim3 grid(2048), block(256);
    if (table) hipLaunchKernelGGL(fill_codes_kernel, grid, block, 0, s, table, rows, uint64_t(sub_index), seed);
    if (hipGetLastError() != hipSuccess) return ENGRAM_EHIP;
    if (scales) hipLaunchKernelGGL(fill_scales_kernel, grid, block, 0, s, scales, rows, uint64_t(sub_index), seed);
    if (hipGetLastError() != hipSuccess) return ENGRAM_EHIP;
    return ENGRAM_OK;
}

extern "C" int engram_synth_fill_e8m0(uint8_t* scales, uint64_t rows, uint32_t sub_index, uint64_t seed, void* stream) {
    using namespace engram;
    if (rows == 0 || rows > (uint64_t(1) << 32)) return ENGRAM_ERANGE;
    if (sub_index >= static_cast<uint32_t>(kSub) || !scales || !aligned(scales, 8)) return ENGRAM_EINVAL;
    hipLaunchKernelGGL(fill_e8m0_kernel, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<uint2*>(scales), rows, uint64_t(sub_index), seed);
    return hipGetLastError() == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}
