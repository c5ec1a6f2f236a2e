// engram_dedup_noalloc: engram_dedup with its workspace in a fixed,
// statically allocated device array instead of a caller buffer, for callers
// that cannot allocate device memory.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy from module load until the process ends.  Host
// code never passes the variable's name to a kernel (in host code that name
// is a host-side stand-in, not a device address): the device address comes
// from hipGetSymbolAddress, taken once per device, on the first call with
// that device current, and kept.  The kernels are those of engram_dedup; the
// workspace keeps a small state between calls that needs no clearing.
#include <mutex>

#include "engram_internal.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[ENGRAM_DEDUP_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (set up on first use).
hipError_t scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int engram_dedup_noalloc(engram_plan_t p, const int32_t* ids, const int32_t* history, int64_t n_seq,
                                    int64_t seq_len, int32_t* perm, int32_t* offsets, int32_t* n_unique,
                                    void* stream) {
    using namespace engram;
    if (!p) return ENGRAM_EINVAL;
    if (n_seq < 0 || seq_len < 0) return ENGRAM_EINVAL;
    if (n_seq != 0 && seq_len > kMaxTokens / n_seq) return ENGRAM_ERANGE;
    const int64_t n_tok = n_seq * seq_len;
    if (n_tok > kMaxDedupTokens) return ENGRAM_ERANGE;
    if (!offsets || !n_unique || !aligned(offsets, 4) || !aligned(n_unique, 4)) return ENGRAM_EINVAL;
    if (n_tok > 0) {
        if (!ids || !perm || !aligned(ids, 4) || !aligned(perm, 4)) return ENGRAM_EINVAL;
        if (history && !aligned(history, 4)) return ENGRAM_EINVAL;
    }
    if (dedup_workspace_bytes(uint32_t(n_tok), p->vocab_size) > ENGRAM_DEDUP_SCRATCH_BYTES) return ENGRAM_EWORKSPACE;
    void* ws = nullptr;
    if (scratch_for_current_device(&ws) != hipSuccess) return ENGRAM_EHIP;
    const hipError_t e = launch_dedup(ids, history, uint32_t(n_tok), uint32_t(seq_len), p->vocab_size, perm, offsets,
                                      n_unique, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP;
}
