// gdr2_fwd_noalloc: the inference forward with its workspace in a fixed device array of
// the library instead of a caller's buffer, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). See include/gdr2.h for the contract.
//
// The array `scratch` (GDR2_NOALLOC_SCRATCH_BYTES) is a file-scope __device__ variable:
// every GPU the library runs on holds its own copy, at its own address, until the
// process ends. In host code its name is only a host-side stand-in, so the device
// address is looked up once per device, with that device current, by
// hipGetSymbolAddress, and that address (never the name) is what the kernels receive.
// The forward writes every workspace array before it reads it, so nothing needs to be
// cleared between calls.
#include "../../include/gdr2.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr2_kernels.hpp"

namespace {

static __device__ __align__(256) char scratch[GDR2_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
void* g_scratch[MAX_DEVICES];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch`, looked up on the first call on that device.
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int gdr2_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* b,
                                const void* w, const float* h0, void* o, float* ht, int B, int T, int H, int dk,
                                int dv, int chunk, int dtype, void* stream) {
    size_t need = 0;
    const int st = gdr2::fwd_validate(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, &need);
    if (st != GDR2_OK) return st;
    if (need > GDR2_NOALLOC_SCRATCH_BYTES) return GDR2_ERR_SCRATCH;
    void* ws = nullptr;  // a call without tokens needs no workspace
    if (need > 0 && scratch_address(&ws) != hipSuccess) return GDR2_ERR_HIP;
    return gdr2::fwd_with_workspace(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, ws,
                                    GDR2_NOALLOC_SCRATCH_BYTES, stream);
}
