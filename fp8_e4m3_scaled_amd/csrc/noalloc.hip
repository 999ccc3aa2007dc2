// Device scratch of paged_attn_decode_noalloc, the decode entry point for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the split-K partials
// go into a fixed array that the library's code object carries, so a call
// needs no workspace.  Each device the library runs on holds its own copy
// until the process ends.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

static __device__ __align__(256) uint8_t scratch[kvf8::kNoAllocScratchBytes];

namespace kvf8 {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

}  // namespace

// The device address of this device's copy of `scratch`.  Looked up once per
// device with that device current (the array's host-side name is only a
// stand-in for it); later calls return the kept address.
hipError_t noalloc_scratch(int device, void **ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[device]) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != device) {
            const hipError_t e2 = hipSetDevice(prev);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[device] = p;
    }
    *ptr = g_scratch[device];
    return hipSuccess;
}

}  // namespace kvf8
