// noalloc.hip — the fixed device workspace of paged_attn_decode_fused_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation) get the single-launch decode step with its split partials and
// merge counters in one library-owned array per GPU.  The array is part of the library's
// code object: the runtime places it in each GPU's memory when the library is first used on
// that GPU, zero-filled, and it stays there until the process ends.
//
// Host code never uses the array's name as a device address (on the host it names a
// host-side stand-in): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that pointer is handed to
// kernels.
#include <atomic>

#include "common.h"

namespace pa {

namespace {

// The first 1 MiB holds the merge counters and nothing else (8192 of them, one per 128-byte
// line): they start at zero (the array is zero-filled) and every call leaves them at zero.
// The rest holds a call's partials, up to 15 MiB: e.g. 16 sequences x 64 query heads x 16
// splits at head_dim 128 (8.5 MB).
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    static std::atomic<void*> cached[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = cached[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        cached[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace pa
