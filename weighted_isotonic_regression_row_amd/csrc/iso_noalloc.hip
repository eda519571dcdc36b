// iso_fit_noalloc: iso_fit with its workspace in a static device array of the
// library, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// entry point itself allocates nothing: the array is part of the library's
// code object, so each GPU the library runs on holds one copy of it from the
// library's first launch there until the process ends.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/iso.h"
#include "iso_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)ISO_NOALLOC_SCRATCH_BYTES;

// The workspace of every iso_fit_noalloc call on a device.  In host code this
// name is a stand-in, not a device address: only the pointer that
// hipGetSymbolAddress returns for the current device may be passed on.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[iso::kMaxDevices] = {};

// Device address of `scratch` on device `dev`, which is current; looked up
// on the first call on that device and kept.  nullptr if the lookup fails.
void* scratch_on(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int iso_fit_noalloc(const void* y, const void* w, int64_t rows, int64_t n, int increasing, double y_min,
                               double y_max, int dtype, void* fit, iso_blocks* blocks_out, void* blocks_mem,
                               void* stream) {
    if (rows < 0 || n < 0 || (dtype != ISO_F32 && dtype != ISO_F64)) return ISO_EINVAL;
    if (rows == 0 || n == 0)  // nothing is queued: iso_fit fills the handle and returns
        return iso_fit(y, w, rows, n, increasing, y_min, y_max, dtype, fit, blocks_out, blocks_mem, nullptr, 0,
                       stream);
    const size_t need = iso_workspace_bytes(rows, n, dtype);
    if (need == 0) return ISO_EINVAL;
    if (need > kScratchBytes) return ISO_ETOOBIG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ISO_EHIP;
    if (dev < 0 || dev >= iso::kMaxDevices) return ISO_EINVAL;
    void* ws = scratch_on(dev);
    if (ws == nullptr) return ISO_EHIP;
    // the same checks, kernels and launches as iso_fit, on this device's scratch
    return iso_fit(y, w, rows, n, increasing, y_min, y_max, dtype, fit, blocks_out, blocks_mem, ws, kScratchBytes,
                   stream);
}
