// noalloc.hip -- scan_fwd_noalloc: the forward scan for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// Its scratch is the file-scope array `scratch` below, a fixed
// LRSCAN_NOALLOC_SCRATCH_BYTES per device, held by every device the library
// runs on until the process ends.  Each device has its own copy at its own
// address: the first call on a device takes that address with
// hipGetSymbolAddress (that device current) and keeps it; host code passes
// the address, never the array's name, to kernels.  Every call initialises
// the part of the array it uses with a kernel (no memset node, nothing
// carried over from the previous call), so calls on one device must not
// overlap: two at once would race on the same array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lrscan.h"

namespace lrscan {
int fwd_on_fixed_scratch(const void* a, const void* b, void* out, float* last, int64_t B,
                         int64_t T, int64_t D, int dtype, void* stream, const lrscan_opts* opts,
                         size_t cap, int (*acquire)(void**));
}

namespace {
constexpr size_t kScratchBytes = LRSCAN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mutex;
void* g_device_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up on the first call on it.
int device_scratch(void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LRSCAN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_device_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LRSCAN_ERR_HIP;
        g_device_ptr[dev] = p;
    }
    *ptr = g_device_ptr[dev];
    return LRSCAN_OK;
}

}  // namespace

extern "C" LRSCAN_API int scan_fwd_noalloc(const void* a, const void* b, void* out, float* last,
                                           int64_t B, int64_t T, int64_t D, int dtype,
                                           void* stream, const lrscan_opts* opts) {
    return lrscan::fwd_on_fixed_scratch(a, b, out, last, B, T, D, dtype, stream, opts,
                                        kScratchBytes, device_scratch);
}
