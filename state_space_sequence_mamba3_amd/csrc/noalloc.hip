// The allocation-free variant of the segmented scan: its workspace is a library-owned device
// array instead of caller memory, for callers that cannot allocate device memory.
//
// The array lives at file scope in device memory: every GPU the library runs on holds its own
// copy (MAMBA3_NOALLOC_SCRATCH_BYTES) from the moment the library's code is loaded there until the
// process ends. Host code never uses the array's name as an address (on the host it is only a
// stand-in for the device symbol); the first call on a device, with that device current, takes the
// array's device address with hipGetSymbolAddress and keeps it per device, and every later call
// passes that address to the kernels as their workspace. Nothing here allocates.
#include <mutex>

#include "m3_common.h"

static __device__ __align__(256) unsigned char scratch[MAMBA3_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once taken

// The scratch array's address on the current device (which must own `stream`).
mamba3_status scratch_address(void *stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAMBA3_EHIP;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return MAMBA3_EHIP;
        if (sdev != dev) return MAMBA3_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MAMBA3_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MAMBA3_OK;
}

}  // namespace

extern "C" {

mamba3_status mamba3_scan_segmented_noalloc(const mamba3_scan_segmented_args *args, void *stream) {
    if (!args) return MAMBA3_EINVAL;
    if (args->workspace || args->workspace_bytes) return MAMBA3_EINVAL;
    // the array's size first, then its address (no work is enqueued by either); the segmented
    // scan then checks every argument, the workspace included, before it launches anything
    mamba3_scan_segmented_args a = *args;
    if (mamba3_scan_segmented_workspace_size(&a) > (size_t)MAMBA3_NOALLOC_SCRATCH_BYTES) return MAMBA3_EWORKSPACE;
    void *ws = nullptr;
    mamba3_status st = scratch_address(stream, &ws);
    if (st != MAMBA3_OK) return st;
    a.workspace = ws;
    a.workspace_bytes = MAMBA3_NOALLOC_SCRATCH_BYTES;
    return mamba3_scan_segmented(&a, stream);
}

}  // extern "C"
