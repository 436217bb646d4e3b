// gs_noalloc.hip -- DeformConv on the channels-last matrix-core kernel with
// its scratch space in a file-scope device array, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array `scratch` is a device symbol: each GPU the library runs on holds
// its own copy, at its own address, until the process ends.  On the first
// call on a device (that device current), the host looks that address up with
// hipGetSymbolAddress and keeps it per device; every later use of the array
// from the host goes through that pointer, never through the symbol's name
// (in host code the name is only a stand-in for the symbol).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gsample.h"

namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Address of this device's `scratch` (looked up once per device), or NULL
// with the HIP error in *err.
void *scratch_address(int *err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = GS_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *err = GS_ERR_HIP;
            return nullptr;
        }
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

int gs_deform_conv_noalloc(const void *X, int dtype, const int64_t *x_shape, int x_rank,
                           const void *W, const int64_t *w_shape, const void *offset,
                           const void *B, const void *mask, const int64_t *strides,
                           const int64_t *pads, const int64_t *dilations, int group,
                           int offset_group, void *Y, void *stream) {
    int64_t need = 0;
    const int rc = gs_deform_conv_workspace_size(dtype, x_shape, x_rank, w_shape, strides, pads,
                                                 dilations, group, offset_group, &need);
    if (rc != GS_OK) return rc;
    if (need > kScratchBytes) return GS_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (need > 0) {
        int err = GS_OK;
        ws = scratch_address(&err);
        if (!ws) return err;
    }
    return gs_deform_conv(X, dtype, x_shape, x_rank, W, w_shape, offset, B, mask, strides, pads,
                          dilations, group, offset_group, Y, ws, need, stream);
}

}  // extern "C"
