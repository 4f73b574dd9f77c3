// dsa3d_noalloc.hip -- dsa3d_backward_noalloc: the backward of dsa3d_backward
// with its scratch memory (the per-cell sample index of the deformable path,
// or the per-query statistics of the fixed window) taken from a fixed device
// array of this library instead of a caller's workspace, for callers that
// cannot allocate device memory.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the variable's name is only a stand-in for the device object, so the
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsa3d.h"
#include "dsa3d_internal.h"

namespace {

constexpr size_t kScratchBytes = DSA3D_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null: not looked up yet)

// The device address of the current device's copy of `scratch`, looked up at
// the first call on that device.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DSA3D_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DSA3D_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSA3D_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA3D_OK;
}

}  // namespace

extern "C" int dsa3d_backward_noalloc(const dsa3d_desc* d, const void* q, const void* k, const void* v,
                                      const void* offsets, const void* out, const float* lse, const void* dout,
                                      void* dq, void* dk, void* dv, void* doffsets, void* stream) {
    int rc = dsa3d_validate(d);
    if (rc != DSA3D_OK) return rc;
    const size_t need = offsets != nullptr ? dsa3d::bwd_workspace_bytes(*d, 1) : dsa3d::fixed_bwd_workspace_bytes(*d);
    if (need == 0) return DSA3D_ERR_UNSUPPORTED;  // sample or cell numbers of one head exceed 32 bits
    if (need > kScratchBytes) return DSA3D_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != DSA3D_OK) return rc;
    // Every kernel of the backward that reads scratch memory first clears it
    // or writes it itself (bucket counts and the large-bucket queue are zeroed
    // by a fill kernel at each pass), so what a previous call left there does
    // not matter.
    return dsa3d_backward(d, q, k, v, offsets, out, lse, dout, dq, dk, dv, doffsets, ws, kScratchBytes, stream);
}
