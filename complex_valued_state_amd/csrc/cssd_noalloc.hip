// cssd_forward_noalloc: cssd_forward with its workspace in a fixed device array
// of this library (declared in include/cssd.h), for callers that cannot
// allocate device memory.
//
// `scratch` below is a file-scope device array.  In host code its name is only a
// host-side stand-in: its device address is fetched once per device with
// hipGetSymbolAddress, with that device current, and only that address is ever
// handed to kernels.  Each GPU holds its own copy of the array for the life of
// the process; every call on one GPU uses that GPU's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cssd.h"

static __device__ __align__(256) unsigned char scratch[CSSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchAddrs {
    std::mutex mu;
    void* ptr[kMaxDevices] = {};
};

ScratchAddrs& addrs() {
    static ScratchAddrs a;
    return a;
}

// Device address of `scratch` on device `dev`, looked up on the first call for
// that device (with that device current) and kept.
hipError_t scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchAddrs& a = addrs();
    std::lock_guard<std::mutex> g(a.mu);
    if (a.ptr[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        a.ptr[dev] = p;
    }
    *out = a.ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int cssd_forward_noalloc(int64_t batch, int64_t seqlen, int64_t nheads,
                                    int64_t headdim, int64_t dstate, int64_t chunk,
                                    int32_t in_dtype, const void* x_re, const void* x_im,
                                    const void* B_re, const void* B_im, const void* C_re,
                                    const void* C_im, const float* dt, const float* A_re,
                                    const float* A_im, const float* Dskip, const float* h0_re,
                                    const float* h0_im, float* y_re, float* y_im, float* hT_re,
                                    float* hT_im, void* stream) {
    size_t need = 0;
    const int st = cssd_forward_workspace_size(batch, seqlen, nheads, headdim, dstate, chunk, &need);
    if (st != CSSD_OK) return st;
    if (need > (size_t)CSSD_NOALLOC_SCRATCH_BYTES) return CSSD_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (need > 0) {
        // the array of the device the stream belongs to (the current device for NULL)
        int dev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
            return CSSD_ERR_HIP;
        if (scratch_on(dev, &ws) != hipSuccess) return CSSD_ERR_HIP;
    }
    // the forward writes every workspace region it later reads (the cumsums, the
    // decays and every chunk's carry-in state) before reading it, so what an
    // earlier call left in the array needs no clearing
    return cssd_forward(batch, seqlen, nheads, headdim, dstate, chunk, in_dtype, x_re, x_im, B_re,
                        B_im, C_re, C_im, dt, A_re, A_im, Dskip, h0_re, h0_im, y_re, y_im, hT_re,
                        hT_im, ws, need > 0 ? (size_t)CSSD_NOALLOC_SCRATCH_BYTES : 0, stream);
}
