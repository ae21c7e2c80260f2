// w8a8_linear for callers that cannot allocate: the INT8 path's workspace
// (the quantized activation and its block scales) lives in a fixed device
// array of this file instead of caller memory.
//
// `scratch` is a file-scope __device__ array: every GPU the library is loaded
// on holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side stand-in, so the device address is taken
// with hipGetSymbolAddress, once per device with that device current, and
// kept; only that address is ever handed to kernels.  Nothing in the array
// needs to start at zero (the activation quantizer writes every code and
// scale the GEMM reads), and calls on one GPU share it, so calls that overlap
// in time on one GPU race on its contents.
#include <mutex>

#include "w8a8.h"
#include "w8a8_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[W8A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up on first use with the
// device current (the caller's current device is restored afterwards).
hipError_t scratch_address(int device, void **out) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        g_scratch[device] = p;
    }
    *out = g_scratch[device];
    return hipSuccess;
}

}  // namespace

extern "C" int w8a8_linear_noalloc(const void *x, int x_dtype, int64_t M, int64_t K, int64_t N, const void *w_bf16,
                                   const int8_t *qw, const float *sw, const void *bias_bf16, void *y_bf16,
                                   hipStream_t stream, int *path_out) {
    if (!x || !w_bf16 || !y_bf16 || M <= 0 || K <= 0 || N <= 0) return W8A8_ERR_INVALID_ARG;
    int device = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &device) : hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= kMaxDevices)) e = hipErrorInvalidDevice;
    void *ws = nullptr;
    if (e == hipSuccess) e = scratch_address(device, &ws);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return w8a8::hip_failure(e);
    }
    // a call whose INT8 path needs more than the array gets W8A8_ERR_UNSUPPORTED
    // (the guard decides the path first, so a call that falls back runs)
    return w8a8::guarded_linear(x, x_dtype, M, K, N, w_bf16, qw, sw, bias_bf16, y_bf16, ws,
                                W8A8_NOALLOC_SCRATCH_BYTES, stream, path_out, W8A8_ERR_UNSUPPORTED);
}
