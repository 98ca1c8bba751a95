// ssm_noalloc.hip - the library's static device scratch: the workspace of
// ssm_scan_fwd_noalloc, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its
// own copy, at its own address, from the first use of the library's code object on that
// GPU until the process ends. In host code its name is only a host-side stand-in, so the
// device address is looked up once per device (with that device current) and kept; every
// host use of the scratch goes through that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssm_internal.h"

namespace ssm {

namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(hipStream_t stream, void** out) {
    *out = nullptr;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    // the stream's device (a stream of another device than the current one gets that
    // device's copy of the array); the null stream runs on the current device
    int dev = cur;
    if (stream) {
        hipDevice_t sd = -1;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return e;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace ssm
