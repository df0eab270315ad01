// Built-in split-K scratch for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): one file-scope device array per GPU, of kNoAllocScratchBytes,
// held until the process ends.
//
// On the host the array's name is only a stand-in for the device copy, so
// host code never passes it to a kernel or a copy: the device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and kept, and every later use goes through that pointer.  The first
// kCounterBytes hold the tiled kernel's arrival counters, which must start at
// zero: they are cleared by a fill kernel on the caller's stream at set-up,
// and every call leaves them at zero.  The rest is scratch (partial tiles).
// Calls that use the array on one GPU share it, so they must not overlap in
// time on that GPU.
#include <mutex>

#include "internal.h"

namespace q4 {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void* ptr = nullptr;
    bool ready = false;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ void clear_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch& d = g_dev[dev];
    if (!d.ready) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e == hipSuccess) {
            constexpr int kWords = (int)(kWsCounterBytes / 4);
            hipLaunchKernelGGL(clear_words, dim3(kWords / 256), dim3(256), 0, s, static_cast<uint32_t*>(p), kWords);
            e = hipGetLastError();
        }
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        d.ptr = p;
        // A clear recorded into a graph under capture only runs when the
        // graph does: set-up then repeats on the next call (the array is
        // also zero when the code object loads, and every call leaves the
        // counters at zero, so a repeated clear changes nothing).
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (s && hipStreamIsCapturing(s, &cs) != hipSuccess) cs = hipStreamCaptureStatusActive;
        d.ready = cs == hipStreamCaptureStatusNone;
    }
    *out = d.ptr;
    return hipSuccess;
}

}  // namespace q4
