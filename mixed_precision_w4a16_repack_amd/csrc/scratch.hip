// scratch.hip -- the device scratch of w4a16_gemm_noalloc: the skinny
// kernels' split-K arrival counters and partial sums in a file-scope device
// array, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array (in the code
// object loaded on that device) until the process ends. Its host-side name
// is not a device address: the address of the current device's copy comes
// from hipGetSymbolAddress, once per device, and only that pointer is ever
// passed to a kernel.
#include <mutex>

#include "internal.h"

namespace w4a16 {
namespace {

// Counters first (kCounterRegionBytes), then the partial sums.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void clear_words_kernel(uint32_t* p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        // The counters must start at zero (every split-K launch leaves them
        // at zero again). A fill kernel, not a memset, so that a first call
        // under graph capture records an ordinary kernel node.
        constexpr int words = (int)(kCounterRegionBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t*>(p), words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace w4a16
