// ceiling.hip -- a plain streaming-read kernel, built into its own library
// (libw4a16_ceiling.so) for the benchmark only: the HBM read rate one launch
// of a given size reaches on this GPU, the practical ceiling of the
// weight-streaming skinny kernels. It is not part of the W4A16 path.
//
// Workgroup b of the grid reads the 16-byte chunks [b*per, (b+1)*per) of the
// buffer (per = ceil(chunks / grid)), each thread U nontemporal 16-byte loads
// at a time, and folds them with XOR; a store that no real data triggers keeps
// the loads from being removed.
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ void stream_read_kernel(const u32x4* src, uint64_t chunks, uint32_t* sink) {
    const uint64_t per = (chunks + gridDim.x - 1) / gridDim.x;
    const uint64_t beg = (uint64_t)blockIdx.x * per;
    const uint64_t end = beg + per < chunks ? beg + per : chunks;
    uint32_t x = 0;
    for (uint64_t i = beg + threadIdx.x; i < end; i += (uint64_t)blockDim.x * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = i + (uint64_t)u * blockDim.x;
            v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from the device buffer `src` with `grid`
// workgroups of `threads` threads (a multiple of 64, at most 1024), `unroll`
// in {1, 2, 4, 8, 16} loads in flight per thread; `sink` holds `grid` words
// (written only in the unlikely case the XOR of the data hits a constant).
// Returns 0, or -1 for bad arguments (nothing launched), or the HIP error.
int w4a16_ceiling_read(const void* src, size_t bytes, uint32_t* sink, int grid, int threads, int unroll,
                       hipStream_t stream) {
    if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 || grid <= 0 || threads <= 0 ||
        threads > 1024 || threads % 64 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
        return -1;
    const uint64_t chunks = bytes / 16;
    const auto* s = static_cast<const u32x4*>(src);
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(threads), 0, stream, s, chunks, sink); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(threads), 0, stream, s, chunks, sink); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(threads), 0, stream, s, chunks, sink); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(threads), 0, stream, s, chunks, sink); break;
        case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(threads), 0, stream, s, chunks, sink); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
