// exchange.h -- cross-workgroup exchange of split-K partial sums, shared by
// the skinny and tiled kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace w4a16 {

// Cross-workgroup exchange of split-K partial sums. Every access carries the
// sc1 cache policy (write-through to, or read from, the agent-wide coherence
// point): stores are agent-scope relaxed atomic stores of 64 bits, which the
// compiler lowers to sc1 stores; loads are sc1 loads in inline assembly.
__device__ __forceinline__ void store_coherent(float* p, const floatx4& v) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, __builtin_bit_cast(uint64_t, __builtin_shufflevector(v, v, 0, 1)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, __builtin_bit_cast(uint64_t, __builtin_shufflevector(v, v, 2, 3)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
// Four coherent 16-byte loads and the wait for them, in one asm statement so
// that no compiler-inserted instruction can read the destination registers
// while the loads are in flight (the compiler does not track asm loads).
__device__ __forceinline__ void load_coherent4(const float* p0, const float* p1, const float* p2, const float* p3,
                                               floatx4& v0, floatx4& v1, floatx4& v2, floatx4& v3) {
    asm volatile(
        "global_load_dwordx4 %0, %4, off sc1\n\t"
        "global_load_dwordx4 %1, %5, off sc1\n\t"
        "global_load_dwordx4 %2, %6, off sc1\n\t"
        "global_load_dwordx4 %3, %7, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
        : "memory");
}
// One coherent 16-byte read as two agent-scope atomic 64-bit loads (sc1),
// which the compiler tracks like ordinary loads: many can be in flight.
__device__ __forceinline__ floatx4 load_coherent(const float* p) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float2 a = __builtin_bit_cast(float2, lo), b = __builtin_bit_cast(float2, hi);
    return floatx4{a.x, a.y, b.x, b.y};
}
// Waits until every vector memory access this wave issued has completed
// (write-through stores: reached the coherence point).
__device__ __forceinline__ void wait_vector_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace w4a16
