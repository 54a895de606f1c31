// lds_stage.h -- staging operand tiles from HBM/L2 straight into LDS, for the
// tiled GEMM kernels (mfma.hip, w4a8.hip).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace w4a16 {

// 16 bytes per lane from buffer `rs` (lane offset voff + scalar offset soff)
// straight into LDS at dst + 16 * lane (dst wave-uniform). dst keeps its
// __shared__ array identity so that the compiler knows which LDS object the
// load writes (reads of the other buffer then need not wait for it).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, unsigned char* dst, uint32_t voff, uint32_t soff) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// Waits until at most N vector memory operations of this wave are
// outstanding (also the direct-to-LDS loads, which no register tracks).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the staged kernels. __syncthreads() carries a
// workgroup-scope fence, which the compiler lowers to a wait for every
// outstanding vector-memory operation, including the direct-to-LDS loads of
// stages still in flight, and so serialises the pipeline. Here each wave
// first waits for exactly the stage the next step reads (wait_vmcnt), and its
// LDS reads of the current stage are complete (lgkmcnt(0)) before any wave
// may overwrite that stage. The memory clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace w4a16
