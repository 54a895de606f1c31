// internal.h -- host-side plumbing shared by the C-ABI and the kernel files
// of libw4a16.so (not installed, not part of the ABI).
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace w4a16 {

// Geometry of one packed weight (see the layout in include/w4a16.h).
struct Geometry {
    int64_t N = 0, K = 0;
    int64_t Np = 0;       // N padded to a multiple of 16 (the packed layout's N)
    int64_t Kp = 0;       // K padded to a multiple of 128 (the packed layout's K)
    int32_t Ge = 0;       // effective group size
    int64_t Kg = 0;       // groups per row stored in the layout (Kp / Ge, or 1)
    int64_t Kg_ck = 0;    // groups per row of the checkpoint (K / Ge)
    int32_t gshift = 0;   // log2(Ge) when Kg > 1 (Ge is then a power of two)
    int32_t qtype = 0;    // 0 uint4b8, 1 uint4
    size_t codes_bytes = 0, scales_off = 0, zeros_off = 0, total_bytes = 0;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Skinny launch plan (M <= 16 rows per launch).
// Wide-weight variants (full_k; mode kRegisters / kResident / kStreamed):
// n_groups x ksplit workgroups of up to 8 waves; workgroup (g, c) owns at
// most nn_max n-tiles (g + i * n_groups) and K chunk c (all of K unless
// kRegisters splits it into chunks of kc_tiles k-tiles); wave w takes
// k-tiles [w * ktw, (w + 1) * ktw) of its chunk.
// Split-K variant (mode kSplitK): a workgroup is 4 waves; each wave owns NW
// consecutive n-tiles (16 rows each) and all KT k-tiles (128 k each) of the
// workgroup's K range, so the workgroup covers 4*NW n-tiles x KT k-tiles and
// ksplit workgroups split K.
struct SkinnyPlan {
    enum Mode { kSplitK = 0, kRegisters = 1, kResident = 2, kStreamed = 3 };
    Mode mode = kSplitK;
    bool full_k = false;  // mode != kSplitK: one of the wide-weight variants
    int nn_max = 1;       // full-K: n-tiles per workgroup, at most
    int ktw = 1;          // full-K: k-tiles per wave
    int kc_tiles = 0;     // kRegisters with ksplit > 1: k-tiles per K chunk
    int NW = 2;
    int KT = 4;
    int ksplit = 1;
    int64_t n_groups = 0;      // workgroups along N
    size_t partial_bytes = 0;  // fp32 partial sums in the workspace (16 rows)
    size_t counter_bytes = 0;  // arrival counters in the workspace
};

// Tiled MFMA launch plan.
struct MfmaPlan {
    int BM = 128;  // rows per workgroup
    int BN = 256;  // columns per workgroup
    bool splitk = false;       // medium-M tiles with K split over workgroups
    int64_t ksplit = 1;        // workgroups per tile along K
    int64_t spk = 0;           // K steps of 128 per split
    size_t partial_bytes = 0;  // fp32 partial tiles in the workspace
};

// Raises a kernel's dynamic-LDS limit (needed above 64 KB); cached per kernel
// (the template parameter is the kernel itself, so each has its own cache).
template <auto Kernel>
inline hipError_t allow_lds(size_t bytes) {
    static size_t granted = 64 * 1024;
    if (bytes <= granted) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) granted = bytes;
    return e;
}

// The full-K skinny variants (no split of K across workgroups) are used
// when N/16 reaches this many n-tiles, enough to occupy most of the CUs.
constexpr int64_t kFullKMinTiles = 192;
constexpr int64_t kCUs = 256;          // MI355X compute units
constexpr int64_t kMaxTilesPerWG = 16; // full-K: n-tiles per workgroup (LDS for the wave partials)

constexpr size_t kCounterRegionBytes = 64 * 1024;  // 16384 u32 arrival counters

// The static device scratch of w4a16_gemm_noalloc: the counter region and
// up to 8 MiB of split-K partial sums.
constexpr size_t kScratchBytes = kCounterRegionBytes + ((size_t)8 << 20);
// Device address of the current device's scratch (set up on the first call
// on that device: its counters cleared by a fill kernel on `stream`).
hipError_t noalloc_scratch(hipStream_t stream, void** out);

SkinnyPlan plan_skinny(int64_t M, const Geometry& g);
// workspace_cap: the most workspace the call may use (split-K partials and
// counters); the plan splits K no further than that allows.
MfmaPlan plan_mfma(int64_t M, const Geometry& g, size_t workspace_cap);
size_t mfma_workspace(const MfmaPlan& p);

// W4A8 launch plan: MI row blocks of 16 per wave, the grid, and the K split
// (partial results in the workspace when ksplit > 1).
// ring >= 0 selects the tiled ring kernel for large M instead (128 x 256
// tiles, no K split): 0 for one group per row, else the 64-k slices per group.
struct W4a8Plan {
    int MI = 1;
    int64_t blocks_n = 0, blocks_m = 0;
    int64_t kc = 0;
    int64_t ksplit = 1;
    size_t partial_bytes = 0;
    int ring = -1;
    int64_t m_tiles = 0, n_blocks = 0;
};
// qa16: the activation codes are 16-byte aligned with ldq % 16 == 0; c16: C
// is 16-byte aligned with ldc % 8 == 0 (the ring kernel's loads and stores
// need both; the workspace size assumes they do not hold).
W4a8Plan plan_w4a8(int64_t M, const Geometry& g, bool qa16 = false, int64_t ldq = 0, bool c16 = false);

// Launchers; each returns hipSuccess or the launch error. Shapes are already
// validated by the caller.
// Orientation of the checkpoint tensors read by launch_repack.
struct CheckpointLayout {
    bool weight_n_first = true;   // weight words [Nw][Kw] (else [Kw][Nw])
    bool weight_k_packed = true;  // eight consecutive k per word (else eight n)
    bool scale_n_first = true;    // scales [N][Kg] (else [Kg][N])
    bool zero_n_first = true;     // zero-point words [N/8][Kg] (else [Kg][N/8])
};

hipError_t launch_repack(const int32_t* wq, const uint16_t* ws, const int32_t* wzp, const CheckpointLayout& lay,
                         const Geometry& g, void* packed, hipStream_t stream);
hipError_t launch_unpack(const void* packed, const Geometry& g, uint8_t* codes, uint16_t* scale_bits, uint8_t* zeros,
                         hipStream_t stream);
hipError_t launch_skinny(const void* A, int64_t M, int64_t lda, const void* packed, const Geometry& g, int dtype,
                         const void* bias, void* C, int64_t ldc, const SkinnyPlan& p, void* workspace,
                         hipStream_t stream);
hipError_t launch_mfma(const void* A, int64_t M, int64_t lda, const void* packed, const Geometry& g, int dtype,
                       const void* bias, void* C, int64_t ldc, const MfmaPlan& p, void* workspace,
                       hipStream_t stream);
hipError_t launch_dequant(const void* packed, const Geometry& g, int dtype, void* dense, int64_t ldw,
                          hipStream_t stream);
hipError_t launch_a8_quant(const void* A, int64_t M, int64_t K, int64_t lda, int dtype, int8_t* qa, int64_t ldq,
                           float* xs, hipStream_t stream);
hipError_t launch_w4a8(const int8_t* qa, const float* xs, int64_t M, int64_t ldq, const void* packed, const Geometry& g,
                       int dtype, const void* bias, void* C, int64_t ldc, const W4a8Plan& p, void* workspace,
                       hipStream_t stream);
// hipBLASLt GEMM on a dense weight; returns a hipblasStatus_t value (0 on
// success) and names the failing step in *what.
int dense_gemm(const void* A, int64_t M, int64_t lda, const void* W, int64_t N, int64_t K, int64_t ldw, int dtype,
               const void* bias, void* C, int64_t ldc, void* workspace, size_t workspace_bytes, hipStream_t stream,
               const char** what);

}  // namespace w4a16
