// dense.hip -- the dense-weight prefill variant: dequantise the packed
// buffer once into a dense [N, K] activation-dtype matrix, then run a plain
// library GEMM on it.
//
// This is the pages' second prefill strategy ("rdna_hybrid_w4a16" page,
// build 61746): `_cache_dequant_weight` builds a dense copy of each W4A16
// weight with `dequantize_w4a16` (four times the int4 bytes, kept at the
// expense of KV cache), and `_rdna_hybrid_w4a16_apply_impl` sends M >=
// MIN_DENSE_M to an unquantized GEMM on that copy. Here the copy is written
// by a HIP kernel from the gfx950 packed layout into caller-owned memory, and
// the GEMM is hipBLASLt (a plain library GEMM; the fused tiled kernel in
// mfma.hip is the path that reads the 4-bit weights directly).
#include <hipblaslt/hipblaslt.h>

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace w4a16 {
namespace {

// One 64-lane wave per 1 KB weight tile (nt, kt): lane l holds row
// n = 16*nt + l%16 and, in word s, the codes at k = 128*kt + 32*s + 8*(l/16)
// + i (i = 0..7). Each word becomes eight consecutive outputs
// RN((q - z) * s) (the rounding of `dequantize_w4a16`), one 16-byte store.
template <int DT, int QT>
__global__ __launch_bounds__(256) void dequant_kernel(const u32x4* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros, int64_t KTT, int64_t Kg,
                                                      int gshift, int one_group, int64_t tiles, int64_t N, int64_t K,
                                                      uint16_t* __restrict__ dense, int64_t ldw) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= tiles) return;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g4 = lane >> 4;
    const int64_t nt = t / KTT, kt = t - nt * KTT;
    const u32x4 w = __builtin_nontemporal_load(codes + t * 64 + lane);
    const int64_t n = nt * 16 + r;
    if (n >= N) return;  // padding of N
    uint32_t mask = 0x000F000Fu, magic = kMagic<DT>;
    asm volatile("" : "+v"(mask), "+v"(magic));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int64_t k0 = kt * 128 + 32 * s + 8 * g4;
        if (k0 >= K) continue;  // padding of K (K % 8 == 0: all eight or none)
        const int64_t g = one_group ? 0 : (k0 >> gshift);
        const int64_t idx = (nt * Kg + g) * 16 + r;
        const int z = QT ? (int)zeros[idx] : 8;
        const u32x4 out = Dequant<DT>::apply(w[s], Dequant<DT>::make(scales[idx], z), mask, magic);
        *reinterpret_cast<u32x4*>(dense + n * ldw + k0) = out;
    }
}

// hipBLASLt handles, one per device, created on first use and kept for the
// life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_blas_mu;
hipblasLtHandle_t g_blas[kMaxDevices] = {};

hipblasStatus_t blas_handle(hipblasLtHandle_t* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HIPBLAS_STATUS_INVALID_VALUE;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    if (g_blas[dev] == nullptr) {
        hipblasStatus_t st = hipblasLtCreate(&g_blas[dev]);
        if (st != HIPBLAS_STATUS_SUCCESS) {
            g_blas[dev] = nullptr;
            return st;
        }
    }
    *out = g_blas[dev];
    return HIPBLAS_STATUS_SUCCESS;
}

// Descriptors of one call, released on every return path.
struct BlasCall {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t lw = nullptr, la = nullptr, lc = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    ~BlasCall() {
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (lc) hipblasLtMatrixLayoutDestroy(lc);
        if (la) hipblasLtMatrixLayoutDestroy(la);
        if (lw) hipblasLtMatrixLayoutDestroy(lw);
        if (op) hipblasLtMatmulDescDestroy(op);
    }
};

}  // namespace

hipError_t launch_dequant(const void* packed, const Geometry& g, int dtype, void* dense, int64_t ldw,
                          hipStream_t stream) {
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    const u32x4* codes = reinterpret_cast<const u32x4*>(base);
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(base + g.scales_off);
    const uint8_t* zeros = g.qtype == 1 ? base + g.zeros_off : nullptr;
    const int64_t KTT = g.Kp / 128;
    const int64_t tiles = (g.Np / 16) * KTT;
    const dim3 grid((unsigned)((tiles + 3) / 4));
    const int one = g.Kg == 1;
    uint16_t* out = static_cast<uint16_t*>(dense);
    if (dtype == 0) {
        if (g.qtype) hipLaunchKernelGGL((dequant_kernel<0, 1>), grid, dim3(256), 0, stream, codes, scales, zeros, KTT, g.Kg, g.gshift, one, tiles, g.N, g.K, out, ldw);
        else hipLaunchKernelGGL((dequant_kernel<0, 0>), grid, dim3(256), 0, stream, codes, scales, zeros, KTT, g.Kg, g.gshift, one, tiles, g.N, g.K, out, ldw);
    } else {
        if (g.qtype) hipLaunchKernelGGL((dequant_kernel<1, 1>), grid, dim3(256), 0, stream, codes, scales, zeros, KTT, g.Kg, g.gshift, one, tiles, g.N, g.K, out, ldw);
        else hipLaunchKernelGGL((dequant_kernel<1, 0>), grid, dim3(256), 0, stream, codes, scales, zeros, KTT, g.Kg, g.gshift, one, tiles, g.N, g.K, out, ldw);
    }
    return hipGetLastError();
}

// C[M, N] = A[M, K] @ W[N, K]^T (+ bias) with hipBLASLt. In column-major
// terms C^T (N x M, ld ldc) = W' ^T (W' = K x N, ld ldw) times A' (K x M, ld
// lda): the "TN" product, fp32 accumulation, one rounding of D, bias added in
// the epilogue before that rounding.
int dense_gemm(const void* A, int64_t M, int64_t lda, const void* W, int64_t N, int64_t K, int64_t ldw, int dtype,
               const void* bias, void* C, int64_t ldc, void* workspace, size_t workspace_bytes, hipStream_t stream,
               const char** what) {
    const hipDataType t = dtype == 0 ? HIP_R_16F : HIP_R_16BF;
    hipblasLtHandle_t h;
    hipblasStatus_t st = blas_handle(&h);
    *what = "hipblasLtCreate";
    if (st != HIPBLAS_STATUS_SUCCESS) return (int)st;
    BlasCall c;
    *what = "hipBLASLt descriptor setup";
    if ((st = hipblasLtMatmulDescCreate(&c.op, HIPBLAS_COMPUTE_32F, HIP_R_32F)) != HIPBLAS_STATUS_SUCCESS) return (int)st;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    if ((st = hipblasLtMatmulDescSetAttribute(c.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta))) != HIPBLAS_STATUS_SUCCESS ||
        (st = hipblasLtMatmulDescSetAttribute(c.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb))) != HIPBLAS_STATUS_SUCCESS)
        return (int)st;
    if (bias != nullptr) {
        const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
        const int32_t bt = (int32_t)t;
        if ((st = hipblasLtMatmulDescSetAttribute(c.op, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi))) != HIPBLAS_STATUS_SUCCESS ||
            (st = hipblasLtMatmulDescSetAttribute(c.op, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias))) != HIPBLAS_STATUS_SUCCESS ||
            (st = hipblasLtMatmulDescSetAttribute(c.op, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof(bt))) != HIPBLAS_STATUS_SUCCESS)
            return (int)st;
    }
    if ((st = hipblasLtMatrixLayoutCreate(&c.lw, t, (uint64_t)K, (uint64_t)N, ldw)) != HIPBLAS_STATUS_SUCCESS ||
        (st = hipblasLtMatrixLayoutCreate(&c.la, t, (uint64_t)K, (uint64_t)M, lda)) != HIPBLAS_STATUS_SUCCESS ||
        (st = hipblasLtMatrixLayoutCreate(&c.lc, t, (uint64_t)N, (uint64_t)M, ldc)) != HIPBLAS_STATUS_SUCCESS)
        return (int)st;
    if ((st = hipblasLtMatmulPreferenceCreate(&c.pref)) != HIPBLAS_STATUS_SUCCESS) return (int)st;
    const uint64_t ws = workspace != nullptr ? (uint64_t)workspace_bytes : 0;
    if ((st = hipblasLtMatmulPreferenceSetAttribute(c.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws))) != HIPBLAS_STATUS_SUCCESS)
        return (int)st;
    hipblasLtMatmulHeuristicResult_t heur[1];
    int found = 0;
    *what = "hipblasLtMatmulAlgoGetHeuristic";
    st = hipblasLtMatmulAlgoGetHeuristic(h, c.op, c.lw, c.la, c.lc, c.lc, c.pref, 1, heur, &found);
    if (st != HIPBLAS_STATUS_SUCCESS) return (int)st;
    if (found < 1) return (int)HIPBLAS_STATUS_NOT_SUPPORTED;
    const float alpha = 1.0f, beta = 0.0f;
    *what = "hipblasLtMatmul";
    st = hipblasLtMatmul(h, c.op, &alpha, W, c.lw, A, c.la, &beta, C, c.lc, C, c.lc, &heur[0].algo,
                         ws ? workspace : nullptr, ws, stream);
    return (int)st;
}

}  // namespace w4a16
