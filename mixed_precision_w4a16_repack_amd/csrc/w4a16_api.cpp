// w4a16_api.cpp -- the C ABI of libw4a16.so (declared in include/w4a16.h):
// argument validation, geometry of the packed buffer, the dispatch on M and
// error reporting. No kernel code lives here.
//
// Validation follows the eligibility rules and launcher asserts of the pages
// (`can_implement` on the "rdna_hybrid_w4a16" pages and the MI300
// "triton_w4a16.py" page: supported quant types, fp16/bf16 activations,
// group sizes {-1, 32, 64, 128, 256}, K % group_size; the launcher asserts of
// `triton_w4a16_skinny_fmt_gemm`: unit column stride, N % 8 with zero points),
// plus the N % 16 and K % 128 alignment the gfx950 layout needs. Every message
// names the rule that failed.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"
#include "w4a16.h"

static_assert(W4A16_NOALLOC_MAX_WORKSPACE_BYTES == w4a16::kScratchBytes, "header and library agree on the scratch");

namespace w4a16 {
namespace {

thread_local char g_err[512] = "";

w4a16_status fail(w4a16_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = '\0'; }

w4a16_status hip_fail(const char* what, hipError_t e) {
    return fail(W4A16_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Bounds that keep every size and offset computation of the calls within
// 64-bit arithmetic: N and K (the packed sizes are products of the two) and
// row strides in elements.
constexpr int64_t kMaxDim = (int64_t)1 << 32;
constexpr int64_t kMaxStride = (int64_t)1 << 40;

w4a16_status check_stride(const char* name, int64_t ld) {
    if (ld > kMaxStride)
        return fail(W4A16_ERR_UNSUPPORTED, "%s=%lld is too large: row strides must be at most 2^40 elements", name,
                    (long long)ld);
    return W4A16_OK;
}

int ilog2(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

// Shape and type rules shared by every call that takes a weight.
w4a16_status make_geometry(int64_t N, int64_t K, int32_t group_size, int32_t qtype, Geometry* g) {
    if (N <= 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "N=%lld and K=%lld must be positive", (long long)N, (long long)K);
    if (N > kMaxDim || K > kMaxDim)
        return fail(W4A16_ERR_UNSUPPORTED, "N=%lld and K=%lld must be at most 2^32", (long long)N, (long long)K);
    if (qtype != W4A16_UINT4B8 && qtype != W4A16_UINT4)
        return fail(W4A16_ERR_INVALID_ARG, "qtype=%d is not a w4a16_qtype (0 uint4b8, 1 uint4)", qtype);
    if (N % 8 != 0) return fail(W4A16_ERR_UNSUPPORTED, "N=%lld must be divisible by 8", (long long)N);
    if (K % 8 != 0) return fail(W4A16_ERR_UNSUPPORTED, "K=%lld must be divisible by 8", (long long)K);
    const int64_t Ge = group_size == -1 ? K : group_size;
    const bool listed = group_size == -1 || group_size == 32 || group_size == 64 || group_size == 128 ||
                        group_size == 256 || (int64_t)group_size == K;
    if (!listed)
        return fail(W4A16_ERR_UNSUPPORTED, "group_size=%d not supported; supported: -1, 32, 64, 128, 256 or K=%lld",
                    group_size, (long long)K);
    if (K % Ge != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "K=%lld must be divisible by group_size=%d", (long long)K, group_size);
    g->N = N;
    g->Np = (N + 15) / 16 * 16;
    g->K = K;
    g->Kp = (K + 127) / 128 * 128;
    g->Ge = (int32_t)Ge;
    g->Kg_ck = K / Ge;
    if (g->Kg_ck > 1 && !is_pow2(Ge))
        return fail(W4A16_ERR_UNSUPPORTED, "group_size=%d must be a power of two when K/group_size > 1", group_size);
    // The layout stores the groups of the padded K (zero scales past K / Ge).
    g->Kg = g->Kg_ck == 1 ? 1 : g->Kp / Ge;
    g->gshift = g->Kg > 1 ? ilog2(Ge) : 0;
    g->qtype = qtype;
    g->codes_bytes = (size_t)g->Np * (size_t)g->Kp / 2;
    g->scales_off = align256(g->codes_bytes);
    size_t end = g->scales_off + (size_t)g->Np * (size_t)g->Kg * 2;
    if (qtype == W4A16_UINT4) {
        g->zeros_off = align256(end);
        end = g->zeros_off + (size_t)g->Np * (size_t)g->Kg;
    } else {
        g->zeros_off = 0;
    }
    g->total_bytes = align256(end);
    return W4A16_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t resolve_path(int64_t M, int32_t path, int32_t skinny_max_m) {
    const int64_t t = skinny_max_m <= 0 ? 16 : skinny_max_m;
    if (path == W4A16_PATH_SKINNY || path == W4A16_PATH_MFMA) return path;
    return M <= t ? W4A16_PATH_SKINNY : W4A16_PATH_MFMA;
}

size_t skinny_workspace(const SkinnyPlan& p) {
    return p.ksplit > 1 ? kCounterRegionBytes + p.partial_bytes : 0;
}

w4a16_status repack_impl(const int32_t* weight, const void* weight_scale, const int32_t* weight_zero_point,
                         const CheckpointLayout& lay, int64_t N, int64_t K, int32_t group_size, int32_t qtype,
                         void* packed, size_t packed_bytes, hipStream_t stream) {
    Geometry g;
    w4a16_status st = make_geometry(N, K, group_size, qtype, &g);
    if (st != W4A16_OK) return st;
    if (weight == nullptr) return fail(W4A16_ERR_INVALID_ARG, "weight_packed is NULL");
    if (weight_scale == nullptr) return fail(W4A16_ERR_INVALID_ARG, "weight_scale is NULL");
    if (packed == nullptr) return fail(W4A16_ERR_INVALID_ARG, "packed is NULL");
    if ((reinterpret_cast<uintptr_t>(weight) & 3u) || (reinterpret_cast<uintptr_t>(weight_scale) & 1u) ||
        (reinterpret_cast<uintptr_t>(weight_zero_point) & 3u))
        return fail(W4A16_ERR_INVALID_ARG, "checkpoint tensors must be aligned to their element size");
    if (reinterpret_cast<uintptr_t>(packed) & 255u) return fail(W4A16_ERR_INVALID_ARG, "packed must be 256-byte aligned");
    if (packed_bytes < g.total_bytes)
        return fail(W4A16_ERR_SIZE, "packed_bytes=%zu is smaller than the %zu bytes the layout needs", packed_bytes,
                    g.total_bytes);
    hipError_t e = launch_repack(weight, static_cast<const uint16_t*>(weight_scale),
                                 qtype == W4A16_UINT4 ? weight_zero_point : nullptr, lay, g, packed, stream);
    if (e != hipSuccess) return hip_fail("repack launch", e);
    return W4A16_OK;
}

}  // namespace
}  // namespace w4a16

using namespace w4a16;

extern "C" {

int32_t w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_last_error(void) { return g_err; }

size_t w4a16_workspace_counter_bytes(void) { return kCounterRegionBytes; }

w4a16_status w4a16_packed_size(int64_t N, int64_t K, int32_t group_size, int32_t qtype, size_t* out_bytes) {
    clear_error();
    if (out_bytes == nullptr) return fail(W4A16_ERR_INVALID_ARG, "out_bytes is NULL");
    Geometry g;
    w4a16_status st = make_geometry(N, K, group_size, qtype, &g);
    if (st != W4A16_OK) return st;
    *out_bytes = g.total_bytes;
    return W4A16_OK;
}


w4a16_status w4a16_repack(const int32_t* weight_packed, const void* weight_scale, const int32_t* weight_zero_point,
                          int64_t N, int64_t K, int32_t group_size, int32_t qtype, void* packed, size_t packed_bytes,
                          hipStream_t stream) {
    clear_error();
    return repack_impl(weight_packed, weight_scale, weight_zero_point, CheckpointLayout{}, N, K, group_size, qtype,
                       packed, packed_bytes, stream);
}

w4a16_status w4a16_repack_layout(const int32_t* weight, int32_t weight_output_dim, int32_t weight_packed_dim,
                                 const void* weight_scale, int32_t scale_output_dim, const int32_t* weight_zero_point,
                                 int32_t zero_output_dim, int64_t N, int64_t K, int32_t group_size, int32_t qtype,
                                 void* packed, size_t packed_bytes, hipStream_t stream) {
    clear_error();
    const int32_t dims[4] = {weight_output_dim, weight_packed_dim, scale_output_dim, zero_output_dim};
    const char* names[4] = {"weight_output_dim", "weight_packed_dim", "scale_output_dim", "zero_output_dim"};
    for (int i = 0; i < 4; ++i)
        if (dims[i] != 0 && dims[i] != 1) return fail(W4A16_ERR_INVALID_ARG, "%s=%d must be 0 or 1", names[i], dims[i]);
    CheckpointLayout lay;
    lay.weight_n_first = weight_output_dim == 0;
    lay.weight_k_packed = weight_packed_dim != weight_output_dim;
    lay.scale_n_first = scale_output_dim == 0;
    lay.zero_n_first = zero_output_dim == 0;
    return repack_impl(weight, weight_scale, weight_zero_point, lay, N, K, group_size, qtype, packed, packed_bytes,
                       stream);
}

w4a16_status w4a16_unpack(const void* packed, int64_t N, int64_t K, int32_t group_size, int32_t qtype,
                          uint8_t* codes, uint16_t* scale_bits, uint8_t* zeros, hipStream_t stream) {
    clear_error();
    Geometry g;
    w4a16_status st = make_geometry(N, K, group_size, qtype, &g);
    if (st != W4A16_OK) return st;
    if (packed == nullptr) return fail(W4A16_ERR_INVALID_ARG, "packed is NULL");
    if (reinterpret_cast<uintptr_t>(packed) & 255u) return fail(W4A16_ERR_INVALID_ARG, "packed must be 256-byte aligned");
    if (reinterpret_cast<uintptr_t>(scale_bits) & 1u) return fail(W4A16_ERR_INVALID_ARG, "scale_bits must be 2-byte aligned");
    hipError_t e = launch_unpack(packed, g, codes, scale_bits, zeros, stream);
    if (e != hipSuccess) return hip_fail("unpack launch", e);
    return W4A16_OK;
}

int32_t w4a16_select_path(int64_t M, int32_t path, int32_t skinny_max_m) {
    clear_error();
    if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_MFMA)
        return fail(W4A16_ERR_INVALID_ARG, "path=%d is not a w4a16_path (0 auto, 1 skinny, 2 mfma)", path);
    return resolve_path(M, path, skinny_max_m);
}

w4a16_status w4a16_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t path,
                                  int32_t skinny_max_m, size_t* out_bytes) {
    clear_error();
    if (out_bytes == nullptr) return fail(W4A16_ERR_INVALID_ARG, "out_bytes is NULL");
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M=%lld must be >= 0", (long long)M);
    if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_MFMA)
        return fail(W4A16_ERR_INVALID_ARG, "path=%d is not a w4a16_path (0 auto, 1 skinny, 2 mfma)", path);
    Geometry g;
    // The workspace does not depend on qtype; uint4b8 has the simpler rules.
    w4a16_status st = make_geometry(N, K, group_size, W4A16_UINT4B8, &g);
    if (st != W4A16_OK) return st;
    *out_bytes = 0;
    if (M > 0 && resolve_path(M, path, skinny_max_m) == W4A16_PATH_MFMA) {
        *out_bytes = mfma_workspace(plan_mfma(M, g, (size_t)-1));
        return W4A16_OK;
    }
    if (M > 0 && resolve_path(M, path, skinny_max_m) == W4A16_PATH_SKINNY) {
        const SkinnyPlan p = plan_skinny(M < 16 ? M : 16, g);
        if (p.n_groups * (int64_t)sizeof(uint32_t) > (int64_t)kCounterRegionBytes)
            return fail(W4A16_ERR_UNSUPPORTED, "N=%lld needs more split-K counters than the workspace holds",
                        (long long)N);
        *out_bytes = skinny_workspace(p);
    }
    return W4A16_OK;
}

}  // extern "C"

namespace w4a16 {
namespace {

// w4a16_gemm and w4a16_gemm_noalloc. With from_scratch, the workspace is the
// library's static device scratch, fetched only once every argument has
// passed validation and the call is known to need it.
w4a16_status gemm_impl(const void* A, int64_t M, int64_t lda, const void* packed, int64_t N, int64_t K,
                       int32_t group_size, int32_t qtype, int32_t dtype, const void* bias, void* C, int64_t ldc,
                       int32_t path, int32_t skinny_max_m, void* workspace, size_t workspace_bytes,
                       bool from_scratch, hipStream_t stream) {
    Geometry g;
    w4a16_status st = make_geometry(N, K, group_size, qtype, &g);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16)
        return fail(W4A16_ERR_INVALID_ARG, "dtype=%d is not a w4a16_dtype (0 fp16, 1 bf16)", dtype);
    if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_MFMA)
        return fail(W4A16_ERR_INVALID_ARG, "path=%d is not a w4a16_path (0 auto, 1 skinny, 2 mfma)", path);
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return W4A16_OK;
    if (A == nullptr || packed == nullptr || C == nullptr)
        return fail(W4A16_ERR_INVALID_ARG, "A, packed and C must not be NULL");
    if (lda < K) return fail(W4A16_ERR_INVALID_ARG, "lda=%lld must be >= K=%lld", (long long)lda, (long long)K);
    if (ldc < N) return fail(W4A16_ERR_INVALID_ARG, "ldc=%lld must be >= N=%lld", (long long)ldc, (long long)N);
    if ((st = check_stride("lda", lda)) != W4A16_OK || (st = check_stride("ldc", ldc)) != W4A16_OK) return st;
    if (!aligned16(A) || lda % 8 != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "A must be 16-byte aligned with lda %% 8 == 0 (lda=%lld)", (long long)lda);
    if (reinterpret_cast<uintptr_t>(packed) & 255u) return fail(W4A16_ERR_INVALID_ARG, "packed must be 256-byte aligned");
    if ((reinterpret_cast<uintptr_t>(C) & 1u) || (reinterpret_cast<uintptr_t>(bias) & 1u))
        return fail(W4A16_ERR_INVALID_ARG, "C and bias must be 2-byte aligned");

    const int32_t which = resolve_path(M, path, skinny_max_m);
    if (which == W4A16_PATH_MFMA) {
        // The tiled kernels address one workgroup's tile (at most 128 rows
        // of A, 16 n-tiles = 128*K bytes of codes) with 32-bit byte offsets;
        // lda >= K makes this bound cover both.
        if ((128 * lda + K) * 2 >= (int64_t)1 << 31)
            return fail(W4A16_ERR_UNSUPPORTED, "lda=%lld is too large for the tiled path: need (128*lda + K)*2 < 2^31",
                        (long long)lda);
        // Medium M splits K over workgroups as far as the workspace holds the
        // partial tiles (none given: no split); the static scratch for the
        // allocation-free entry.
        size_t cap = from_scratch ? kScratchBytes : (workspace != nullptr ? workspace_bytes : 0);
        const MfmaPlan p = plan_mfma(M, g, cap);
        const size_t need = mfma_workspace(p);
        if (need > 0 && from_scratch) {
            hipError_t e = noalloc_scratch(stream, &workspace);
            if (e != hipSuccess) return hip_fail("static scratch set-up", e);
        }
        if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u))
            return fail(W4A16_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        hipError_t e = launch_mfma(A, M, lda, packed, g, dtype, bias, C, ldc, p, need > 0 ? workspace : nullptr,
                                   stream);
        if (e != hipSuccess) return hip_fail("mfma kernel launch", e);
        return W4A16_OK;
    }

    // The skinny kernels address the activation rows of one launch (at most
    // 16) with 32-bit byte offsets.
    const int64_t rows = M < 16 ? M : 16;
    if (((rows - 1) * lda + K) * 2 > (int64_t)INT32_MAX)
        return fail(W4A16_ERR_UNSUPPORTED, "lda=%lld is too large for the skinny path: need ((M-1)*lda + K)*2 < 2^31",
                    (long long)lda);
    const SkinnyPlan p = plan_skinny(rows, g);
    if (p.n_groups * (int64_t)sizeof(uint32_t) > (int64_t)kCounterRegionBytes)
        return fail(W4A16_ERR_UNSUPPORTED, "N=%lld needs more split-K counters than the workspace holds", (long long)N);
    const size_t need = skinny_workspace(p);
    if (need > 0 && from_scratch) {
        if (need > kScratchBytes)
            return fail(W4A16_ERR_SIZE,
                        "this call needs %zu bytes of split-K workspace, more than the %zu bytes of the static "
                        "scratch; use w4a16_gemm with a caller workspace",
                        need, kScratchBytes);
        hipError_t e = noalloc_scratch(stream, &workspace);
        if (e != hipSuccess) return hip_fail("static scratch set-up", e);
        workspace_bytes = kScratchBytes;
    }
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(W4A16_ERR_SIZE, "workspace of %zu bytes is smaller than the %zu bytes this call needs",
                        workspace == nullptr ? (size_t)0 : workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(W4A16_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }
    // M > 16 on the forced skinny path: 16-row slices, one launch each.
    const uint16_t* a16 = static_cast<const uint16_t*>(A);
    uint16_t* c16 = static_cast<uint16_t*>(C);
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int64_t mm = M - m0 < 16 ? M - m0 : 16;
        hipError_t e = launch_skinny(a16 + m0 * lda, mm, lda, packed, g, dtype, bias, c16 + m0 * ldc, ldc, p,
                                     need > 0 ? workspace : nullptr, stream);
        if (e != hipSuccess) return hip_fail("skinny kernel launch", e);
    }
    return W4A16_OK;
}

}  // namespace
}  // namespace w4a16

extern "C" {

w4a16_status w4a16_gemm(const void* A, int64_t M, int64_t lda, const void* packed, int64_t N, int64_t K,
                        int32_t group_size, int32_t qtype, int32_t dtype, const void* bias, void* C, int64_t ldc,
                        int32_t path, int32_t skinny_max_m, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    clear_error();
    return gemm_impl(A, M, lda, packed, N, K, group_size, qtype, dtype, bias, C, ldc, path, skinny_max_m, workspace,
                     workspace_bytes, false, stream);
}

w4a16_status w4a16_gemm_noalloc(const void* A, int64_t M, int64_t lda, const void* packed, int64_t N, int64_t K,
                                int32_t group_size, int32_t qtype, int32_t dtype, const void* bias, void* C,
                                int64_t ldc, int32_t path, int32_t skinny_max_m, hipStream_t stream) {
    clear_error();
    return gemm_impl(A, M, lda, packed, N, K, group_size, qtype, dtype, bias, C, ldc, path, skinny_max_m, nullptr, 0,
                     true, stream);
}


w4a16_status w4a8_quantize(const void* A, int64_t M, int64_t K, int64_t lda, int32_t dtype, int8_t* qa, int64_t ldq,
                           float* xs, hipStream_t stream) {
    clear_error();
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M=%lld must be >= 0", (long long)M);
    if (K <= 0) return fail(W4A16_ERR_INVALID_ARG, "K=%lld must be positive", (long long)K);
    if (dtype != W4A16_F16 && dtype != W4A16_BF16)
        return fail(W4A16_ERR_INVALID_ARG, "dtype=%d is not a w4a16_dtype (0 fp16, 1 bf16)", dtype);
    if (K % 8 != 0) return fail(W4A16_ERR_UNSUPPORTED, "K=%lld must be divisible by 8", (long long)K);
    if (lda < K) return fail(W4A16_ERR_INVALID_ARG, "lda=%lld must be >= K=%lld", (long long)lda, (long long)K);
    if (ldq < K) return fail(W4A16_ERR_INVALID_ARG, "ldq=%lld must be >= K=%lld", (long long)ldq, (long long)K);
    if (K > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "K=%lld must be at most 2^32", (long long)K);
    w4a16_status st = check_stride("lda", lda);
    if (st != W4A16_OK || (st = check_stride("ldq", ldq)) != W4A16_OK) return st;
    if (M >= ((int64_t)1 << 31)) return fail(W4A16_ERR_UNSUPPORTED, "M=%lld is too large (one workgroup per row)", (long long)M);
    if (M == 0) return W4A16_OK;
    if (A == nullptr || qa == nullptr || xs == nullptr) return fail(W4A16_ERR_INVALID_ARG, "A, qa and xs must not be NULL");
    if (!aligned16(A) || lda % 8 != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "A must be 16-byte aligned with lda %% 8 == 0 (lda=%lld)", (long long)lda);
    if ((reinterpret_cast<uintptr_t>(qa) & 7u) || ldq % 8 != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "qa must be 8-byte aligned with ldq %% 8 == 0 (ldq=%lld)", (long long)ldq);
    if (reinterpret_cast<uintptr_t>(xs) & 3u) return fail(W4A16_ERR_INVALID_ARG, "xs must be 4-byte aligned");
    hipError_t e = launch_a8_quant(A, M, K, lda, dtype, qa, ldq, xs, stream);
    if (e != hipSuccess) return hip_fail("quantize kernel launch", e);
    return W4A16_OK;
}

w4a16_status w4a8_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size, size_t* out_bytes) {
    clear_error();
    if (out_bytes == nullptr) return fail(W4A16_ERR_INVALID_ARG, "out_bytes is NULL");
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M=%lld must be >= 0", (long long)M);
    Geometry g;
    w4a16_status st = make_geometry(N, K, group_size, W4A16_UINT4B8, &g);
    if (st != W4A16_OK) return st;
    // The larger of the two kernels' needs: the call picks the ring kernel
    // only for 16-byte aligned activation and output rows.
    const size_t reg = M > 0 ? plan_w4a8(M, g).partial_bytes : 0;
    const size_t ring = M > 0 ? plan_w4a8(M, g, true, K, true).partial_bytes : 0;
    *out_bytes = reg > ring ? reg : ring;
    return W4A16_OK;
}

w4a16_status w4a8_gemm(const int8_t* qa, const float* xs, int64_t M, int64_t ldq, const void* packed, int64_t N,
                       int64_t K, int32_t group_size, int32_t dtype, const void* bias, void* C, int64_t ldc,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    clear_error();
    Geometry g;
    // The weights are symmetric (uint4b8), as the pages' W4A8 kernel requires.
    w4a16_status st = make_geometry(N, K, group_size, W4A16_UINT4B8, &g);
    if (st != W4A16_OK) return st;
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M=%lld must be >= 0", (long long)M);
    if (dtype != W4A16_F16 && dtype != W4A16_BF16)
        return fail(W4A16_ERR_INVALID_ARG, "dtype=%d is not a w4a16_dtype (0 fp16, 1 bf16)", dtype);
    if (ldq < K) return fail(W4A16_ERR_INVALID_ARG, "ldq=%lld must be >= K=%lld", (long long)ldq, (long long)K);
    if (ldc < N) return fail(W4A16_ERR_INVALID_ARG, "ldc=%lld must be >= N=%lld", (long long)ldc, (long long)N);
    if ((st = check_stride("ldq", ldq)) != W4A16_OK || (st = check_stride("ldc", ldc)) != W4A16_OK) return st;
    if (M == 0) return W4A16_OK;
    if (qa == nullptr || xs == nullptr || packed == nullptr || C == nullptr)
        return fail(W4A16_ERR_INVALID_ARG, "qa, xs, packed and C must not be NULL");
    if (reinterpret_cast<uintptr_t>(packed) & 255u) return fail(W4A16_ERR_INVALID_ARG, "packed must be 256-byte aligned");
    if ((reinterpret_cast<uintptr_t>(qa) & 7u) || ldq % 8 != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "qa must be 8-byte aligned with ldq %% 8 == 0 (ldq=%lld)", (long long)ldq);
    if ((reinterpret_cast<uintptr_t>(xs) & 3u) || (reinterpret_cast<uintptr_t>(C) & 1u) ||
        (reinterpret_cast<uintptr_t>(bias) & 1u))
        return fail(W4A16_ERR_INVALID_ARG, "xs must be 4-byte and C, bias 2-byte aligned");
    const bool qa16 = (reinterpret_cast<uintptr_t>(qa) & 15u) == 0 && ldq % 16 == 0;
    const bool c16 = (reinterpret_cast<uintptr_t>(C) & 15u) == 0 && ldc % 8 == 0;
    const W4a8Plan p = plan_w4a8(M, g, qa16, ldq, c16);
    if (p.blocks_m > 65535 || p.ksplit > 65535)
        return fail(W4A16_ERR_UNSUPPORTED, "M=%lld is too large for one W4A8 launch", (long long)M);
    if (p.partial_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < p.partial_bytes)
            return fail(W4A16_ERR_SIZE, "a workspace of %zu bytes is smaller than the %zu bytes this call needs",
                        workspace == nullptr ? (size_t)0 : workspace_bytes, p.partial_bytes);
        if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(W4A16_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    }
    hipError_t e = launch_w4a8(qa, xs, M, ldq, packed, g, dtype, bias, C, ldc, p, workspace, stream);
    if (e != hipSuccess) return hip_fail("w4a8 kernel launch", e);
    return W4A16_OK;
}

w4a16_status w4a16_dequant(const void* packed, int64_t N, int64_t K, int32_t group_size, int32_t qtype, int32_t dtype,
                           void* dense, int64_t ldw, hipStream_t stream) {
    clear_error();
    Geometry g;
    w4a16_status st = make_geometry(N, K, group_size, qtype, &g);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16)
        return fail(W4A16_ERR_INVALID_ARG, "dtype=%d is not a w4a16_dtype (0 fp16, 1 bf16)", dtype);
    if (packed == nullptr || dense == nullptr) return fail(W4A16_ERR_INVALID_ARG, "packed and dense must not be NULL");
    if (reinterpret_cast<uintptr_t>(packed) & 255u) return fail(W4A16_ERR_INVALID_ARG, "packed must be 256-byte aligned");
    if (ldw < K) return fail(W4A16_ERR_INVALID_ARG, "ldw=%lld must be >= K=%lld", (long long)ldw, (long long)K);
    if ((st = check_stride("ldw", ldw)) != W4A16_OK) return st;
    if (!aligned16(dense) || ldw % 8 != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "dense must be 16-byte aligned with ldw %% 8 == 0 (ldw=%lld)", (long long)ldw);
    hipError_t e = launch_dequant(packed, g, dtype, dense, ldw, stream);
    if (e != hipSuccess) return hip_fail("dequant kernel launch", e);
    return W4A16_OK;
}

w4a16_status w4a16_gemm_dense(const void* A, int64_t M, int64_t lda, const void* dense, int64_t N, int64_t K,
                              int64_t ldw, int32_t dtype, const void* bias, void* C, int64_t ldc, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    clear_error();
    if (N <= 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "N=%lld and K=%lld must be positive", (long long)N, (long long)K);
    if (dtype != W4A16_F16 && dtype != W4A16_BF16)
        return fail(W4A16_ERR_INVALID_ARG, "dtype=%d is not a w4a16_dtype (0 fp16, 1 bf16)", dtype);
    if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return W4A16_OK;
    if (A == nullptr || dense == nullptr || C == nullptr)
        return fail(W4A16_ERR_INVALID_ARG, "A, dense and C must not be NULL");
    if (lda < K) return fail(W4A16_ERR_INVALID_ARG, "lda=%lld must be >= K=%lld", (long long)lda, (long long)K);
    if (ldw < K) return fail(W4A16_ERR_INVALID_ARG, "ldw=%lld must be >= K=%lld", (long long)ldw, (long long)K);
    if (ldc < N) return fail(W4A16_ERR_INVALID_ARG, "ldc=%lld must be >= N=%lld", (long long)ldc, (long long)N);
    w4a16_status st = check_stride("lda", lda);
    if (st != W4A16_OK || (st = check_stride("ldw", ldw)) != W4A16_OK || (st = check_stride("ldc", ldc)) != W4A16_OK)
        return st;
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(dense) | reinterpret_cast<uintptr_t>(C) |
         reinterpret_cast<uintptr_t>(bias)) & 1u)
        return fail(W4A16_ERR_INVALID_ARG, "A, dense, C and bias must be 2-byte aligned");
    const char* what = "";
    const int bst = dense_gemm(A, M, lda, dense, N, K, ldw, dtype, bias, C, ldc, workspace, workspace_bytes, stream, &what);
    if (bst != 0) return fail(W4A16_ERR_HIP, "%s failed: hipblasStatus %d", what, bst);
    return W4A16_OK;
}

}  // extern "C"
