/*
 * w4a16.h -- C ABI of libw4a16.so, a fused W4A16 linear layer for AMD
 * Instinct MI355X (gfx950):
 *
 *     C[M, N] = A[M, K] @ dequant(W)^T (+ bias),   dequant(W)[n, k] = (q - z) * s
 *
 * W is N x K 4-bit codes q with one fp16/bf16 scale s per row and group of G
 * consecutive k, and a zero z that is the constant 8 (symmetric "uint4b8") or
 * a stored 4-bit zero point (asymmetric "uint4"). A, scales, bias and C share
 * one activation dtype (fp16 or bf16); products accumulate in fp32 and C is
 * rounded once (round to nearest even).
 *
 * Where the operations come from (page title, section):
 *  - the checkpoint layout the repack accepts: "triton_w4a16.py" (Triton-based
 *    W4A16 GEMM for ROCm MI300), module docstring -- weight_packed [N, K/8]
 *    int32 with GPTQ sequential packing (eight codes per word, code i at bits
 *    4i), weight_scale [N, K/G], weight_zero_point [N/8, K/G] int32 packed
 *    along N (row n at bits 4*(n%8) of word n/8, as the
 *    `_triton_w4a16_skinny_fmt_kernel` docstring of the "rdna_hybrid_w4a16"
 *    page, build 58181, states).
 *  - dequantisation w = (q - z) * s with z = 8 for uint4b8: the
 *    `triton_w4a16_gemm_kernel` docstring (MI300 page) and
 *    `dequantize_w4a16` ("rdna_hybrid_w4a16", build 61746).
 *  - group_size -1 meaning K, and uint4b8 ignoring any zero-point tensor:
 *    `apply_weights` (MI300 page).
 *  - one weight buffer serving a small-M ("skinny") kernel and a tiled
 *    prefill kernel, with a dispatch on M: the module docstring and
 *    `_rdna_hybrid_w4a16_apply_impl` ("rdna_hybrid_w4a16", both builds).
 *  - the load-time repack into a kernel-native layout: `process_weights_after_
 *    loading` on both pages (here a GPU kernel into the layout defined below).
 *  - the bias added to the output: `apply_weights` (both pages); here it is
 *    fused in fp32 before the single rounding of C.
 *
 * Conventions shared by every call:
 *  - Pointers are device pointers unless a parameter says "host". All device
 *    memory is owned by the caller; the library never allocates, frees or
 *    synchronises (calls are asynchronous on `stream`, NULL = default stream).
 *    The one exception is w4a16_gemm_dense (see there).
 *  - Every call validates its arguments before any HIP call. A failure
 *    returns a negative w4a16_status and sets a message readable with
 *    w4a16_last_error() on the same thread (e.g. "K=4100 must be divisible by
 *    group_size=128"). Nothing is launched after a validation failure. The
 *    library never aborts and no exception crosses the ABI.
 *  - qtype is a w4a16_qtype, dtype a w4a16_dtype, path a w4a16_path (passed
 *    as int32_t so the ABI does not depend on enum sizes).
 *  - Shapes: N % 8 == 0 (zero points, and AWQ words, pack eight values along
 *    N), K % 8 == 0 (the checkpoint packs eight codes per word); group_size
 *    in {-1, 32, 64, 128, 256} or group_size == K, with K % group_size == 0.
 *    Other shapes return W4A16_ERR_UNSUPPORTED. Neither N need be a multiple
 *    of 16 nor K of 128 (shards of a layer often are not): the packed layout
 *    pads both, the kernels read the activation columns past K as zeros
 *    (never touching them) and store no column of C past N, so A needs only
 *    lda >= K, C ldc >= N and bias N elements.
 *
 * Device layout of the packed buffer (written by w4a16_repack, read by
 * w4a16_gemm; Ge = K if group_size == -1 else group_size; Np = N rounded up
 * to a multiple of 16; Kp = K rounded up to a multiple of 128; Kg = 1 if
 * K == Ge, else Kp / Ge stored groups, of which the first K / Ge are the
 * checkpoint's; align256(x) rounds x up to a multiple of 256; words are
 * little-endian):
 *  - Codes at byte 0, Np*Kp/2 bytes: 1024-byte tiles; tile (nt, kt), nt in
 *    [0, Np/16), kt in [0, Kp/128), starts at ((nt * (Kp/128)) + kt) * 1024.
 *    32-bit word 4*l + s of a tile (l in [0, 64), s in [0, 4)) holds the codes
 *    of row n = 16*nt + l%16 at k = 128*kt + 32*s + 8*(l/16) + i, i = 0..7,
 *    code i in bits [4*(i/2) + 16*(i%2), +4); codes at n >= N or k >= K are
 *    0. One 16-byte load per lane of a 64-wide wavefront moves a whole tile,
 *    and word s of lane l is the B operand of a 16x16x32 fp16/bf16 MFMA over
 *    k in [128*kt + 32*s, +32).
 *  - Scales at S0 = align256(Np*Kp/2): Np*Kg raw 2-byte fp16/bf16 values;
 *    element (nt, g, r) = weight_scale[16*nt + r][g] at
 *    S0 + ((nt*Kg + g)*16 + r)*2, and 0 for rows 16*nt + r >= N and for the
 *    groups g >= K / Ge.
 *  - Zeros (uint4 only) at Z0 = align256(S0 + Np*Kg*2): Np*Kg bytes, element
 *    (nt, g, r) = zero of (row 16*nt + r, group g) at Z0 + (nt*Kg + g)*16 + r,
 *    0 for rows >= N and g >= K / Ge; all 0 when the checkpoint has no zero
 *    points.
 *  - Total size = align256(end of the last region) = w4a16_packed_size().
 *  When N % 16 == 0 and K % 128 == 0, Np = N, Kp = K and Kg = K / Ge.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 1

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum, stride < width */
    W4A16_ERR_UNSUPPORTED = -2, /* a shape or group size the device layout cannot hold */
    W4A16_ERR_SIZE = -3,        /* a caller buffer (packed, workspace) is too small */
    W4A16_ERR_HIP = -4          /* a HIP call or kernel launch failed */
} w4a16_status;

typedef enum { W4A16_UINT4B8 = 0, W4A16_UINT4 = 1 } w4a16_qtype;
typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1 } w4a16_dtype;
typedef enum { W4A16_PATH_AUTO = 0, W4A16_PATH_SKINNY = 1, W4A16_PATH_MFMA = 2 } w4a16_path;

/* The ABI version this library implements (W4A16_ABI_VERSION). */
int32_t w4a16_abi_version(void);

/* The message of the last failed call on this thread ("" if none). The pointer
 * stays valid until the next library call on this thread. */
const char *w4a16_last_error(void);

/* Bytes of the packed buffer for an N x K weight (layout above). out_bytes is
 * a host pointer. Fails like w4a16_repack on an unsupported shape. */
w4a16_status w4a16_packed_size(int64_t N, int64_t K, int32_t group_size, int32_t qtype, size_t *out_bytes);

/* One-time repack of a checkpoint into the packed buffer (bit-exact and
 * deterministic; checkpoint layout as above):
 *   weight_packed     [N, K/8] int32, row-major, contiguous
 *   weight_scale      [N, Kg] fp16/bf16 bits (copied as raw 16-bit values)
 *   weight_zero_point [N/8, Kg] int32, or NULL; read only for uint4 (NULL
 *                     means every zero is 0); ignored for uint4b8
 *   packed            output, packed_bytes >= w4a16_packed_size(...)
 * The inputs must not overlap the output. W4A16_ERR_SIZE if packed_bytes is
 * too small. */
w4a16_status w4a16_repack(const int32_t *weight_packed, const void *weight_scale, const int32_t *weight_zero_point,
                          int64_t N, int64_t K, int32_t group_size, int32_t qtype, void *packed, size_t packed_bytes,
                          hipStream_t stream);

/* w4a16_repack for checkpoints in the other orientations the MI300 Triton
 * W4A16 page accepts ("triton_w4a16.py": process_weights_after_loading, and
 * the zero-point handling of its MI300 kernel section). Each packed tensor is
 * described as the page describes a parameter: output_dim is its dimension
 * that runs over the N output features, packed_dim the dimension whose eight
 * consecutive entries share one int32 word (entry 8j + i of that dimension in
 * bits [4i, 4i+4) of word j). All tensors row-major and contiguous:
 *   weight             output_dim 0, packed_dim 1: [N, K/8]  (compressed-tensors)
 *                      output_dim 0, packed_dim 0: [N/8, K]
 *                      output_dim 1, packed_dim 1: [K, N/8]  (AWQ)
 *                      output_dim 1, packed_dim 0: [K/8, N]  (AutoGPTQ)
 *   weight_scale       scale_output_dim 0: [N, Kg]; 1: [Kg, N] (raw 16-bit values)
 *   weight_zero_point  eight zeros per word along N; zero_output_dim 0:
 *                      [N/8, Kg]; 1: [Kg, N/8] (AutoGPTQ); NULL and qtype
 *                      rules as for w4a16_repack
 * The packed buffer is byte-identical to what w4a16_repack writes for the
 * same codes, scales and zeros; with dims (0, 1, 0, 0) this is w4a16_repack.
 * Nibble orders other than the sequential one above (for instance an
 * interleaved order some AWQ exporters use) must be undone by the caller.
 * W4A16_ERR_INVALID_ARG if a dim is not 0 or 1; otherwise fails like
 * w4a16_repack. */
w4a16_status w4a16_repack_layout(const int32_t *weight, int32_t weight_output_dim, int32_t weight_packed_dim,
                                 const void *weight_scale, int32_t scale_output_dim,
                                 const int32_t *weight_zero_point, int32_t zero_output_dim, int64_t N, int64_t K,
                                 int32_t group_size, int32_t qtype, void *packed, size_t packed_bytes,
                                 hipStream_t stream);

/* Test support: the inverse of w4a16_repack. Reads the packed buffer and
 * writes codes [N, K] (one code per byte, row-major), scale_bits [N, Kg]
 * (raw 16-bit values) and, for uint4, zeros [N, Kg] bytes. Any output may be
 * NULL to skip it (zeros is ignored for uint4b8). */
w4a16_status w4a16_unpack(const void *packed, int64_t N, int64_t K, int32_t group_size, int32_t qtype,
                          uint8_t *codes, uint16_t *scale_bits, uint8_t *zeros, hipStream_t stream);

/* Bytes of device workspace w4a16_gemm needs for these arguments (0 if none).
 * out_bytes is a host pointer. The workspace starts with a region of
 * w4a16_workspace_counter_bytes() bytes of arrival counters, followed by
 * split-K partial sums: of the skinny kernels (M <= 16: narrow weights, and
 * K > 4096 unless M <= 4 with one fold block per 128 k; these also use the
 * counters) and of the tiled kernel for medium M (17 rows up to where its
 * 128 x 256 tiles fill the CUs on their own; partial sums only). The size
 * for M = 16 serves every M <= 16. Its first
 * w4a16_workspace_counter_bytes() bytes must be
 * zero before it is first used; every completed w4a16_gemm call leaves them
 * zero again, so a workspace can be reused for any shape. Calls that share a
 * workspace must be ordered (same stream); overlapping calls race. */
w4a16_status w4a16_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t path,
                                  int32_t skinny_max_m, size_t *out_bytes);

/* Size of the counter region at the start of every workspace (a constant). */
size_t w4a16_workspace_counter_bytes(void);

/* Which kernel w4a16_gemm runs for M rows: W4A16_PATH_SKINNY when
 * path == AUTO and M <= skinny_max_m (skinny_max_m <= 0 means 16), else the
 * forced path; W4A16_PATH_MFMA otherwise. Returns a negative status for a
 * bad path. */
int32_t w4a16_select_path(int64_t M, int32_t path, int32_t skinny_max_m);

/* C[M, N] = A[M, K] @ dequant(W)^T (+ bias):
 *   A       [M, lda] act dtype, row-major, lda >= K (unit column stride)
 *   packed  the buffer written by w4a16_repack for the same N, K,
 *           group_size and qtype (the call cannot check this)
 *   bias    [N] act dtype, or NULL
 *   C       [M, ldc] act dtype, ldc >= N; must not overlap A, packed or bias
 *   path    AUTO dispatches on M (see w4a16_select_path); SKINNY forces the
 *           small-M kernel (M > 16 runs it over 16-row slices); MFMA forces
 *           the tiled kernel
 *   workspace, workspace_bytes  device workspace, >= w4a16_workspace_size();
 *           may be NULL when that size is 0. The skinny path returns
 *           W4A16_ERR_SIZE for a smaller one; the tiled path splits K no
 *           further than the given workspace holds (NULL: no split), so it
 *           only runs slower
 * M == 0 is a no-op. The result does not depend on the workspace contents or
 * on earlier calls (no float atomics: the order of every sum is fixed).
 * The skinny kernel addresses the (at most 16) rows of one launch with 32-bit
 * byte offsets: it returns W4A16_ERR_UNSUPPORTED when
 * ((min(M, 16) - 1) * lda + K) * 2 >= 2^31. The tiled kernel does the same
 * per workgroup tile (A and the weight may be of any size): it returns
 * W4A16_ERR_UNSUPPORTED when (128 * lda + K) * 2 >= 2^31. */
w4a16_status w4a16_gemm(const void *A, int64_t M, int64_t lda, const void *packed, int64_t N, int64_t K,
                        int32_t group_size, int32_t qtype, int32_t dtype, const void *bias, void *C, int64_t ldc,
                        int32_t path, int32_t skinny_max_m, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* w4a16_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, result and errors as w4a16_gemm, without the workspace:
 * the split-K partial sums and arrival counters live in a static device
 * array of the library, W4A16_NOALLOC_MAX_WORKSPACE_BYTES bytes (64 KiB of
 * counters + 8 MiB of partial sums) per GPU, held until the process ends. A
 * skinny call that needs more workspace than that (a larger
 * w4a16_workspace_size()) returns W4A16_ERR_SIZE without launching anything;
 * use w4a16_gemm with a caller workspace for it. The tiled path splits K no
 * further than the array holds. The call allocates nothing:
 * no hipMalloc, hipFree or allocating library routine. On the first call
 * that needs the array on a device (that device current), the library looks
 * up its address and clears its counters with a small kernel on `stream`;
 * every later call on that device uses the same array, whose counters every
 * completed call leaves at zero. All calls on one GPU share the array: calls
 * that overlap in time on one GPU (different streams, or threads without
 * ordering) race and must be serialised by the caller. */
#define W4A16_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)(64 * 1024) + ((size_t)8 << 20))
w4a16_status w4a16_gemm_noalloc(const void *A, int64_t M, int64_t lda, const void *packed, int64_t N, int64_t K,
                                int32_t group_size, int32_t qtype, int32_t dtype, const void *bias, void *C,
                                int64_t ldc, int32_t path, int32_t skinny_max_m, hipStream_t stream);

/* Dense dequantisation of the packed buffer, the first half of the pages'
 * second prefill strategy ("rdna_hybrid_w4a16" page, build 61746:
 * `dequantize_w4a16` and `_cache_dequant_weight`, which keep a dense copy of
 * each weight, four times its int4 bytes, for prefill):
 *   dense[n, k] = RN_act((q - z) * s)   (one rounding, as `dequantize_w4a16`)
 *   packed  the buffer written by w4a16_repack for the same N, K,
 *           group_size and qtype (the call cannot check this)
 *   dense   [N, ldw] act dtype, row-major, ldw >= K, 16-byte aligned with
 *           ldw % 8 == 0 (W4A16_ERR_UNSUPPORTED otherwise); N * ldw * 2
 *           bytes owned by the caller, who decides whether the memory budget
 *           allows a dense copy
 * Shapes and group sizes as for w4a16_repack. */
w4a16_status w4a16_dequant(const void *packed, int64_t N, int64_t K, int32_t group_size, int32_t qtype,
                           int32_t dtype, void *dense, int64_t ldw, hipStream_t stream);

/* C[M, N] = A[M, K] @ W[N, K]^T (+ bias) for a dense act-dtype weight W
 * (for example written by w4a16_dequant), the second half of that strategy:
 * `_rdna_hybrid_w4a16_apply_impl` sends M >= MIN_DENSE_M to an unquantized
 * GEMM on the dense copy. The product runs in hipBLASLt (fp32 accumulation,
 * bias added before the single rounding of C):
 *   A       [M, lda] act dtype, row-major, lda >= K
 *   W       [N, ldw] act dtype, row-major, ldw >= K
 *   bias    [N] act dtype, or NULL
 *   C       [M, ldc] act dtype, ldc >= N; must not overlap A, W or bias
 *   workspace, workspace_bytes  optional hipBLASLt workspace (NULL: none)
 * Every pointer must be 2-byte aligned. M == 0 is a no-op. Unlike the other
 * calls, this one relies on a library: on the first call on each device it
 * creates a hipBLASLt handle, which holds host and device state until the
 * process ends. A hipBLASLt failure returns W4A16_ERR_HIP with the
 * hipblasStatus_t value in the message. */
w4a16_status w4a16_gemm_dense(const void *A, int64_t M, int64_t lda, const void *W, int64_t N, int64_t K,
                              int64_t ldw, int32_t dtype, const void *bias, void *C, int64_t ldc, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* W4A8: int8 activations with the int4 weights, as the "mixed_precision"
 * package page describes XPUW4A8IntLinearKernel (class docstring and
 * `apply_weights`): each row of A is quantised dynamically to symmetric int8
 * with one scale per row, and the int8 rows are multiplied by symmetric int4
 * weights with the row scale and the group scales. Two calls.
 *
 * w4a8_quantize: per-token symmetric int8 quantisation of A.
 *   xs[m]     = fp32(max_k |A[m, k]|) / 127   (fp32, IEEE division)
 *   qa[m, k]  = rint(A[m, k] / xs[m])         (round half to even; always in
 *               [-127, 127]); a row of zeros gets xs[m] = 0 and codes 0
 *   A   [M, lda] act dtype, lda >= K, 16-byte aligned with lda % 8 == 0
 *   qa  [M, ldq] int8, ldq >= K, 8-byte aligned with ldq % 8 == 0. Each
 *       run of 8 codes (k = 8c .. 8c + 7) is stored in the order
 *       k = 8c + 0, 4, 1, 5, 2, 6, 3, 7: the order in which a packed weight
 *       word gives its codes to the int8 MFMA, so w4a8_gemm uses them as
 *       stored. Codes from elsewhere must be stored the same way.
 *   xs  [M] fp32
 * K % 8 == 0. M == 0 is a no-op. */
w4a16_status w4a8_quantize(const void *A, int64_t M, int64_t K, int64_t lda, int32_t dtype, int8_t *qa, int64_t ldq,
                           float *xs, hipStream_t stream);

/* Bytes of device workspace w4a8_gemm needs for these arguments (0 if none):
 * split-K partial results. out_bytes is a host pointer. */
w4a16_status w4a8_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size, size_t *out_bytes);

/* C[M, N] = xs[m] * sum_g s[n, g] * sum_{k in g} qa[m, k] * (q[n, k] - 8)
 * (+ bias[n]), rounded once to the act dtype:
 *   qa, xs   as written by w4a8_quantize (qa [M, ldq] int8, xs [M] fp32)
 *   packed   the buffer w4a16_repack writes for the same N, K, group_size
 *            and qtype W4A16_UINT4B8 (symmetric weights only, as on the
 *            pages; the call cannot check this)
 *   bias     [N] act dtype, or NULL; C [M, ldc] act dtype, ldc >= N
 *   workspace, workspace_bytes  at least w4a8_workspace_size() bytes (may
 *            be NULL when that is 0); calls that share one must be ordered.
 *            The call writes partial results from the start of the
 *            workspace: a buffer it shares with w4a16_gemm must have its
 *            first w4a16_workspace_counter_bytes() bytes zeroed again before
 *            the next w4a16_gemm call
 * The integer group sums are exact (int8 MFMA, int32 accumulation); each
 * group's sum is scaled in fp32. Shapes as for w4a16_repack. qa must be
 * 8-byte aligned with ldq % 8 == 0. At M >= 64, with qa 16-byte aligned,
 * ldq % 16 == 0, C 16-byte aligned and ldc % 8 == 0, a tiled kernel runs;
 * other calls take a kernel that works in registers. Both give the same
 * result when neither splits K. M == 0 is a no-op. W4A16_ERR_SIZE if the
 * workspace is too small. */
w4a16_status w4a8_gemm(const int8_t *qa, const float *xs, int64_t M, int64_t ldq, const void *packed, int64_t N,
                       int64_t K, int32_t group_size, int32_t dtype, const void *bias, void *C, int64_t ldc,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
