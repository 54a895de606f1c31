/*
 * w4a16_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, obviously correct CPU oracle for the fused W4A16 linear layer
 *     C[M,N] = A[M,K] @ dequant(W)^T (+ bias).
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load it. The HIP library never links or calls it, and the two share no
 * code, header, table or constant.
 *
 * Everything is computed in fp64. A 4-bit code minus a 4-bit zero, times an
 * fp16/bf16 scale, is exact in fp64, so dequantisation is exact; the product
 * is a plain k-ordered sum in fp64.
 *
 * Sources, cited by page title and section (the pages are vLLM API pages and a
 * fork's copy of vLLM's MI300 Triton kernel):
 *  [TRITON-MI300] "triton_w4a16.py" (Triton-based W4A16 GEMM for ROCm MI300):
 *      module docstring -- checkpoint layout weight_packed [N, K/8] int32,
 *      weight_scale [N, K/G], weight_zero_point [N/8, K/G]; GPTQ sequential
 *      packing, eight int4 values per int32 at shifts 0,4,...,28.
 *      `process_weights_after_loading` / `repack_w_q`, steps 2 and 4 -- the
 *      unpack (shift, mask 0xF) and the pack (sum of (v & 0xF) << shift).
 *      `triton_w4a16_gemm_kernel` docstring -- w = (w_int4 - zero) * scale,
 *      zero = 8 for symmetric uint4b8.
 *      `apply_weights` -- group_size -1 means K; a type with a built-in bias
 *      (uint4b8) ignores any zero-point tensor; uint4 without zeros uses 0.
 *  [HYBRID-58181] "rdna_hybrid_w4a16" (vLLM docs, build 58181),
 *      `_triton_w4a16_skinny_fmt_kernel` docstring -- row n's raw zero point
 *      sits in word [n/8] of [N/8, K/G] at bits 4*(n%8); dequant is
 *      (nibble - zp_raw) * scale.
 *  [HYBRID-61746] "rdna_hybrid_w4a16" (vLLM docs, build 61746),
 *      `dequantize_w4a16` -- group g of row n covers the G consecutive k of
 *      the view [N, K/G, G]; w = (q - zp) * scale.
 *  [PKG-58588] "mixed_precision" package page (vLLM docs, build 58588),
 *      zentorch W4A16 section -- an [N, K/8] int32 tensor is the same memory as
 *      [N, K/2] bytes in little-endian order (used by the tests as a pin);
 *      XPUW4A8IntLinearKernel -- symmetric int4 weights, activations
 *      quantised per token to symmetric int8 (the W4A8 functions at the end).
 *
 * The device-layout encoder at the end follows the layout this project
 * defines for its gfx950 kernels (the specification is restated beside the
 * function); it is written from that specification, not from the kernels.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define W4O_UINT4B8 0 /* symmetric, implicit zero 8 */
#define W4O_UINT4 1   /* asymmetric, explicit zero points (0 when absent) */

int w4o_version(void) { return 1; }

int w4o_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* [TRITON-MI300] module docstring and repack_w_q step 2: code k = 8j + i of
 * row n is bits [4i, 4i+4) of word (n, j). Words are handled as raw 32-bit
 * patterns, so a set top bit (a negative int32) needs no care. */
void w4o_unpack_codes(const uint32_t *words, int64_t N, int64_t K, uint8_t *codes) {
    const int64_t K8 = K / 8;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint32_t w = words[n * K8 + k / 8];
            codes[n * K + k] = (uint8_t)((w >> (4 * (k % 8))) & 0xFu);
        }
}

/* [TRITON-MI300] repack_w_q step 4, applied along K: word (n, j) is the OR of
 * (code & 0xF) << 4i over its eight codes (the bit ranges are disjoint, so the
 * page's sum equals this OR). */
void w4o_pack_codes(const uint8_t *codes, int64_t N, int64_t K, uint32_t *words) {
    const int64_t K8 = K / 8;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K8; ++j) {
            uint32_t w = 0;
            for (int i = 0; i < 8; ++i) w |= ((uint32_t)(codes[n * K + 8 * j + i] & 0xFu)) << (4 * i);
            words[n * K8 + j] = w;
        }
}

/* [HYBRID-58181] kernel docstring: zero of (row n, group g) is bits
 * [4*(n%8), +4) of word (n/8, g) of the [N/8, Kg] tensor. */
void w4o_unpack_zeros(const uint32_t *zp_words, int64_t N, int64_t Kg, uint8_t *zeros) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < Kg; ++g)
            zeros[n * Kg + g] = (uint8_t)((zp_words[(n / 8) * Kg + g] >> (4 * (n % 8))) & 0xFu);
}

void w4o_pack_zeros(const uint8_t *zeros, int64_t N, int64_t Kg, uint32_t *zp_words) {
    for (int64_t b = 0; b < N / 8; ++b)
        for (int64_t g = 0; g < Kg; ++g) {
            uint32_t w = 0;
            for (int i = 0; i < 8; ++i) w |= ((uint32_t)(zeros[(8 * b + i) * Kg + g] & 0xFu)) << (4 * i);
            zp_words[b * Kg + g] = w;
        }
}

/* [TRITON-MI300] apply_weights: group_size -1 means one group over all of K. */
static int64_t effective_group(int64_t K, int64_t G) { return G == -1 ? K : G; }

/* The zero of (row n, group g). [TRITON-MI300] kernel docstring and
 * apply_weights: uint4b8 subtracts the constant 8 and ignores a zero-point
 * tensor; uint4 subtracts the stored nibble, or 0 when there is none. */
static int zero_of(int qtype, const uint32_t *zp_words, int64_t Kg, int64_t n, int64_t g) {
    if (qtype == W4O_UINT4B8) return 8;
    if (zp_words == NULL) return 0;
    return (int)((zp_words[(n / 8) * Kg + g] >> (4 * (n % 8))) & 0xFu);
}

/* Dequantise row n into out[0..K): out[k] = (q[n,k] - z[n,g(k)]) * s[n,g(k)]
 * with g(k) = k / G ([HYBRID-61746] dequantize_w4a16). Exact in fp64. */
static void dequant_row(const uint32_t *words, const double *scales, const uint32_t *zp_words, int qtype,
                        int64_t K, int64_t G, int64_t n, double *out) {
    const int64_t Ge = effective_group(K, G), Kg = K / Ge, K8 = K / 8;
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / Ge;
        int q = (int)((words[n * K8 + k / 8] >> (4 * (k % 8))) & 0xFu);
        int z = zero_of(qtype, zp_words, Kg, n, g);
        out[k] = (double)(q - z) * scales[n * Kg + g];
    }
}

/* The dense weight W[N,K] in fp64. */
void w4o_dequant(const uint32_t *words, const double *scales, const uint32_t *zp_words, int qtype, int64_t N,
                 int64_t K, int64_t G, double *W) {
    for (int64_t n = 0; n < N; ++n) dequant_row(words, scales, zp_words, qtype, K, G, n, W + n * K);
}

/* C[m,n] = sum_k A[m,k] * W[n,k] (+ bias[n]), fp64, k in order 0..K-1.
 * A is [M, lda] fp64 (row m starts at A + m*lda), C is [M, N] fp64.
 * Rows of W are dequantised one at a time into a per-thread buffer; threads
 * split the N rows and never share an output. Returns the thread count used,
 * or -1 when a buffer cannot be allocated. */
int w4o_gemm(const double *A, int64_t M, int64_t lda, const uint32_t *words, const double *scales,
             const uint32_t *zp_words, int qtype, int64_t N, int64_t K, int64_t G, const double *bias, double *C,
             int nthreads) {
    int used = 1, failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *wrow = (double *)malloc((size_t)K * sizeof(double));
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        if (wrow == NULL) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
        for (int64_t n = 0; n < N; ++n) {
            if (wrow == NULL) continue;
            dequant_row(words, scales, zp_words, qtype, K, G, n, wrow);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                const double *a = A + m * lda;
                for (int64_t k = 0; k < K; ++k) acc += a[k] * wrow[k];
                if (bias != NULL) acc += bias[n];
                C[m * N + n] = acc;
            }
        }
        free(wrow);
    }
    return failed ? -1 : used;
}

/*
 * Device layout ("packed buffer") used by this project's gfx950 kernels.
 * Requires N % 8 == 0, K % 8 == 0, Ge | K with Ge in {32, 64, 128, 256} or
 * Ge == K; Kg = K / Ge groups. N is padded to Np, the next multiple of 16,
 * K to Kp, the next multiple of 128, and the groups to
 * Kgp = (Kg == 1 ? 1 : Kp / Ge) (Np = N, Kp = K and Kgp = Kg when N % 16 == 0
 * and K % 128 == 0). All offsets in bytes; words are little-endian uint32.
 *
 *  Q region at 0, Np*Kp/2 bytes: 1024-byte tiles, tile (nt, kt) for
 *    nt in [0, Np/16), kt in [0, Kp/128) at ((nt * (Kp/128)) + kt) * 1024.
 *    Word 4*l + s of a tile (lane l in [0,64), s in [0,4)) holds the codes of
 *    row n = 16*nt + l%16 at k = 128*kt + 32*s + 8*(l/16) + i, i = 0..7,
 *    code i in bits [4*(i/2) + 16*(i%2), +4); codes at n >= N or k >= K
 *    are 0.
 *  S region at S0 = align256(Np*Kp/2): Np*Kgp 2-byte scales (the raw
 *    fp16/bf16 bits), element (nt, g, r) = scale[16*nt + r][g] at
 *    S0 + ((nt*Kgp + g)*16 + r)*2, and 0 for 16*nt + r >= N or g >= Kg.
 *  Z region (uint4 only) at Z0 = align256(S0 + Np*Kgp*2): Np*Kgp bytes,
 *    element (nt, g, r) = zero nibble of (row 16*nt + r, group g) at
 *    Z0 + (nt*Kgp + g)*16 + r, 0 for rows >= N or g >= Kg; all zero when the
 *    checkpoint has no zero points.
 *  Total size = align256(end of the last region).
 */
static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
static int64_t padded_k(int64_t K) { return (K + 127) / 128 * 128; }
static int64_t padded_n(int64_t N) { return (N + 15) / 16 * 16; }
static int64_t stored_groups(int64_t K, int64_t G) {
    const int64_t Ge = effective_group(K, G);
    return K / Ge == 1 ? 1 : padded_k(K) / Ge;
}

int64_t w4o_device_size(int64_t N, int64_t K, int64_t G, int qtype) {
    const int64_t Kgp = stored_groups(K, G), Np = padded_n(N);
    int64_t end = align256(Np * padded_k(K) / 2) + Np * Kgp * 2;
    if (qtype == W4O_UINT4) end = align256(end) + Np * Kgp;
    return align256(end);
}

/* codes [N, K] (one per byte), scale_bits [N, Kg] (raw 16-bit patterns),
 * zeros [N, Kg] or NULL; out must hold w4o_device_size bytes (padding is
 * written as 0). */
void w4o_encode_device(const uint8_t *codes, const uint16_t *scale_bits, const uint8_t *zeros, int qtype, int64_t N,
                       int64_t K, int64_t G, uint8_t *out) {
    const int64_t Kg = K / effective_group(K, G), Kp = padded_k(K), KT = Kp / 128;
    const int64_t Kgp = stored_groups(K, G), Np = padded_n(N);
    memset(out, 0, (size_t)w4o_device_size(N, K, G, qtype));
    for (int64_t nt = 0; nt < Np / 16; ++nt)
        for (int64_t kt = 0; kt < KT; ++kt)
            for (int l = 0; l < 64; ++l)
                for (int s = 0; s < 4; ++s) {
                    const int64_t n = 16 * nt + l % 16;
                    const int64_t k0 = 128 * kt + 32 * s + 8 * (l / 16);
                    uint32_t w = 0;
                    for (int i = 0; i < 8; ++i)
                        if (n < N && k0 + i < K)
                            w |= (uint32_t)(codes[n * K + k0 + i] & 0xFu) << (4 * (i / 2) + 16 * (i % 2));
                    const int64_t off = (nt * KT + kt) * 1024 + (4 * l + s) * 4;
                    for (int b = 0; b < 4; ++b) out[off + b] = (uint8_t)(w >> (8 * b));
                }
    const int64_t S0 = align256(Np * Kp / 2);
    for (int64_t nt = 0; nt < Np / 16; ++nt)
        for (int64_t g = 0; g < Kg; ++g)
            for (int r = 0; r < 16 && 16 * nt + r < N; ++r) {
                const uint16_t v = scale_bits[(16 * nt + r) * Kg + g];
                const int64_t off = S0 + ((nt * Kgp + g) * 16 + r) * 2;
                out[off] = (uint8_t)(v & 0xFF);
                out[off + 1] = (uint8_t)(v >> 8);
            }
    if (qtype == W4O_UINT4) {
        const int64_t Z0 = align256(S0 + Np * Kgp * 2);
        for (int64_t nt = 0; nt < Np / 16; ++nt)
            for (int64_t g = 0; g < Kg; ++g)
                for (int r = 0; r < 16 && 16 * nt + r < N; ++r)
                    out[Z0 + (nt * Kgp + g) * 16 + r] = zeros ? (uint8_t)(zeros[(16 * nt + r) * Kg + g] & 0xFu) : 0;
    }
}

/*
 * W4A8: activations quantised per token to symmetric int8, weights
 * symmetric int4 ("mixed_precision" package page, XPUW4A8IntLinearKernel:
 * its class docstring and `apply_weights`, which quantises each row of x
 * dynamically to symmetric int8 and multiplies the int8 rows by the int4
 * weights with the row scale and the group scales). The pages do not print
 * the quantiser; the reading taken (stated where the project documents its
 * readings): the row scale is fp32(max |x|) / 127 in fp32 with IEEE
 * division, each value is rint(fp32(x) / scale) (round half to even)
 * clamped to [-127, 127], and a row of zeros has scale 0 and codes 0.
 */
void w4o_quant_rows_a8(const double *A, int64_t M, int64_t K, int8_t *q, float *xs) {
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf((float)A[m * K + k]);
            if (v > amax) amax = v;
        }
        const float s = amax / 127.0f;
        xs[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            int v = 0;
            if (amax > 0.0f) {
                const float t = rintf((float)A[m * K + k] / s);
                /* |x / s| is within a few ulps of 127 at most, so the clamp
                 * never binds; it is kept as the rule's statement. */
                v = t > 127.0f ? 127 : (t < -127.0f ? -127 : (int)t);
            }
            q[m * K + k] = (int8_t)v;
        }
    }
}

/* C[m, n] = xs[m] * sum_g s[n, g] * sum_{k in g} q[m, k] * (code[n, k] - 8)
 * (+ bias[n]), in fp64: the integer sums are exact, and so is their product
 * with an fp32 row scale and an fp16/bf16 group scale. */
void w4o_gemm_w4a8(const int8_t *q, const float *xs, int64_t M, int64_t K, const uint32_t *words, const double *scales,
                   int64_t N, int64_t G, const double *bias, double *C) {
    const int64_t Ge = effective_group(K, G), Kg = K / Ge, K8 = K / 8;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t g = 0; g < Kg; ++g) {
                int64_t isum = 0;
                for (int64_t k = g * Ge; k < (g + 1) * Ge; ++k) {
                    const int code = (int)((words[n * K8 + k / 8] >> (4 * (k % 8))) & 0xFu);
                    isum += (int64_t)q[m * K + k] * (code - 8);
                }
                acc += scales[n * Kg + g] * (double)isum;
            }
            acc *= (double)xs[m];
            if (bias) acc += bias[n];
            C[n + m * N] = acc;
        }
    }
}
