/* Host driver for the sanitizer build of the oracle (test_sanitizers.py):
 * runs every oracle routine on small shapes with N and K tails, both zero
 * conventions and several group sizes, and checks a few identities that hold
 * exactly (pack/unpack round trips, the GEMM against a sum over the dequantised
 * weight, the device encoding of a code against its position). Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer; any out-of-bounds access,
 * overflow or undefined shift aborts the run. Prints "ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void w4o_unpack_codes(const uint32_t *words, int64_t N, int64_t K, uint8_t *codes);
void w4o_pack_codes(const uint8_t *codes, int64_t N, int64_t K, uint32_t *words);
void w4o_unpack_zeros(const uint32_t *zp_words, int64_t N, int64_t Kg, uint8_t *zeros);
void w4o_pack_zeros(const uint8_t *zeros, int64_t N, int64_t Kg, uint32_t *zp_words);
void w4o_dequant(const uint32_t *words, const double *scales, const uint32_t *zp_words, int qtype, int64_t N,
                 int64_t K, int64_t G, double *W);
int w4o_gemm(const double *A, int64_t M, int64_t lda, const uint32_t *words, const double *scales,
             const uint32_t *zp_words, int qtype, int64_t N, int64_t K, int64_t G, const double *bias, double *C,
             int nthreads);
int64_t w4o_device_size(int64_t N, int64_t K, int64_t G, int qtype);
void w4o_encode_device(const uint8_t *codes, const uint16_t *scale_bits, const uint8_t *zeros, int qtype, int64_t N,
                       int64_t K, int64_t G, uint8_t *out);
void w4o_quant_rows_a8(const double *A, int64_t M, int64_t K, int8_t *q, float *xs);
void w4o_gemm_w4a8(const int8_t *q, const float *xs, int64_t M, int64_t K, const uint32_t *words,
                   const double *scales, int64_t N, int64_t G, const double *bias, double *C);

static uint64_t state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) { /* xorshift64*, a fixed test sequence */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 2685821657736338717ull) >> 32);
}

static int failures = 0;
#define CHECK(cond, ...)                  \
    do {                                  \
        if (!(cond)) {                    \
            printf("FAIL: " __VA_ARGS__); \
            printf("\n");                 \
            ++failures;                   \
        }                                 \
    } while (0)

static void run_case(int64_t M, int64_t N, int64_t K, int64_t G, int qtype) {
    const int64_t Ge = G == -1 ? K : G, Kg = K / Ge;
    uint8_t *codes = malloc((size_t)(N * K)), *codes2 = malloc((size_t)(N * K));
    uint32_t *words = malloc((size_t)(N * K / 8) * 4);
    uint8_t *zeros = malloc((size_t)(N * Kg)), *zeros2 = malloc((size_t)(N * Kg));
    uint32_t *zpw = malloc((size_t)(N / 8 * Kg) * 4);
    double *scales = malloc((size_t)(N * Kg) * 8);
    uint16_t *sbits = malloc((size_t)(N * Kg) * 2);
    double *A = malloc((size_t)(M * K) * 8), *W = malloc((size_t)(N * K) * 8), *C = malloc((size_t)(M * N) * 8);
    double *bias = malloc((size_t)N * 8);
    for (int64_t i = 0; i < N * K; ++i) codes[i] = (uint8_t)(next_u32() & 15u);
    for (int64_t i = 0; i < N * Kg; ++i) {
        zeros[i] = (uint8_t)(next_u32() & 15u);
        sbits[i] = (uint16_t)(0x2000u + (next_u32() & 0x0FFFu)); /* fp16 values in [2^-7, 2^-6) */
        scales[i] = ldexp(1.0 + (sbits[i] & 0x3FF) / 1024.0, ((sbits[i] >> 10) & 31) - 15);
    }
    for (int64_t i = 0; i < M * K; ++i) A[i] = ((int)(next_u32() % 2001) - 1000) / 256.0;
    for (int64_t n = 0; n < N; ++n) bias[n] = ((int)(next_u32() % 201) - 100) / 64.0;
    w4o_pack_codes(codes, N, K, words);
    w4o_unpack_codes(words, N, K, codes2);
    CHECK(memcmp(codes, codes2, (size_t)(N * K)) == 0, "codes round trip N=%lld K=%lld", (long long)N, (long long)K);
    w4o_pack_zeros(zeros, N, Kg, zpw);
    w4o_unpack_zeros(zpw, N, Kg, zeros2);
    CHECK(memcmp(zeros, zeros2, (size_t)(N * Kg)) == 0, "zeros round trip");
    const uint32_t *zp = qtype == 1 ? zpw : NULL;
    w4o_dequant(words, scales, zp, qtype, N, K, G, W);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int z = qtype == 1 ? zeros[n * Kg + k / Ge] : 8;
            CHECK(W[n * K + k] == (codes[n * K + k] - z) * scales[n * Kg + k / Ge], "dequant at %lld,%lld",
                  (long long)n, (long long)k);
        }
    CHECK(w4o_gemm(A, M, K, words, scales, zp, qtype, N, K, G, bias, C, 2) >= 1, "gemm threads");
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += A[m * K + k] * W[n * K + k];
            CHECK(C[m * N + n] == acc + bias[n], "gemm at %lld,%lld", (long long)m, (long long)n);
        }
    const int64_t bytes = w4o_device_size(N, K, G, qtype);
    uint8_t *dev = malloc((size_t)bytes);
    w4o_encode_device(codes, sbits, qtype == 1 ? zeros : NULL, qtype, N, K, G, dev);
    /* code (n, k): tile (n/16, k/128), lane 16*((k%32)/8) + n%16, word (k%128)/32, bits 4*(i/2) + 16*(i%2) */
    for (int64_t n = 0; n < N; n += 7)
        for (int64_t k = 0; k < K; k += 5) {
            const int64_t KT = (K + 127) / 128, l = 16 * ((k % 32) / 8) + n % 16, s = (k % 128) / 32, i = k % 8;
            const int64_t off = ((n / 16) * KT + k / 128) * 1024 + (4 * l + s) * 4;
            const uint32_t w = (uint32_t)dev[off] | (uint32_t)dev[off + 1] << 8 | (uint32_t)dev[off + 2] << 16 |
                               (uint32_t)dev[off + 3] << 24;
            CHECK(((w >> (4 * (i / 2) + 16 * (i % 2))) & 15u) == codes[n * K + k], "encode at %lld,%lld",
                  (long long)n, (long long)k);
        }
    int8_t *q = malloc((size_t)(M * K));
    float *xs = malloc((size_t)M * 4);
    w4o_quant_rows_a8(A, M, K, q, xs);
    w4o_gemm_w4a8(q, xs, M, K, words, scales, N, G, bias, C);
    free(dev);
    free(q);
    free(xs);
    free(codes);
    free(codes2);
    free(words);
    free(zeros);
    free(zeros2);
    free(zpw);
    free(scales);
    free(sbits);
    free(A);
    free(W);
    free(C);
    free(bias);
}

int main(void) {
    run_case(3, 24, 136, -1, 1); /* N and K tails, one group */
    run_case(2, 40, 256, 32, 1);
    run_case(1, 16, 128, 128, 0);
    run_case(4, 48, 512, 64, 0);
    run_case(2, 8, 264, 8 * 33, 1); /* G == K */
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
