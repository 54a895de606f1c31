// w4a8.hip -- the W4A8 variant: activations quantised per token to symmetric
// int8, symmetric int4 weights from the same packed buffer, int8 MFMA.
//
// The operation is the one the "mixed_precision" package page gives for
// XPUW4A8IntLinearKernel (class docstring and `apply_weights`): each row of x
// is quantised dynamically to symmetric int8 with one scale per row, and the
// int8 rows are multiplied by the int4 weights (uint4b8, zero 8) with the row
// scale and the weight's group scales:
//     C[m, n] = xs[m] * sum_g s[n, g] * sum_{k in g} qa[m, k] * (q[n, k] - 8)
// The integer sums run on the int8 matrix cores and are exact; the group
// scale is applied to each group's integer sum in fp32, the row scale and
// bias at the end, and C is rounded once. Two GEMM kernels:
//  * w4a8_ring_kernel (M >= 64 with enough tiles or a long K): 128 x 256
//    tiles, operands staged through a four-stage LDS ring,
//    v_mfma_i32_16x16x64_i8 on signed weight bytes 16 (q - 8);
//  * w4a8_kernel (the rest, decode included): operands straight into
//    registers, v_mfma_i32_16x16x32_i8 on unsigned codes with a row-sum
//    correction, K split across workgroups.
#include "device_common.h"
#include "internal.h"
#include "lds_stage.h"

namespace w4a16 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr int kA8DecodeChunk = 4;      // k-tiles per K chunk (and register stages) for up to 16 rows
constexpr int64_t kA8RingMinM = 64;     // the ring kernel from this many rows ...
constexpr int64_t kA8RingMinTiles = 48; // ... and this many 128 x 256 tiles or
constexpr int64_t kA8RingMinK = 8192;   // ... this long a K (split into chunks)
constexpr int64_t kA8RingMinChunk = 8;  // k-tiles per K chunk of the ring kernel, at least

// ---------------------------------------------------------------- quantiser

// One workgroup of 256 threads per row. The scale is fp32(max |x|) / 127
// (IEEE division); each value becomes rint(x / scale) (half to even),
// which stays within [-127, 127] because |x| <= max |x|; a row of zeros
// gets scale 0 and codes 0. K % 8 == 0: each thread handles 8-element chunks.
// Each chunk of 8 codes is stored in the order 0,4,1,5,2,6,3,7: the order in
// which a packed weight word's two nibble masks give its codes, so that the
// GEMM kernels use the bytes as they are.
template <int DT>
__global__ __launch_bounds__(256) void a8_quant_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t K,
                                                       int8_t* __restrict__ q, int64_t ldq, float* __restrict__ xs) {
    const int64_t m = blockIdx.x;
    const uint16_t* row = A + m * lda;
    const int64_t chunks = K / 8;
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < chunks; c += 256) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax = fmaxf(amax, fabsf(act_to_float<DT>((uint16_t)(v[e] & 0xFFFFu))));
            amax = fmaxf(amax, fabsf(act_to_float<DT>((uint16_t)(v[e] >> 16))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) xs[m] = s;
    int8_t* qrow = q + m * ldq;
    for (int64_t c = threadIdx.x; c < chunks; c += 256) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
        uint32_t out[2] = {0u, 0u};
        if (amax > 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t bits = (uint16_t)(e & 1 ? v[e >> 1] >> 16 : v[e >> 1] & 0xFFFFu);
                const float t = __builtin_rintf(act_to_float<DT>(bits) / s);
                const int iv = t > 127.0f ? 127 : (t < -127.0f ? -127 : (int)t);
                const int pos = e < 4 ? 2 * e : 2 * e - 7;  // pair order 0,4,1,5,2,6,3,7
                out[pos >> 2] |= ((uint32_t)iv & 0xFFu) << (8 * (pos & 3));
            }
        }
        *reinterpret_cast<uint2*>(qrow + 8 * c) = make_uint2(out[0], out[1]);
    }
}

// The same quantiser with the row held in registers between its two
// passes, so that it is read from memory once: CPT 16-byte chunks per
// thread, for K <= 8 * 256 * CPT.
template <int DT, int CPT>
__global__ __launch_bounds__(256) void a8_quant_reg_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t K,
                                                           int8_t* __restrict__ q, int64_t ldq, float* __restrict__ xs) {
    const int64_t m = blockIdx.x;
    const uint16_t* row = A + m * lda;
    const int64_t chunks = K / 8;
    u32x4 v[CPT];
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
        const int64_t c = threadIdx.x + 256 * t;
        v[t] = c < chunks ? *reinterpret_cast<const u32x4*>(row + 8 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax = fmaxf(amax, fabsf(act_to_float<DT>((uint16_t)(v[t][e] & 0xFFFFu))));
            amax = fmaxf(amax, fabsf(act_to_float<DT>((uint16_t)(v[t][e] >> 16))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) xs[m] = s;
    int8_t* qrow = q + m * ldq;
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
        const int64_t c = threadIdx.x + 256 * t;
        if (c >= chunks) break;
        uint32_t out[2] = {0u, 0u};
        if (amax > 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t bits = (uint16_t)(e & 1 ? v[t][e >> 1] >> 16 : v[t][e >> 1] & 0xFFFFu);
                const float r = __builtin_rintf(act_to_float<DT>(bits) / s);
                const int iv = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r);
                const int pos = e < 4 ? 2 * e : 2 * e - 7;  // pair order 0,4,1,5,2,6,3,7
                out[pos >> 2] |= ((uint32_t)iv & 0xFFu) << (8 * (pos & 3));
            }
        }
        *reinterpret_cast<uint2*>(qrow + 8 * c) = make_uint2(out[0], out[1]);
    }
}

// ---------------------------------------------------------------- GEMM

struct A8Args {
    const int8_t* qa;
    const float* xs;
    int64_t M, ldq, K;
    const u32x4* codes;
    const uint16_t* scales;
    int64_t NT, N, KTT, Kg, Ge;  // NT: n-tiles of the padded N; N: columns of C
    int one_group;
    int64_t kc;                  // k-tiles per K chunk (split-K)
    const uint16_t* bias;
    uint16_t* C;
    int64_t ldc;
    float* partials;             // [ksplit][M][16*NT] when ksplit > 1
    int64_t n_blocks;            // ring kernel: 256-column blocks of C
};

// One activation chunk (k .. k+7 of a row, stored in pair order by the
// quantiser) as the 8 bytes of an MFMA operand.
__device__ __forceinline__ int64_t a_operand(uint2 v) {
    return (int64_t)(((uint64_t)v.y << 32) | v.x);
}

// The eight codes of a packed word (pair order: code i at 4*(i/2) + 16*(i%2))
// as bytes 0..15: the low nibbles give codes 0,4,1,5, the high ones 2,6,3,7.
__device__ __forceinline__ int64_t b_operand(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A wave owns MI row blocks of 16 and 4 n-tiles; a workgroup of 4 waves owns
// 16*MI rows x 256 columns over one K chunk (blockIdx.z). Lane l of a 16x16
// output block holds rows 4*(l/16) .. +3 of column l%16. The loads of NS
// k-tiles are in flight at a time (a ring of register stages): with NS equal
// to the chunk length every load is issued before the first MFMA.
template <int DT, int MI, int NS>
__global__ __launch_bounds__(256) void w4a8_kernel(A8Args a) {
    constexpr int NJ = 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    const int64_t nt0 = (int64_t)blockIdx.x * 16 + wave * NJ;
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MI;
    const int64_t kt0 = (int64_t)blockIdx.z * a.kc;
    const int64_t kt1 = kt0 + a.kc < a.KTT ? kt0 + a.kc : a.KTT;

    i32x4 acc[MI][NJ], S[MI];
    floatx4 accf[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        S[i] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            acc[i][j] = i32x4{0, 0, 0, 0};
            accf[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const int64_t ones = 0x0101010101010101ll;

    // Group scale of n-tile j for group g (lane column r); 0 past N's tiles.
    auto fold = [&](int64_t g) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t nt = nt0 + j;
            const float sc = nt < a.NT ? act_to_float<DT>(a.scales[(nt * a.Kg + g) * 16 + r]) : 0.f;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    accf[i][j][jj] = __builtin_fmaf(sc, (float)(acc[i][j][jj] - 8 * S[i][jj]), accf[i][j][jj]);
                acc[i][j] = i32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) S[i] = i32x4{0, 0, 0, 0};
    };

    // Stage u holds k-tile kt: the weight words of the wave's n-tiles (tiles
    // past the padded N read tile NT-1 and are never stored) and the
    // activation chunks of rows m0 + 16i + r at k = 128kt + 32s + 8g4 (rows
    // past M and columns past K read as zero, never loaded).
    u32x4 w[NS][NJ];
    uint2 av[NS][MI][4];
    auto load = [&](int u, int64_t kt) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t nt = nt0 + j < a.NT ? nt0 + j : a.NT - 1;
            w[u][j] = __builtin_nontemporal_load(a.codes + (nt * a.KTT + kt) * 64 + lane);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int64_t m = m0 + 16 * i + r;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int64_t k = kt * 128 + 32 * s + 8 * g4;
                uint2 v = make_uint2(0u, 0u);
                if (m < a.M && k < a.K) v = *reinterpret_cast<const uint2*>(a.qa + m * a.ldq + k);
                av[u][i][s] = v;
            }
        }
    };
    auto compute = [&](int u, int64_t kt) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            int64_t A8[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                A8[i] = a_operand(av[u][i][s]);
                S[i] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A8[i], ones, S[i], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int64_t B8 = b_operand(w[u][j][s]);
#pragma unroll
                for (int i = 0; i < MI; ++i) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A8[i], B8, acc[i][j], 0, 0, 0);
            }
            // A group ends with this slice: fold its integer sums.
            const int64_t kend = kt * 128 + 32 * (s + 1);
            if (!a.one_group && kend % a.Ge == 0) fold((kend - 1) / a.Ge);
        }
    };

#pragma unroll
    for (int u = 0; u < NS; ++u)
        if (kt0 + u < kt1) load(u, kt0 + u);
    for (int64_t kt = kt0; kt < kt1; kt += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            if (kt + u < kt1) {
                compute(u, kt + u);
                if (kt + u + NS < kt1) load(u, kt + u + NS);
            }
        }
    }
    // The rest of a group cut by the chunk's end (or the only group).
    if (a.one_group) fold(0);
    else if ((kt1 * 128) % a.Ge != 0) fold((kt1 * 128 - 1) / a.Ge);

    const int64_t ldp = a.NT * 16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int64_t n = (nt0 + j) * 16 + r;
        if (nt0 + j >= a.NT) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int64_t m = m0 + 16 * i + 4 * g4 + jj;
                if (m >= a.M) continue;
                if (a.partials != nullptr) {
                    a.partials[((int64_t)blockIdx.z * a.M + m) * ldp + n] = accf[i][j][jj];
                } else if (n < a.N) {
                    const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
                    a.C[m * a.ldc + n] = to_act_bits<DT>(__builtin_fmaf(a.xs[m], accf[i][j][jj], bv));
                }
            }
        }
    }
}

// C = xs[m] * (sum of the K chunks' partial results) + bias, one thread per
// element of C.
template <int DT>
__global__ __launch_bounds__(256) void w4a8_reduce_kernel(const float* __restrict__ partials, int ksplit, int64_t M,
                                                          int64_t N, int64_t ldp, const float* __restrict__ xs,
                                                          const uint16_t* __restrict__ bias, uint16_t* __restrict__ C,
                                                          int64_t ldc) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= M * N) return;
    const int64_t m = t / N, n = t - m * N;
    float sum = 0.f;
    for (int c = 0; c < ksplit; ++c) sum += partials[((int64_t)c * M + m) * ldp + n];
    const float bv = bias ? act_to_float<DT>(bias[n]) : 0.f;
    C[m * ldc + n] = to_act_bits<DT>(__builtin_fmaf(xs[m], sum, bv));
}


// Tiled ring kernel for large M (K % 128 == 0, one group per row or groups
// of 64, 128 or 256 k). A workgroup of 8 waves computes a 128 x 256 tile of C;
// wave (wm, wn) owns rows 64 wm .. +63 (4 row blocks) and n-tiles 4 wn .. +3.
//  * Per K step of 128, the 128 x 128-byte activation tile and the
//    workgroup's 16 packed weight tiles go from HBM/L2 straight into LDS
//    with direct 16-byte buffer loads. Activation block 2 rb + h (1 KB) holds
//    rows 16 rb .. +15 at k = 64 h .. +63; lane l's 16 bytes (row l % 16,
//    k = 64 h + 16 (l / 16) .. +15) sit at 16 l.
//  * Four LDS stages form a ring: step t reads stage t % 4 while the loads
//    of steps t + 1 .. t + 3 are in flight. One barrier per step.
//  * v_mfma_i32_16x16x64_i8 takes two packed words per lane (64 k). A word
//    becomes signed bytes 16 (q - 8) without a zero-point term: with the
//    sign bit of each nibble flipped, a nibble is the 4-bit two's complement
//    of q - 8, and placed in the high half of a byte it reads as 16 (q - 8).
//    The low nibbles (codes 0, 4, 1, 5 in pair order) move up by a shift;
//    the quantiser stores each 8-byte activation chunk in the same order.
//  * Integer sums are exact (|16 (q - 8) qa| <= 16256; a chunk of at most
//    131072 k stays below 2^31). GP = 0: one group per row, the scale is
//    applied in the epilogue. GP > 0: a group spans GP slices of 64 k; at
//    its end each sum is scaled by s / 16 into an fp32 result and the
//    integer sum restarts.
template <int DT, int GP>
__global__ __launch_bounds__(512) void w4a8_ring_kernel(A8Args a) {
    static_assert(GP == 0 || GP == 1 || GP == 2 || GP == 4, "groups of 64, 128 or 256 k, or one group");
    constexpr int MI = 4, NJ = 4;
    constexpr int NSC = GP == 0 ? 1 : (GP == 1 ? 2 : 1) * NJ;  // scale registers per stage
    __shared__ __attribute__((aligned(1024))) unsigned char a0[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a1[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a2[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a3[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b0[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b1[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b2[16 * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b3[16 * 1024];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int r = lane & 15, g4 = lane >> 4;
    const int64_t lin = blockIdx.x;
    const int64_t ty = lin / a.n_blocks, tx = lin - ty * a.n_blocks;
    const int64_t m0 = ty * 128;
    const int64_t ntb = tx * 16;  // first n-tile of the workgroup
    // K chunk blockIdx.y: k-tiles [kt0, kt0 + steps) (one chunk unless the
    // tiles are too few for the chip; chunks start at group boundaries).
    const int64_t kt0 = (int64_t)blockIdx.y * a.kc;
    const int64_t steps = (a.KTT - kt0 < a.kc ? a.KTT - kt0 : a.kc);

    // The workgroup's operands as buffers based at its tile: rows
    // [mb, mb + mr) of the activation codes (rows past M clamp to M - 1) and
    // n-tiles [ntb, ntb + nn) of the packed weight (tiles past it clamp).
    const int64_t mb = m0 < a.M - 1 ? m0 : a.M - 1;
    const int64_t mr = a.M - mb < 128 ? a.M - mb : 128;
    const int64_t nn = a.NT - ntb < 16 ? a.NT - ntb : 16;
    const int8_t* abase = a.qa + mb * a.ldq;
    const uint32_t a_bytes = (uint32_t)((mr - 1) * a.ldq + a.K);
    const u32x4* cbase = a.codes + ntb * a.KTT * 64;
    const uint32_t c_bytes = (uint32_t)(nn * a.KTT * 1024);
    const uint16_t* sbase = a.scales + ntb * a.Kg * 16;
    const uint32_t s_bytes = (uint32_t)(nn * a.Kg * 32);
    auto rsrc = [&](const void* base, uint32_t bytes, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, live ? (int)bytes : 0, 0x00020000);
    };
    // This wave loads activation blocks 2 wave + h (row block `wave`) and
    // weight tiles 2 wave + t of the workgroup.
    int64_t arow = m0 + 16 * wave + r;
    if (arow > a.M - 1) arow = a.M - 1;
    const uint32_t a_off = (uint32_t)((arow - mb) * a.ldq + 16 * g4);
    const uint32_t lane16 = (uint32_t)lane * 16;
    // LDS offset of this lane's first activation chunk in the wave's rows.
    const uint32_t a_rd = (uint32_t)(8 * wm * 1024 + 16 * (16 * (g4 >> 1) + r) + 8 * (g4 & 1));
    uint32_t b_tile[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t nt = ntb + 2 * wave + t;
        b_tile[t] = (uint32_t)((nt < a.NT ? nt : a.NT - 1) - ntb);
    }
    auto nt_ld = [&](int j) {
        const int64_t nt = ntb + 4 * wn + j;
        return nt < a.NT ? nt : a.NT - 1;
    };

    // Part h (0, 1) of the loads of step st: activation block h and weight
    // tile h of the wave.
    auto issue = [&](int64_t st, int h, unsigned char* abuf, unsigned char* bbuf) {
        const bool live = st < steps;
        load_lds16(rsrc(abase, a_bytes, live), abuf + (2 * wave + h) * 1024, a_off,
                   (uint32_t)((kt0 + st) * 128 + 64 * h));
        load_lds16(rsrc(cbase, c_bytes, live), bbuf + (2 * wave + h) * 1024, lane16,
                   (uint32_t)((b_tile[h] * a.KTT + kt0 + st) * 1024));
    };
    // The scales of the groups that end in step st (GP = 4: only odd steps
    // end a group), for the wave's four columns.
    auto issue_scales = [&](int64_t st, uint32_t (&sb)[NSC]) {
        if (GP == 0) return;
        const __amdgpu_buffer_rsrc_t rs = rsrc(sbase, s_bytes, st < steps);
        constexpr int NG = GP == 1 ? 2 : 1;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t kt = kt0 + st;
            const int64_t g = GP == 1 ? 2 * kt + q : (GP == 2 ? kt : kt / 2);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t so = (uint32_t)(((nt_ld(j) - ntb) * a.Kg + g) * 16);
                sb[q * NJ + j] = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)r * 2, so * 2, 0);
            }
        }
    };
    // Scale loads per step, over two consecutive steps.
    constexpr int SC2 = GP == 0 ? 0 : (GP == 4 ? NSC : 2 * NSC);

    i32x4 acc[MI][NJ];
    floatx4 accf[GP > 0 ? MI : 1][GP > 0 ? NJ : 1];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            acc[i][j] = i32x4{0, 0, 0, 0};
            if (GP > 0) accf[GP > 0 ? i : 0][GP > 0 ? j : 0] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    const i32x4 zero4 = {0, 0, 0, 0};

    // Step st (u = st % 4, known at compile time after inlining) reads stage
    // u, loads the scales of step st + 2 (into the registers of stage
    // (u + 2) % 4) and then the operands of step st + 3 (into stage
    // (u + 3) % 4). A step's scales are loaded before the operands of the
    // step after it, so waiting for them never waits for later operands.
    // tail (a compile-time value at each call): 0 in the loop; in the at
    // most three steps after it, 1 for the first (it requests only the
    // scales of the third, which that step reads if it runs) and 2 for the
    // others (nothing to request). Tail steps wait for every load before
    // their barrier. (Requesting loads whose registers no step reads would
    // let the compiler drop them and break the count of the wait.)
    auto step = [&](int64_t st, int u, unsigned char* abuf, unsigned char* bbuf, const uint32_t (&sb)[NSC],
                    uint32_t (&ssb)[NSC], unsigned char* nabuf, unsigned char* nbbuf, int tail) {
        if (tail <= 1 && (GP == 1 || GP == 2 || (GP == 4 && (u & 1)))) issue_scales(st + 2, ssb);
        u32x4 raw[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) raw[j] = *reinterpret_cast<const u32x4*>(bbuf + (4 * wn + j) * 1024 + lane16);
        // The activation chunks of slice 0; those of slice 1 are read while
        // slice 0 is multiplied.
        uint64_t av[2][MI][2];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const unsigned char* ap = abuf + (a_rd + (2 * i) * 1024);
            av[0][i][0] = *reinterpret_cast<const uint64_t*>(ap);
            av[0][i][1] = *reinterpret_cast<const uint64_t*>(ap + 512);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __builtin_amdgcn_sched_barrier(0);
            if (tail == 0) issue(st + 3, h, nabuf, nbbuf);
            __builtin_amdgcn_sched_barrier(0);
            if (h == 0) {
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const unsigned char* ap = abuf + (a_rd + (2 * i + 1) * 1024);
                    av[1][i][0] = *reinterpret_cast<const uint64_t*>(ap);
                    av[1][i][1] = *reinterpret_cast<const uint64_t*>(ap + 512);
                }
            }
            i32x4 B[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t w = raw[j][2 * h + e];
                    B[j][2 * e] = (int32_t)(((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u);
                    B[j][2 * e + 1] = (int32_t)((w & 0xF0F0F0F0u) ^ 0x80808080u);
                }
            }
            const bool start = GP > 0 && ((2 * u + h) % (GP > 0 ? GP : 1)) == 0;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const uint64_t v0 = av[h][i][0], v1 = av[h][i][1];
                const i32x4 A = {(int32_t)(uint32_t)v0, (int32_t)(uint32_t)(v0 >> 32), (int32_t)(uint32_t)v1,
                                 (int32_t)(uint32_t)(v1 >> 32)};
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B[j], start ? zero4 : acc[i][j], 0, 0, 0);
            }
            // A slice ends a group: fold the integer sums with s / 16.
            if (GP > 0 && ((2 * u + h + 1) % (GP > 0 ? GP : 1)) == 0) {
                const int q = GP == 1 ? h : 0;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const float sc = 0.0625f * act_to_float<DT>((uint16_t)sb[q * NJ + j]);
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            accf[GP > 0 ? i : 0][GP > 0 ? j : 0][jj] =
                                __builtin_fmaf(sc, (float)acc[i][j][jj], accf[GP > 0 ? i : 0][GP > 0 ? j : 0][jj]);
                }
            }
        }
        // Stage st + 1 has landed once only the loads issued in steps st - 1
        // and st (operands of steps st + 2, st + 3 and their scales) may be
        // outstanding; the barrier then also frees stage u for step st + 4.
        if (tail) wait_vmcnt<0>();
        else wait_vmcnt<8 + SC2>();
        stage_barrier();
    };

    uint32_t sb0[NSC], sb1[NSC], sb2[NSC], sb3[NSC];
    // Operands of steps 0 .. 2 and scales of steps 0 and 1, in the order the
    // steps keep (the scales of step k before the operands of step k + 1).
#pragma unroll
    for (int h = 0; h < 2; ++h) issue(0, h, a0, b0);
    if (GP == 1 || GP == 2) issue_scales(0, sb0);
#pragma unroll
    for (int h = 0; h < 2; ++h) issue(1, h, a1, b1);
    if (GP != 0) issue_scales(1, sb1);
#pragma unroll
    for (int h = 0; h < 2; ++h) issue(2, h, a2, b2);
    wait_vmcnt<8 + SC2>();
    stage_barrier();
    int64_t st = 0;
    for (; st + 4 <= steps; st += 4) {
        step(st, 0, a0, b0, sb0, sb2, a3, b3, 0);
        step(st + 1, 1, a1, b1, sb1, sb3, a0, b0, 0);
        step(st + 2, 2, a2, b2, sb2, sb0, a1, b1, 0);
        step(st + 3, 3, a3, b3, sb3, sb1, a2, b2, 0);
    }
    if (st < steps) step(st, 0, a0, b0, sb0, sb2, a3, b3, 1);
    if (st + 1 < steps) step(st + 1, 1, a1, b1, sb1, sb3, a0, b0, 2);
    if (st + 2 < steps) step(st + 2, 2, a2, b2, sb2, sb0, a1, b1, 2);
    wait_vmcnt<0>();

    // With K in chunks: this chunk's fp32 results (the row scale and bias
    // follow in w4a8_reduce_kernel).
    if (a.partials != nullptr) {
        const int64_t ldp = a.NT * 16;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t nt = ntb + 4 * wn + j;
            if (nt >= a.NT) continue;
            const int64_t n = nt * 16 + r;
            const float sc = GP == 0 ? 0.0625f * act_to_float<DT>(a.scales[nt * a.Kg * 16 + r]) : 0.f;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t m = m0 + 64 * wm + 16 * i + 4 * g4 + jj;
                    if (m >= a.M || n >= a.N) continue;
                    a.partials[((int64_t)blockIdx.y * a.M + m) * ldp + n] =
                        GP == 0 ? sc * (float)acc[i][j][jj] : accf[GP > 0 ? i : 0][GP > 0 ? j : 0][jj];
                }
        }
        return;
    }

    // Epilogue. The tile goes through LDS so that C is written in whole
    // 16-byte row chunks: once every wave's loads have landed (the steps past
    // K load zeros into the stages), rows 32 q .. 32 q + 31 of the tile go to
    // stage buffer a_q, 512 bytes per row. Chunk c (8 columns) of tile row m
    // sits at chunk c ^ 2 ((m / 4) % 4), which puts the four row groups of a
    // 16 x 16 block on different LDS banks.
    stage_barrier();
    // Lane l holds rows 4 (l / 16) .. +3 of column l % 16 of each block.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        int64_t nt = ntb + 4 * wn + j;
        nt = nt < a.NT ? nt : a.NT - 1;
        const int64_t n = nt * 16 + r;
        const float bv = a.bias && n < a.N ? act_to_float<DT>(a.bias[n]) : 0.f;
        const float sc = GP == 0 ? 0.0625f * act_to_float<DT>(a.scales[nt * a.Kg * 16 + r]) : 0.f;
        const uint32_t col = (uint32_t)(16 * (4 * wn + j) + r);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            unsigned char* rows = wm ? (i < 2 ? a2 : a3) : (i < 2 ? a0 : a1);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                int64_t m = m0 + 64 * wm + 16 * i + 4 * g4 + jj;
                m = m < a.M ? m : a.M - 1;
                const float v = GP == 0 ? sc * (float)acc[i][j][jj] : accf[GP > 0 ? i : 0][GP > 0 ? j : 0][jj];
                const uint32_t row = (uint32_t)(16 * (i & 1) + 4 * g4 + jj);
                const uint32_t off = row * 512 + ((((col >> 3) ^ (2u * (uint32_t)g4)) << 4) | ((col & 7) << 1));
                *reinterpret_cast<uint16_t*>(rows + off) = to_act_bits<DT>(__builtin_fmaf(a.xs[m], v, bv));
            }
        }
    }
    stage_barrier();
    // Thread t stores chunk t % 32 of tile rows 16 p + t / 32, p = 0 .. 7.
    const uint32_t ch = threadIdx.x & 31;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t row = 16 * (p & 1) + (threadIdx.x >> 5);  // row within a_q, q = p / 2
        const unsigned char* rows = p < 2 ? a0 : (p < 4 ? a1 : (p < 6 ? a2 : a3));
        const u32x4 v = *reinterpret_cast<const u32x4*>(rows + row * 512 + ((ch ^ (2u * ((row >> 2) & 3u))) << 4));
        const int64_t m = m0 + 16 * p + (threadIdx.x >> 5);
        const int64_t n = ntb * 16 + 8 * ch;
        if (m < a.M && n < a.N) *reinterpret_cast<u32x4*>(a.C + m * a.ldc + n) = v;
    }
}
}  // namespace

W4a8Plan plan_w4a8(int64_t M, const Geometry& g, bool qa16, int64_t ldq, bool c16) {
    W4a8Plan p;
    p.MI = M <= 16 ? 1 : 2;
    const int64_t KTT = g.Kp / 128;
    p.blocks_n = (g.Np / 16 + 15) / 16;
    p.blocks_m = (M + 16 * p.MI - 1) / (16 * p.MI);
    // Split K until there are about two workgroups per CU; up to 16 rows,
    // chunks of at most 4 k-tiles, whose loads are all in flight at once.
    const int64_t blocks = p.blocks_n * p.blocks_m;
    int64_t ks = (2 * kCUs + blocks - 1) / blocks;
    if (ks > KTT) ks = KTT;
    if (ks < 1) ks = 1;
    p.kc = (KTT + ks - 1) / ks;
    if (p.MI == 1 && p.kc > kA8DecodeChunk) p.kc = kA8DecodeChunk;
    p.ksplit = (KTT + p.kc - 1) / p.kc;
    p.partial_bytes = p.ksplit > 1 ? (size_t)p.ksplit * (size_t)M * (size_t)g.Np * sizeof(float) : 0;

    // The ring kernel from 64 rows when it has 48 tiles of 128 x 256 or K is
    // long enough to split well (on the decode-layer shapes measured it beat
    // this kernel there, by up to 4x at a few hundred rows) and its
    // constraints hold: no K tail, one group per row (at most 131072
    // k, so that the integer sums fit in 32 bits) or groups of 64 to 256 k,
    // 16-byte aligned activation and output rows, and per-tile offsets below
    // 2^31.
    const int64_t m_tiles = (M + 127) / 128, n_blocks = (g.Np / 16 + 15) / 16;
    const bool groups_ok = g.Kg == 1 ? g.Kp <= 131072 : (g.Ge >= 64 && g.Ge <= 256);
    const int64_t rtiles = m_tiles * n_blocks;
    const bool big_enough = M >= kA8RingMinM && (rtiles >= kA8RingMinTiles || g.K >= kA8RingMinK);
    const bool offsets_ok = rtiles <= (1 << 22) && 128 * ldq + g.K < ((int64_t)1 << 31) &&
                            16 * (g.Kp / 128) * 1024 < ((int64_t)1 << 31);
    if (qa16 && c16 && g.Kp == g.K && groups_ok && big_enough && offsets_ok) {
        p.ring = g.Kg == 1 ? 0 : (int)(g.Ge / 64);
        p.m_tiles = m_tiles;
        p.n_blocks = n_blocks;
        // Fewer tiles than CUs: K in chunks of at least kA8RingMinChunk k-tiles
        // (whole groups of 256 k), up to about one workgroup per CU.
        int64_t ks = (kCUs + rtiles - 1) / rtiles;
        if (ks > KTT / kA8RingMinChunk) ks = KTT / kA8RingMinChunk;
        if (ks < 1) ks = 1;
        int64_t kc = (KTT + ks - 1) / ks;
        if (p.ring == 4 && (kc & 1)) ++kc;
        p.kc = kc;
        p.ksplit = (KTT + kc - 1) / kc;
        p.partial_bytes = p.ksplit > 1 ? (size_t)p.ksplit * (size_t)M * (size_t)g.Np * sizeof(float) : 0;
    }
    return p;
}

hipError_t launch_a8_quant(const void* A, int64_t M, int64_t K, int64_t lda, int dtype, int8_t* qa, int64_t ldq,
                           float* xs, hipStream_t stream) {
    const uint16_t* a = static_cast<const uint16_t*>(A);
    const int64_t cpt = (K / 8 + 255) / 256;  // 16-byte chunks per thread
    const dim3 grid((unsigned)M), block(256);
#define A8Q(D, C) hipLaunchKernelGGL((a8_quant_reg_kernel<D, C>), grid, block, 0, stream, a, lda, K, qa, ldq, xs)
    if (cpt <= 8) {
        if (dtype == 0) {
            if (cpt <= 1) A8Q(0, 1);
            else if (cpt <= 2) A8Q(0, 2);
            else if (cpt <= 4) A8Q(0, 4);
            else A8Q(0, 8);
        } else {
            if (cpt <= 1) A8Q(1, 1);
            else if (cpt <= 2) A8Q(1, 2);
            else if (cpt <= 4) A8Q(1, 4);
            else A8Q(1, 8);
        }
    } else if (dtype == 0) {
        hipLaunchKernelGGL((a8_quant_kernel<0>), grid, block, 0, stream, a, lda, K, qa, ldq, xs);
    } else {
        hipLaunchKernelGGL((a8_quant_kernel<1>), grid, block, 0, stream, a, lda, K, qa, ldq, xs);
    }
#undef A8Q
    return hipGetLastError();
}

hipError_t launch_w4a8(const int8_t* qa, const float* xs, int64_t M, int64_t ldq, const void* packed, const Geometry& g,
                       int dtype, const void* bias, void* C, int64_t ldc, const W4a8Plan& p, void* workspace,
                       hipStream_t stream) {
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    A8Args a;
    a.qa = qa;
    a.xs = xs;
    a.M = M;
    a.ldq = ldq;
    a.K = g.K;
    a.codes = reinterpret_cast<const u32x4*>(base);
    a.scales = reinterpret_cast<const uint16_t*>(base + g.scales_off);
    a.NT = g.Np / 16;
    a.N = g.N;
    a.KTT = g.Kp / 128;
    a.Kg = g.Kg;
    a.Ge = g.Ge;
    a.one_group = g.Kg == 1;
    a.kc = p.kc;
    a.bias = static_cast<const uint16_t*>(bias);
    a.C = static_cast<uint16_t*>(C);
    a.ldc = ldc;
    a.partials = p.ksplit > 1 ? static_cast<float*>(workspace) : nullptr;
    a.n_blocks = p.n_blocks;
    if (p.ring >= 0) {
        const dim3 rgrid((unsigned)(p.m_tiles * p.n_blocks), (unsigned)p.ksplit);
#define W4A8_RING(D, G) hipLaunchKernelGGL((w4a8_ring_kernel<D, G>), rgrid, dim3(512), 0, stream, a)
        if (dtype == 0) {
            if (p.ring == 0) W4A8_RING(0, 0);
            else if (p.ring == 1) W4A8_RING(0, 1);
            else if (p.ring == 2) W4A8_RING(0, 2);
            else W4A8_RING(0, 4);
        } else {
            if (p.ring == 0) W4A8_RING(1, 0);
            else if (p.ring == 1) W4A8_RING(1, 1);
            else if (p.ring == 2) W4A8_RING(1, 2);
            else W4A8_RING(1, 4);
        }
#undef W4A8_RING
    } else {
        const dim3 grid((unsigned)p.blocks_n, (unsigned)p.blocks_m, (unsigned)p.ksplit);
        if (dtype == 0) {
            if (p.MI == 1) hipLaunchKernelGGL((w4a8_kernel<0, 1, kA8DecodeChunk>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((w4a8_kernel<0, 2, 2>), grid, dim3(256), 0, stream, a);
        } else {
            if (p.MI == 1) hipLaunchKernelGGL((w4a8_kernel<1, 1, kA8DecodeChunk>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((w4a8_kernel<1, 2, 2>), grid, dim3(256), 0, stream, a);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ksplit == 1) return e;
    const dim3 rgrid((unsigned)((M * g.N + 255) / 256));
    const uint16_t* b = static_cast<const uint16_t*>(bias);
    uint16_t* c = static_cast<uint16_t*>(C);
    if (dtype == 0)
        hipLaunchKernelGGL((w4a8_reduce_kernel<0>), rgrid, dim3(256), 0, stream, a.partials, p.ksplit, M, g.N, g.Np, xs, b, c, ldc);
    else
        hipLaunchKernelGGL((w4a8_reduce_kernel<1>), rgrid, dim3(256), 0, stream, a.partials, p.ksplit, M, g.N, g.Np, xs, b, c, ldc);
    return hipGetLastError();
}

}  // namespace w4a16
