// w4a8.hip -- the W4A8 variant: activations quantised per token to symmetric
// int8, symmetric int4 weights from the same packed buffer, int8 MFMA.
//
// The operation is the one the "mixed_precision" package page gives for
// XPUW4A8IntLinearKernel (class docstring and `apply_weights`): each row of x
// is quantised dynamically to symmetric int8 with one scale per row, and the
// int8 rows are multiplied by the int4 weights (uint4b8, zero 8) with the row
// scale and the weight's group scales:
//     C[m, n] = xs[m] * sum_g s[n, g] * sum_{k in g} qa[m, k] * (q[n, k] - 8)
// The integer sums run on v_mfma_i32_16x16x32_i8 and are exact; the group
// scale is applied to each group's integer sum in fp32, the row scale and
// bias at the end, and C is rounded once.
#include "device_common.h"
#include "internal.h"

namespace w4a16 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr int kA8DecodeChunk = 4;  // k-tiles per K chunk (and register stages) for up to 16 rows

// ---------------------------------------------------------------- quantiser

// One workgroup of 256 threads per row. The scale is fp32(max |x|) / 127
// (IEEE division); each value becomes rint(x / scale) (half to even),
// which stays within [-127, 127] because |x| <= max |x|; a row of zeros
// gets scale 0 and codes 0. K % 8 == 0: each thread handles 8-element chunks.
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
                out[e >> 2] |= ((uint32_t)iv & 0xFFu) << (8 * (e & 3));
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
};

// Bytes of one activation chunk (k .. k+7 of a row) in the order the packed
// weight word gives its codes after the nibble split below: 0,4,1,5 | 2,6,3,7.
__device__ __forceinline__ int64_t a_operand(uint2 v) {
    const uint32_t lo = __builtin_amdgcn_perm(v.y, v.x, 0x05010400u);
    const uint32_t hi = __builtin_amdgcn_perm(v.y, v.x, 0x07030602u);
    return (int64_t)(((uint64_t)hi << 32) | lo);
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

}  // namespace

W4a8Plan plan_w4a8(int64_t M, const Geometry& g) {
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
    return p;
}

hipError_t launch_a8_quant(const void* A, int64_t M, int64_t K, int64_t lda, int dtype, int8_t* qa, int64_t ldq,
                           float* xs, hipStream_t stream) {
    const uint16_t* a = static_cast<const uint16_t*>(A);
    if (dtype == 0) hipLaunchKernelGGL((a8_quant_kernel<0>), dim3((unsigned)M), dim3(256), 0, stream, a, lda, K, qa, ldq, xs);
    else hipLaunchKernelGGL((a8_quant_kernel<1>), dim3((unsigned)M), dim3(256), 0, stream, a, lda, K, qa, ldq, xs);
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
    const dim3 grid((unsigned)p.blocks_n, (unsigned)p.blocks_m, (unsigned)p.ksplit);
    if (dtype == 0) {
        if (p.MI == 1) hipLaunchKernelGGL((w4a8_kernel<0, 1, kA8DecodeChunk>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((w4a8_kernel<0, 2, 2>), grid, dim3(256), 0, stream, a);
    } else {
        if (p.MI == 1) hipLaunchKernelGGL((w4a8_kernel<1, 1, kA8DecodeChunk>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((w4a8_kernel<1, 2, 2>), grid, dim3(256), 0, stream, a);
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
