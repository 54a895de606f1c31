// skinny.hip -- W4A16 GEMM for M <= 16 rows (decode), bound by the weight
// stream from HBM.
//
// Prior art: the HIP skinny kernel the "rdna_hybrid_w4a16" pages dispatch to
// for small M (`_rdna_hybrid_w4a16_apply_impl`, `wvSplitK_int4_g`: wave-level
// split-K sized by the CU count, activations staged in LDS). Its source is not
// on the pages; this kernel is designed for gfx950 from the packed layout:
//
//  * Work unit: one wave streams KT consecutive 1 KB tiles of one n-tile (16
//    rows x 128 k each) with one 16-byte load per lane per tile, all issued
//    before any arithmetic, so a workgroup keeps WN*WK*KT KB in flight.
//  * A workgroup is WN x WK waves: WN n-tiles share one K range whose
//    activation rows are staged once in LDS; WK waves split that range.
//  * ksplit workgroups split K further. Each writes fp32 partial sums to the
//    workspace and bumps an arrival counter; the last to arrive sums the
//    partials in a fixed order, adds the bias and writes C, then clears the
//    counter. No float atomics: the result is deterministic.
//  * The inner product is one v_mfma_f32_16x16x32 per word (M padded to 16
//    with zeros), so the VALU only dequantises (about two ops per code).
//  * Workgroups that share an n-group are numbered so that round-robin
//    dispatch places them on the same XCD, keeping their partials and counter
//    in one L2.
#include "device_common.h"
#include "internal.h"

namespace w4a16 {
namespace {

struct SkinnyArgs {
    const uint16_t* A;
    int64_t lda;
    int M;
    const u32x4* codes;
    const uint16_t* scales;
    const uint8_t* zeros;
    int64_t KTT;  // K / 128
    int64_t Kg;
    int gshift;
    int one_group;
    const uint16_t* bias;
    uint16_t* C;
    int64_t ldc;
    float* partials;
    uint32_t* counters;
    int WN, WK, ksplit;
    int64_t n_groups;
    int xcd_map;
};

template <int DT, int QT, int KT, int SPT>
__global__ __launch_bounds__(1024) void skinny_kernel(SkinnyArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % a.WN, wk = wave / a.WN;
    const int r = lane & 15, g4 = lane >> 4;

    // Block -> (n-group, k-split). With xcd_map, the blocks of XCD x (block
    // ids congruent to x mod 8) take a contiguous run of (ng, ks) pairs that
    // holds whole n-groups.
    int64_t p = blockIdx.x;
    if (a.xcd_map) {
        const int64_t per = (a.n_groups * a.ksplit) >> 3;
        p = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int64_t ng = p / a.ksplit;
    const int ks = (int)(p - ng * a.ksplit);

    const int64_t nt = ng * a.WN + wn;
    const int64_t kt_wg = (int64_t)ks * (a.WK * KT);
    const int64_t kt0 = kt_wg + (int64_t)wk * KT;

    // 1. Weight stream: KT 16-byte loads per lane, issued first.
    u32x4 wq[KT];
    const u32x4* src = a.codes + (nt * a.KTT + kt0) * 64 + lane;
#pragma unroll
    for (int j = 0; j < KT; ++j) wq[j] = __builtin_nontemporal_load(src + j * 64);

    // Scales (and zeros): SPT groups per tile; word s uses sub-block s / (4 / SPT).
    uint16_t sb[KT][SPT];
    uint8_t zb[KT][SPT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int64_t k = (kt0 + j) * 128 + u * (128 / SPT);
            const int64_t g = a.one_group ? 0 : (k >> a.gshift);
            const int64_t idx = (nt * a.Kg + g) * 16 + r;
            sb[j][u] = a.scales[idx];
            zb[j][u] = QT ? a.zeros[idx] : (uint8_t)8;
        }
    }

    // 2. Stage A[0:M, kt_wg*128 : +KR] in LDS, row stride KR + 8 elements.
    const int KR = a.WK * KT * 128;
    const int lds_ld = KR + 8;
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);
    {
        const int cpr = KR / 8;  // 16-byte chunks per row
        const int total = a.M * cpr;
        for (int c = threadIdx.x; c < total; c += blockDim.x) {
            const int m = c / cpr, cc = c - m * cpr;
            const u32x4 v = *reinterpret_cast<const u32x4*>(a.A + (int64_t)m * a.lda + kt_wg * 128 + cc * 8);
            *reinterpret_cast<u32x4*>(As + m * lds_ld + cc * 8) = v;
        }
    }
    __syncthreads();

    // 3. Dequantise and multiply.
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool row_live = r < a.M;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int u = s / (4 / SPT);
            const typename Dequant<DT>::Params dp = Dequant<DT>::make(sb[j][u], zb[j][u]);
            const u32x4 b = Dequant<DT>::apply(wq[j][s], dp);
            u32x4 av = {0u, 0u, 0u, 0u};
            if (row_live)
                av = *reinterpret_cast<const u32x4*>(As + r * lds_ld + (wk * KT + j) * 128 + 32 * s + 8 * g4);
            acc = mfma16x16x32<DT>(av, b, acc);
        }
    }

    // 4. Reduce the WK waves of each n-tile in LDS (fixed order).
    float* red = reinterpret_cast<float*>(smem + (size_t)a.M * lds_ld * 2);
    if (a.WK > 1) {
        *reinterpret_cast<floatx4*>(red + ((size_t)wave * 64 + lane) * 4) = acc;
        __syncthreads();
        if (wk == 0) {
            for (int q = 1; q < a.WK; ++q)
                acc += *reinterpret_cast<const floatx4*>(red + ((size_t)(q * a.WN + wn) * 64 + lane) * 4);
        }
    }

    const int64_t n = nt * 16 + r;
    if (a.ksplit == 1) {
        if (wk == 0) {
            const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 4 * g4 + jj;
                if (m < a.M) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(acc[jj] + bv);
            }
        }
        return;
    }

    // 5. Split-K across workgroups: partials [ng][ks][m][16*WN].
    const int width = 16 * a.WN;
    float* part = a.partials + (ng * a.ksplit) * (int64_t)a.M * width;
    if (wk == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int m = 4 * g4 + jj;
            if (m < a.M) part[((int64_t)ks * a.M + m) * width + wn * 16 + r] = acc[jj];
        }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counters + ng, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(a.ksplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int entries = a.M * width;
    for (int e = threadIdx.x; e < entries; e += blockDim.x) {
        const int m = e / width, col = e - m * width;
        float sum = 0.f;
        for (int q = 0; q < a.ksplit; ++q)
            sum += __builtin_nontemporal_load(part + ((int64_t)q * a.M + m) * width + col);
        const int64_t nn = ng * width + col;
        if (a.bias) sum += act_to_float<DT>(a.bias[nn]);
        a.C[(int64_t)m * a.ldc + nn] = to_act_bits<DT>(sum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + ng, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int QT, int KT>
hipError_t launch_skinny_kt(const SkinnyArgs& a, int spt, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
    hipError_t e = hipSuccess;
    switch (spt) {
        case 1:
            e = allow_lds<skinny_kernel<DT, QT, KT, 1>>(lds);
            if (e == hipSuccess) hipLaunchKernelGGL((skinny_kernel<DT, QT, KT, 1>), grid, block, lds, stream, a);
            break;
        case 2:
            e = allow_lds<skinny_kernel<DT, QT, KT, 2>>(lds);
            if (e == hipSuccess) hipLaunchKernelGGL((skinny_kernel<DT, QT, KT, 2>), grid, block, lds, stream, a);
            break;
        default:
            e = allow_lds<skinny_kernel<DT, QT, KT, 4>>(lds);
            if (e == hipSuccess) hipLaunchKernelGGL((skinny_kernel<DT, QT, KT, 4>), grid, block, lds, stream, a);
            break;
    }
    return e != hipSuccess ? e : hipGetLastError();
}

template <int DT, int QT>
hipError_t launch_skinny_q(const SkinnyArgs& a, int KT, int spt, dim3 grid, dim3 block, size_t lds,
                           hipStream_t stream) {
    switch (KT) {
        case 1: return launch_skinny_kt<DT, QT, 1>(a, spt, grid, block, lds, stream);
        case 2: return launch_skinny_kt<DT, QT, 2>(a, spt, grid, block, lds, stream);
        case 4: return launch_skinny_kt<DT, QT, 4>(a, spt, grid, block, lds, stream);
        default: return launch_skinny_kt<DT, QT, 8>(a, spt, grid, block, lds, stream);
    }
}

}  // namespace

// LDS bytes of a skinny workgroup holding m rows of activations.
static size_t skinny_lds_bytes(int64_t m, int WN, int WK, int KT) {
    size_t lds = (size_t)m * (WK * KT * 128 + 8) * 2;
    lds = (lds + 15) / 16 * 16;
    if (WK > 1) lds += (size_t)WN * WK * 64 * 4 * sizeof(float);
    return lds;
}

SkinnyPlan plan_skinny(int64_t M, const Geometry& g) {
    (void)M;  // the plan is sized for 16 rows so one workspace fits every M
    SkinnyPlan p;
    const int64_t NT = g.N / 16, KTT = g.K / 128;
    p.WN = NT % 4 == 0 ? 4 : (NT % 2 == 0 ? 2 : 1);
    p.KT = KTT % 4 == 0 ? 4 : (KTT % 2 == 0 ? 2 : 1);
    const int64_t chunks = KTT / p.KT;  // k-chunks of KT tiles
    p.n_groups = NT / p.WN;
    // Aim for at least 512 workgroups of at most 16 waves and 96 KB of LDS;
    // prefer splitting K inside a workgroup (WK) over splitting it across
    // workgroups (ksplit), whose partial sums cost workspace traffic.
    p.ksplit = (int)chunks;
    for (int64_t ks = 1; ks <= chunks; ++ks) {
        if (chunks % ks) continue;
        const int64_t wk = chunks / ks;
        if (p.WN * wk > 16 || skinny_lds_bytes(16, p.WN, (int)wk, p.KT) > 96 * 1024) continue;
        p.ksplit = (int)ks;
        if (p.n_groups * ks >= 512) break;
    }
    p.WK = (int)(chunks / p.ksplit);
    if (p.ksplit > 1) p.partial_bytes = (size_t)p.ksplit * 16 * (size_t)g.N * sizeof(float);
    p.counter_bytes = p.ksplit > 1 ? (size_t)p.n_groups * sizeof(uint32_t) : 0;
    return p;
}

hipError_t launch_skinny(const void* A, int64_t M, int64_t lda, const void* packed, const Geometry& g, int dtype,
                         const void* bias, void* C, int64_t ldc, const SkinnyPlan& p, void* workspace,
                         hipStream_t stream) {
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    SkinnyArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.lda = lda;
    a.M = (int)M;
    a.codes = reinterpret_cast<const u32x4*>(base);
    a.scales = reinterpret_cast<const uint16_t*>(base + g.scales_off);
    a.zeros = g.qtype == 1 ? base + g.zeros_off : nullptr;
    a.KTT = g.K / 128;
    a.Kg = g.Kg;
    a.gshift = g.gshift;
    a.one_group = g.Kg == 1;
    a.bias = static_cast<const uint16_t*>(bias);
    a.C = static_cast<uint16_t*>(C);
    a.ldc = ldc;
    a.counters = static_cast<uint32_t*>(workspace);
    a.partials = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kCounterRegionBytes) : nullptr;
    a.WN = p.WN;
    a.WK = p.WK;
    a.ksplit = p.ksplit;
    a.n_groups = p.n_groups;
    const int64_t nblocks = p.n_groups * p.ksplit;
    a.xcd_map = (nblocks % 8 == 0) && ((nblocks / 8) % p.ksplit == 0);
    const int spt = g.Kg == 1 ? 1 : (g.Ge >= 128 ? 1 : 128 / g.Ge);
    const dim3 grid((unsigned)nblocks), block((unsigned)(64 * p.WN * p.WK));
    const size_t lds = skinny_lds_bytes(M, p.WN, p.WK, p.KT);
    const int qt = g.qtype;
    if (dtype == 0)
        return qt ? launch_skinny_q<0, 1>(a, p.KT, spt, grid, block, lds, stream)
                  : launch_skinny_q<0, 0>(a, p.KT, spt, grid, block, lds, stream);
    return qt ? launch_skinny_q<1, 1>(a, p.KT, spt, grid, block, lds, stream)
              : launch_skinny_q<1, 0>(a, p.KT, spt, grid, block, lds, stream);
}

}  // namespace w4a16
