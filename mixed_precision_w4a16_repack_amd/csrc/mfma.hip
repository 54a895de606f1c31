// mfma.hip -- W4A16 GEMM for large M (prefill), a dense contraction on the
// gfx950 matrix cores.
//
// Prior art: the fused dequant-GEMM Triton kernels of the pages
// (`_triton_w4a16_skinny_fmt_kernel` on the "rdna_hybrid_w4a16" pages,
// `triton_w4a16_gemm_kernel` on the MI300 "triton_w4a16.py" page): per K step
// they load an activation tile and a packed weight tile, unpack, subtract the
// zero, scale, and accumulate a dot product in fp32. This kernel keeps that
// arithmetic and lays the work out for CDNA4:
//
//  * A workgroup of 4 wavefronts computes a BM x (64*WNT) tile of C. All four
//    waves share the BM activation rows; each wave owns WNT distinct 16-column
//    n-tiles, so every weight word is loaded and dequantised exactly once per
//    workgroup, in registers, straight from one 16-byte load per lane of the
//    packed tile (which is already in MFMA B-operand order).
//  * The activation tile (BM x 128 per K step) is staged in LDS in
//    "fragment order": 1 KB per (16 rows x 32 k) block, lane l's 16 bytes at
//    offset 16*l, so every A-operand read is one conflict-free ds_read_b128.
//    Two LDS buffers alternate: the next tile is fetched while the current
//    one feeds the MFMAs; one barrier per K step.
//  * Each wave issues v_mfma_f32_16x16x32_{f16,bf16}; (BM/16) x WNT
//    accumulators of 4 fp32 per lane (256 fp32 at BM = 256, WNT = 4) live in
//    the accumulation registers.
//  * Epilogue: + bias in fp32, one rounding to the act dtype, store.
#include "device_common.h"
#include "internal.h"

namespace w4a16 {
namespace {

struct MfmaArgs {
    const uint16_t* A;
    int64_t lda;
    int64_t M;
    const u32x4* codes;
    const uint16_t* scales;
    const uint8_t* zeros;
    int64_t N;
    int64_t KTT;  // K / 128
    int64_t Kg;
    int gshift;
    int one_group;
    const uint16_t* bias;
    uint16_t* C;
    int64_t ldc;
    int64_t m_tiles, n_blocks;
};

template <int DT, int QT, int BM, int WNT, int SPT>
__global__ __launch_bounds__(256) void mfma_kernel(MfmaArgs a) {
    constexpr int MB = BM / 16;            // 16-row blocks per tile
    constexpr int CHUNKS = MB * 4;         // 1 KB A chunks per K step
    constexpr int CPW = CHUNKS / 4;        // chunks loaded per wave
    constexpr int BUF_BYTES = BM * 128 * 2;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;

    const int64_t b = blockIdx.x;
    const int64_t nb_idx = b % a.n_blocks;
    const int64_t mt = b / a.n_blocks;
    const int64_t m0 = mt * BM;
    const int64_t NT = a.N / 16;

    // This wave's n-tiles (clamped for loads when N is not a multiple of the
    // workgroup width; clamped tiles are never stored).
    int64_t nt_of[WNT];
    int64_t nt_ld[WNT];
#pragma unroll
    for (int nb = 0; nb < WNT; ++nb) {
        nt_of[nb] = nb_idx * (4 * WNT) + wave * WNT + nb;
        nt_ld[nb] = nt_of[nb] < NT ? nt_of[nb] : NT - 1;
    }

    // A chunk c = wave * CPW + i covers rows 16*(c/4) .. +15, k 32*(c%4) .. +31
    // of the current K step; lane l loads row 16*(c/4) + l%16 (clamped to
    // M - 1) at k offset 32*(c%4) + 8*(l/16).
    const uint16_t* a_src[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = wave * CPW + i;
        int64_t row = m0 + 16 * (c >> 2) + r;
        if (row > a.M - 1) row = a.M - 1;
        a_src[i] = a.A + row * a.lda + 32 * (c & 3) + 8 * g4;
    }

    auto load_a = [&](int64_t kt, u32x4 (&regs)[CPW]) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) regs[i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * 128);
    };
    auto store_a = [&](int buf, const u32x4 (&regs)[CPW]) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = wave * CPW + i;
            *reinterpret_cast<u32x4*>(smem + buf * BUF_BYTES + (c * 64 + lane) * 16) = regs[i];
        }
    };
    auto load_b = [&](int64_t kt, u32x4 (&raw)[WNT], uint16_t (&sb)[WNT][SPT], uint8_t (&zb)[WNT][SPT]) {
#pragma unroll
        for (int nb = 0; nb < WNT; ++nb) {
            raw[nb] = __builtin_nontemporal_load(a.codes + (nt_ld[nb] * a.KTT + kt) * 64 + lane);
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int64_t k = kt * 128 + u * (128 / SPT);
                const int64_t g = a.one_group ? 0 : (k >> a.gshift);
                const int64_t idx = (nt_ld[nb] * a.Kg + g) * 16 + r;
                sb[nb][u] = a.scales[idx];
                zb[nb][u] = QT ? a.zeros[idx] : (uint8_t)8;
            }
        }
    };

    // Dequant operands in registers (see and_or).
    uint32_t dq_mask = 0x000F000Fu, dq_magic = kMagic<DT>;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));

    floatx4 acc[MB][WNT];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < WNT; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

    u32x4 areg[CPW];
    u32x4 braw[WNT];
    uint16_t sb[WNT][SPT];
    uint8_t zb[WNT][SPT];
    load_a(0, areg);
    load_b(0, braw, sb, zb);
    store_a(0, areg);
    __syncthreads();

    for (int64_t kt = 0; kt < a.KTT; ++kt) {
        const int buf = (int)(kt & 1);
        const bool more = kt + 1 < a.KTT;
        u32x4 braw_n[WNT];
        uint16_t sb_n[WNT][SPT];
        uint8_t zb_n[WNT][SPT];
        if (more) {
            load_a(kt + 1, areg);
            load_b(kt + 1, braw_n, sb_n, zb_n);
        }
        const unsigned char* abase = smem + buf * BUF_BYTES + lane * 16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 bq[WNT];
#pragma unroll
            for (int nb = 0; nb < WNT; ++nb) {
                const int u = s / (4 / SPT);
                bq[nb] = Dequant<DT>::apply(braw[nb][s], Dequant<DT>::make(sb[nb][u], zb[nb][u]), dq_mask, dq_magic);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(abase + (mb * 4 + s) * 1024);
#pragma unroll
                for (int nb = 0; nb < WNT; ++nb) acc[mb][nb] = mfma16x16x32<DT>(av, bq[nb], acc[mb][nb]);
            }
        }
        if (more) {
            store_a(buf ^ 1, areg);
#pragma unroll
            for (int nb = 0; nb < WNT; ++nb) {
                braw[nb] = braw_n[nb];
#pragma unroll
                for (int u = 0; u < SPT; ++u) {
                    sb[nb][u] = sb_n[nb][u];
                    zb[nb][u] = zb_n[nb][u];
                }
            }
        }
        __syncthreads();
    }

    // Epilogue: lane l holds rows 4*(l/16) .. +3 of column l%16 of each block.
#pragma unroll
    for (int nb = 0; nb < WNT; ++nb) {
        if (nt_of[nb] >= NT) continue;
        const int64_t n = nt_of[nb] * 16 + r;
        const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int64_t m = m0 + 16 * mb + 4 * g4 + jj;
                if (m < a.M) a.C[m * a.ldc + n] = to_act_bits<DT>(acc[mb][nb][jj] + bv);
            }
        }
    }
}

template <int DT, int QT, int BM, int WNT>
hipError_t launch_mfma_t(const MfmaArgs& a, int spt, dim3 grid, hipStream_t stream) {
    const size_t lds = 2 * (size_t)BM * 128 * 2;
    hipError_t e = hipSuccess;
    switch (spt) {
        case 1:
            e = allow_lds<mfma_kernel<DT, QT, BM, WNT, 1>>(lds);
            if (e == hipSuccess) hipLaunchKernelGGL((mfma_kernel<DT, QT, BM, WNT, 1>), grid, dim3(256), lds, stream, a);
            break;
        case 2:
            e = allow_lds<mfma_kernel<DT, QT, BM, WNT, 2>>(lds);
            if (e == hipSuccess) hipLaunchKernelGGL((mfma_kernel<DT, QT, BM, WNT, 2>), grid, dim3(256), lds, stream, a);
            break;
        default:
            e = allow_lds<mfma_kernel<DT, QT, BM, WNT, 4>>(lds);
            if (e == hipSuccess) hipLaunchKernelGGL((mfma_kernel<DT, QT, BM, WNT, 4>), grid, dim3(256), lds, stream, a);
            break;
    }
    return e != hipSuccess ? e : hipGetLastError();
}

template <int DT, int QT>
hipError_t launch_mfma_q(const MfmaArgs& a, const MfmaPlan& p, int spt, dim3 grid, hipStream_t stream) {
    if (p.BM == 256) {
        return p.BN == 256 ? launch_mfma_t<DT, QT, 256, 4>(a, spt, grid, stream)
                           : launch_mfma_t<DT, QT, 256, 2>(a, spt, grid, stream);
    }
    return p.BN == 256 ? launch_mfma_t<DT, QT, 128, 4>(a, spt, grid, stream)
                       : launch_mfma_t<DT, QT, 128, 2>(a, spt, grid, stream);
}

}  // namespace

MfmaPlan plan_mfma(int64_t M, const Geometry& g) {
    MfmaPlan p;
    p.BM = M > 128 ? 256 : 128;
    // Prefer the wider tile unless it leaves most of the 256 CUs idle.
    const int64_t mt = (M + p.BM - 1) / p.BM;
    const int64_t wide = mt * ((g.N + 255) / 256);
    p.BN = wide >= 256 ? 256 : 128;
    return p;
}

hipError_t launch_mfma(const void* A, int64_t M, int64_t lda, const void* packed, const Geometry& g, int dtype,
                       const void* bias, void* C, int64_t ldc, const MfmaPlan& p, hipStream_t stream) {
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    MfmaArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.lda = lda;
    a.M = M;
    a.codes = reinterpret_cast<const u32x4*>(base);
    a.scales = reinterpret_cast<const uint16_t*>(base + g.scales_off);
    a.zeros = g.qtype == 1 ? base + g.zeros_off : nullptr;
    a.N = g.N;
    a.KTT = g.K / 128;
    a.Kg = g.Kg;
    a.gshift = g.gshift;
    a.one_group = g.Kg == 1;
    a.bias = static_cast<const uint16_t*>(bias);
    a.C = static_cast<uint16_t*>(C);
    a.ldc = ldc;
    a.m_tiles = (M + p.BM - 1) / p.BM;
    a.n_blocks = (g.N + p.BN - 1) / p.BN;
    const dim3 grid((unsigned)(a.m_tiles * a.n_blocks));
    const int spt = g.Kg == 1 ? 1 : (g.Ge >= 128 ? 1 : 128 / g.Ge);
    if (dtype == 0) return g.qtype ? launch_mfma_q<0, 1>(a, p, spt, grid, stream) : launch_mfma_q<0, 0>(a, p, spt, grid, stream);
    return g.qtype ? launch_mfma_q<1, 1>(a, p, spt, grid, stream) : launch_mfma_q<1, 0>(a, p, spt, grid, stream);
}

}  // namespace w4a16
