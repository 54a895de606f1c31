// mfma.hip -- W4A16 GEMM for large M (prefill), a dense contraction on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_{f16,bf16}).
//
// Prior art: the fused dequant-GEMM Triton kernels of the pages
// (`_triton_w4a16_skinny_fmt_kernel` on the "rdna_hybrid_w4a16" pages,
// `triton_w4a16_gemm_kernel` on the MI300 "triton_w4a16.py" page): per K step
// they load an activation tile and a packed weight tile, unpack, subtract the
// zero, scale, and accumulate a dot product in fp32. Three kernels keep that
// arithmetic and lay the work out for CDNA4:
//
//  * mfma_wide_kernel / mfma_wide_grouped_kernel: 128 x 512 tiles for large
//    M and N (one group per row; groups of 128 k or more), double-buffered
//    in LDS, the group scales of the grouped one applied by rescaling one
//    set of accumulators.
//  * mfma_ring_kernel: 128 x 256 tiles when they give at least one
//    workgroup per CU, for one group per row or groups of 128 k or more.
//    Activation and weight tiles go from HBM/L2 straight into a three-stage
//    LDS ring (direct 16-byte buffer loads).
//    These three dequantise offset-corrected: exact values 1 + q/16 into
//    the MFMA (TopNibble), the offset removed with row sums and the scale
//    applied once per row or group.
//  * mfma_splitk_kernel + splitk_reduce_kernel: medium M (tens to a few
//    hundred rows), any group size, K split over workgroups so that the
//    tiles fill the CUs; scale first, per weight, as the pages do.
//  * mfma_lds_kernel: 64-column tiles (a K tail, or a workspace too small
//    for split-K); activation tiles go straight into two LDS buffers, the
//    weights into registers.
// All address a workgroup's operands through buffer descriptors based at
// its own tile, so A and the packed weight may be of any size.
// Every kernel stages activations in LDS in "fragment order" (1 KB per
// 16 rows x 32 k, lane l's 16 bytes at 16*l) so that each A-operand read is
// one conflict-free ds_read_b128, reads the packed weight tiles, which are
// already in B-operand order, and ends with bias in fp32, one rounding to
// the act dtype, and the store.
#include <type_traits>

#include "device_common.h"
#include "exchange.h"
#include "internal.h"
#include "lds_stage.h"

namespace w4a16 {
namespace {

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N - 1 (compile-time
// indices, e.g. of named LDS stages).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_impl<I + 1, N>(f);
    }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<0, N>(f);
}

struct MfmaArgs {
    const uint16_t* A;
    int64_t lda;
    int64_t M;
    const u32x4* codes;
    const uint16_t* scales;
    const uint8_t* zeros;
    int64_t N;    // N rounded up to 16: the n-tiles of the packed weight
    int64_t KTT;  // padded K / 128
    int64_t K;    // K: activation columns past it read as zero
    int64_t Kg;
    int gshift;
    int one_group;
    const uint16_t* bias;
    uint16_t* C;
    int64_t ldc;
    int64_t m_tiles, n_blocks;
    int64_t tile0;  // mfma_ring_kernel: first 128 x 256 tile (row-major over m-tiles x n-blocks)
    int64_t Nst;    // columns of C (N above is rounded up to 16); stores and bias stop at Nst
    // mfma_splitk_kernel: K steps split over ksplit workgroups of spk steps;
    // partial tiles in the workspace, after its counter region (which the
    // tiled kernels leave untouched).
    int64_t ksplit, spk;
    float* partials;
};

// One workgroup's operands as buffer bases and byte extents: rows
// [mb, mb + rows) of A with mb = min(m0, M - 1) (a half tile may start past
// a ragged M; its rows then all clamp to M - 1 >= mb), and n-tiles
// [nt0, nt0 + ntn) of the packed weight (nt0 < N/16).
// The kernels form 32-bit offsets from these per-workgroup bases, which stay
// below 2^31 whatever the sizes of A and of the weight (the host checks
// (128 * lda + K) * 2 < 2^31, which with lda >= K also bounds the 128*K bytes
// of codes of 16 n-tiles).
struct TileBufs {
    int64_t mb;  // row of A at the base
    const uint16_t* A;
    const u32x4* codes;
    const uint16_t* scales;
    const uint8_t* zeros;
    uint32_t a_bytes, codes_bytes, scales_bytes, zeros_bytes;
};

__device__ __forceinline__ TileBufs tile_bufs(const MfmaArgs& a, int64_t m0, int64_t rows, int64_t nt0, int64_t ntn) {
    const int64_t NT = a.N / 16;
    TileBufs t;
    t.mb = m0 < a.M - 1 ? m0 : a.M - 1;
    const int64_t mr = a.M - t.mb < rows ? a.M - t.mb : rows;  // >= 1 rows of A
    const int64_t nn = NT - nt0 < ntn ? NT - nt0 : ntn;        // >= 1 n-tiles
    t.A = a.A + t.mb * a.lda;
    t.a_bytes = (uint32_t)(((mr - 1) * a.lda + a.K) * 2);
    t.codes = a.codes + nt0 * a.KTT * 64;
    t.codes_bytes = (uint32_t)(nn * a.KTT * 1024);
    t.scales = a.scales + nt0 * a.Kg * 16;
    t.scales_bytes = (uint32_t)(nn * a.Kg * 32);
    t.zeros = a.zeros != nullptr ? a.zeros + nt0 * a.Kg * 16 : nullptr;
    t.zeros_bytes = a.zeros != nullptr ? (uint32_t)(nn * a.Kg * 16) : 0u;
    return t;
}

// Output staging of the tiled kernels' epilogues: a wave's rows x 64
// columns of C in LDS, 128 bytes per row, the 16-byte chunks of a row
// XOR-swizzled by row/2 so that the 16 rows one write instruction touches
// (lane l: row l%16, 8 bytes at column 4*(l/16)) fall in distinct banks.
__device__ __forceinline__ int stage_chunk(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

// The four adjacent outputs (packed act values) of lane (r, g4) for row
// `row` and n-tile j of the wave.
__device__ __forceinline__ void stage_put(unsigned char* stage, int row, int j, int g4, uint2 packed) {
    *reinterpret_cast<uint2*>(stage + stage_chunk(row, 2 * j + (g4 >> 1)) + 8 * (g4 & 1)) = packed;
}

// Stores the wave's ROWS x 64 staged outputs to C rows mrow0 + row, columns
// n0 .. n0 + 63: per instruction 8 rows x 128 bytes, lane l chunk l%8 of row
// l/8. N is a multiple of 8, so a 16-byte chunk lies wholly inside or wholly
// past it; rows past M are not stored. The wave's own LDS writes complete in
// order before these reads.
template <int ROWS>
__device__ __forceinline__ void stage_flush(const unsigned char* stage, int lane, uint16_t* C, int64_t ldc, int64_t M,
                                            int64_t Nst, int64_t mrow0, int64_t n0) {
#pragma unroll
    for (int q = 0; q < ROWS / 8; ++q) {
        const int row = 8 * q + (lane >> 3), c = lane & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + stage_chunk(row, c));
        const int64_t m = mrow0 + row, n = n0 + 8 * c;
        if (m < M && n < Nst) *reinterpret_cast<u32x4*>(C + m * ldc + n) = v;
    }
}

// Tile (ty, tx) of tile `local` of a launch of `count` tiles that covers
// positions tile0 .. tile0 + count - 1 of the tile order. Workgroups go to
// the 8 XCDs round-robin (blockIdx % 8); each XCD takes a contiguous eighth
// of the launch's positions, and the order runs over groups of 4 m-tiles
// with the n-blocks inside a group, so that the workgroups one XCD runs at a
// time share 4 activation row blocks and about 8 weight column blocks in its
// L2. 32-bit arithmetic (fewer than 2^31 tiles) made explicitly wave-uniform,
// so that the tile's buffer descriptors stay scalar.
__device__ __forceinline__ void xcd_tile(const MfmaArgs& a, uint32_t local, uint32_t count, int64_t& ty,
                                         int64_t& tx) {
    const uint32_t nb = (uint32_t)a.n_blocks, mt = (uint32_t)a.m_tiles;
    const uint32_t idx = (uint32_t)a.tile0 + (count % 8 == 0 ? (local % 8) * (count / 8) + local / 8 : local);
    constexpr uint32_t GM = 4;
    const uint32_t grp = idx / (GM * nb), off = idx - grp * GM * nb;
    const uint32_t rows = mt - grp * GM < GM ? mt - grp * GM : GM;
    ty = (int64_t)__builtin_amdgcn_readfirstlane(grp * GM + off % rows);
    tx = (int64_t)__builtin_amdgcn_readfirstlane(off / rows);
}

// Tiled variant with the activation tile loaded straight into LDS.
// A workgroup of 8 waves computes a BM x BN tile of C, the waves in a
// WM x (8/WM) grid; wave (wm, wn) owns MI = BM/(16*WM) row blocks and NJ
// n-tiles (BN = (8/WM) * NJ * 16), so it holds MI*NJ accumulators of 16x16.
// K advances in steps of KS k-tiles (128 k each). Per step, the BM x 128*KS
// activation tile goes from HBM/L2 to LDS with direct 16-byte buffer loads
// (no registers), in MFMA fragment order (1 KB per 16 x 32 block, lane l's
// 16 bytes at 16*l: conflict-free ds_read_b128), double-buffered: step t+1
// is in flight while step t is multiplied. Each wave streams its NJ x KS
// weight tiles (one 16-byte load per lane each, already in B-operand
// order), dequantises each word once, scale first as the pages do, and
// reuses it for its MI row blocks. One barrier per step. Small tiles use
// KS = 2 or 4 so that each step carries enough loads to cover the memory
// latency.
// All loads go through buffer descriptors based at the workgroup's tile
// whose per-wave part of the offset is scalar, which keeps the vector
// registers for the accumulators.
// OCM: 0 scale-first dequantisation; 1 offset-corrected with one group per
// row (operand 1 + q/16, offset and scale applied in the epilogue).
template <int DT, int QT, int SPT, int BM, int WM, int NJ, int KS, int OCM, int KT = 0>
__global__ __launch_bounds__(512) void mfma_lds_kernel(MfmaArgs a) {
    static_assert(OCM == 0 || OCM == 1, "scale first, or one group per row");
    constexpr bool OC = OCM != 0;
    constexpr int WN = 8 / WM;
    constexpr int MI = BM / (16 * WM);
    constexpr int BN = WN * NJ * 16;
    constexpr int NBLK = BM / 16 * 4 * KS;  // 1 KB fragment blocks per step
    constexpr int BPW = NBLK / 8;           // blocks staged per wave
    constexpr int BUF = NBLK * 1024;        // bytes of one LDS buffer
    // Weight loads per wave per step (with OC the scales and zeros are
    // loaded once, before the K loop).
    constexpr int NB_LOADS = NJ * KS * (OCM == 1 ? 1 : 1 + SPT * (1 + QT));
    static_assert(BPW >= 1, "at least one block per wave");
    // Two separate LDS objects (not one array) for the two activation
    // buffers: the loads into one and the reads of the other then need not
    // wait for each other.
    __shared__ __attribute__((aligned(1024))) unsigned char abuf0[BUF];
    __shared__ __attribute__((aligned(1024))) unsigned char abuf1[BUF];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave - wm * WN;
    const int r = lane & 15, g4 = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t NT = a.N / 16;
    const int64_t steps = (a.KTT + KS - 1) / KS;

    // Descriptors of A and of the packed weight; with live == false they
    // have size 0, so loads past K or after the last step read zeros without
    // a memory access and every step issues the same loads (a conditional
    // load would make the compiler's counter waits pessimistic).
    auto rsrc = [&](const void* base, uint32_t bytes, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, live ? (int)bytes : 0, 0x00020000);
    };

    // The workgroup's operands, based at its tile (offsets below 2^31).
    const int64_t ntw = (int64_t)blockIdx.x * (BN / 16);  // first n-tile of the workgroup
    const TileBufs tb = tile_bufs(a, m0, BM, ntw, BN / 16);

    // Activation blocks this wave stages: block b = wave*BPW + t is row
    // block rb = b / (4*KS), k-tile kk = (b / 4) % KS, word s = b % 4 of the
    // step: rows m0 + 16*rb + (0..15), k 128*kk + 32*s + (0..31). Lane l
    // loads row 16*rb + l%16 (clamped to M-1) at k offset 8*(l/16).
    uint32_t a_off[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int b = wave * BPW + t;
        int64_t row = m0 + 16 * (b / (4 * KS)) + r;
        if (row > a.M - 1) row = a.M - 1;
        a_off[t] = (uint32_t)(((row - tb.mb) * a.lda + 8 * g4) * 2);
    }
    // KT (K % 128 != 0): a lane whose 8 columns start at or past K reads
    // zeros (offset 2^31 is past the descriptor's range: no memory access).
    const int32_t k_end = (int32_t)a.K - 8 * g4;
    auto stage_a = [&](int64_t st, int buf, bool live) {
#pragma unroll
        for (int t = 0; t < BPW; ++t) {
            const int b = wave * BPW + t;
            const int kk = (b / 4) % KS, s = b % 4;
            const int64_t kt = st * KS + kk;
            const __amdgpu_buffer_rsrc_t rs_a = rsrc(tb.A, tb.a_bytes, live && kt < a.KTT);
            const uint32_t voff = KT && (int32_t)(kt * 128 + 32 * s) >= k_end ? 0x80000000u : a_off[t];
            load_lds16(rs_a, (buf ? abuf1 : abuf0) + b * 1024, voff, (uint32_t)((kt * 128 + 32 * s) * 2));
        }
    };

    // This wave's n-tiles (clamped for loads past N; never stored).
    const int64_t nt0 = ntw + wn * NJ;
    auto nt_ld = [&](int j) { return nt0 + j < NT ? nt0 + j : NT - 1; };
    const uint32_t lane16 = (uint32_t)lane * 16;
    // Scales and zeros stay one per 32-bit register: packing two freshly
    // loaded 16-bit values would make the step wait for loads just issued.
    u32x4 raw0[NJ][KS], raw1[NJ][KS];
    uint32_t sb0[NJ][KS][SPT], sb1[NJ][KS][SPT];
    uint32_t zb0[NJ][KS][SPT], zb1[NJ][KS][SPT];
    auto load_b = [&](int64_t st, u32x4 (&raw)[NJ][KS], uint32_t (&sb)[NJ][KS][SPT], uint32_t (&zb)[NJ][KS][SPT],
                      bool live) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int64_t kt = st * KS + kk;
            const bool ok = live && kt < a.KTT;
            const __amdgpu_buffer_rsrc_t rs_c = rsrc(tb.codes, tb.codes_bytes, ok);
            const __amdgpu_buffer_rsrc_t rs_s = rsrc(tb.scales, tb.scales_bytes, ok);
            const __amdgpu_buffer_rsrc_t rs_z = rsrc(tb.zeros, tb.zeros_bytes, ok);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int64_t nt = nt_ld(j) - ntw;  // relative to the workgroup's first n-tile
                raw[j][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rs_c, lane16, (uint32_t)((nt * a.KTT + kt) * 1024), 2));
#pragma unroll
                for (int u = 0; u < SPT && OCM != 1; ++u) {
                    const int64_t k = kt * 128 + u * (128 / SPT);
                    const int64_t g = a.one_group ? 0 : (k >> a.gshift);
                    const uint32_t so = (uint32_t)((nt * a.Kg + g) * 16);
                    sb[j][kk][u] = __builtin_amdgcn_raw_buffer_load_b16(rs_s, (uint32_t)r * 2, so * 2, 0);
                    if (QT) zb[j][kk][u] = __builtin_amdgcn_raw_buffer_load_b8(rs_z, (uint32_t)r, so, 0);
                }
            }
        }
    };

    uint32_t dq_mask = OC ? TopNibble<DT>::kMask : 0x000F000Fu, dq_magic = OC ? TopNibble<DT>::kOne : kMagic<DT>;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));

    floatx4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    // OC (one group per row): offset-corrected dequantisation. The B
    // operand is the exact value 1 + q/16 (TopNibble: a shift and one
    // v_and_or_b32 per pair of codes), acc sums A*(1 + q/16) over all of K,
    // S sums A over K (one MFMA against an all-ones B per activation
    // fragment, shared by the NJ n-tiles), and the epilogue applies
    // C = 16*s * (acc - (1 + z/16) * S): the scale multiplies an
    // exact-weight sum once instead of every weight.
    floatx4 S[OC ? MI : 1];
#pragma unroll
    for (int i = 0; i < (OC ? MI : 1); ++i) S[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4 ones = {one2, one2, one2, one2};

    // One step on LDS buffer `buf` with the weights in (raw, sb, zb); the
    // next step's activation tile and then its weights are requested first
    // (in that order: the wait at the end counts the weight loads). The
    // last step (a compile-time flag at each call) requests nothing and
    // needs no wait: no step reads what it would load.
    auto step = [&](int64_t st, int buf, const u32x4 (&raw)[NJ][KS], const uint32_t (&sb)[NJ][KS][SPT],
                    const uint32_t (&zb)[NJ][KS][SPT], u32x4 (&nraw)[NJ][KS], uint32_t (&nsb)[NJ][KS][SPT],
                    uint32_t (&nzb)[NJ][KS][SPT], bool last) {
        if (!last) {
            const bool more = st + 1 < steps;
            stage_a(st + 1, buf ^ 1, more);
            __builtin_amdgcn_sched_barrier(0);
            load_b(st + 1, nraw, nsb, nzb, more);
        }
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* abase = (buf ? abuf1 : abuf0) + lane * 16;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u32x4 bq[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (OC) {
                        const uint32_t w = raw[j][kk][s];
                        bq[j] = u32x4{and_or(top_pair_shift<DT, 0>(w), dq_mask, dq_magic),
                                      and_or(top_pair_shift<DT, 1>(w), dq_mask, dq_magic),
                                      and_or(top_pair_shift<DT, 2>(w), dq_mask, dq_magic),
                                      and_or(top_pair_shift<DT, 3>(w), dq_mask, dq_magic)};
                    } else {
                        const int u = s / (4 / SPT);
                        bq[j] = Dequant<DT>::apply(
                            raw[j][kk][s], Dequant<DT>::make((uint16_t)sb[j][kk][u], QT ? (int)zb[j][kk][u] : 8),
                            dq_mask, dq_magic);
                    }
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const int blk = ((wm * MI + i) * KS + kk) * 4 + s;
                    const u32x4 av = *reinterpret_cast<const u32x4*>(abase + blk * 1024);
                    if (OC) S[i] = mfma16x16x32<DT>(av, ones, S[i]);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32<DT>(av, bq[j], acc[i][j]);
                }
            }
        }
        // The next activation tile has landed once only the weight loads
        // issued after it may be outstanding; then every wave is done with
        // this buffer and sees the next one.
        if (!last) {
            wait_vmcnt<NB_LOADS>();
            stage_barrier();
        }
    };

    stage_a(0, 0, true);
    __builtin_amdgcn_sched_barrier(0);
    load_b(0, raw0, sb0, zb0, true);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<NB_LOADS>();
    stage_barrier();
    int64_t st = 0;
    for (; st + 1 < steps; st += 2) {
        step(st, 0, raw0, sb0, zb0, raw1, sb1, zb1, false);
        step(st + 1, 1, raw1, sb1, zb1, raw0, sb0, zb0, false);
    }
    if (st < steps) step(st, 0, raw0, sb0, zb0, raw1, sb1, zb1, true);

    // Epilogue: lane l holds rows 4*(l/16) .. +3 of column l%16 of each block.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (nt0 + j >= NT) continue;
        const int64_t n = (nt0 + j) * 16 + r;
        const float bv = a.bias && n < a.Nst ? act_to_float<DT>(a.bias[n]) : 0.f;
        float sf = 1.f, zf = 0.f;
        if (OCM == 1) {  // the row's only scale and zero (exact in fp32)
            sf = 16.0f * act_to_float<DT>(a.scales[n]);
            zf = -(1.0f + (QT ? (float)a.zeros[n] : 8.0f) * 0.0625f);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int64_t m = m0 + wm * (BM / WM) + 16 * i + 4 * g4 + jj;
                float v = acc[i][j][jj];
                if (OCM == 1) v = sf * __builtin_fmaf(zf, S[OC ? i : 0][jj], v);
                if (m < a.M && n < a.Nst) a.C[m * a.ldc + n] = to_act_bits<DT>(v + bv);
            }
        }
    }
}

// Ring variant of the tiled kernel for 128 x 256 tiles with offset-corrected
// dequantisation (one group per row, or groups of 128 k or more).
//  * Both operands go from HBM/L2 straight into LDS with direct 16-byte
//    buffer loads: per K step of 128 the activation tile (32 fragment blocks
//    of 1 KB) and the workgroup's 16 weight tiles (1 KB each, already in
//    B-operand order), so every weight word is fetched once per workgroup.
//  * Three LDS stages form a ring: step t computes on stage t % 3 while the
//    loads of step t + 2 are in flight, which covers two steps of latency.
//    One barrier per step.
//  * The activation sums S (one MFMA per 16 x 32 block against an all-ones
//    B) are split over the four waves that share a row half: wave wn sums
//    row block wn of the half (one extra fragment read per K slice), and
//    the sums meet in LDS.
//  * The B operand is the exact value 1 + q/16 (TopNibble), and
//    P = sum A*(1 + q/16) runs over all of K. OCM 1 (one group per row):
//    the epilogue applies C = 16*s * (P - (1 + z/16) * S). OCM 2 (groups of
//    G >= 128): each group end adds (s_g - s_{g+1}) * P to the result, which
//    sums to sum_g s_g * P_g without ever clearing P, the correction
//    -s_g * (1 + z_g/16) * S_g is applied one step later, once the row sums
//    of the group have passed the step's barrier, and the epilogue scales
//    the whole by 16. With the offset at 16 code steps (not 1024 as with
//    the magic 1024 + q), P stays within a small factor of the result even
//    when sum A grows with K.
template <int DT, int QT, int OCM, int BM, int KT>
__global__ __launch_bounds__(512) void mfma_ring_kernel(MfmaArgs a) {
    static_assert(OCM == 1 || OCM == 2, "offset-corrected modes only");
    // KT: K is not a multiple of 128 (possible with one group per row only:
    // groups of 128 or 256 divide K), so the last step masks the activation.
    static_assert(KT == 0 || OCM == 1, "a K tail needs one group per row");
    static_assert(BM == 128 || BM == 64, "whole or half tiles");
    constexpr int WN = 4, MI = BM / 32, NJ = 4;
    constexpr int ABLK = BM / 4, BBLK = 16;         // 1 KB blocks per stage
    constexpr int APW = ABLK / 8, BPW = BBLK / 8;   // blocks loaded per wave
    constexpr int NSC = OCM == 2 ? NJ * (1 + QT) : 0;  // scale/zero loads per wave per step
    constexpr int STAGE_LOADS = APW + BPW + NSC;
    __shared__ __attribute__((aligned(1024))) unsigned char a0[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a1[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a2[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b0[BBLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b1[BBLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b2[BBLK * 1024];
    // Row sums: [group parity][wm][row block wn][row].
    __shared__ float sx[2][2][WN][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave - wm * WN;
    const int r = lane & 15, g4 = lane >> 4;
    // Tile of the workgroup: tile blockIdx.x of the launch, or with BM = 64
    // half (blockIdx.x & 1) of tile blockIdx.x / 2.
    int64_t ty, tx;
    if (BM == 128) xcd_tile(a, blockIdx.x, gridDim.x, ty, tx);
    else xcd_tile(a, blockIdx.x >> 1, gridDim.x >> 1, ty, tx);
    const int64_t m0 = ty * 128 + (BM == 64 ? (int64_t)(blockIdx.x & 1) * 64 : 0);
    const int64_t NT = a.N / 16;
    const int64_t steps = a.KTT;
    const int64_t ntb = tx * 16;  // first n-tile of the workgroup
    // The workgroup's operands, based at its tile (offsets below 2^31).
    const TileBufs tb = tile_bufs(a, m0, BM, ntb, 16);

    auto rsrc = [&](const void* base, uint32_t bytes, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, live ? (int)bytes : 0, 0x00020000);
    };
    // Activation block b = wave*APW + t: row block b/4, K slice s = b%4 of
    // the step; lane l loads row 16*(b/4) + l%16 (clamped to M-1) at k
    // offset 32*s + 8*(l/16).
    uint32_t a_off[APW];
#pragma unroll
    for (int t = 0; t < APW; ++t) {
        const int b = wave * APW + t;
        int64_t row = m0 + 16 * (b >> 2) + r;
        if (row > a.M - 1) row = a.M - 1;
        a_off[t] = (uint32_t)(((row - tb.mb) * a.lda + 8 * g4) * 2);
    }
    // Weight block b = wave*BPW + t: n-tile ntb + b (clamped; never stored),
    // as an index relative to ntb.
    uint32_t b_tile[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int64_t nt = ntb + wave * BPW + t;
        b_tile[t] = (uint32_t)((nt < NT ? nt : NT - 1) - ntb);
    }
    const uint32_t lane16 = (uint32_t)lane * 16;
    const int32_t k_end = (int32_t)a.K - 8 * g4;
    auto nt_of = [&](int j) { return ntb + wn * NJ + j; };
    auto nt_ld = [&](int j) { return nt_of(j) < NT ? nt_of(j) : NT - 1; };

    // Per n-tile of the wave: the scales (4 x 16 bits) and zero points
    // (4 x 8 bits) of the lane's four columns 4*(l/16) .. +3.
    uint2 sb0[NJ], sb1[NJ], sb2[NJ];
    uint32_t zb0[NJ], zb1[NJ], zb2[NJ];
    // Requests part p (0..3) of step st: activation block p of the wave,
    // weight block p (p < BPW), and with p == 2 the scales and zeros of the
    // step's group. A step's loads are spread over its four K slices so that
    // the waves do not all queue their requests at the barrier.
    auto issue = [&](int64_t st, int p, unsigned char* abuf, unsigned char* bbuf, uint2 (&sb)[NJ],
                     uint32_t (&zb)[NJ]) {
        const bool live = st < steps;
        const int b = wave * APW + p;
        // With a K tail, a lane whose 8 columns start at or past K reads
        // zeros (offset 2^31 is past the descriptor's range: no memory access).
        if (p < APW)
            load_lds16(rsrc(tb.A, tb.a_bytes, live), abuf + b * 1024,
                       KT && (int32_t)(st * 128 + 32 * (b & 3)) >= k_end ? 0x80000000u : a_off[p],
                       (uint32_t)((st * 128 + 32 * (b & 3)) * 2));
        if (p < BPW)
            load_lds16(rsrc(tb.codes, tb.codes_bytes, live), bbuf + (wave * BPW + p) * 1024, lane16,
                       (uint32_t)((b_tile[p] * a.KTT + st) * 1024));
        if (OCM == 2 && p == 2) {
            const __amdgpu_buffer_rsrc_t rs_s = rsrc(tb.scales, tb.scales_bytes, live);
            const __amdgpu_buffer_rsrc_t rs_z = rsrc(tb.zeros, tb.zeros_bytes, live);
            const int64_t g = (st * 128) >> a.gshift;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t so = (uint32_t)(((nt_ld(j) - ntb) * a.Kg + g) * 16);
                sb[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs_s, (uint32_t)g4 * 8, so * 2, 0));
                if (QT) zb[j] = __builtin_amdgcn_raw_buffer_load_b32(rs_z, (uint32_t)g4 * 4, so, 0);
            }
        }
    };
    static_assert(APW <= 4 && BPW <= 2, "at most one activation block per K slice");

    uint32_t dq_mask = TopNibble<DT>::kMask, dq_magic = TopNibble<DT>::kOne;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));
    // Two slices' operands at once (one 64-bit shift per pair position for
    // both words) except in the grouped mode with zero points, which has no
    // registers for the second slice's operands: one slice at a time there.
    constexpr bool kPairs = !(OCM == 2 && QT);
    // Operand values 1 + q/16 of two consecutive words: b0 from w0, b1 from
    // w1 (one 64-bit shift per pair position serves both words).
    auto dequant_pair = [&](uint32_t w0, uint32_t w1, u32x4& b0, u32x4& b1) {
        const uint64_t x = ((uint64_t)w1 << 32) | w0;
        auto put = [&](int p, uint64_t xp) {
            b0[p] = and_or((uint32_t)xp, dq_mask, dq_magic);
            b1[p] = and_or((uint32_t)(xp >> 32), dq_mask, dq_magic);
        };
        put(0, top_pair_shift64<DT, 0>(x));
        put(1, top_pair_shift64<DT, 1>(x));
        put(2, top_pair_shift64<DT, 2>(x));
        put(3, top_pair_shift64<DT, 3>(x));
    };
    const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4 ones = {one2, one2, one2, one2};

    // S: row block wn % MI of the wave's half (with half tiles two waves
    // sum each row block; the sums read back are those of waves 0..MI-1).
    floatx4 acc[MI][NJ], S = {0.f, 0.f, 0.f, 0.f};
    floatx4 P[OCM == 2 ? MI : 1][OCM == 2 ? NJ : 1];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < (OCM == 2 ? NJ : 1); ++j) P[OCM == 2 ? i : 0][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // Pending group correction (OCM 2): -s*(1 + z/16) per n column of the lane.
    float cz[NJ][4];
    int par = 0;          // parity of the group whose S partials are written next
    bool pending = false; // a group ended in the previous step

    // Writes this wave's row sums for parity p: with the transposed products
    // every lane holds the sum of row l%16 of its row block.
    auto put_s = [&](int p) {
        if (g4 == 0) sx[p][wm][wn][r] = S[0];
        S = floatx4{0.f, 0.f, 0.f, 0.f};
    };
    // Row sums of the lane's row (l%16) in each of the wave's row blocks.
    auto get_s = [&](int p, float (&Sf)[MI]) {
#pragma unroll
        for (int i = 0; i < MI; ++i) Sf[i] = sx[p][wm][i][r];
    };

    // sb, zb: scales and zeros of step st; sbn: scales of step st + 1 (0
    // past the last step). A tail step (one of the at most two after the
    // loop; a compile-time flag at each call) requests nothing, since the
    // step two ahead does not exist, and waits for every load before its
    // barrier. (Requesting loads whose registers no step reads would let
    // the compiler drop them and break the count of the wait.)
    auto step = [&](int64_t st, unsigned char* abuf, unsigned char* bbuf, const uint2 (&sb)[NJ],
                    const uint32_t (&zb)[NJ], const uint2 (&sbn)[NJ], unsigned char* nabuf, unsigned char* nbbuf,
                    uint2 (&nsb)[NJ], uint32_t (&nzb)[NJ], bool tail) {
        if (OCM == 2 && pending) {
            float Sf[MI];
            get_s(par ^ 1, Sf);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][j][jj] = __builtin_fmaf(cz[j][jj], Sf[i], acc[i][j][jj]);
            pending = false;
        }
        u32x4 raw[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) raw[j] = *reinterpret_cast<const u32x4*>(bbuf + (wn * NJ + j) * 1024 + lane16);
        const unsigned char* abase = abuf + lane16;
        u32x4 bq2[2][NJ];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // The loads of step st + 2 stay at their slice. With one group per
            // row, LDS reads, VALU and MFMA may move across that point (mask
            // 0x18F), so the next slice's fragment reads are hoisted over the
            // current MFMAs; with groups the register budget is spent and the
            // point is a full scheduling barrier.
            __builtin_amdgcn_sched_barrier(OCM == 1 ? 0x18F : 0);
            if (!tail) issue(st + 2, s, nabuf, nbbuf, nsb, nzb);
            __builtin_amdgcn_sched_barrier(OCM == 1 ? 0x18F : 0);
            if (kPairs && (s & 1) == 0) {
                // Slices s and s + 1 together: their words are adjacent
                // registers, so one 64-bit shift serves both.
#pragma unroll
                for (int j = 0; j < NJ; ++j) dequant_pair(raw[j][s], raw[j][s + 1], bq2[0][j], bq2[1][j]);
            } else if (!kPairs) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const uint32_t w = raw[j][s];
                    bq2[s & 1][j] = u32x4{and_or(top_pair_shift<DT, 0>(w), dq_mask, dq_magic),
                                          and_or(top_pair_shift<DT, 1>(w), dq_mask, dq_magic),
                                          and_or(top_pair_shift<DT, 2>(w), dq_mask, dq_magic),
                                          and_or(top_pair_shift<DT, 3>(w), dq_mask, dq_magic)};
                }
            }
            const u32x4 (&bq)[NJ] = bq2[s & 1];
            // Transposed products (weights as the first operand): lane l
            // ends with row l%16, columns 4*(l/16) .. +3 of each tile, and
            // the row sum of row l%16.
            const u32x4 as = *reinterpret_cast<const u32x4*>(abase + ((wm * MI + wn % MI) * 4 + s) * 1024);
            S = mfma16x16x32<DT>(ones, as, S);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(abase + ((wm * MI + i) * 4 + s) * 1024);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (OCM == 2) P[OCM == 2 ? i : 0][OCM == 2 ? j : 0] = mfma16x16x32<DT>(bq[j], av, P[OCM == 2 ? i : 0][OCM == 2 ? j : 0]);
                    else acc[i][j] = mfma16x16x32<DT>(bq[j], av, acc[i][j]);
                }
            }
        }
        if (OCM == 2 && (((st + 1) << 7) & ((1 << a.gshift) - 1)) == 0) {
            // Last step of group g: P runs over all of K (never reset), so
            // sum_g s_g * P_g = sum_g (s_g - s_{g+1}) * P(end of g), with
            // s_{G+1} = 0 after the last group. The S part waits for the
            // row sums of the other waves (next step, after the barrier).
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const uint32_t sw = jj < 2 ? sb[j].x : sb[j].y, nw = jj < 2 ? sbn[j].x : sbn[j].y;
                    const float sf = act_to_float<DT>((uint16_t)(sw >> (16 * (jj & 1))));
                    const float d = sf - act_to_float<DT>((uint16_t)(nw >> (16 * (jj & 1))));
                    const float z = QT ? (float)((zb[j] >> (8 * jj)) & 0xFFu) : 8.0f;
                    cz[j][jj] = -sf * (1.0f + z * 0.0625f);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        const floatx4& p = P[OCM == 2 ? i : 0][OCM == 2 ? j : 0];
                        acc[i][j][jj] = __builtin_fmaf(d, p[jj], acc[i][j][jj]);
                    }
                }
            }
            put_s(par);
            par ^= 1;
            pending = true;
        }
        // Stage st + 1 has landed once only the loads of step st + 2 may be
        // outstanding; the barrier then also frees stage st for step st + 3.
        if (tail) wait_vmcnt<0>();
        else wait_vmcnt<STAGE_LOADS>();
        stage_barrier();
    };

#pragma unroll
    for (int p = 0; p < 4; ++p) issue(0, p, a0, b0, sb0, zb0);
#pragma unroll
    for (int p = 0; p < 4; ++p) issue(1, p, a1, b1, sb1, zb1);
    wait_vmcnt<STAGE_LOADS>();
    stage_barrier();
    int64_t st = 0;
    for (; st + 3 <= steps; st += 3) {
        step(st, a0, b0, sb0, zb0, sb1, a2, b2, sb2, zb2, false);
        step(st + 1, a1, b1, sb1, zb1, sb2, a0, b0, sb0, zb0, false);
        step(st + 2, a2, b2, sb2, zb2, sb0, a1, b1, sb1, zb1, false);
    }
    // Tail: the scales of the first tail step's successor were requested
    // by the loop (or the prologue); the second tail step is the last, and
    // its successor's scale is 0.
    const uint2 no_scale[NJ] = {};
    if (st < steps) step(st, a0, b0, sb0, zb0, sb1, a2, b2, sb2, zb2, true);
    if (st + 1 < steps) step(st + 1, a1, b1, sb1, zb1, no_scale, a0, b0, sb0, zb0, true);
    wait_vmcnt<0>();

    float Sf[MI];
    if (OCM == 1) {
        put_s(0);
        stage_barrier();
        get_s(0, Sf);
    } else {
        // The last group's correction (its partials passed the last barrier).
        get_s(par ^ 1, Sf);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[i][j][jj] = __builtin_fmaf(cz[j][jj], Sf[i], acc[i][j][jj]);
    }

    // Epilogue. Per tile, lane l holds row l%16 of the row block, columns
    // 4*(l/16) .. +3 of the n-tile. Where C's rows are 16-byte aligned, the
    // wave stages its BM/2 x 64 outputs in its own part of the (now idle)
    // activation stages and writes whole 128-byte row segments; otherwise
    // each lane stores its four outputs (one 8-byte store where C's rows
    // keep them 8-byte aligned).
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool vec16 = ((a.ldc & 7) == 0) && ((cbase & 15) == 0);
    const bool vec = ((a.ldc & 3) == 0) && ((cbase & 7) == 0);
    unsigned char* stage = (wave < 4 ? a0 : a1) + (wave & 3) * (BM * 64);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (nt_of(j) >= NT) continue;
        const int64_t n0 = nt_of(j) * 16 + 4 * g4;
        // OCM 1: the column's only scale and zero; OCM 2: the folded sum is
        // in units of 1/16 code step. Both factors are exact in fp32.
        float sf[4], zf[4], bv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int64_t n = n0 + jj;
            bv[jj] = a.bias && n < a.Nst ? act_to_float<DT>(a.bias[n]) : 0.f;
            sf[jj] = 16.0f;
            zf[jj] = 0.f;
            if (OCM == 1) {
                sf[jj] = 16.0f * act_to_float<DT>(a.scales[n]);
                zf[jj] = -(1.0f + (QT ? (float)a.zeros[n] : 8.0f) * 0.0625f);
            }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int64_t m = m0 + wm * (BM / 2) + 16 * i + r;
            uint16_t o[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float v = acc[i][j][jj];
                o[jj] = to_act_bits<DT>((OCM == 1 ? sf[jj] * __builtin_fmaf(zf[jj], Sf[i], v) : sf[jj] * v) + bv[jj]);
            }
            const uint2 packed = uint2{(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
            if (vec16) {
                stage_put(stage, 16 * i + r, j, g4, packed);
                continue;
            }
            if (m >= a.M) continue;
            uint16_t* dst = a.C + m * a.ldc + n0;
            if (vec && n0 + 3 < a.Nst) {
                *reinterpret_cast<uint2*>(dst) = packed;
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (n0 + jj < a.Nst) dst[jj] = o[jj];
            }
        }
    }
    if (vec16) stage_flush<BM / 2>(stage, lane, a.C, a.ldc, a.M, a.Nst, m0 + wm * (BM / 2), nt_of(0) * 16);
}

// 128 x 512 tiles for one group per row, for large M and N: twice the
// columns per activation tile of the ring kernel, so every activation byte
// brought from L2 serves twice the MFMA work. On MI355X the shader clock of
// these GEMMs is set by the power limit, and the activation traffic from L2
// into the CUs is what lowers it (with half of it the clock rises from about
// 2.05 to 2.27 GHz); the wider tile cuts the bytes moved per MFMA by a
// quarter.
//  * 8 waves side by side: wave w computes all 128 rows of n-tiles
//    4*w .. 4*w + 3 (32 accumulators of 16 x 16), so each weight word is
//    dequantised once per workgroup and serves 8 row blocks.
//  * Per K step of 128 both operands go straight into LDS (32 activation
//    blocks and 32 weight tiles of 1 KB), double-buffered: the step's loads
//    are requested in its first two slices and waited for at its end, a
//    whole step (33 MFMAs per wave and slice) later.
//  * Same offset-corrected arithmetic as the ring kernel with one group per
//    row: operand 1 + q/16 (TopNibble), row sums S by MFMA against ones
//    (wave w sums row block w), C = 16*s * (P - (1 + z/16) * S) in the
//    epilogue.
template <int DT, int QT, int KT>
__global__ __launch_bounds__(512) void mfma_wide_kernel(MfmaArgs a) {
    constexpr int MI = 8, NJ = 4;
    constexpr int ABLK = 32, BBLK = 32;  // 1 KB blocks per stage
    constexpr int APW = ABLK / 8, BPW = BBLK / 8;
    __shared__ __attribute__((aligned(1024))) unsigned char a0[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a1[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b0[BBLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b1[BBLK * 1024];
    __shared__ float sx[MI][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g4 = lane >> 4;
    int64_t ty, tx;
    xcd_tile(a, blockIdx.x, gridDim.x, ty, tx);
    const int64_t m0 = ty * 128;
    const int64_t NT = a.N / 16;
    const int64_t steps = a.KTT;
    const int64_t ntb = tx * 32;  // first n-tile of the workgroup
    const TileBufs tb = tile_bufs(a, m0, 128, ntb, 32);

    auto rsrc = [&](const void* base, uint32_t bytes, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, live ? (int)bytes : 0, 0x00020000);
    };
    // Activation block b = wave*APW + t: row block b/4, K slice b%4.
    uint32_t a_off[APW];
#pragma unroll
    for (int t = 0; t < APW; ++t) {
        const int b = wave * APW + t;
        int64_t row = m0 + 16 * (b >> 2) + r;
        if (row > a.M - 1) row = a.M - 1;
        a_off[t] = (uint32_t)(((row - tb.mb) * a.lda + 8 * g4) * 2);
    }
    // Weight block b = wave*BPW + t: n-tile ntb + b (clamped; never stored).
    uint32_t b_tile[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int64_t nt = ntb + wave * BPW + t;
        b_tile[t] = (uint32_t)((nt < NT ? nt : NT - 1) - ntb);
    }
    const uint32_t lane16 = (uint32_t)lane * 16;
    const int32_t k_end = (int32_t)a.K - 8 * g4;
    auto nt_of = [&](int j) { return ntb + wave * NJ + j; };

    // Requests half h (0, 1) of step st: two activation blocks and two
    // weight tiles of the wave.
    auto issue = [&](int64_t st, int h, unsigned char* abuf, unsigned char* bbuf) {
        const bool live = st < steps;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = 2 * h + u;
            const int b = wave * APW + p;
            const uint32_t kcol = (uint32_t)(st * 128 + 32 * (b & 3));
            load_lds16(rsrc(tb.A, tb.a_bytes, live), abuf + b * 1024,
                       KT && (int32_t)kcol >= k_end ? 0x80000000u : a_off[p], kcol * 2);
            load_lds16(rsrc(tb.codes, tb.codes_bytes, live), bbuf + (wave * BPW + p) * 1024, lane16,
                       (uint32_t)((b_tile[p] * a.KTT + st) * 1024));
        }
    };

    uint32_t dq_mask = TopNibble<DT>::kMask, dq_magic = TopNibble<DT>::kOne;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));
    const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4 ones = {one2, one2, one2, one2};

    floatx4 acc[MI][NJ], S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Step st multiplies stage (abuf, bbuf) and fills the other stage with
    // step st + 1 (past the last step the descriptors have size 0: the loads
    // write zeros without a memory access, and no step reads them).
    auto step = [&](int64_t st, const unsigned char* abuf, const unsigned char* bbuf, unsigned char* nabuf,
                    unsigned char* nbbuf) {
        const unsigned char* abase = abuf + lane16;
        u32x4 bq2[2][NJ];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            if (s < 2) issue(st + 1, s, nabuf, nbbuf);
            if ((s & 1) == 0) {
                // Words s and s + 1 of each n-tile (k 32*s .. 32*s + 63 of the
                // step): adjacent, so one 64-bit shift per pair position
                // serves both.
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const uint64_t x =
                        *reinterpret_cast<const uint64_t*>(bbuf + (wave * NJ + j) * 1024 + lane16 + 4 * s);
                    auto put = [&](int p, uint64_t xp) {
                        bq2[0][j][p] = and_or((uint32_t)xp, dq_mask, dq_magic);
                        bq2[1][j][p] = and_or((uint32_t)(xp >> 32), dq_mask, dq_magic);
                    };
                    put(0, top_pair_shift64<DT, 0>(x));
                    put(1, top_pair_shift64<DT, 1>(x));
                    put(2, top_pair_shift64<DT, 2>(x));
                    put(3, top_pair_shift64<DT, 3>(x));
                }
            }
            const u32x4 (&bq)[NJ] = bq2[s & 1];
            // Transposed products (weights as the first operand): lane l
            // ends with C[row l%16][columns 4*(l/16) .. +3] of each tile,
            // four adjacent outputs, and the row sum of row l%16.
            const u32x4 as = *reinterpret_cast<const u32x4*>(abase + (wave * 4 + s) * 1024);
            S = mfma16x16x32<DT>(ones, as, S);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(abase + (i * 4 + s) * 1024);
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32<DT>(bq[j], av, acc[i][j]);
            }
        }
        // The next stage has landed once no load is outstanding; the barrier
        // also frees this stage for the step after next.
        wait_vmcnt<0>();
        stage_barrier();
    };

    issue(0, 0, a0, b0);
    issue(0, 1, a0, b0);
    wait_vmcnt<0>();
    stage_barrier();
    int64_t st = 0;
    for (; st + 2 <= steps; st += 2) {
        step(st, a0, b0, a1, b1);
        step(st + 1, a1, b1, a0, b0);
    }
    if (st < steps) step(st, a0, b0, a1, b1);

    // Row sums: wave w summed row block w (every lane holds the sum of its
    // row l%16).
    if (g4 == 0) sx[wave][r] = S[0];
    stage_barrier();

    // Epilogue. Per tile, lane l holds row 16*i + l%16, columns
    // 4*(l/16) .. +3 of the n-tile. Where C's rows are 16-byte aligned, the
    // wave stages its 128 x 64 outputs in its own 16 KB of the (now idle)
    // stage buffers, then writes whole 128-byte row segments: 16 stores of
    // 8 rows x 128 bytes. Otherwise each lane stores its four outputs (one
    // 8-byte store where C's rows keep them 8-byte aligned).
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool vec16 = ((a.ldc & 7) == 0) && ((cbase & 15) == 0);
    const bool vec8 = ((a.ldc & 3) == 0) && ((cbase & 7) == 0);
    unsigned char* stage = (wave < 2 ? a0 : wave < 4 ? a1 : wave < 6 ? b0 : b1) + (wave & 1) * 16384;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (nt_of(j) >= NT) continue;
        const int64_t n0 = nt_of(j) * 16 + 4 * g4;
        float sf[4], zf[4], bv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int64_t n = n0 + jj;
            bv[jj] = a.bias && n < a.Nst ? act_to_float<DT>(a.bias[n]) : 0.f;
            sf[jj] = 16.0f * act_to_float<DT>(a.scales[n]);
            zf[jj] = -(1.0f + (QT ? (float)a.zeros[n] : 8.0f) * 0.0625f);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int64_t m = m0 + 16 * i + r;
            const float Sr = sx[i][r];
            uint16_t o[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o[jj] = to_act_bits<DT>(sf[jj] * __builtin_fmaf(zf[jj], Sr, acc[i][j][jj]) + bv[jj]);
            const uint2 packed = uint2{(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
            if (vec16) {
                stage_put(stage, 16 * i + r, j, g4, packed);
                continue;
            }
            if (m >= a.M) continue;
            uint16_t* dst = a.C + m * a.ldc + n0;
            if (vec8 && n0 + 3 < a.Nst) {
                *reinterpret_cast<uint2*>(dst) = packed;
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (n0 + jj < a.Nst) dst[jj] = o[jj];
            }
        }
    }
    if (vec16) stage_flush<128>(stage, lane, a.C, a.ldc, a.M, a.Nst, m0, nt_of(0) * 16);
}

// 128 x 512 tiles for groups of 128 k or more (G a power of two, K a
// multiple of 128): the same tile, loads and dequantisation as the one-group
// kernel, with the group scales applied by rescaling the accumulators.
// With b = 1 + q/16 into the MFMA and c_g = 1 + z_g/16, the result is
// C = 16 * sum_g s_g * (P_g - c_g * S_g), P_g and S_g the group's products and
// row sums. The accumulators hold that sum in units of the current group's
// scale u_g (u_g = s_g, or 1 for a zero scale): the MFMAs add P_g directly,
// and at each group end every column is multiplied by u_g / u_{g+1}; the
// zero-point term -c_g * S_g (times that ratio) follows one step later, once
// the row sums of the group have met in LDS; the epilogue multiplies by
// 16 * u of the last group. A group whose scale is zero contributes nothing:
// its operand mask and magic are zero (b = 0) and its row-sum term is
// dropped. Only one set of accumulators is needed (the ring kernel keeps a
// second set for P), so the 128 x 512 tile fits. The products are not
// transposed here: each lane owns one column per n-tile (n-tile row l%16),
// so the per-column scale work is four values per lane and the operand mask
// of that column is the lane's own.
template <int DT, int QT>
__global__ __launch_bounds__(512) void mfma_wide_grouped_kernel(MfmaArgs a) {
    constexpr int MI = 8, NJ = 4;
    constexpr int ABLK = 32, BBLK = 32;
    constexpr int APW = ABLK / 8, BPW = BBLK / 8;
    __shared__ __attribute__((aligned(1024))) unsigned char a0[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char a1[ABLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b0[BBLK * 1024];
    __shared__ __attribute__((aligned(1024))) unsigned char b1[BBLK * 1024];
    // Row sums of a group: [parity][row block][4 row groups] of floatx4.
    __shared__ floatx4 sx[2][MI][4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g4 = lane >> 4;
    int64_t ty, tx;
    xcd_tile(a, blockIdx.x, gridDim.x, ty, tx);
    const int64_t m0 = ty * 128;
    const int64_t NT = a.N / 16;
    const int64_t steps = a.KTT;
    const int64_t ntb = tx * 32;
    const TileBufs tb = tile_bufs(a, m0, 128, ntb, 32);
    const int64_t gsteps = (int64_t)1 << (a.gshift - 7);  // K steps per group

    auto rsrc = [&](const void* base, uint32_t bytes, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, live ? (int)bytes : 0, 0x00020000);
    };
    uint32_t a_off[APW];
#pragma unroll
    for (int t = 0; t < APW; ++t) {
        const int b = wave * APW + t;
        int64_t row = m0 + 16 * (b >> 2) + r;
        if (row > a.M - 1) row = a.M - 1;
        a_off[t] = (uint32_t)(((row - tb.mb) * a.lda + 8 * g4) * 2);
    }
    uint32_t b_tile[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int64_t nt = ntb + wave * BPW + t;
        b_tile[t] = (uint32_t)((nt < NT ? nt : NT - 1) - ntb);
    }
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto nt_of = [&](int j) { return ntb + wave * NJ + j; };
    auto nt_ld = [&](int j) { return nt_of(j) < NT ? nt_of(j) : NT - 1; };

    auto issue = [&](int64_t st, int h, unsigned char* abuf, unsigned char* bbuf) {
        const bool live = st < steps;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = 2 * h + u;
            const int b = wave * APW + p;
            const uint32_t kcol = (uint32_t)(st * 128 + 32 * (b & 3));
            load_lds16(rsrc(tb.A, tb.a_bytes, live), abuf + b * 1024, a_off[p], kcol * 2);
            load_lds16(rsrc(tb.codes, tb.codes_bytes, live), bbuf + (wave * BPW + p) * 1024, lane16,
                       (uint32_t)((b_tile[p] * a.KTT + st) * 1024));
        }
    };
    // The scale (and zero point) of group g for the lane's column of each
    // n-tile (zero past the last group).
    auto load_group = [&](int64_t g, uint32_t (&sraw)[NJ], uint32_t (&zraw)[NJ]) {
        const bool live = g < a.Kg;
        const __amdgpu_buffer_rsrc_t rs_s = rsrc(tb.scales, tb.scales_bytes, live);
        const __amdgpu_buffer_rsrc_t rs_z = rsrc(tb.zeros, tb.zeros_bytes, live);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint32_t so = (uint32_t)(((nt_ld(j) - ntb) * a.Kg + g) * 16);
            sraw[j] = __builtin_amdgcn_raw_buffer_load_b16(rs_s, (uint32_t)r * 2, so * 2, 0);
            if (QT) zraw[j] = __builtin_amdgcn_raw_buffer_load_b8(rs_z, (uint32_t)r, so, 0);
        }
    };

    const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4 ones = {one2, one2, one2, one2};

    floatx4 acc[MI][NJ], S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Current group: scale and zero of the lane's column per n-tile, the
    // operand mask and magic (zero for a zero scale); next group: raw loads.
    float sc[NJ], zc[NJ], cz[NJ];
    uint32_t msk[NJ], mag[NJ], sn[NJ], zn[NJ];
    auto set_group = [&](const uint32_t (&sraw)[NJ], const uint32_t (&zraw)[NJ]) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            sc[j] = act_to_float<DT>((uint16_t)sraw[j]);
            zc[j] = QT ? (float)(zraw[j] & 0xFFu) : 8.0f;
            msk[j] = sc[j] != 0.0f ? TopNibble<DT>::kMask : 0u;
            mag[j] = sc[j] != 0.0f ? TopNibble<DT>::kOne : 0u;
        }
    };
    int par = 0;
    bool pending = false;

    auto step = [&](int64_t st, const unsigned char* abuf, const unsigned char* bbuf, unsigned char* nabuf,
                    unsigned char* nbbuf) {
        if (pending) {
            // Zero-point term of the group that ended last step: its row sums
            // passed that step's barrier.
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const floatx4 Sf = sx[par ^ 1][i][g4];
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][j][jj] = __builtin_fmaf(cz[j], Sf[jj], acc[i][j][jj]);
            }
            pending = false;
        }
        const unsigned char* abase = abuf + lane16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            if (s < 2) issue(st + 1, s, nabuf, nbbuf);
            if (s == 0 && (st & (gsteps - 1)) == 0) load_group((st >> (a.gshift - 7)) + 1, sn, zn);
            // Word s of each n-tile (one slice at a time: the group state
            // takes the registers of a second slice).
            u32x4 bq[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(bbuf + (wave * NJ + j) * 1024 + lane16 + 4 * s);
                bq[j] = u32x4{and_or(top_pair_shift<DT, 0>(w), msk[j], mag[j]),
                              and_or(top_pair_shift<DT, 1>(w), msk[j], mag[j]),
                              and_or(top_pair_shift<DT, 2>(w), msk[j], mag[j]),
                              and_or(top_pair_shift<DT, 3>(w), msk[j], mag[j])};
            }
            const u32x4 as = *reinterpret_cast<const u32x4*>(abase + (wave * 4 + s) * 1024);
            S = mfma16x16x32<DT>(as, ones, S);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(abase + (i * 4 + s) * 1024);
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32<DT>(av, bq[j], acc[i][j]);
            }
        }
        if (((st + 1) & (gsteps - 1)) == 0) {
            // End of a group: hand its row sums over, move the accumulators to
            // the next group's scale, and keep the zero-point factor.
            if (r == 0) sx[par][wave][g4] = S;
            S = floatx4{0.f, 0.f, 0.f, 0.f};
            const bool last = st + 1 >= steps;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float s_next = last ? 0.0f : act_to_float<DT>((uint16_t)sn[j]);
                const float u_cur = sc[j] != 0.0f ? sc[j] : 1.0f;
                const float u_next = s_next != 0.0f ? s_next : 1.0f;
                const float ratio = last ? 1.0f : u_cur / u_next;
                cz[j] = sc[j] != 0.0f ? -(1.0f + zc[j] * 0.0625f) * ratio : 0.0f;
                if (!last) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc[i][j][jj] *= ratio;
                }
            }
            if (!last) set_group(sn, zn);
            par ^= 1;
            pending = true;
        }
        wait_vmcnt<0>();
        stage_barrier();
    };

    {
        uint32_t s0[NJ], z0[NJ];
        load_group(0, s0, z0);
        set_group(s0, z0);
    }
    issue(0, 0, a0, b0);
    issue(0, 1, a0, b0);
    wait_vmcnt<0>();
    stage_barrier();
    int64_t st = 0;
    for (; st + 2 <= steps; st += 2) {
        step(st, a0, b0, a1, b1);
        step(st + 1, a1, b1, a0, b0);
    }
    if (st < steps) step(st, a0, b0, a1, b1);
    if (pending) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const floatx4 Sf = sx[par ^ 1][i][g4];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[i][j][jj] = __builtin_fmaf(cz[j], Sf[jj], acc[i][j][jj]);
        }
    }

    // Epilogue: lane l holds rows 4*(l/16) .. +3 of column l%16 of each tile.
    // Where C's rows are 16-byte aligned the wave stages its 128 x 64 outputs
    // (2-byte writes) and stores whole 128-byte row segments.
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(a.C);
    const bool vec16 = ((a.ldc & 7) == 0) && ((cbase & 15) == 0);
    unsigned char* stage = (wave < 2 ? a0 : wave < 4 ? a1 : wave < 6 ? b0 : b1) + (wave & 1) * 16384;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (nt_of(j) >= NT) continue;
        const int64_t n = nt_of(j) * 16 + r;
        const float bv = a.bias && n < a.Nst ? act_to_float<DT>(a.bias[n]) : 0.f;
        const float sf = 16.0f * (sc[j] != 0.0f ? sc[j] : 1.0f);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * i + 4 * g4 + jj;
                const uint16_t o = to_act_bits<DT>(sf * acc[i][j][jj] + bv);
                if (vec16) {
                    *reinterpret_cast<uint16_t*>(stage + stage_chunk(row, 2 * j + (r >> 3)) + 2 * (r & 7)) = o;
                } else {
                    const int64_t m = m0 + row;
                    if (m < a.M && n < a.Nst) a.C[m * a.ldc + n] = o;
                }
            }
        }
    }
    if (vec16) stage_flush<128>(stage, lane, a.C, a.ldc, a.M, a.Nst, m0, nt_of(0) * 16);
}

// Waves of the split-K tiled kernel; each owns kSplitkNJ of the tile's 16
// n-tiles and all of its rows.
constexpr int kSplitkWaves = 8;
constexpr int kSplitkNJ = 16 / kSplitkWaves;

// Medium M (up to a few hundred rows), any group size, K a multiple of 128:
// tiles of BM (32, 64 or 128) rows x 256 columns, K split over `ksplit`
// workgroups so that the tiles of a narrow M still occupy every CU.
//  * 8 waves side by side: wave w owns n-tiles 2w and 2w + 1 of the tile and
//    all BM rows, so each weight word is dequantised once per workgroup and
//    serves BM/16 row blocks.
//  * The weight stream sets the pace at these M, so the operands go through
//    a ring of NS LDS stages (3 for 128 rows, 4 for 64, 6 for 32: as deep as
//    160 KB allows): the loads of step st + NS - 1 (activation and weight
//    blocks straight into LDS, the step's scales and zero points into
//    registers) are requested during step st, and each step ends waiting for
//    the next one's loads only, with the later NS - 2 steps' loads still in
//    flight (hand-counted: the counter retires loads in issue order).
//  * Scale first, as the pages do: each word becomes RN((q - z) * s) in the
//    act dtype (Dequant), so the MFMA sums are the result; no row sums and no
//    offset correction, which suits groups of 32 or 64 k.
//  * With ksplit > 1 each workgroup writes its fp32 partial tile to the
//    workspace with ordinary stores, and splitk_reduce_kernel, the next
//    launch on the stream, adds the partials in split order (a fixed order),
//    adds the bias and writes C. The kernel boundary makes the partials
//    visible, which costs less than write-through stores and coherent
//    reads by the last workgroup of a tile to arrive.
template <int DT, int QT, int BM, int SPT, int NS>
__global__ __launch_bounds__(64 * kSplitkWaves) void mfma_splitk_kernel(MfmaArgs a) {
    static_assert(BM == 32 || BM == 64 || BM == 128, "32, 64 or 128 rows");
    static_assert(SPT == 1 || SPT == 2 || SPT == 4, "groups per K step");
    static_assert(NS >= 3 && NS <= 6, "three to six stages");
    constexpr int NW = kSplitkWaves;
    constexpr int MI = BM / 16, NJ = kSplitkNJ;
    constexpr int ABLK = BM / 16 * 4, BBLK = 16;
    constexpr int APW = ABLK / NW, BPW = BBLK / NW;  // 1 KB blocks per wave and step
    static_assert(ABLK % NW == 0, "whole activation blocks per wave");
    constexpr int ASZ = ABLK * 1024, BSZ = BBLK * 1024;
    // Loads per wave and step: activation and weight blocks, then one scale
    // (and zero point) per group of the step and n-tile of the wave.
    constexpr int STEP_LOADS = APW + BPW + SPT * NJ * (1 + QT);
    static_assert(NS * (ASZ + BSZ) <= 160 * 1024, "stages fit the LDS");
    static_assert((NS - 2) * STEP_LOADS <= 63, "the loads in flight fit the vmcnt counter");
    // One LDS object per stage, so that the compiler knows which stage a
    // direct-to-LDS load writes (the reads of the others need not wait).
    __shared__ __attribute__((aligned(1024))) unsigned char sa0[ASZ], sb0[BSZ];
    __shared__ __attribute__((aligned(1024))) unsigned char sa1[ASZ], sb1[BSZ];
    __shared__ __attribute__((aligned(1024))) unsigned char sa2[ASZ], sb2[BSZ];
    __shared__ __attribute__((aligned(1024))) unsigned char sa3[NS > 3 ? ASZ : 16], sb3[NS > 3 ? BSZ : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char sa4[NS > 4 ? ASZ : 16], sb4[NS > 4 ? BSZ : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char sa5[NS > 5 ? ASZ : 16], sb5[NS > 5 ? BSZ : 16];
    auto abuf = [&](auto I) -> unsigned char* {
        constexpr int i = decltype(I)::value;
        if constexpr (i == 0) return sa0;
        else if constexpr (i == 1) return sa1;
        else if constexpr (i == 2) return sa2;
        else if constexpr (i == 3) return sa3;
        else if constexpr (i == 4) return sa4;
        else return sa5;
    };
    auto bbuf = [&](auto I) -> unsigned char* {
        constexpr int i = decltype(I)::value;
        if constexpr (i == 0) return sb0;
        else if constexpr (i == 1) return sb1;
        else if constexpr (i == 2) return sb2;
        else if constexpr (i == 3) return sb3;
        else if constexpr (i == 4) return sb4;
        else return sb5;
    };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g4 = lane >> 4;
    const int64_t tile = blockIdx.x / a.ksplit, kc = blockIdx.x - tile * a.ksplit;
    const int64_t ty = tile / a.n_blocks, tx = tile - ty * a.n_blocks;
    const int64_t m0 = ty * BM;
    const int64_t NT = a.N / 16;
    const int64_t ntb = tx * 16;
    const int64_t st0 = kc * a.spk;
    const int64_t st1 = st0 + a.spk < a.KTT ? st0 + a.spk : a.KTT;
    const TileBufs tb = tile_bufs(a, m0, BM, ntb, 16);

    auto rsrc = [&](const void* base, uint32_t bytes, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, live ? (int)bytes : 0, 0x00020000);
    };
    // Activation block b = wave*APW + t: row block b/4, K slice b%4.
    uint32_t a_off[APW];
#pragma unroll
    for (int t = 0; t < APW; ++t) {
        const int b = wave * APW + t;
        int64_t row = m0 + 16 * (b >> 2) + r;
        if (row > a.M - 1) row = a.M - 1;
        a_off[t] = (uint32_t)(((row - tb.mb) * a.lda + 8 * g4) * 2);
    }
    uint32_t b_tile[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
        const int64_t nt = ntb + wave * BPW + t;
        b_tile[t] = (uint32_t)((nt < NT ? nt : NT - 1) - ntb);
    }
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto nt_of = [&](int j) { return ntb + wave * NJ + j; };
    auto nt_ld = [&](int j) { return nt_of(j) < NT ? nt_of(j) : NT - 1; };

    // Scales and zero points of the steps in flight, one slot per stage.
    uint32_t sraw[NS][SPT][NJ], zraw[NS][SPT][NJ];

    // Requests every load of step st into stage I (past the split's last
    // step the descriptors have size 0: no memory access, zeros written, and
    // the same number of loads, which the hand-counted waits rely on).
    auto issue = [&](int64_t st, auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const bool live = st < st1;
#pragma unroll
        for (int p = 0; p < APW; ++p) {
            const int b = wave * APW + p;
            load_lds16(rsrc(tb.A, tb.a_bytes, live), abuf(I) + b * 1024, a_off[p],
                       (uint32_t)((st * 128 + 32 * (b & 3)) * 2));
        }
#pragma unroll
        for (int p = 0; p < BPW; ++p)
            load_lds16(rsrc(tb.codes, tb.codes_bytes, live), bbuf(I) + (wave * BPW + p) * 1024, lane16,
                       (uint32_t)((b_tile[p] * a.KTT + st) * 1024));
        const __amdgpu_buffer_rsrc_t rs_s = rsrc(tb.scales, tb.scales_bytes, live);
        const __amdgpu_buffer_rsrc_t rs_z = rsrc(tb.zeros, tb.zeros_bytes, live);
#pragma unroll
        for (int gi = 0; gi < SPT; ++gi) {
            const int64_t g = a.one_group ? 0 : ((st * 128) >> a.gshift) + gi;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t so = (uint32_t)(((nt_ld(j) - ntb) * a.Kg + g) * 16);
                sraw[i][gi][j] = __builtin_amdgcn_raw_buffer_load_b16(rs_s, (uint32_t)r * 2, so * 2, 0);
                if (QT) zraw[i][gi][j] = __builtin_amdgcn_raw_buffer_load_b8(rs_z, (uint32_t)r, so, 0);
            }
        }
    };

    uint32_t dq_mask = 0x000F000Fu, dq_magic = DT == 0 ? 0x64006400u : 0x43004300u;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));

    floatx4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Step st on stage I; with `more`, it first requests step st + NS - 1
    // into the stage the previous step freed, and ends waiting for step
    // st + 1 only; the last NS - 1 steps of the split request nothing and
    // wait for every load.
    auto step = [&](int64_t st, auto I, bool more) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        constexpr int inext = (i + NS - 1) % NS;
        if (more) issue(st + NS - 1, std::integral_constant<int, inext>{});
        const unsigned char* abase = abuf(I) + lane16;
        const unsigned char* bb = bbuf(I);
        typename Dequant<DT>::Params prm[NJ];
        // The dequantised words (bq) and activation fragments (av) of slice s
        // are ready before its MFMAs; those of slice s + 1 are read and
        // dequantised in slice s's scheduling region, so that their LDS and
        // VALU work interleaves with slice s's MFMAs.
        u32x4 bq[NJ];
        auto dequant_slice = [&](int s, u32x4 (&out)[NJ]) __attribute__((always_inline)) {
            if (s % (4 / SPT) == 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    prm[j] = Dequant<DT>::make((uint16_t)sraw[i][s / (4 / SPT)][j],
                                               QT ? (int)zraw[i][s / (4 / SPT)][j] : 8);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(bb + (wave * NJ + j) * 1024 + lane16 + 4 * s);
                out[j] = Dequant<DT>::apply(w, prm[j], dq_mask, dq_magic);
            }
        };
        u32x4 av[MI];
        auto read_a = [&](int s, u32x4 (&out)[MI]) __attribute__((always_inline)) {
#pragma unroll
            for (int ii = 0; ii < MI; ++ii) out[ii] = *reinterpret_cast<const u32x4*>(abase + (ii * 4 + s) * 1024);
        };
        __builtin_amdgcn_sched_barrier(0);
        read_a(0, av);
        dequant_slice(0, bq);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            u32x4 bqn[NJ], avn[MI];
            if (s < 3) {
                read_a(s + 1, avn);
                dequant_slice(s + 1, bqn);
            }
#pragma unroll
            for (int ii = 0; ii < MI; ++ii)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[ii][j] = mfma16x16x32<DT>(av[ii], bq[j], acc[ii][j]);
            if (s < 3) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) bq[j] = bqn[j];
#pragma unroll
                for (int ii = 0; ii < MI; ++ii) av[ii] = avn[ii];
            }
        }
        if (more) wait_vmcnt<(NS - 2) * STEP_LOADS>();
        else wait_vmcnt<0>();
        stage_barrier();
    };

    // Prologue: steps st0 .. st0 + NS - 2 into stages 0 .. NS - 2.
    static_for<NS - 1>([&](auto I) { issue(st0 + decltype(I)::value, I); });
    wait_vmcnt<(NS - 2) * STEP_LOADS>();
    stage_barrier();
    int64_t st = st0;
    for (; st + NS <= st1; st += NS) static_for<NS>([&](auto I) { step(st + decltype(I)::value, I, true); });
    // The last (st1 - st) < NS steps: their loads are all requested.
    static_for<NS - 1>([&](auto I) {
        if (st + decltype(I)::value < st1) step(st + decltype(I)::value, I, false);
    });
    // Every load has landed (the dead ones of the loop's last steps too)
    // before the workgroup may leave.
    wait_vmcnt<0>();

    if (a.ksplit > 1) {
        // Partial tile of split kc: per wave, per (i, j) accumulator, the
        // 64 lanes' floatx4 (1 KB). Ordinary stores: splitk_reduce_kernel,
        // the next launch on the stream, reads them after the kernel
        // boundary has made them visible.
        float* part = a.partials + (tile * a.ksplit + kc) * (int64_t)(BM * 256) + (int64_t)wave * (MI * NJ * 256);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) *reinterpret_cast<floatx4*>(part + ((i * NJ + j) * 64 + lane) * 4) = acc[i][j];
        return;
    }

    // Epilogue: lane l holds rows 4*(l/16) .. +3 of column l%16 of each tile.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (nt_of(j) >= NT) continue;
        const int64_t n = nt_of(j) * 16 + r;
        if (n >= a.Nst) continue;
        const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int64_t m = m0 + 16 * i + 4 * g4 + jj;
                if (m < a.M) a.C[m * a.ldc + n] = to_act_bits<DT>(acc[i][j][jj] + bv);
            }
    }
}

// Second half of a split-K launch: C = sum of the ksplit partial tiles in
// split order (((p0 + p1) + p2) + ..., a fixed order) + bias. Thread t of the
// grid takes unit t of the partial layout (tile, wave, accumulator (i, j),
// lane: rows 4*(lane/16) .. +3 of column lane%16 of the 16 x 16 block), so
// the loads of a wave are 1 KB contiguous per split.
template <int DT, int BM>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(MfmaArgs a) {
    constexpr int MI = BM / 16, NJ = kSplitkNJ;
    constexpr int UNITS = BM * 256 / 4;  // floatx4 units per partial tile
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tile = u / UNITS;
    if (tile >= a.m_tiles * a.n_blocks) return;
    const int rem = (int)(u - tile * UNITS);
    const int wave = rem / (MI * NJ * 64), acc_idx = (rem / 64) % (MI * NJ), lane = rem % 64;
    const int i = acc_idx / NJ, j = acc_idx % NJ;
    const int64_t ty = tile / a.n_blocks, tx = tile - ty * a.n_blocks;
    const int64_t n = (tx * 16 + wave * NJ + j) * 16 + (lane & 15);
    const int64_t mrow = ty * BM + 16 * i + 4 * (lane >> 4);
    if (n >= a.Nst || mrow >= a.M) return;
    const float* p = a.partials + tile * a.ksplit * (int64_t)(BM * 256) + (int64_t)rem * 4;
    floatx4 sum = *reinterpret_cast<const floatx4*>(p);
    for (int64_t q = 1; q < a.ksplit; ++q) sum += *reinterpret_cast<const floatx4*>(p + q * (int64_t)(BM * 256));
    const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
        if (mrow + jj < a.M) a.C[(mrow + jj) * a.ldc + n] = to_act_bits<DT>(sum[jj] + bv);
}

template <int DT, int QT, int OCM, int KT>
hipError_t launch_ring_ocm(MfmaArgs a, hipStream_t stream) {
    // 128 x 256 tiles, row-major over m-tiles x n-blocks, one workgroup per
    // CU at a time. When the last round of workgroups would be at most half
    // full, its tiles run as 64-row halves in a second launch: twice the
    // workgroups at half the work each, so the last round takes half as long.
    const int64_t tiles = a.m_tiles * a.n_blocks;
    const int64_t tail = tiles % kCUs;
    const int64_t full = tiles > kCUs && tail > 0 && 2 * tail <= kCUs ? tiles - tail : tiles;
    a.tile0 = 0;
    hipLaunchKernelGGL((mfma_ring_kernel<DT, QT, OCM, 128, KT>), dim3((unsigned)full), dim3(512), 0, stream, a);
    if (full < tiles) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        a.tile0 = full;
        hipLaunchKernelGGL((mfma_ring_kernel<DT, QT, OCM, 64, KT>), dim3((unsigned)(2 * (tiles - full))), dim3(512), 0,
                           stream, a);
    }
    return hipGetLastError();
}

// Whether `wide` 128 x 512 tiles beat the 128 x 256 ring tiles: when they
// fill whole rounds of the CUs, or the last, partial round is at most a fifth
// of the work, or (`late_round`) it is at least three quarters full. Measured
// on 2048 x 14336 x 4096 (448 wide tiles, 1.75 rounds, against 3.5 rounds of
// ring tiles): one group per row 170 us wide against 183 us ring; groups of
// 256 with zero points 242 against 259 us; without zero points 236 against
// 227 us, so that mode does not take the late round.
inline bool wide_tiles_fit(int64_t wide, bool late_round) {
    if (wide < kCUs) return false;
    if (wide % kCUs == 0 || wide >= 4 * kCUs) return true;
    return late_round && 4 * (wide % kCUs) >= 3 * kCUs;
}

template <int DT, int QT>
hipError_t launch_ring_t(MfmaArgs a, hipStream_t stream) {
    a.m_tiles = (a.M + 127) / 128;
    if (a.one_group) {
        const int64_t wide = a.m_tiles * ((a.N + 511) / 512);
        if (wide_tiles_fit(wide, true)) {
            a.n_blocks = (a.N + 511) / 512;
            a.tile0 = 0;
            if (a.K % 128) hipLaunchKernelGGL((mfma_wide_kernel<DT, QT, 1>), dim3((unsigned)wide), dim3(512), 0, stream, a);
            else hipLaunchKernelGGL((mfma_wide_kernel<DT, QT, 0>), dim3((unsigned)wide), dim3(512), 0, stream, a);
            return hipGetLastError();
        }
    }
    if (!a.one_group) {
        const int64_t wide = a.m_tiles * ((a.N + 511) / 512);
        if (wide_tiles_fit(wide, QT == 1)) {
            a.n_blocks = (a.N + 511) / 512;
            a.tile0 = 0;
            hipLaunchKernelGGL((mfma_wide_grouped_kernel<DT, QT>), dim3((unsigned)wide), dim3(512), 0, stream, a);
            return hipGetLastError();
        }
    }
    a.n_blocks = (a.N + 255) / 256;
    if (!a.one_group) return launch_ring_ocm<DT, QT, 2, 0>(a, stream);
    return a.K % 128 ? launch_ring_ocm<DT, QT, 1, 1>(a, stream) : launch_ring_ocm<DT, QT, 1, 0>(a, stream);
}

template <int DT, int QT, int BM, int WM, int NJ, int KS>
hipError_t launch_lds_t(const MfmaArgs& a, int spt, hipStream_t stream) {
    constexpr int BN = (8 / WM) * NJ * 16;
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    // Static LDS: two activation buffers of BM x 128*KS. One group per row:
    // offset-corrected dequantisation; otherwise scale first.
    if (a.one_group) {
        hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 1, BM, WM, NJ, KS, 1>), grid, dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    switch (spt) {  // spt == 1: groups of 128 k or more
        case 1: hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 1, BM, WM, NJ, KS, 0>), grid, dim3(512), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 2, BM, WM, NJ, KS, 0>), grid, dim3(512), 0, stream, a); break;
        default: hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 4, BM, WM, NJ, KS, 0>), grid, dim3(512), 0, stream, a); break;
    }
    return hipGetLastError();
}


// 128 x 256 staged tiles for groups of 32 or 64 k (scale first); every
// other G at this tile size runs on the ring.
template <int DT, int QT>
hipError_t launch_lds_wide(const MfmaArgs& a, int spt, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)((a.M + 127) / 128));
    if (spt == 2) hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 2, 128, 2, 4, 1, 0>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 4, 128, 2, 4, 1, 0>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

// K % 128 != 0 with groups below 128 or a narrow launch: one tile shape of
// the staged kernel, built with the K mask (the other shapes stay without it).
template <int DT, int QT>
hipError_t launch_lds_ktail(const MfmaArgs& a, int spt, hipStream_t stream) {
    constexpr int BM = 64, WM = 2, NJ = 1, KS = 2, BN = (8 / WM) * NJ * 16;
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    if (a.one_group) {
        hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 1, BM, WM, NJ, KS, 1, 1>), grid, dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    switch (spt) {  // a K tail leaves groups of 32 or 64 only
        case 2: hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 2, BM, WM, NJ, KS, 0, 1>), grid, dim3(512), 0, stream, a); break;
        default: hipLaunchKernelGGL((mfma_lds_kernel<DT, QT, 4, BM, WM, NJ, KS, 0, 1>), grid, dim3(512), 0, stream, a); break;
    }
    return hipGetLastError();
}

// Stages of the split-K ring: as many as 160 KB of LDS holds, and as the
// vmcnt counter (at most 63 outstanding) can count for the steps in flight.
constexpr int splitk_stages(int BM, int SPT, int QT) {
    const int by_lds = BM == 128 ? 3 : (BM == 64 ? 4 : 6);
    const int step_loads = BM / (4 * kSplitkWaves) + 16 / kSplitkWaves + SPT * kSplitkNJ * (1 + QT);
    const int by_count = 2 + 63 / step_loads;
    return by_lds < by_count ? by_lds : by_count;
}

template <int DT, int QT, int BM>
hipError_t launch_splitk_t(const MfmaArgs& a, const MfmaPlan& p, hipStream_t stream) {
    const dim3 grid((unsigned)(a.m_tiles * a.n_blocks * a.ksplit));
    // Groups per K step: 4 (G = 32), 2 (G = 64), else 1.
    const int spt = a.one_group || a.gshift >= 7 ? 1 : 1 << (7 - a.gshift);
    switch (spt) {
        case 4:
            hipLaunchKernelGGL((mfma_splitk_kernel<DT, QT, BM, 4, splitk_stages(BM, 4, QT)>), grid, dim3(64 * kSplitkWaves), 0,
                               stream, a);
            break;
        case 2:
            hipLaunchKernelGGL((mfma_splitk_kernel<DT, QT, BM, 2, splitk_stages(BM, 2, QT)>), grid, dim3(64 * kSplitkWaves), 0,
                               stream, a);
            break;
        default:
            hipLaunchKernelGGL((mfma_splitk_kernel<DT, QT, BM, 1, splitk_stages(BM, 1, QT)>), grid, dim3(64 * kSplitkWaves), 0,
                               stream, a);
            break;
    }
    if (a.ksplit == 1) return hipGetLastError();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t units = a.m_tiles * a.n_blocks * (BM * 256 / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<DT, BM>), dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int QT>
hipError_t launch_mfma_q(const MfmaArgs& a, const MfmaPlan& p, int spt, hipStream_t stream) {
    if (p.splitk) {
        switch (p.BM) {
            case 32: return launch_splitk_t<DT, QT, 32>(a, p, stream);
            case 64: return launch_splitk_t<DT, QT, 64>(a, p, stream);
            default: return launch_splitk_t<DT, QT, 128>(a, p, stream);
        }
    }
    // The ring kernel masks a K tail itself (one group per row); every other
    // K % 128 != 0 case takes the staged kernel's masked instance.
    if (a.K % 128 != 0 && !(p.BN == 256 && spt == 1)) return launch_lds_ktail<DT, QT>(a, spt, stream);
    if (p.BN == 256) {
        // Offset-corrected modes run on the three-stage ring.
        return spt == 1 ? launch_ring_t<DT, QT>(a, stream) : launch_lds_wide<DT, QT>(a, spt, stream);
    }
    switch (p.BM) {  // BN = 64: one n-tile per wave, 2 or 4 k-tiles per step
        case 32: return launch_lds_t<DT, QT, 32, 2, 1, 4>(a, spt, stream);
        case 64: return launch_lds_t<DT, QT, 64, 2, 1, 2>(a, spt, stream);
        default: return launch_lds_t<DT, QT, 128, 2, 1, 2>(a, spt, stream);
    }
}

}  // namespace

MfmaPlan plan_mfma(int64_t M, const Geometry& g, size_t workspace_cap) {
    MfmaPlan p;
    // 128 x 256 tiles while they give at least one workgroup per CU (the
    // ring kernel, or 128 x 512 tiles when those fill whole rounds).
    const int64_t wide = ((M + 127) / 128) * ((g.Np + 255) / 256);
    if (wide >= kCUs) {
        p.BM = 128;
        p.BN = 256;
        return p;
    }
    const int64_t KTT = g.Kp / 128;
    if (g.K % 128 == 0) {
        // Medium M: BM x 256 tiles with K split so that the tiles fill the
        // CUs (each split at least 4 K steps), as far as the workspace holds
        // the partial tiles; with too small a workspace for half the CUs,
        // the 64-column tiles below.
        const int bm = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
        const int64_t tiles = ((M + bm - 1) / bm) * ((g.Np + 255) / 256);
        int64_t ks = kCUs / tiles;
        if (ks > KTT / 4) ks = KTT / 4;
        for (; ks > 1; --ks) {
            const size_t need = kCounterRegionBytes + (size_t)tiles * ks * bm * 256 * sizeof(float);
            if (need <= workspace_cap) break;
        }
        if (ks < 1) ks = 1;
        if (tiles * ks < kCUs / 2) goto narrow;
        p.splitk = true;
        p.BM = bm;
        p.BN = 256;
        p.spk = (KTT + ks - 1) / ks;
        p.ksplit = (KTT + p.spk - 1) / p.spk;
        p.partial_bytes = p.ksplit > 1 ? (size_t)tiles * p.ksplit * bm * 256 * sizeof(float) : 0;
        return p;
    }
narrow:
    // A K tail (or a small workspace): 64-column tiles (four times the
    // workgroups) with as few rows as M needs, so that the weight stream
    // still spreads over the chip.
    p.BM = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
    p.BN = 64;
    return p;
}

size_t mfma_workspace(const MfmaPlan& p) { return p.ksplit > 1 ? kCounterRegionBytes + p.partial_bytes : 0; }

hipError_t launch_mfma(const void* A, int64_t M, int64_t lda, const void* packed, const Geometry& g, int dtype,
                       const void* bias, void* C, int64_t ldc, const MfmaPlan& p, void* workspace,
                       hipStream_t stream) {
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    MfmaArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.lda = lda;
    a.M = M;
    a.codes = reinterpret_cast<const u32x4*>(base);
    a.scales = reinterpret_cast<const uint16_t*>(base + g.scales_off);
    a.zeros = g.qtype == 1 ? base + g.zeros_off : nullptr;
    a.N = g.Np;
    a.Nst = g.N;
    a.KTT = g.Kp / 128;
    a.K = g.K;
    a.Kg = g.Kg;
    a.gshift = g.gshift;
    a.one_group = g.Kg == 1;
    a.bias = static_cast<const uint16_t*>(bias);
    a.C = static_cast<uint16_t*>(C);
    a.ldc = ldc;
    a.m_tiles = (M + p.BM - 1) / p.BM;
    a.n_blocks = (g.Np + p.BN - 1) / p.BN;
    a.tile0 = 0;
    a.ksplit = p.ksplit;
    a.spk = p.splitk ? p.spk : a.KTT;
    a.partials = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kCounterRegionBytes) : nullptr;
    const int spt = g.Kg == 1 ? 1 : (g.Ge >= 128 ? 1 : 128 / g.Ge);
    if (dtype == 0) return g.qtype ? launch_mfma_q<0, 1>(a, p, spt, stream) : launch_mfma_q<0, 0>(a, p, spt, stream);
    return g.qtype ? launch_mfma_q<1, 1>(a, p, spt, stream) : launch_mfma_q<1, 0>(a, p, spt, stream);
}

}  // namespace w4a16
