// skinny.hip -- W4A16 GEMM for M <= 16 rows (decode), bound by the weight
// stream from HBM.
//
// Prior art: the HIP skinny kernel the "rdna_hybrid_w4a16" pages dispatch to
// for small M (`_rdna_hybrid_w4a16_apply_impl`, `wvSplitK_int4_g`: wave-level
// split-K sized by the CU count). Its source is not on the pages; this kernel
// is designed for gfx950 from the packed layout:
//
//  * A workgroup of 4 waves covers 4*NW n-tiles (16 rows each) by KT k-tiles
//    (128 k each); each wave owns NW n-tiles and the whole K range of the
//    workgroup. Per lane, everything the wave needs is requested up front in
//    the order it is consumed: the activation fragments of the K range
//    (small and L2-resident, so they arrive first), the scales, then one
//    16-byte weight load per n-tile and k-tile.
//  * Each activation fragment feeds NW MFMAs, so the activation traffic per
//    weight byte falls by NW * 4 compared with one n-tile per workgroup.
//  * The inner product is one v_mfma_f32_16x16x32 per weight word (M padded
//    to 16; rows past M read row M-1 and are never stored), so the VALU only
//    dequantises.
//  * ksplit workgroups split K. Each writes its fp32 partial tile through to
//    the agent-wide coherence point (sc1 stores), waits for the writes, and
//    bumps an arrival counter with an agent-scope atomic add; the last to
//    arrive reads all partials back (sc1 loads, all in flight at once, spread
//    over its 256 threads), sums them in a fixed order, adds the bias, rounds
//    once, writes C and clears the counter. No workgroup ever waits for
//    another, no float atomics are used (the result is deterministic), and
//    no release/acquire fence is needed: every value that crosses
//    workgroups travels with the sc1 policy, which is how the compiler
//    implements agent-scope atomic stores and loads (a release fence would
//    write back the XCD's whole L2).
//
// That kernel serves narrow weights (fewer than 192 n-tiles) and N or K
// tails. Wide weights (the decode layers) use three variants that keep K
// whole in a workgroup where they can and give each CU up to 16 waves:
//  * skinny_reg_kernel: 2-4 n-tiles per workgroup sharing the activation
//    fragments, 2 k-tiles per wave; K over 4096 split in chunks whose
//    partials meet as above.
//  * skinny_res_kernel: one n-tile per workgroup, the M real activation rows
//    staged in LDS; 2 k-tiles per wave, or 8 for K up to 16384 at up to 4
//    rows; at up to 8 rows one row-sum MFMA serves several k-tiles.
//  * skinny_str_kernel: a ring of weight units in flight per wave.
// A wave computes only after its loads are issued, and issuing waits for
// room in the CU's memory queue, so more waves per CU (and, for the long-K
// waves, requesting a few k-tiles ahead) let MFMAs overlap loads.
#include "device_common.h"
#include "exchange.h"
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
    int64_t NT;   // n-tiles: N rounded up to 16, / 16
    int64_t KTT;  // padded K / 128
    int64_t Kg;
    int gshift;
    int one_group;
    const uint16_t* bias;
    uint16_t* C;
    int64_t ldc;
    float* partials;
    uint32_t* counters;
    int ksplit;
    int64_t n_groups;
    int xcd_map;
    uint32_t mask, magic;  // dequant operands, kept in registers (see Dequant)
    uint32_t a_bytes;      // bytes from A to the end of row M-1: ((M-1)*lda + K)*2 < 2^31
    int kc_tiles;          // split register variant: k-tiles per K chunk
    int nn_max;            // full-K variants: n-tiles per workgroup, at most
    uint32_t codes_bytes, scales_bytes, zeros_bytes;  // region sizes (< 2^31 on the full-K paths)
    int64_t K;    // activation columns past K read as zero (split kernel; the full-K paths need K % 128 == 0)
    int64_t N;    // columns of C (NT covers N rounded up to 16); the split kernel's stores and bias stop at N
};

template <int DT, int QT, int NW, int KT, int SPT>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a) {
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;

    // Block -> (n-group, k-chunk). With xcd_map, the blocks that round-robin
    // dispatch sends to XCD x (ids congruent to x mod 8) take a contiguous run
    // of (ng, kc) pairs that holds whole n-groups.
    int64_t p = blockIdx.x;
    if (a.xcd_map) {
        const int64_t per = (a.n_groups * a.ksplit) >> 3;
        p = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int64_t ng = p / a.ksplit;
    const int kc = (int)(p - ng * a.ksplit);
    const int64_t kt0 = (int64_t)kc * KT;

    // This wave's n-tiles; tiles past N (a ragged last group) load tile NT-1
    // and are never stored.
    int64_t nt[NW], ntl[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        nt[i] = ng * (4 * NW) + wave * NW + i;
        ntl[i] = nt[i] < a.NT ? nt[i] : a.NT - 1;
    }

    // 1. Activation fragments: lane (r, g4) of word s of tile j holds
    //    A[r][128*(kt0+j) + 32*s + 8*g4 .. +7]; rows past M read row M-1.
    //    A k-tile past the last one (a ragged last chunk) and the columns
    //    past K (K % 128 != 0) contribute zeros and are not read.
    const int rr = r < a.M ? r : a.M - 1;
    const uint16_t* arow = a.A + (int64_t)rr * a.lda + 8 * g4;
    u32x4 av[KT][4];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
        const int64_t kt = kt0 + j;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (kt < a.KTT && (int32_t)(kt * 128 + 32 * s + 8 * g4) < (int32_t)a.K)
                v = *reinterpret_cast<const u32x4*>(arow + kt * 128 + 32 * s);
            av[j][s] = v;
        }
    }

    // 2. Scales (and zeros): SPT groups per tile; word s uses sub-block s / (4 / SPT).
    uint16_t sb[NW][KT][SPT];
    uint8_t zb[NW][KT][SPT];
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const int64_t kt = kt0 + j < a.KTT ? kt0 + j : a.KTT - 1;
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int64_t k = kt * 128 + u * (128 / SPT);
                const int64_t g = a.one_group ? 0 : (k >> a.gshift);
                const int64_t idx = (ntl[i] * a.Kg + g) * 16 + r;
                sb[i][j][u] = a.scales[idx];
                zb[i][j][u] = QT ? a.zeros[idx] : (uint8_t)8;
            }
        }

    // 3. Weight stream: one 16-byte load per lane per (k-tile, n-tile), in
    //    the order they are consumed.
    u32x4 wq[KT][NW];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
        const int64_t kt = kt0 + j < a.KTT ? kt0 + j : a.KTT - 1;
#pragma unroll
        for (int i = 0; i < NW; ++i) wq[j][i] = __builtin_nontemporal_load(a.codes + (ntl[i] * a.KTT + kt) * 64 + lane);
    }

    // Keep every load above this point: the scheduler would otherwise sink
    // loads into the compute below to save registers, serialising round trips.
    __builtin_amdgcn_sched_barrier(0);

    // 4. Dequantise and multiply (mask and magic in opaque registers, so
    // that each pair is one v_and_or_b32).
    uint32_t dq_mask = a.mask, dq_magic = a.magic;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));
    floatx4 acc[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KT; ++j) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int u = s / (4 / SPT);
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const u32x4 b = Dequant<DT>::apply(wq[j][i][s], Dequant<DT>::make(sb[i][j][u], zb[i][j][u]), dq_mask,
                                                   dq_magic);
                acc[i] = mfma16x16x32<DT>(av[j][s], b, acc[i]);
            }
        }
    }

    // 5a. One workgroup over K: add the bias, round once, store.
    if (a.ksplit == 1) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            if (nt[i] >= a.NT) continue;
            const int64_t n = nt[i] * 16 + r;
            const float bv = a.bias && n < a.N ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 4 * g4 + jj;
                if (m < a.M && n < a.N) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(acc[i][jj] + bv);
            }
        }
        return;
    }

    // 5b. Split K. Partial tile of workgroup (ng, kc): [64*NW columns][16
    //     rows] fp32, lane (c, g4) of n-tile i holding rows 4*g4 .. +3 of
    //     column 16*(wave*NW + i) + c: one 16-byte write-through store.
    constexpr int W = 64 * NW;
    float* part = a.partials + (ng * a.ksplit) * (int64_t)(W * 16);
#pragma unroll
    for (int i = 0; i < NW; ++i)
        store_coherent(part + ((int64_t)kc * W + (wave * NW + i) * 16 + r) * 16 + 4 * g4, acc[i]);
    wait_vector_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counters + ng, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(a.ksplit - 1);
    }
    __syncthreads();
    if (!s_last) return;

    // Last to arrive: units are (column, 4-row quad) float4s of live rows.
    // Thread t takes unit t % units and the k-chunks q = t / units + G*i;
    // all its loads are in flight together; the G per-thread sums meet in
    // LDS and are added in group order (a fixed order for every call).
    __shared__ floatx4 red[256];
    const int quads = (a.M + 3) >> 2;
    const int units = W * quads;
    const int G = units >= 256 ? 1 : 256 / units;
    for (int u0 = 0; u0 < units; u0 += 256 / G) {
        const int t = threadIdx.x;
        const int grp = t / (256 / G), uu = u0 + t % (256 / G);
        const bool active = grp < G && uu < units;
        const int col = active ? uu / quads : 0, qd = active ? uu % quads : 0;
        floatx4 sum = {0.f, 0.f, 0.f, 0.f};
        if (active) {
            constexpr int B = 4;  // loads in flight per batch
            for (int q0 = grp; q0 < a.ksplit; q0 += B * G) {
                const float* src[B];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int q = q0 + b * G;
                    const int qc = q < a.ksplit ? q : grp;
                    src[b] = part + ((int64_t)qc * W + col) * 16 + 4 * qd;
                }
                floatx4 v[B];
                load_coherent4(src[0], src[1], src[2], src[3], v[0], v[1], v[2], v[3]);
#pragma unroll
                for (int b = 0; b < B; ++b)
                    if (q0 + b * G < a.ksplit) sum += v[b];
            }
        }
        red[t] = sum;
        __syncthreads();
        if (t < 256 / G && uu < units) {
            floatx4 tot = red[t];
            for (int g = 1; g < G; ++g) tot += red[g * (256 / G) + t];
            const int64_t n = ng * W + col;
            if (n < a.NT * 16) {
                const float bv = a.bias && n < a.N ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int m = 4 * qd + jj;
                    if (m < a.M && n < a.N) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(tot[jj] + bv);
                }
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + ng, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Full-K streaming variants, used when the n-tiles alone can occupy the chip.
// A workgroup of 8 waves owns n-tiles nt = blockIdx.x + i * gridDim.x
// (i < nn) and the whole K range; wave w takes k-tiles [w*ktw, (w+1)*ktw) of
// each of them, so no partial sum leaves the workgroup. The grid holds
// ceil(NT / nn_max) workgroups, nn_max = ceil(NT / 256), so every workgroup
// gets nn_max or nn_max - 1 n-tiles and no CU gets two workgroups.
//
// A decode GEMM streams each weight byte once and does little arithmetic per
// byte, so its duration is set by how many HBM requests are in flight. Each
// wave therefore requests its data before any arithmetic, in the order it
// is consumed, so the hardware counter waits let it compute on the first
// tiles while the rest arrive:
//  * skinny_res_kernel (at most 4 k-tiles per wave and 16 units per wave):
//    the activation fragments of the wave's k-tiles are loaded once and stay
//    in registers for all its n-tiles; every weight tile, scale and zero of
//    the wave is requested at once.
//  * skinny_str_kernel (longer K ranges or more n-tiles): a ring of D units,
//    each one weight tile with its activation fragments, scales and zeros;
//    unit u + D is requested as soon as unit u is consumed.
// Partial sums over the waves meet in LDS after one barrier; wave q then
// finishes n-tiles q, q + 8, ...: a fixed-order sum, + bias, one rounding.
//
// Offset-corrected dequantisation: the MFMA B operand is the exact magic
// value m + q (m = 1024 for fp16, 128 for bf16), one v_and_or_b32 per pair
// of codes. Over a fold block of FW words (FW*32 consecutive k, never
// crossing a group) the MFMA sums P = sum_k A*(m + q); one more MFMA against
// an all-ones B gives S = sum_k A for the block. Then
// acc += s * (P - (m + z) * S) in fp32, which equals s * sum_k A*(q - z):
// the scale is applied to an exact-integer-weight sum instead of to every
// weight (more accurate than rounding each (q - z) * s, and with A = I it is
// (q - z) * s exactly, rounded once at the end).
constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kResMaxKt = 4;    // K chunks of the split skinny_reg_kernel are multiples of it
constexpr int kRegKt = 2;       // k-tiles per wave in skinny_reg_kernel (up to 16 waves)
constexpr int kResShortKt = 2;  // k-tiles per wave in skinny_res_kernel for K <= 4096 (up to 16 waves)
constexpr int kLongResMaxRows = 4;  // rows of the long-K skinny_res_kernel instances
constexpr int kResAhead = 3;        // k-tiles a wave of skinny_res_kernel requests ahead of the one consumed
constexpr int kStrDepth = 8;  // units in flight per wave in skinny_str_kernel

template <int DT>
__device__ __forceinline__ float magic_base() { return DT == 0 ? 1024.0f : 128.0f; }

template <int DT>
__device__ __forceinline__ u32x4 ones_operand() {
    const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
    return u32x4{one2, one2, one2, one2};
}

// Loads through buffer descriptors. Reads past a descriptor's size return
// zeros without a memory access, which the full-K kernels use twice:
//  * activation lanes of padding rows (r >= M) read past the end of A, so at
//    small M most fragment lanes cost no load bandwidth;
//  * a unit that does not exist (past the wave's k-tiles, past the
//    workgroup's n-tiles, or past the end of a streamed wave's work) gets a
//    descriptor of 0 bytes. Every load is then issued unconditionally and in
//    the order the data is consumed, so the counter wait before each use is
//    exact, and the extra loads cost only issue slots.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Activation rows [0, M) of one launch; a_bytes = ((M-1)*lda + K)*2 < 2^31.
// The full-K variants that use it run only with K % 128 == 0 and
// N % 16 == 0 (the planner sends other shapes to the split kernel), so every
// k-tile and n-tile is whole.
struct ActRows {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lane_off;  // byte offset of this lane's row and 8-element slice
    __device__ ActRows(const SkinnyArgs& a, int r, int g4)
        : rsrc(make_rsrc(a.A, a.a_bytes)),
          lane_off(r < a.M ? (uint32_t)(((int64_t)r * a.lda + 8 * g4) * 2) : 0x80000000u) {}
    // Word s of k-tile kt: A[r][128*kt + 32*s + 8*g4 .. +7]; zeros if !valid.
    __device__ __forceinline__ u32x4 load(int64_t kt, int s, bool valid) const {
        const uint32_t off = (lane_off + (uint32_t)(kt * 256 + 64 * s)) | (valid ? 0u : 0x80000000u);
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
};

// One descriptor per region of the packed weight (codes, scales, zeros);
// a unit that does not exist reads at offset 2^31, past every region.
struct WeightBufs {
    __amdgpu_buffer_rsrc_t codes, scales, zeros;
    __device__ explicit WeightBufs(const SkinnyArgs& a)
        : codes(make_rsrc(a.codes, a.codes_bytes)),
          scales(make_rsrc(a.scales, a.scales_bytes)),
          zeros(make_rsrc(a.zeros, a.zeros_bytes)) {}
};
constexpr uint32_t kNoUnit = 0x80000000u;

// Weight tile (nt, kt) (1 KB, one 16-byte word group per lane), streamed
// once: nontemporal.
__device__ __forceinline__ u32x4 load_tile(const WeightBufs& wb, const SkinnyArgs& a, int64_t nt, int64_t kt,
                                           int lane, bool valid) {
    const uint32_t off = valid ? (uint32_t)(((nt * a.KTT + kt) * 64 + lane) * 16) : kNoUnit;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wb.codes, off, 0, 2));
}

// Scale (and zero) of row 16*nt + r for the fold block that starts at
// k-tile kt, word f*FW.
template <int FW>
__device__ __forceinline__ uint32_t group_of(const SkinnyArgs& a, int64_t kt, int f) {
    const int64_t k = kt * 128 + f * FW * 32;
    return a.one_group ? 0u : (uint32_t)(k >> a.gshift);
}
template <int QT, int FW>
__device__ __forceinline__ void load_scale_zero(const WeightBufs& wb, const SkinnyArgs& a, int64_t nt, int64_t kt,
                                                int f, int r, bool valid, uint16_t& sb, uint8_t& zb) {
    const uint32_t idx = (uint32_t)((nt * a.Kg + group_of<FW>(a, kt, f)) * 16 + r);
    sb = __builtin_amdgcn_raw_buffer_load_b16(wb.scales, valid ? idx * 2 : kNoUnit, 0, 0);
    if (QT) zb = __builtin_amdgcn_raw_buffer_load_b8(wb.zeros, valid ? idx : kNoUnit, 0, 0);
}

// B operand of exact magic values m + q for the 8 codes of word wv.
__device__ __forceinline__ u32x4 magic_operand(uint32_t wv, uint32_t mask, uint32_t magic) {
    u32x4 b;
    b[0] = and_or(wv, mask, magic);
    b[1] = and_or(wv >> 4, mask, magic);
    b[2] = and_or(wv >> 8, mask, magic);
    b[3] = and_or(wv >> 12, mask, magic);
    return b;
}

// (No inline asm may touch sbits or z: the compiler does not wait for a
// pending buffer load before an asm operand tied to its register.)
template <int DT, int QT>
__device__ __forceinline__ void fold(floatx4& acc, const floatx4& P, const floatx4& S, uint16_t sbits, uint8_t z) {
    const float sf = act_to_float<DT>(sbits);
    const float zf = -(magic_base<DT>() + (QT ? (float)z : 8.0f));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[jj] = __builtin_fmaf(sf, __builtin_fmaf(zf, S[jj], P[jj]), acc[jj]);
}

// fold() where `mine`, else acc unchanged: the scale factor is 0 for the
// k-tiles another lane group folds (P and S are finite there, so the term is
// an exact zero).
template <int DT, int QT>
__device__ __forceinline__ void fold_if(floatx4& acc, const floatx4& P, const floatx4& S, uint16_t sbits, uint8_t z,
                                        bool mine) {
    const float sf = mine ? act_to_float<DT>(sbits) : 0.0f;
    const float zf = -(magic_base<DT>() + (QT ? (float)z : 8.0f));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[jj] = __builtin_fmaf(sf, __builtin_fmaf(zf, S[jj], P[jj]), acc[jj]);
}

// Sum over the first nwa waves of red[wave][i][lane], in wave order. The
// LDS holds MAXW waves' slots (launch size MAXW * nn_max KB), so all MAXW
// reads are issued at once and only the additions depend on nwa.
template <int MAXW = kStreamWaves>
__device__ __forceinline__ floatx4 sum_waves(const floatx4* red, int nn, int i, int nwa, int lane) {
    floatx4 v[MAXW];
#pragma unroll
    for (int q = 0; q < MAXW; ++q) v[q] = red[(q * nn + i) * 64 + lane];
    floatx4 tot = v[0];
#pragma unroll
    for (int q = 1; q < MAXW; ++q)
        if (q < nwa) tot += v[q];
    return tot;
}

// The first `nwa` waves have written red[wave][i][lane] for i < nn; wave q
// of the workgroup's nw waves sums them, in wave order, for n-tiles q,
// q + nw, ..., adds the bias, rounds once and stores rows < M.
template <int DT, int MAXW = kStreamWaves>
__device__ __forceinline__ void finish_tiles(const SkinnyArgs& a, const floatx4* red, int nn, int nwa, int64_t g,
                                             int64_t groups) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    const int nw = blockDim.x >> 6;  // short K: fewer than 8 waves
    for (int i = wave; i < nn; i += nw) {
        const floatx4 tot = sum_waves<MAXW>(red, nn, i, nwa, lane);
        const int64_t n = (g + (int64_t)i * groups) * 16 + r;
        const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int m = 4 * g4 + jj;
            if (m < a.M) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(tot[jj] + bv);
        }
    }
}

// Split K across ksplit workgroups per n-group g (chunk c of K each): the
// workgroup's wave-summed tile of each of its n-tiles goes to the workspace
// with write-through stores; the last workgroup of the n-group to arrive
// (agent-scope counter, as in skinny_kernel) reads the ksplit partials back
// with coherent loads and sums them in chunk order, so the result does not
// depend on which one arrives last. Partial (g, c, i): 64 lanes x 16 bytes.
template <int DT, int MAXW = kStreamWaves>
__device__ __forceinline__ void finish_split(const SkinnyArgs& a, const floatx4* red, int* flag, int nn, int nwa,
                                             int64_t g, int c) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    const int nw = blockDim.x >> 6;
    float* part = a.partials + g * a.ksplit * (int64_t)a.nn_max * 256;
    for (int i = wave; i < nn; i += nw) {
        const floatx4 tot = sum_waves<MAXW>(red, nn, i, nwa, lane);
        store_coherent(part + (((int64_t)c * a.nn_max + i) * 64 + lane) * 4, tot);
    }
    wait_vector_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counters + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = prev == (uint32_t)(a.ksplit - 1);
    }
    __syncthreads();
    if (!*flag) return;
    for (int i = wave; i < nn; i += nw) {
        floatx4 tot = {0.f, 0.f, 0.f, 0.f};
        for (int q0 = 0; q0 < a.ksplit; q0 += 4) {
            const float* src[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int q = q0 + b < a.ksplit ? q0 + b : q0;
                src[b] = part + (((int64_t)q * a.nn_max + i) * 64 + lane) * 4;
            }
            floatx4 v[4];
            load_coherent4(src[0], src[1], src[2], src[3], v[0], v[1], v[2], v[3]);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (q0 + b < a.ksplit) tot += v[b];
        }
        const int64_t n = (g + (int64_t)i * a.n_groups) * 16 + r;
        const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int m = 4 * g4 + jj;
            if (m < a.M) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(tot[jj] + bv);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS row stride (halves) of a wave's activation slice of KTW k-tiles: 16
// bytes of padding per row spread the rows over the LDS banks.
template <int KTW>
constexpr int act_lds_ld() { return KTW * 128 + 8; }

// Fold without the zero term: acc += s * P, for P accumulated on top of
// -(m + z) * S (uint4b8: z = 8, the same for every n-tile, so that start
// value is computed once per fold block and shared).
template <int DT>
__device__ __forceinline__ void fold_scaled(floatx4& acc, const floatx4& P, uint16_t sbits) {
    const float sf = act_to_float<DT>(sbits);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[jj] = __builtin_fmaf(sf, P[jj], acc[jj]);
}

// Waves of skinny_reg_kernel, at most (its K chunks are at most 32 k-tiles).
constexpr int kRegMaxWaves = (32 + kRegKt - 1) / kRegKt;

template <int DT, int QT, int FW, int NNM>
__global__ __launch_bounds__(64 * kRegMaxWaves) void skinny_reg_kernel(SkinnyArgs a) {
    constexpr int KTM = kRegKt;  // k-tiles per wave (the grid has ceil(kc_tiles / KTM) waves)
    constexpr int NB = 4 / FW;      // fold blocks per k-tile
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    floatx4* red = reinterpret_cast<floatx4*>(smem);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    const int nwaves = blockDim.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    // Workgroup (K chunk c = blockIdx.x, n-group g = blockIdx.y): n-tiles
    // g + i * n_groups, k-tiles [c * kc_tiles, +kc_tiles) (all of K when
    // ksplit == 1).
    const int c = blockIdx.x;
    const int64_t g = blockIdx.y;
    const int nn = (int)((a.NT - g + a.n_groups - 1) / a.n_groups);
    const int64_t kt0 = (int64_t)c * a.kc_tiles + (int64_t)wave * KTM;
    const int64_t kend = (int64_t)(c + 1) * a.kc_tiles < a.KTT ? (int64_t)(c + 1) * a.kc_tiles : a.KTT;
    const int kc = kt0 >= kend ? 0 : (int)(kend - kt0 < KTM ? kend - kt0 : KTM);

    uint32_t dq_mask = 0x000F000Fu, dq_magic = kMagic<DT>;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));

    // 1. Activation fragments: lane (r, g4) of word s of k-tile j holds
    //    A[r][128*(kt0+j) + 32*s + 8*g4 .. +7]. The lanes of padding rows
    //    (r >= M) issue no load at all: the texture unit's time per load
    //    grows with the active lanes, and at small M most lanes are padding.
    const ActRows act(a, r, g4);
    const WeightBufs wb(a);
    // Lanes of rows past M keep whatever their registers hold (an empty asm
    // defines them without an instruction): row m of an MFMA result depends
    // on row m of A only, and those rows are never stored.
    u32x4 af[KTM][4];
#pragma unroll
    for (int j = 0; j < KTM; ++j) {
#pragma unroll
        for (int s = 0; s < 4; ++s) asm volatile("" : "=v"(af[j][s]));
    }
    if (r < a.M) {
#pragma unroll
        for (int j = 0; j < KTM; ++j) {
#pragma unroll
            for (int s = 0; s < 4; ++s) af[j][s] = act.load(kt0 + j, s, j < kc);
        }
    }
    // 2. Weight tiles, scales and zeros of every (n-tile, k-tile) unit, in
    //    consumption order.
    u32x4 w[NNM][KTM];
    uint16_t sb[NNM][KTM][NB];
    uint8_t zb[NNM][KTM][NB];
#pragma unroll
    for (int i = 0; i < NNM; ++i) {
        const int64_t nt = g + (int64_t)i * a.n_groups;
#pragma unroll
        for (int j = 0; j < KTM; ++j) {
            const bool valid = i < nn && j < kc;
            w[i][j] = load_tile(wb, a, nt, kt0 + j, lane, valid);
#pragma unroll
            for (int f = 0; f < NB; ++f) load_scale_zero<QT, FW>(wb, a, nt, kt0 + j, f, r, valid, sb[i][j][f], zb[i][j][f]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3. S per fold block, once per k-tile (shared by the n-tiles).
    const u32x4 ones = ones_operand<DT>();
    floatx4 S[KTM][NB];
#pragma unroll
    for (int j = 0; j < KTM; ++j) {
#pragma unroll
        for (int f = 0; f < NB; ++f) {
            S[j][f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ww = 0; ww < FW; ++ww) S[j][f] = mfma16x16x32<DT>(af[j][f * FW + ww], ones, S[j][f]);
            if (!QT) S[j][f] *= -(magic_base<DT>() + 8.0f);  // uint4b8: the start value T = -(m + 8) * S
        }
    }

    // 4. Multiply and fold, n-tile by n-tile. k-tiles past the wave's kc are
    //    computed too, without a branch (their activations and scales read as
    //    zeros, so they add exactly 0 to rows < M), so the chains of a wave's
    //    k-tiles can interleave.
#pragma unroll
    for (int i = 0; i < NNM; ++i) {
        if (i >= nn) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KTM; ++j) {
#pragma unroll
            for (int f = 0; f < NB; ++f) {
                floatx4 P = QT ? floatx4{0.f, 0.f, 0.f, 0.f} : S[j][f];
#pragma unroll
                for (int ww = 0; ww < FW; ++ww) {
                    const int word = f * FW + ww;
                    P = mfma16x16x32<DT>(af[j][word], magic_operand(w[i][j][word], dq_mask, dq_magic), P);
                }
                if (QT) fold<DT, QT>(acc, P, S[j][f], sb[i][j][f], zb[i][j][f]);
                else fold_scaled<DT>(acc, P, sb[i][j][f]);
            }
        }
        red[(wave * nn + i) * 64 + lane] = acc;
    }
    __syncthreads();
    if (a.ksplit == 1) finish_tiles<DT, kRegMaxWaves>(a, red, nn, nwaves, g, a.n_groups);
    else finish_split<DT, kRegMaxWaves>(a, red, reinterpret_cast<int*>(red + kRegMaxWaves * a.nn_max * 64), nn, nwaves, g, c);
}

// Waves of skinny_res_kernel, at most: 16 with 2 k-tiles per wave (K <=
// 4096) and with 8 k-tiles per wave (long K, up to 4 rows), else 8. A wave
// computes only after all of its loads are issued, and the loads of a CU
// queue up behind each other: with more waves per CU, one wave's MFMAs
// overlap other waves' loads.
__host__ __device__ constexpr int res_max_waves(int ktw, int mr) {
    return ktw <= kResShortKt || (ktw == 8 && mr <= kLongResMaxRows) ? 16 : kStreamWaves;
}

template <int DT, int QT, int FW, int NNM, int KTW, int MR>
__global__ __launch_bounds__(64 * res_max_waves(KTW, MR)) void skinny_res_kernel(SkinnyArgs a) {
    constexpr int NB = 4 / FW;  // fold blocks per k-tile
    constexpr int LD = act_lds_ld<KTW>();
    constexpr int kMaxRows = MR;  // largest M this instance is launched for
    constexpr int kMaxChunks = (kMaxRows * KTW * 16 + 63) / 64;  // 16-byte activation chunks per lane
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    const int nwaves = blockDim.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    const int nn = (int)((a.NT - blockIdx.x + gridDim.x - 1) / gridDim.x);
    // Wave w takes k-tiles w, w + nwaves, w + 2 nwaves, ...: the waves'
    // loads of one round cover adjacent k-tiles of the n-tile.
    const int64_t kt0 = wave;
    const int kc = (int)((a.KTT - wave + nwaves - 1) / nwaves);  // >= 1, <= KTW: the grid has ceil(KTT / KTW) waves
    uint16_t* As = reinterpret_cast<uint16_t*>(smem) + (size_t)wave * a.M * LD;

    uint32_t dq_mask = 0x000F000Fu, dq_magic = kMagic<DT>;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));

    // 1. The wave's activation slice, rows [0, M) of its kc k-tiles, into
    //    registers (16-byte chunks, row-major over the slice, the wave's
    //    k-tiles side by side). Only the M real rows are read: the padding
    //    rows of the MFMA operand come from LDS later, which has about three
    //    times the return bandwidth. Chunk c is row c / CPR, column chunk
    //    c % CPR (CPR = KTW*16, a constant), that is chunk col % 16 of the
    //    wave's k-tile col / 16; columns past the wave's kc k-tiles are not
    //    loaded. K is a multiple of 128 here, so every loaded column is < K.
    constexpr int CPR = KTW * 16;
    const int nch = a.M * CPR;
    const int ccols = kc * 16;
    u32x4 ach[kMaxChunks];
#pragma unroll
    for (int t = 0; t < kMaxChunks; ++t) {
        const int c = lane + 64 * t;
        const int m = c / CPR, col = c - m * CPR;
        if (c < nch && col < ccols)
            ach[t] = *reinterpret_cast<const u32x4*>(a.A + (int64_t)m * a.lda + (kt0 + (col >> 4) * nwaves) * 128 +
                                                     8 * (col & 15));
    }
    const WeightBufs wb(a);
    // 2. Every weight tile, scale and zero of the wave, in consumption order
    //    (k-tile outer, n-tile inner). Units past the workgroup's n-tiles or
    //    the wave's k-tiles use zero-size descriptors (see make_rsrc). The
    //    first AHEAD k-tiles are requested here, each later one right after
    //    the k-tile AHEAD before it is consumed. (A wave whose request waits
    //    for room in the CU's full memory queue computes nothing meanwhile;
    //    requesting all 8 k-tiles of a long-K wave first left all of its
    //    MFMAs until after its last request. 3 ahead measured fastest with
    //    16 waves.)
    constexpr int AHEAD = KTW < kResAhead ? KTW : kResAhead;
    u32x4 w[KTW][NNM];
    uint16_t sb[KTW][NNM][NB];
    uint8_t zb[KTW][NNM][NB];
    auto issue = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NNM; ++i) {
            const int64_t nt = blockIdx.x + (int64_t)i * gridDim.x;
            const bool valid = i < nn && j < kc;
            w[j][i] = load_tile(wb, a, nt, kt0 + j * nwaves, lane, valid);
#pragma unroll
            for (int f = 0; f < NB; ++f)
                load_scale_zero<QT, FW>(wb, a, nt, kt0 + j * nwaves, f, r, valid, sb[j][i][f], zb[j][i][f]);
        }
    };
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) issue(j);
    __builtin_amdgcn_sched_barrier(0);
    // 3. Activation slice into this wave's LDS region (no other wave reads
    //    it, and a wave's LDS accesses complete in order: no barrier).
#pragma unroll
    for (int t = 0; t < kMaxChunks; ++t) {
        const int c = lane + 64 * t;
        const int m = c / CPR, col = c - m * CPR;
        if (c < nch && col < ccols) *reinterpret_cast<u32x4*>(As + m * LD + 8 * col) = ach[t];
    }

    // 4. k-tile by k-tile: the activation fragments and P for every n-tile.
    //    With one fold block per k-tile and at most 8 rows (MR), one S MFMA
    //    serves TPS = 16 / MR k-tiles: operand row r carries real row
    //    r % MR of k-tile j0 + r / MR, so lane group g (lanes 16g..16g+15,
    //    result rows 4g..4g+3) holds S of k-tile j0 + 4g / MR. The P operand
    //    repeats rows 0..MR-1 in every row block, so every lane group holds
    //    P of its rows for every k-tile, and lane group g folds only the
    //    k-tiles j0 + 4g / MR; the groups' sums meet at the end. With
    //    TPS = 1 this is one S per fold block, every lane folding every
    //    k-tile. Padding rows (r % RG >= M) repeat row M-1. P starts from
    //    zero, so the S and P chains of a k-tile do not wait for each other.
    constexpr int TPS = (FW == 4 && MR <= 8) ? (16 / MR < KTW ? 16 / MR : KTW) : 1;  // k-tiles per S MFMA
    constexpr int RG = 16 / TPS;                              // operand rows per k-tile
    static_assert(KTW % TPS == 0, "the k-tiles of a wave come in groups of TPS");
    const int orow = (r % RG) < a.M ? (r % RG) : a.M - 1;
    const int mytile = (4 * g4) / RG;  // which k-tile of each group this lane group folds
    const u32x4 ones = ones_operand<DT>();
    floatx4 acc[NNM];
#pragma unroll
    for (int i = 0; i < NNM; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j0 = 0; j0 < KTW; j0 += TPS) {
        if (j0 < kc) {
            floatx4 S[NB];
            if constexpr (TPS > 1) {
                // k-tiles past the wave's kc read k-tile kc - 1 (a finite
                // value that no lane folds).
                const int js = j0 + r / RG < kc ? j0 + r / RG : kc - 1;
                S[0] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    S[0] = mfma16x16x32<DT>(*reinterpret_cast<const u32x4*>(As + orow * LD + js * 128 + 32 * q + 8 * g4),
                                            ones, S[0]);
            }
#pragma unroll
            for (int t = 0; t < TPS; ++t) {
                const int j = j0 + t;
                if (j < kc) {
                    u32x4 af[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        af[q] = *reinterpret_cast<const u32x4*>(As + orow * LD + j * 128 + 32 * q + 8 * g4);
                    if constexpr (TPS == 1) {
#pragma unroll
                        for (int f = 0; f < NB; ++f) {
                            S[f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int ww = 0; ww < FW; ++ww) S[f] = mfma16x16x32<DT>(af[f * FW + ww], ones, S[f]);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < NNM; ++i) {
                        if (i < nn) {
#pragma unroll
                            for (int f = 0; f < NB; ++f) {
                                floatx4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int ww = 0; ww < FW; ++ww) {
                                    const int word = f * FW + ww;
                                    P = mfma16x16x32<DT>(af[word], magic_operand(w[j][i][word], dq_mask, dq_magic), P);
                                }
                                if constexpr (TPS == 1) fold<DT, QT>(acc[i], P, S[f], sb[j][i][f], zb[j][i][f]);
                                else fold_if<DT, QT>(acc[i], P, S[0], sb[j][i][0], zb[j][i][0], mytile == t);
                            }
                        }
                    }
                }
                if (j + AHEAD < KTW) {
                    issue(j + AHEAD);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    if constexpr (TPS > 1) {
        // Lane groups 16 (TPS = 4) and 32 apart hold the same rows: sum them,
        // (g0 + g1) + (g2 + g3) in every group alike.
#pragma unroll
        for (int i = 0; i < NNM; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if constexpr (TPS == 4) acc[i][jj] += __shfl_xor(acc[i][jj], 16);
                acc[i][jj] += __shfl_xor(acc[i][jj], 32);
            }
        }
    }
    // 5. Partials over the waves through LDS (reusing the activation area
    //    once every wave is done with it), fixed-order sum, bias, store.
    __syncthreads();
    floatx4* red = reinterpret_cast<floatx4*>(smem);
#pragma unroll
    for (int i = 0; i < NNM; ++i)
        if (i < nn) red[(wave * nn + i) * 64 + lane] = acc[i];
    __syncthreads();
    finish_tiles<DT, res_max_waves(KTW, MR)>(a, red, nn, nwaves, blockIdx.x, gridDim.x);
}

template <int DT, int QT, int FW>
__global__ __launch_bounds__(kStreamThreads) void skinny_str_kernel(SkinnyArgs a, int ktw) {
    constexpr int D = FW == 1 ? kStrDepth - 2 : kStrDepth;  // a scale (and zero) per word: fewer units fit
    constexpr int NB = 4 / FW;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    floatx4* red = reinterpret_cast<floatx4*>(smem);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g4 = lane >> 4;
    const int nn = (int)((a.NT - blockIdx.x + gridDim.x - 1) / gridDim.x);
    const int64_t kt0 = (int64_t)wave * ktw;
    const int kc = kt0 >= a.KTT ? 0 : (int)(a.KTT - kt0 < ktw ? a.KTT - kt0 : ktw);
    const int nwa = (int)((a.KTT + ktw - 1) / ktw);  // waves with k-tiles
    const int U = nn * kc;  // units of this wave: (n-tile i, k-tile j), j fastest

    uint32_t dq_mask = 0x000F000Fu, dq_magic = kMagic<DT>;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));
    const ActRows act(a, r, g4);
    const WeightBufs wb(a);

    struct Slot {
        u32x4 af[4];
        u32x4 w;
        uint16_t sb[NB];
        uint8_t zb[NB];
    };
    Slot ring[D];
    // Requests unit (pi, pj) into a slot and advances. Positions past the
    // wave's units load nothing (zero-size descriptors) and are never
    // consumed, so the ring is refilled unconditionally.
    int pi = 0, pj = 0;
    auto request = [&](Slot& sl) {
        const bool valid = pi < nn && kc > 0;
        const int64_t nt = blockIdx.x + (int64_t)pi * gridDim.x;
        const int64_t kt = kt0 + pj;
#pragma unroll
        for (int s = 0; s < 4; ++s) sl.af[s] = act.load(kt, s, valid);
        sl.w = load_tile(wb, a, nt, kt, lane, valid);
#pragma unroll
        for (int f = 0; f < NB; ++f) load_scale_zero<QT, FW>(wb, a, nt, kt, f, r, valid, sl.sb[f], sl.zb[f]);
        if (++pj >= kc) {
            pj = 0;
            ++pi;
        }
        // Keep the loads of a unit together and in unit order: the counter
        // waits are in issue order, so a unit consumed first must be issued
        // first.
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int s = 0; s < D; ++s) request(ring[s]);

    const u32x4 ones = ones_operand<DT>();
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int ci = 0, cj = 0;  // unit being consumed
    const int rounds = (U + D - 1) / D;
    for (int rnd = 0; rnd < rounds; ++rnd) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            Slot& sl = ring[s];
            if (rnd * D + s < U) {
#pragma unroll
                for (int f = 0; f < NB; ++f) {
                    floatx4 P = {0.f, 0.f, 0.f, 0.f}, S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ww = 0; ww < FW; ++ww) {
                        const int word = f * FW + ww;
                        S = mfma16x16x32<DT>(sl.af[word], ones, S);
                        P = mfma16x16x32<DT>(sl.af[word], magic_operand(sl.w[word], dq_mask, dq_magic), P);
                    }
                    fold<DT, QT>(acc, P, S, sl.sb[f], QT ? sl.zb[f] : (uint8_t)8);
                }
                if (++cj == kc) {
                    red[(wave * nn + ci) * 64 + lane] = acc;
                    acc = floatx4{0.f, 0.f, 0.f, 0.f};
                    cj = 0;
                    ++ci;
                }
            }
            request(sl);
        }
    }
    __syncthreads();
    finish_tiles<DT>(a, red, nn, nwa < kStreamWaves ? nwa : kStreamWaves, blockIdx.x, gridDim.x);
}

template <int DT, int QT, int FW, int NNM>
hipError_t launch_reg(const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
    hipError_t e = allow_lds<skinny_reg_kernel<DT, QT, FW, NNM>>(lds);
    if (e == hipSuccess) hipLaunchKernelGGL((skinny_reg_kernel<DT, QT, FW, NNM>), grid, block, lds, stream, a);
    return e;
}

template <int DT, int QT, int FW, int NNM, int KTW, int MR>
hipError_t launch_res(const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
    hipError_t e = allow_lds<skinny_res_kernel<DT, QT, FW, NNM, KTW, MR>>(lds);
    if (e == hipSuccess) hipLaunchKernelGGL((skinny_res_kernel<DT, QT, FW, NNM, KTW, MR>), grid, block, lds, stream, a);
    return e;
}

template <int DT, int QT, int FW>
hipError_t launch_stream_fw(const SkinnyArgs& a, const SkinnyPlan& p, hipStream_t stream) {
    const dim3 grid((unsigned)p.n_groups);
    const size_t lds = (size_t)kStreamWaves * p.nn_max * 64 * sizeof(floatx4);
    if (p.mode == SkinnyPlan::kRegisters) {
        const dim3 rgrid((unsigned)p.ksplit, (unsigned)p.n_groups);
        const int64_t nw = (p.kc_tiles + kRegKt - 1) / kRegKt;
        if (nw > kRegMaxWaves) return hipErrorInvalidValue;
        const dim3 block((unsigned)(64 * nw));
        // kRegMaxWaves partial slots per n-tile + the last-arrival flag of a split
        const size_t rlds = (size_t)kRegMaxWaves * p.nn_max * 64 * sizeof(floatx4) + 16;
        hipError_t e = hipSuccess;
        if (p.nn_max == 1) e = launch_reg<DT, QT, FW, 1>(a, rgrid, block, rlds, stream);
        else if (p.nn_max == 2 || FW == 1) e = launch_reg<DT, QT, FW, 2>(a, rgrid, block, rlds, stream);
        else e = launch_reg<DT, QT, FW, (FW == 1 ? 2 : 4)>(a, rgrid, block, rlds, stream);
        return e;
    }
    if (p.mode == SkinnyPlan::kResident) {
        // One wave per ktw k-tiles; each holds its activation rows (M rows of
        // ktw*128 + 8 halves) in LDS, and the partial sums reuse the area
        // (res_max_waves slots per n-tile: 8, or 16 for the long-K instance
        // with 8 k-tiles per wave).
        const int64_t nw = (a.KTT + p.ktw - 1) / p.ktw;
        const int64_t maxw = res_max_waves(p.ktw, p.ktw == 8 ? kLongResMaxRows : 16);
        if (nw > maxw) return hipErrorInvalidValue;
        const dim3 block((unsigned)(64 * nw));
        const size_t lds_a = (size_t)(nw > kStreamWaves ? nw : kStreamWaves) * a.M * (p.ktw * 128 + 8) * 2;
        const size_t lds_w = (size_t)maxw * p.nn_max * 64 * sizeof(floatx4);
        const size_t lds_r = lds_w > lds_a ? lds_w : lds_a;
        // The planner picks this variant for one n-tile per workgroup only;
        // up to 8 rows need half the activation registers (and with one fold
        // block per k-tile, up to 4 and 8 rows share S MFMAs over 4 and 2
        // k-tiles). Long K (8 k-tiles per wave, up to 16 waves, or 16
        // k-tiles per wave) only with one fold block per k-tile and up to 4
        // rows.
        if constexpr (FW == 4) {
            if (p.ktw > kResMaxKt && a.M > kLongResMaxRows) return hipErrorInvalidValue;
            if (p.ktw == 8) return launch_res<DT, QT, FW, 1, 8, kLongResMaxRows>(a, grid, block, lds_r, stream);
            if (p.ktw == 16) return launch_res<DT, QT, FW, 1, 16, kLongResMaxRows>(a, grid, block, lds_r, stream);
            if (p.ktw == kResShortKt && a.M <= 4)
                return launch_res<DT, QT, FW, 1, kResShortKt, 4>(a, grid, block, lds_r, stream);
        }
        if (p.ktw != kResShortKt) return hipErrorInvalidValue;
        return a.M <= 8 ? launch_res<DT, QT, FW, 1, kResShortKt, 8>(a, grid, block, lds_r, stream)
                        : launch_res<DT, QT, FW, 1, kResShortKt, 16>(a, grid, block, lds_r, stream);
    }
    hipError_t e = allow_lds<skinny_str_kernel<DT, QT, FW>>(lds);
    if (e == hipSuccess)
        hipLaunchKernelGGL((skinny_str_kernel<DT, QT, FW>), grid, dim3(kStreamThreads), lds, stream, a, p.ktw);
    return e;
}

template <int DT, int QT, int NW, int KT>
void launch_skinny_t(const SkinnyArgs& a, int spt, dim3 grid, hipStream_t stream) {
    switch (spt) {
        case 1: hipLaunchKernelGGL((skinny_kernel<DT, QT, NW, KT, 1>), grid, dim3(256), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((skinny_kernel<DT, QT, NW, KT, 2>), grid, dim3(256), 0, stream, a); break;
        default: hipLaunchKernelGGL((skinny_kernel<DT, QT, NW, KT, 4>), grid, dim3(256), 0, stream, a); break;
    }
}

template <int DT, int QT>
hipError_t launch_stream_q(const SkinnyArgs& a, const SkinnyPlan& p, int spt, hipStream_t stream) {
    // Fold width: words per fold block, at most one group (G / 32 words) and
    // at most 4 (one k-tile); spt = groups per k-tile.
    switch (spt) {
        case 1: return launch_stream_fw<DT, QT, 4>(a, p, stream);
        case 2: return launch_stream_fw<DT, QT, 2>(a, p, stream);
        default: return launch_stream_fw<DT, QT, 1>(a, p, stream);
    }
}

template <int DT, int QT>
void launch_skinny_q(const SkinnyArgs& a, const SkinnyPlan& p, int spt, dim3 grid, hipStream_t stream) {
    if (p.NW == 2) {
        switch (p.KT) {
            case 1: launch_skinny_t<DT, QT, 2, 1>(a, spt, grid, stream); break;
            case 2: launch_skinny_t<DT, QT, 2, 2>(a, spt, grid, stream); break;
            default: launch_skinny_t<DT, QT, 2, 4>(a, spt, grid, stream); break;
        }
    } else {
        switch (p.KT) {
            case 1: launch_skinny_t<DT, QT, 1, 1>(a, spt, grid, stream); break;
            case 2: launch_skinny_t<DT, QT, 1, 2>(a, spt, grid, stream); break;
            default: launch_skinny_t<DT, QT, 1, 4>(a, spt, grid, stream); break;
        }
    }
}

}  // namespace

SkinnyPlan plan_skinny(int64_t M, const Geometry& g) {
    // The plans that split K do not depend on M, so a workspace sized for 16
    // rows serves every M <= 16; the long-K resident plan (M <= 4) needs none.
    SkinnyPlan p;
    const int64_t NT = g.Np / 16, KTT = g.Kp / 128;
    // The wide-weight variants address each region of the packed weight with
    // 32-bit offsets below 2^31 (codes N*K/2 bytes, the largest).
    // The wide-weight variants read whole k-tiles of A and store whole
    // n-tiles of C: K % 128 == 0 and N % 16 == 0 only. Other shapes (the
    // layout pads them) go to the split kernel below, whose activation loads
    // stop at K and whose stores stop at N.
    if (NT >= kFullKMinTiles && g.codes_bytes < ((size_t)1 << 31) && g.K % 128 == 0 && g.N % 16 == 0) {
        // Wide weights: one workgroup per CU while N allows, n-tiles spread
        // evenly.
        p.full_k = true;
        p.ksplit = 1;
        const int64_t per = (NT + kCUs - 1) / kCUs;
        p.nn_max = (int)(per < kMaxTilesPerWG ? per : kMaxTilesPerWG);
        p.n_groups = (NT + p.nn_max - 1) / p.nn_max;
        p.kc_tiles = (int)KTT;
        // Every weight tile of a wave in registers: 2 k-tiles per wave (up
        // to 16 waves) and up to 4 n-tiles per workgroup (2 with a scale per
        // word). The activation fragments either stay in registers for all
        // of the wave's n-tiles (kRegisters: several n-tiles share them), or
        // the M real rows are loaded compactly and staged per wave in LDS
        // (kResident: one n-tile per workgroup, where the fragment loads of
        // 16 rows would cost more texture-unit time than the weights). With
        // K > 4096, K is split into chunks of at most 32 k-tiles and the
        // n-groups shrink so that the chunks of all n-groups still make
        // about one workgroup per CU; the chunk partials meet in the
        // workspace (or, for one n-tile per workgroup and up to 4 rows, all
        // of K stays in one workgroup, below). Otherwise the streamed
        // variant.
        const int nb = g.Kg == 1 || g.Ge >= 128 ? 1 : (int)(128 / g.Ge);  // fold blocks per k-tile
        const int nn_cap = nb < 4 ? 4 : 2;
        if (KTT <= 32 && p.nn_max <= nn_cap) {
            p.mode = p.nn_max >= 2 ? SkinnyPlan::kRegisters : SkinnyPlan::kResident;
            p.ktw = p.nn_max >= 2 ? kResMaxKt : kResShortKt;
            return p;
        }
        // One n-tile per workgroup, at most 4 rows and one fold block per
        // k-tile: all of K in one workgroup (8 k-tiles per wave, up to 16
        // waves), its activation rows staged in LDS (4 rows x 8 k-tiles x
        // 16 waves: 132 KB). No K chunks, so no exchange through the
        // workspace.
        if (p.nn_max == 1 && M <= kLongResMaxRows && nb == 1 && KTT <= 8 * 16) {
            p.mode = SkinnyPlan::kResident;
            p.ktw = 8;
            return p;
        }
        int64_t ks = (KTT + 31) / 32;
        const int64_t kc = ((KTT + ks - 1) / ks + kResMaxKt - 1) / kResMaxKt * kResMaxKt;
        ks = (KTT + kc - 1) / kc;
        const int64_t groups = kCUs / ks > 1 ? kCUs / ks : 1;
        const int64_t nnm = (NT + groups - 1) / groups;
        if (nnm <= nn_cap) {
            p.mode = SkinnyPlan::kRegisters;
            p.ktw = kResMaxKt;
            p.ksplit = (int)ks;
            p.kc_tiles = (int)kc;
            p.nn_max = (int)nnm;
            p.n_groups = (NT + nnm - 1) / nnm;
            p.partial_bytes = (size_t)p.n_groups * p.ksplit * p.nn_max * 64 * sizeof(floatx4);
            p.counter_bytes = (size_t)p.n_groups * sizeof(uint32_t);
            return p;
        }
        p.mode = SkinnyPlan::kStreamed;
        p.ktw = (int)((KTT + kStreamWaves - 1) / kStreamWaves);
        return p;
    }
    // Few n-tiles: split K across workgroups so the grid still covers the
    // chip; prefer 2 n-tiles per wave and 4 k-tiles, then narrower
    // workgroups or shorter K ranges, until there are 256 workgroups.
    static const int cand[][2] = {{2, 4}, {1, 4}, {2, 2}, {1, 2}, {1, 1}};
    for (const auto& c : cand) {
        p.NW = c[0];
        p.KT = c[1];
        p.n_groups = (NT + 4 * p.NW - 1) / (4 * p.NW);
        p.ksplit = (int)((KTT + p.KT - 1) / p.KT);
        if (p.n_groups * p.ksplit >= 256) break;
    }
    if (p.ksplit > 1) {
        p.partial_bytes = (size_t)p.n_groups * p.ksplit * (64 * p.NW) * 16 * sizeof(float);
        p.counter_bytes = (size_t)p.n_groups * sizeof(uint32_t);
    }
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
    a.NT = g.Np / 16;
    a.N = g.N;
    a.KTT = g.Kp / 128;
    a.K = g.K;
    a.Kg = g.Kg;
    a.gshift = g.gshift;
    a.one_group = g.Kg == 1;
    a.bias = static_cast<const uint16_t*>(bias);
    a.C = static_cast<uint16_t*>(C);
    a.ldc = ldc;
    a.counters = static_cast<uint32_t*>(workspace);
    a.partials = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kCounterRegionBytes) : nullptr;
    a.ksplit = p.ksplit;
    a.n_groups = p.n_groups;
    const int64_t nblocks = p.n_groups * p.ksplit;
    a.xcd_map = !p.full_k && (nblocks % 8 == 0) && ((nblocks / 8) % p.ksplit == 0);
    a.a_bytes = (uint32_t)(((M - 1) * lda + g.K) * 2);
    a.kc_tiles = p.kc_tiles;
    a.nn_max = p.nn_max;
    a.codes_bytes = (uint32_t)g.codes_bytes;  // the full-K paths need all three < 2^31
    a.scales_bytes = (uint32_t)(g.Np * g.Kg * 2);
    a.zeros_bytes = g.qtype == 1 ? (uint32_t)(g.Np * g.Kg) : 0u;
    a.mask = 0x000F000Fu;
    a.magic = dtype == 0 ? 0x64006400u : 0x43004300u;
    const int spt = g.Kg == 1 ? 1 : (g.Ge >= 128 ? 1 : 128 / g.Ge);
    const dim3 grid((unsigned)nblocks);
    if (p.full_k) {
        hipError_t e;
        if (dtype == 0) e = g.qtype ? launch_stream_q<0, 1>(a, p, spt, stream) : launch_stream_q<0, 0>(a, p, spt, stream);
        else e = g.qtype ? launch_stream_q<1, 1>(a, p, spt, stream) : launch_stream_q<1, 0>(a, p, spt, stream);
        return e != hipSuccess ? e : hipGetLastError();
    }
    if (dtype == 0) {
        if (g.qtype) launch_skinny_q<0, 1>(a, p, spt, grid, stream);
        else launch_skinny_q<0, 0>(a, p, spt, grid, stream);
    } else {
        if (g.qtype) launch_skinny_q<1, 1>(a, p, spt, grid, stream);
        else launch_skinny_q<1, 0>(a, p, spt, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace w4a16
