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
    int64_t NT;   // N / 16
    int64_t KTT;  // K / 128
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
};

// Cross-workgroup exchange of split-K partial sums. Every access carries the
// sc1 cache policy (write-through to, or read from, the agent-wide coherence
// point): stores are agent-scope relaxed atomic stores of 64 bits, which the
// compiler lowers to sc1 stores; loads are sc1 loads in inline assembly.
__device__ __forceinline__ void store_coherent(float* p, const floatx4& v) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, __builtin_bit_cast(uint64_t, __builtin_shufflevector(v, v, 0, 1)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, __builtin_bit_cast(uint64_t, __builtin_shufflevector(v, v, 2, 3)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
// Four coherent 16-byte loads and the wait for them, in one asm statement so
// that no compiler-inserted instruction can read the destination registers
// while the loads are in flight (the compiler does not track asm loads).
__device__ __forceinline__ void load_coherent4(const float* p0, const float* p1, const float* p2, const float* p3,
                                               floatx4& v0, floatx4& v1, floatx4& v2, floatx4& v3) {
    asm volatile(
        "global_load_dwordx4 %0, %4, off sc1\n\t"
        "global_load_dwordx4 %1, %5, off sc1\n\t"
        "global_load_dwordx4 %2, %6, off sc1\n\t"
        "global_load_dwordx4 %3, %7, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
        : "memory");
}
// Waits until every vector memory access this wave issued has completed
// (write-through stores: reached the coherence point).
__device__ __forceinline__ void wait_vector_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
    //    A k-tile past K (a ragged last chunk) contributes zeros.
    //    (The load itself uses a clamped k-tile, so it is always in bounds.)
    const int rr = r < a.M ? r : a.M - 1;
    const uint16_t* arow = a.A + (int64_t)rr * a.lda + 8 * g4;
    u32x4 av[KT][4];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
        const bool live = kt0 + j < a.KTT;
        const int64_t kt = live ? kt0 + j : a.KTT - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(arow + kt * 128 + 32 * s);
            av[j][s] = live ? v : u32x4{0u, 0u, 0u, 0u};
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

    // 4. Dequantise and multiply.
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
                const u32x4 b = Dequant<DT>::apply(wq[j][i][s], Dequant<DT>::make(sb[i][j][u], zb[i][j][u]), a.mask,
                                                   a.magic);
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
            const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 4 * g4 + jj;
                if (m < a.M) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(acc[i][jj] + bv);
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
                const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int m = 4 * qd + jj;
                    if (m < a.M) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(tot[jj] + bv);
                }
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + ng, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Persistent variant, used when the n-tiles alone can occupy the chip: one
// workgroup of up to 8 waves per CU (grid = min(N/16, CUs)), n-tiles nt =
// blockIdx.x + i * gridDim.x. K is walked in phases of PT = waves * KT
// k-tiles; the activation rows of a phase sit in LDS (staged once per
// workgroup instead of once per n-tile, double-buffered: phase p+1 is
// fetched while phase p is multiplied). Within a phase, wave w takes k-tiles
// [w*KT, +KT) of every n-tile, and the weights of the next (phase, n-tile)
// unit are always in flight while the current one is multiplied.
//
// Offset-corrected dequantisation: the MFMA B operand is the exact magic
// value m + q (m = 1024 for fp16, 128 for bf16), one v_and_or_b32 per pair
// of codes. Over a fold block of FW words (FW*32 consecutive k, never
// crossing a group) the MFMA sums P = sum_k A*(m + q); one more MFMA against
// an all-ones B gives S = sum_k A for the block (once per phase, shared by
// all n-tiles). Then acc += s * (P - (m + z) * S) in fp32, which equals
// s * sum_k A*(q - z): the scale is applied to an exact-integer-weight sum
// instead of to every weight (more accurate than rounding each (q - z) * s,
// and with A = I it is (q - z) * s exactly, rounded once at the end).
constexpr int kMaxTilesPerWG = 4;  // n-tiles per workgroup (accumulators per wave)
constexpr int kPersistThreads = 512;
constexpr int kStageChunks = 8;    // 16-byte A chunks per thread per phase (M * PT <= 256)

struct PersistArgs {
    int PT;        // k-tiles per phase (waves * KT)
    int phases;
    int lds_ld;    // LDS row stride of a staged phase, in elements
    int buf_bytes; // bytes of one phase buffer
};

template <int DT>
__device__ __forceinline__ float magic_base() { return DT == 0 ? 1024.0f : 128.0f; }

template <int DT, int QT, int KT, int FW>
__global__ __launch_bounds__(kPersistThreads) void skinny_persist_kernel(SkinnyArgs a, PersistArgs ph) {
    constexpr int WORDS = 4 * KT;      // weight words per lane per unit
    constexpr int NB = WORDS / FW;     // fold blocks per unit
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    const int rr = r < a.M ? r : a.M - 1;
    const int nn = (int)((a.NT - blockIdx.x + gridDim.x - 1) / gridDim.x);  // n-tiles of this workgroup
    const int Kp = ph.PT * 128;
    floatx4* red = reinterpret_cast<floatx4*>(smem + 2 * ph.buf_bytes);

    // Dequant operands in registers (see and_or) and the all-ones B operand.
    uint32_t dq_mask = 0x000F000Fu, dq_magic = kMagic<DT>;
    asm volatile("" : "+v"(dq_mask), "+v"(dq_magic));
    const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4 ones = {one2, one2, one2, one2};

    // Phase staging: M rows x Kp columns of A, zero past K; chunk c of 8
    // elements -> row c / (Kp/8), column 8 * (c % (Kp/8)).
    const int cpr = Kp / 8;
    const int nchunks = a.M * cpr;
    auto stage_load = [&](int p, u32x4 (&v)[kStageChunks]) {
#pragma unroll
        for (int t = 0; t < kStageChunks; ++t) {
            const int c = threadIdx.x + t * kPersistThreads;
            v[t] = u32x4{0u, 0u, 0u, 0u};
            if (c < nchunks) {
                const int m = c / cpr;
                const int64_t col = (int64_t)p * Kp + 8 * (c - m * cpr);
                if (col < a.KTT * 128) v[t] = *reinterpret_cast<const u32x4*>(a.A + (int64_t)m * a.lda + col);
            }
        }
    };
    auto stage_store = [&](int buf, const u32x4 (&v)[kStageChunks]) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(smem + buf * ph.buf_bytes);
#pragma unroll
        for (int t = 0; t < kStageChunks; ++t) {
            const int c = threadIdx.x + t * kPersistThreads;
            if (c < nchunks) {
                const int m = c / cpr;
                *reinterpret_cast<u32x4*>(dst + m * ph.lds_ld + 8 * (c - m * cpr)) = v[t];
            }
        }
    };

    // One unit = (phase p, n-tile i): this wave's KT weight tiles and the
    // scale (and zero) of each fold block.
    struct Unit {
        u32x4 w[KT];
        uint16_t sb[NB];
        uint8_t zb[NB];
    };
    const int64_t KTT = a.KTT;
    auto unit_load = [&](int p, int i, Unit& u) {
        const int64_t nt = blockIdx.x + (int64_t)i * gridDim.x;
        const int64_t kt0 = (int64_t)p * ph.PT + wave * KT;
        const u32x4* src = a.codes + (nt * KTT + kt0) * 64 + lane;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            u.w[j] = u32x4{0u, 0u, 0u, 0u};
            if (kt0 + j < KTT) u.w[j] = __builtin_nontemporal_load(src + j * 64);
        }
        const int64_t sbase = nt * a.Kg * 16 + r;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            int64_t k = kt0 * 128 + bb * FW * 32;
            if (k >= KTT * 128) k = KTT * 128 - 1;
            const int64_t g = a.one_group ? 0 : (k >> a.gshift);
            u.sb[bb] = a.scales[sbase + g * 16];
            u.zb[bb] = QT ? a.zeros[sbase + g * 16] : (uint8_t)8;
        }
    };

    floatx4 acc[kMaxTilesPerWG];
#pragma unroll
    for (int i = 0; i < kMaxTilesPerWG; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Prologue: the first unit's weights are requested before phase 0 of A
    // is staged, so the two fetches overlap.
    Unit cur, nxt;
    unit_load(0, 0, cur);
    {
        u32x4 v[kStageChunks];
        stage_load(0, v);
        stage_store(0, v);
    }
    __syncthreads();

    for (int p = 0; p < ph.phases; ++p) {
        const int buf = p & 1;
        const bool more = p + 1 < ph.phases;
        u32x4 stg[kStageChunks];
        if (more) stage_load(p + 1, stg);
        const uint16_t* As = reinterpret_cast<const uint16_t*>(smem + buf * ph.buf_bytes);
        const uint16_t* arow = As + rr * ph.lds_ld + wave * KT * 128 + 8 * g4;

        // S of each fold block of this wave's k-range (shared by the n-tiles).
        floatx4 S[NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            S[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ww = 0; ww < FW; ++ww) {
                const int word = bb * FW + ww;
                const u32x4 av = *reinterpret_cast<const u32x4*>(arow + (word >> 2) * 128 + 32 * (word & 3));
                S[bb] = mfma16x16x32<DT>(av, ones, S[bb]);
            }
        }

#pragma unroll
        for (int i = 0; i < kMaxTilesPerWG; ++i) {
            if (i < nn) {
                // Prefetch the next unit: the next n-tile, or the first
                // n-tile of the next phase.
                if (i + 1 < nn) unit_load(p, i + 1, nxt);
                else if (more) unit_load(p + 1, 0, nxt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ww = 0; ww < FW; ++ww) {
                        const int word = bb * FW + ww;
                        const uint32_t wv = cur.w[word >> 2][word & 3];
                        u32x4 bq;
                        bq[0] = and_or(wv, dq_mask, dq_magic);
                        bq[1] = and_or(wv >> 4, dq_mask, dq_magic);
                        bq[2] = and_or(wv >> 8, dq_mask, dq_magic);
                        bq[3] = and_or(wv >> 12, dq_mask, dq_magic);
                        const u32x4 av = *reinterpret_cast<const u32x4*>(arow + (word >> 2) * 128 + 32 * (word & 3));
                        t = mfma16x16x32<DT>(av, bq, t);
                    }
                    const float sf = act_to_float<DT>(cur.sb[bb]);
                    const float zf = -(magic_base<DT>() + (float)cur.zb[bb]);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = __builtin_fmaf(sf, __builtin_fmaf(zf, S[bb][jj], t[jj]), acc[i][jj]);
                }
                cur = nxt;
            }
        }
        if (more) stage_store(buf ^ 1, stg);
        __syncthreads();
    }

    // Reduce each n-tile's accumulators over the waves (fixed order), add the
    // bias, round once, store.
#pragma unroll
    for (int i = 0; i < kMaxTilesPerWG; ++i) {
        if (i < nn) {
            red[wave * 64 + lane] = acc[i];
            __syncthreads();
            if (wave == 0) {
                floatx4 tot = acc[i];
                for (int q = 1; q < nwaves; ++q) tot += red[q * 64 + lane];
                const int64_t n = (blockIdx.x + (int64_t)i * gridDim.x) * 16 + r;
                const float bv = a.bias ? act_to_float<DT>(a.bias[n]) : 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int m = 4 * g4 + jj;
                    if (m < a.M) a.C[(int64_t)m * a.ldc + n] = to_act_bits<DT>(tot[jj] + bv);
                }
            }
            __syncthreads();
        }
    }
}

template <int DT, int QT, int KT, int FW>
hipError_t launch_persist_fw(const SkinnyArgs& a, const PersistArgs& ph, dim3 grid, dim3 block, size_t lds,
                             hipStream_t stream) {
    hipError_t e = allow_lds<skinny_persist_kernel<DT, QT, KT, FW>>(lds);
    if (e == hipSuccess) hipLaunchKernelGGL((skinny_persist_kernel<DT, QT, KT, FW>), grid, block, lds, stream, a, ph);
    return e;
}

template <int DT, int QT, int KT>
hipError_t launch_persist_t(const SkinnyArgs& a, const PersistArgs& ph, int fw, dim3 grid, dim3 block, size_t lds,
                            hipStream_t stream) {
    switch (fw) {
        case 1: return launch_persist_fw<DT, QT, KT, 1>(a, ph, grid, block, lds, stream);
        case 2: return launch_persist_fw<DT, QT, KT, 2>(a, ph, grid, block, lds, stream);
        default: return launch_persist_fw<DT, QT, KT, 4>(a, ph, grid, block, lds, stream);
    }
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
hipError_t launch_persist_q(const SkinnyArgs& a, const SkinnyPlan& p, int spt, hipStream_t stream) {
    PersistArgs ph;
    ph.PT = p.WK * p.KT;
    ph.phases = (int)((a.KTT + ph.PT - 1) / ph.PT);
    ph.lds_ld = ph.PT * 128 + 8;
    ph.buf_bytes = (a.M * ph.lds_ld * 2 + 15) / 16 * 16;
    const size_t lds = 2 * (size_t)ph.buf_bytes + (size_t)p.WK * 64 * sizeof(floatx4);
    const dim3 grid((unsigned)p.n_groups), block((unsigned)(64 * p.WK));
    // Fold width: words per fold block, at most one group (G / 32 words) and
    // at most 4 (one k-tile); spt = groups per k-tile.
    const int fw = spt >= 4 ? 1 : (spt == 2 ? 2 : 4);
    switch (p.KT) {
        case 1: return launch_persist_t<DT, QT, 1>(a, ph, fw, grid, block, lds, stream);
        case 2: return launch_persist_t<DT, QT, 2>(a, ph, fw, grid, block, lds, stream);
        default: return launch_persist_t<DT, QT, 4>(a, ph, fw, grid, block, lds, stream);
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
    (void)M;  // sized for 16 rows, so one workspace serves every M <= 16
    SkinnyPlan p;
    const int64_t NT = g.N / 16, KTT = g.K / 128;
    if (NT >= kFullKMinTiles) {
        // Persistent: one workgroup of up to 8 waves per CU, at most
        // kMaxTilesPerWGHost n-tiles each. Phases of PT = waves * KT k-tiles
        // with M * PT <= 256, so two phase buffers of M rows take at most
        // 129 KB of LDS; as many k-tiles per wave as that allows, up to 4.
        p.full_k = true;
        p.NW = 1;
        p.n_groups = NT < kCUs ? NT : kCUs;
        if ((NT + p.n_groups - 1) / p.n_groups > kMaxTilesPerWGHost)
            p.n_groups = (NT + kMaxTilesPerWGHost - 1) / kMaxTilesPerWGHost;
        const int64_t m = M < 1 ? 1 : M;
        p.WK = (int)(KTT < 8 ? KTT : 8);
        p.KT = 1;
        while (p.KT < 4 && (int64_t)p.WK * p.KT * 2 * m <= 256 && (int64_t)p.WK * p.KT * 2 <= KTT) p.KT *= 2;
        p.ksplit = 1;
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
    a.NT = g.N / 16;
    a.KTT = g.K / 128;
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
    a.mask = 0x000F000Fu;
    a.magic = dtype == 0 ? 0x64006400u : 0x43004300u;
    const int spt = g.Kg == 1 ? 1 : (g.Ge >= 128 ? 1 : 128 / g.Ge);
    const dim3 grid((unsigned)nblocks);
    if (p.full_k) {
        hipError_t e;
        if (dtype == 0) e = g.qtype ? launch_persist_q<0, 1>(a, p, spt, stream) : launch_persist_q<0, 0>(a, p, spt, stream);
        else e = g.qtype ? launch_persist_q<1, 1>(a, p, spt, stream) : launch_persist_q<1, 0>(a, p, spt, stream);
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
