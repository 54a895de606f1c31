// device_common.h -- device helpers shared by the skinny and tiled W4A16
// kernels: operand types, the in-register dequantisation of one packed word
// into a 16x16x32 MFMA B operand, the MFMA call and the output rounding.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Activation dtypes: 0 = fp16, 1 = bf16. Quant types: 0 = uint4b8 (zero 8),
// 1 = uint4 (zero from the packed buffer).

// Dequantisation of one word (eight codes in pair order: codes 2p and 2p+1
// at bits 4p and 16+4p) into eight act-dtype values RN((q - z) * s), exactly
// the rounding of the pages' `dequantize_w4a16` ("rdna_hybrid_w4a16", build
// 61746): q - z is a small integer, so one rounding of the product is the
// whole error.
//
// fp16: OR-ing a nibble into the low mantissa of 1024.0 (0x6400) gives the
// fp16 value 1024 + q (the `_int4_pair_to_fp16x2` idea of that page), two
// nibbles per v_and_or_b32. Adding -(1024 + z) is exact; the multiply by s
// rounds once.
//
// bf16: 0x4300 is 128.0 and its mantissa has 7 bits, so OR-ing a nibble gives
// 128 + q exactly. v_dot2_f32_bf16 with (s, 0) or (0, s) and the fp32
// constant c = -(128 + z) * s (exact: an 8-bit integer times an 8-bit
// significand) yields (q - z) * s exactly in fp32 (every partial sum is
// representable); v_cvt_pk_bf16_f32 then rounds to nearest even once.
//
// The pair extraction (w >> 4p) & 0x000F000F | magic is one v_and_or_b32 per
// pair (plus the shift). The mask and magic are passed in registers (callers
// keep them opaque with an empty asm): gfx9 VOP3 instructions cannot encode
// two literal constants, and given literals the compiler splits the
// operation into v_and_b32 + v_or_b32. Plain C rather than inline asm: the
// result often feeds an MFMA directly, and only an instruction the compiler
// knows gets the wait states the hardware needs between a VALU write of a
// register and an MFMA that reads it (an asm result does not).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) { return (x & mask) | magic; }

template <int DT>
struct Dequant;

template <>
struct Dequant<0> {
    struct Params {
        half2_t zz;  // -(1024 + z), both halves
        half2_t ss;  // s, both halves
    };
    static __device__ __forceinline__ Params make(uint16_t sbits, int z) {
        Params p;
        const _Float16 s = __builtin_bit_cast(_Float16, sbits);
        const _Float16 zz = (_Float16)(-(1024 + z));  // exact
        p.zz = half2_t{zz, zz};
        p.ss = half2_t{s, s};
        return p;
    }
    // mask = 0x000F000F, magic = 0x64006400.
    static __device__ __forceinline__ u32x4 apply(uint32_t w, const Params& p, uint32_t mask, uint32_t magic) {
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t x = and_or(w >> (4 * q), mask, magic);
            half2_t h = __builtin_bit_cast(half2_t, x);
            h = (h + p.zz) * p.ss;
            out[q] = __builtin_bit_cast(uint32_t, h);
        }
        return out;
    }
};

template <>
struct Dequant<1> {
    struct Params {
        bf16x2_t slo;  // (s, 0)
        bf16x2_t shi;  // (0, s)
        float c;       // -(128 + z) * s, exact in fp32
    };
    static __device__ __forceinline__ Params make(uint16_t sbits, int z) {
        Params p;
        p.slo = __builtin_bit_cast(bf16x2_t, (uint32_t)sbits);
        p.shi = __builtin_bit_cast(bf16x2_t, (uint32_t)sbits << 16);
        const float s = __builtin_bit_cast(float, (uint32_t)sbits << 16);
        p.c = -(128.0f + (float)z) * s;
        return p;
    }
    // mask = 0x000F000F, magic = 0x43004300.
    static __device__ __forceinline__ u32x4 apply(uint32_t w, const Params& p, uint32_t mask, uint32_t magic) {
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t x = and_or(w >> (4 * q), mask, magic);
            const bf16x2_t b = __builtin_bit_cast(bf16x2_t, x);
            const float lo = __builtin_amdgcn_fdot2_f32_bf16(b, p.slo, p.c, false);
            const float hi = __builtin_amdgcn_fdot2_f32_bf16(b, p.shi, p.c, false);
            const bf16x2_t r = bf16x2_t{(__bf16)lo, (__bf16)hi};
            out[q] = __builtin_bit_cast(uint32_t, r);
        }
        return out;
    }
};

// Offset-corrected B operand of the tiled kernels: code q becomes the exact
// act value 1 + q/16, the nibble OR-ed into the top four mantissa bits of 1.0
// (fp16 bits 6..9 of each half, bf16 bits 3..6). Pair p of a word (codes 2p
// and 2p+1 at bits 4p and 16+4p) moves there with one shift by kPos - 4p and
// one v_and_or_b32. A product sum P = sum A*(1 + q/16) then carries the
// offset sum A with weight 1 against code steps of 1/16, so
// sum A*(q - z) = 16*P - (16 + z)*S (S = sum A) cancels only a few bits even
// when sum A grows with K (the magic 1024 + q of the skinny kernels would
// carry the offset 1024 times one code step).
template <int DT>
struct TopNibble {
    static constexpr int kPos = DT == 0 ? 6 : 3;  // lowest bit of the nibble in each half
    static constexpr uint32_t kMask = (0xFu << kPos) * 0x00010001u;
    static constexpr uint32_t kOne = DT == 0 ? 0x3C003C00u : 0x3F803F80u;  // 1.0 in both halves
};

// Word w shifted so that its pair P lands at the nibble position.
template <int DT, int P>
__device__ __forceinline__ uint32_t top_pair_shift(uint32_t w) {
    constexpr int sh = TopNibble<DT>::kPos - 4 * P;
    if constexpr (sh >= 0) {
        return w << sh;
    } else {
        return w >> (-sh);
    }
}

// The same shift of two consecutive words held as one 64-bit value (word 0
// low): one v_lshlrev_b64 / v_lshrrev_b64 serves both. The bits that cross
// between the halves land outside the nibble masks. The empty asm (no
// instruction) keeps the compiler from narrowing the shift into one per
// word; the shift itself stays a compiler-emitted instruction, so its
// register hazards against in-flight MFMAs are tracked.
template <int DT, int P>
__device__ __forceinline__ uint64_t top_pair_shift64(uint64_t x) {
    constexpr int sh = TopNibble<DT>::kPos - 4 * P;
    uint64_t y;
    if constexpr (sh > 0) {
        y = x << sh;
    } else if constexpr (sh < 0) {
        y = x >> -sh;
    } else {
        y = x;
    }
    asm("" : "+v"(y));
    return y;
}

// acc += A_frag (16 rows x 32 k) * B_frag (32 k x 16 cols), fp32 accumulate.
// Lane l holds A[l%16][8(l/16) .. +7] and B[8(l/16) .. +7][l%16]; the result
// lane l holds rows 4(l/16) .. +3 of column l%16.
template <int DT>
__device__ __forceinline__ floatx4 mfma16x16x32(const u32x4& a, const u32x4& b, const floatx4& acc);

template <>
__device__ __forceinline__ floatx4 mfma16x16x32<0>(const u32x4& a, const u32x4& b, const floatx4& acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), acc,
                                                  0, 0, 0);
}

template <>
__device__ __forceinline__ floatx4 mfma16x16x32<1>(const u32x4& a, const u32x4& b, const floatx4& acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   acc, 0, 0, 0);
}

// The magic constant of the pair extraction for each act dtype.
template <int DT>
constexpr uint32_t kMagic = DT == 0 ? 0x64006400u : 0x43004300u;

// fp32 -> act dtype bits, round to nearest even; and act bits -> fp32.
template <int DT>
__device__ __forceinline__ uint16_t to_act_bits(float x) {
    if constexpr (DT == 0) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    } else {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
}

template <int DT>
__device__ __forceinline__ float act_to_float(uint16_t b) {
    if constexpr (DT == 0) {
        return (float)__builtin_bit_cast(_Float16, b);
    } else {
        return __builtin_bit_cast(float, (uint32_t)b << 16);
    }
}

}  // namespace w4a16
