// repack.hip -- one-time repack of a compressed-tensors GPTQ checkpoint into
// the gfx950 packed buffer, and its inverse (test support).
//
// The checkpoint layout is the one "triton_w4a16.py" (Triton-based W4A16 GEMM
// for ROCm MI300) lists in its module docstring: weight_packed [N, K/8] int32
// with code k = 8j + i of row n at bits 4i of word j, weight_scale [N, K/G],
// weight_zero_point [N/8, K/G] int32 with row n at bits 4*(n%8) of word n/8.
// The pages repack on the host at load time (`process_weights_after_loading`,
// `repack_w_q`); here it is one pass of three small GPU kernels, bit-exact.
//
// The same kernels read the other orientations the page's
// `process_weights_after_loading` and zero-point handling accept: a packed
// tensor is described by the dimension over N (output_dim) and the dimension
// whose eight consecutive entries share a word (packed_dim), value i of a
// word at bits 4i. AWQ weights arrive as (K, N/8) (packed along N), AutoGPTQ
// ones as (K/8, N), scales as (K/G, N), AutoGPTQ zero points as (K/G, N/8).
#include "internal.h"

namespace w4a16 {
namespace {

// GPTQ order (code i at bits 4i) -> pair order (code i at 4*(i/2) + 16*(i%2)):
// even codes move to the low half-word, odd codes to the high half-word, so
// that (w >> 4p) & 0x000F000F holds codes 2p and 2p+1 in separate halves.
__device__ __forceinline__ uint32_t gptq_to_pair_order(uint32_t w) {
    uint32_t even = 0, odd = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        even |= ((w >> (8 * p)) & 0xFu) << (4 * p);
        odd |= ((w >> (8 * p + 4)) & 0xFu) << (4 * p);
    }
    return even | (odd << 16);
}

__device__ __forceinline__ uint32_t pair_to_gptq_order(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        out |= ((w >> (4 * p)) & 0xFu) << (8 * p);
        out |= ((w >> (16 + 4 * p)) & 0xFu) << (8 * p + 4);
    }
    return out;
}

// Index of checkpoint word (nw, kw) in a tensor of Nw x Kw words stored with
// N first ([Nw][Kw]) or K first ([Kw][Nw]).
template <bool NFIRST>
__device__ __forceinline__ int64_t word_index(int64_t nw, int64_t kw, int64_t Nw, int64_t Kw) {
    return NFIRST ? nw * Kw + kw : kw * Nw + nw;
}

// One thread per (tile, lane): builds the four words that lane l of tile
// (nt, kt) holds (codes of row n at k0 .. k0+7, k0 = 128kt + 32s + 8(l/16))
// and writes them as one 16-byte store. Packed along K, each is one
// checkpoint word with its nibbles reordered; packed along N, its eight codes
// come from nibble n%8 of eight words, one per k.
template <bool NFIRST, bool KPACKED>
__global__ __launch_bounds__(256) void repack_codes_kernel(const uint32_t* __restrict__ wq, uint4* __restrict__ out,
                                                           int64_t N, int64_t Np, int64_t K, int64_t Kp) {
    const int64_t KT = Kp / 128;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (Np / 16) * KT * 64;
    if (t >= total) return;
    const int64_t tile = t >> 6;
    const int l = (int)(t & 63);
    const int64_t nt = tile / KT, kt = tile - nt * KT;
    const int64_t n = 16 * nt + (l & 15);
    const int64_t k = 128 * kt + 8 * (l >> 4);
    uint32_t w[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int64_t k0 = k + 32 * s;
        if (n >= N || k0 >= K) {  // padding of N up to Np, of K up to Kp (K % 8 == 0)
            w[s] = 0u;
        } else if constexpr (KPACKED) {
            w[s] = gptq_to_pair_order(wq[word_index<NFIRST>(n, k0 / 8, N, K / 8)]);
        } else {
            const int shift = 4 * (int)(n & 7);
            uint32_t v = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t q = (wq[word_index<NFIRST>(n >> 3, k0 + i, N / 8, K)] >> shift) & 0xFu;
                v |= q << (4 * (i >> 1) + 16 * (i & 1));
            }
            w[s] = v;
        }
    }
    out[t] = make_uint4(w[0], w[1], w[2], w[3]);
}

// One thread per (row, group): scales to [N/16][Kg][16], zeros likewise.
// Kg stored groups per row; the checkpoint holds Kg_ck <= Kg of them, and
// the rest (groups of the padding of K), like the rows of the padding of N,
// get scale 0 and zero 0.
template <bool SNFIRST, bool ZNFIRST>
__global__ __launch_bounds__(256) void repack_scales_kernel(const uint16_t* __restrict__ ws,
                                                            const uint32_t* __restrict__ wzp,
                                                            uint16_t* __restrict__ s_out, uint8_t* __restrict__ z_out,
                                                            int64_t N, int64_t Np, int64_t Kg, int64_t Kg_ck) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= Np * Kg) return;
    // t enumerates the destination order so the stores are contiguous.
    const int r = (int)(t & 15);
    const int64_t ng = t >> 4;  // nt * Kg + g
    const int64_t nt = ng / Kg, g = ng - nt * Kg;
    const int64_t n = 16 * nt + r;
    const bool real = n < N && g < Kg_ck;
    s_out[t] = real ? ws[SNFIRST ? n * Kg_ck + g : g * N + n] : (uint16_t)0;
    if (z_out != nullptr) {
        uint8_t z = 0;
        if (wzp != nullptr && real)
            z = (uint8_t)((wzp[word_index<ZNFIRST>(n >> 3, g, N / 8, Kg_ck)] >> (4 * (n & 7))) & 0xFu);
        z_out[t] = z;
    }
}

__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint4* __restrict__ in, uint8_t* __restrict__ codes,
                                                           int64_t N, int64_t Np, int64_t K, int64_t Kp) {
    const int64_t KT = Kp / 128;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (Np / 16) * KT * 64;
    if (t >= total) return;
    const int64_t tile = t >> 6;
    const int l = (int)(t & 63);
    const int64_t nt = tile / KT, kt = tile - nt * KT;
    const int64_t n = 16 * nt + (l & 15);
    if (n >= N) return;  // padding of N
    const uint4 v = in[t];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int64_t k0 = 128 * kt + 32 * s + 8 * (l >> 4);
        if (k0 >= K) continue;  // padding of K
        const uint32_t g = pair_to_gptq_order(w[s]);
        uint8_t* dst = codes + n * K + k0;
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = (uint8_t)((g >> (4 * i)) & 0xFu);
    }
}

__global__ __launch_bounds__(256) void unpack_scales_kernel(const uint16_t* __restrict__ s_in,
                                                            const uint8_t* __restrict__ z_in,
                                                            uint16_t* __restrict__ s_out, uint8_t* __restrict__ z_out,
                                                            int64_t N, int64_t Np, int64_t Kg, int64_t Kg_ck) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= Np * Kg) return;
    const int r = (int)(t & 15);
    const int64_t ng = t >> 4;
    const int64_t nt = ng / Kg, g = ng - nt * Kg;
    const int64_t n = 16 * nt + r;
    if (n >= N || g >= Kg_ck) return;  // padding of N or of K
    if (s_out != nullptr) s_out[n * Kg_ck + g] = s_in[t];
    if (z_out != nullptr && z_in != nullptr) z_out[n * Kg_ck + g] = z_in[t];
}

// Zero-fills [begin, end) of the packed buffer (alignment padding), byte by
// byte; the gaps are at most 255 bytes each.
__global__ __launch_bounds__(256) void zero_gap_kernel(uint8_t* __restrict__ base, size_t begin, size_t end) {
    const size_t i = begin + threadIdx.x;
    if (i < end) base[i] = 0;
}

inline unsigned blocks_for(int64_t threads, int per_block) { return (unsigned)((threads + per_block - 1) / per_block); }

}  // namespace

hipError_t launch_repack(const int32_t* wq, const uint16_t* ws, const int32_t* wzp, const CheckpointLayout& lay,
                         const Geometry& g, void* packed, hipStream_t stream) {
    uint8_t* base = static_cast<uint8_t*>(packed);
    const int64_t code_threads = (g.Np / 16) * (g.Kp / 128) * 64;
    const dim3 cgrid(blocks_for(code_threads, 256));
    const uint32_t* src = reinterpret_cast<const uint32_t*>(wq);
    uint4* dst = reinterpret_cast<uint4*>(base);
    if (lay.weight_n_first && lay.weight_k_packed)
        hipLaunchKernelGGL((repack_codes_kernel<true, true>), cgrid, dim3(256), 0, stream, src, dst, g.N, g.Np, g.K, g.Kp);
    else if (lay.weight_n_first)
        hipLaunchKernelGGL((repack_codes_kernel<true, false>), cgrid, dim3(256), 0, stream, src, dst, g.N, g.Np, g.K, g.Kp);
    else if (lay.weight_k_packed)
        hipLaunchKernelGGL((repack_codes_kernel<false, true>), cgrid, dim3(256), 0, stream, src, dst, g.N, g.Np, g.K, g.Kp);
    else
        hipLaunchKernelGGL((repack_codes_kernel<false, false>), cgrid, dim3(256), 0, stream, src, dst, g.N, g.Np, g.K, g.Kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint8_t* z_out = g.qtype == 1 ? base + g.zeros_off : nullptr;
    const uint32_t* zp = g.qtype == 1 ? reinterpret_cast<const uint32_t*>(wzp) : nullptr;
    uint16_t* s_out = reinterpret_cast<uint16_t*>(base + g.scales_off);
    const dim3 sgrid(blocks_for(g.Np * g.Kg, 256));
    if (lay.scale_n_first && lay.zero_n_first)
        hipLaunchKernelGGL((repack_scales_kernel<true, true>), sgrid, dim3(256), 0, stream, ws, zp, s_out, z_out, g.N, g.Np, g.Kg, g.Kg_ck);
    else if (lay.scale_n_first)
        hipLaunchKernelGGL((repack_scales_kernel<true, false>), sgrid, dim3(256), 0, stream, ws, zp, s_out, z_out, g.N, g.Np, g.Kg, g.Kg_ck);
    else if (lay.zero_n_first)
        hipLaunchKernelGGL((repack_scales_kernel<false, true>), sgrid, dim3(256), 0, stream, ws, zp, s_out, z_out, g.N, g.Np, g.Kg, g.Kg_ck);
    else
        hipLaunchKernelGGL((repack_scales_kernel<false, false>), sgrid, dim3(256), 0, stream, ws, zp, s_out, z_out, g.N, g.Np, g.Kg, g.Kg_ck);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Padding bytes between and after the regions are part of the contract
    // (zero), so the whole buffer is a pure function of the checkpoint. Each
    // gap is shorter than 256 bytes (alignment padding only).
    const size_t gaps[3][2] = {
        {g.codes_bytes, g.scales_off},
        {g.scales_off + (size_t)(g.Np * g.Kg * 2), g.qtype == 1 ? g.zeros_off : g.total_bytes},
        {g.qtype == 1 ? g.zeros_off + (size_t)(g.Np * g.Kg) : g.total_bytes, g.total_bytes},
    };
    for (auto& gap : gaps) {
        if (gap[1] > gap[0]) {
            hipLaunchKernelGGL(zero_gap_kernel, dim3(1), dim3(256), 0, stream, base, gap[0], gap[1]);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_unpack(const void* packed, const Geometry& g, uint8_t* codes, uint16_t* scale_bits, uint8_t* zeros,
                         hipStream_t stream) {
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    if (codes != nullptr) {
        const int64_t code_threads = (g.Np / 16) * (g.Kp / 128) * 64;
        hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks_for(code_threads, 256)), dim3(256), 0, stream,
                           reinterpret_cast<const uint4*>(base), codes, g.N, g.Np, g.K, g.Kp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    uint8_t* z_out = g.qtype == 1 ? zeros : nullptr;
    if (scale_bits != nullptr || z_out != nullptr) {
        hipLaunchKernelGGL(unpack_scales_kernel, dim3(blocks_for(g.Np * g.Kg, 256)), dim3(256), 0, stream,
                           reinterpret_cast<const uint16_t*>(base + g.scales_off),
                           g.qtype == 1 ? base + g.zeros_off : nullptr, scale_bits, z_out, g.N, g.Np, g.Kg, g.Kg_ck);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace w4a16
