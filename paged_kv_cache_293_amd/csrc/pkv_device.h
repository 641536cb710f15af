// Device helpers shared by the cache-write and attention kernels.  Not part
// of the public ABI.
#pragma once

#include "pkv_internal.h"

namespace pkv {

enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_INT8 = 3, KV_INT4 = 4 };

// Code element types carry a float32 scale per (layer, KV head).
template <int KVT> constexpr bool kv_scaled() { return KVT == KV_FP8 || KVT == KV_INT8 || KVT == KV_INT4; }

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// E4M3 code of x * inv: the product is one float32 multiply (round to nearest
// even), saturated to +-448 by comparisons that let NaN through, then
// converted with round-to-nearest-even by the hardware converter.
__device__ __forceinline__ unsigned quantize_e4m3(float x, float inv) {
    float y = __fmul_rn(x, inv);
    y = (y > 448.f) ? 448.f : y;
    y = (y < -448.f) ? -448.f : y;
    return static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false)) & 0xffu;
}

// Symmetric int8 code of x * inv: one float32 multiply (round to nearest
// even), NaN -> 0, round to the nearest integer with ties to even, saturate to
// +-127 (the code -128 is never written).
__device__ __forceinline__ unsigned quantize_i8(float x, float inv) {
    float y = __fmul_rn(x, inv);
    y = (y == y) ? y : 0.f;
    y = __builtin_rintf(fminf(fmaxf(y, -127.f), 127.f));
    return static_cast<unsigned>(static_cast<int>(y)) & 0xffu;
}

// Symmetric int4 code (the low nibble of the result): as int8, saturated to
// +-7 (the code -8 is never written).
__device__ __forceinline__ unsigned quantize_i4(float x, float inv) {
    float y = __fmul_rn(x, inv);
    y = (y == y) ? y : 0.f;
    y = __builtin_rintf(fminf(fmaxf(y, -7.f), 7.f));
    return static_cast<unsigned>(static_cast<int>(y)) & 0xfu;
}

template <int KVT>
__device__ __forceinline__ unsigned quantize_code(float x, float inv) {
    if constexpr (KVT == KV_INT8) return quantize_i8(x, inv);
    else if constexpr (KVT == KV_INT4) return quantize_i4(x, inv);
    else return quantize_e4m3(x, inv);
}

// Element i of an input row as float (float32 or bfloat16 input).
template <int IN>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
    if constexpr (IN == KV_F32) return reinterpret_cast<const float*>(p)[i];
    else return __uint_as_float(static_cast<unsigned>(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

// Write one token's K and V, heads [h0, h0 + nh), at offset `off` of a
// physical block (page "KV cache & continuous batching", section
// "2. PagedAttention (vLLM)": the token's slot is block * 16 + offset).
//   blk    first tile of the block in this layer, tile (l, p, h = 0, K)
//   k_row  the token's K input, [H_kv][D] elements of type IN (same for v_row)
//   k_inv, v_inv  fp8 pools: per-head 1/scale arrays of this layer ([H_kv])
// K goes in 16-byte chunks (element ((i / X) * 16 + off) * X + i % X of the
// K tile), V element by element (element i * 16 + off of the V tile).
// Threads tid = 0 .. nthr-1 of the caller share the work.
template <int KVT, int IN, int D>
__device__ __forceinline__ void write_token(uint8_t* blk, int64_t tile_bytes, int off, const void* k_row,
                                            const void* v_row, int h0, int nh, const float* k_scale,
                                            const float* v_scale, int tid, int nthr);

// Nibbles [n0, n0 + 8) of an int4 run as one 32-bit word, code j = value
// index `first + stride * j` of the row (low nibble first).
template <int IN>
__device__ __forceinline__ unsigned pack8_i4(const void* row, int64_t first, int stride, float inv) {
    unsigned w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= quantize_i4(load_in<IN>(row, first + stride * j), inv) << (4 * j);
    return w;
}

// int4 pools (layout in the library header): per token, K is four runs of
// D / 4 nibbles (lane groups g), V one byte in every fourth byte of sixteen
// runs (columns c); every byte written belongs to this token alone.
template <int IN, int D>
__device__ __forceinline__ void write_token_i4(uint8_t* blk, int64_t tile_bytes, int off, const void* k_row,
                                               const void* v_row, int h0, int nh, const float* k_scale,
                                               const float* v_scale, int tid, int nthr) {
    constexpr int W = D / 4;                 // nibbles per lane run
    for (int it = tid; it < nh * 4; it += nthr) {          // K: run (g, off)
        const int h = h0 + it / 4;
        const int g = it % 4;
        const float inv = 1.0f / k_scale[h];
        uint8_t* run = blk + static_cast<int64_t>(h) * 2 * tile_bytes + (g * 16 + off) * (W / 2);
        const int64_t src = static_cast<int64_t>(h) * D;
        // dims 32 s + 8 g + e at nibble 8 s + e
        if constexpr (D == 128) {
            u32x4_t w;
#pragma unroll
            for (int st = 0; st < 4; ++st) w[st] = pack8_i4<IN>(k_row, src + 32 * st + 8 * g, 1, inv);
            *reinterpret_cast<u32x4_t*>(run) = w;
        } else {
            const unsigned w0 = pack8_i4<IN>(k_row, src + 8 * g, 1, inv);
            const unsigned w1 = pack8_i4<IN>(k_row, src + 32 + 8 * g, 1, inv);
            reinterpret_cast<unsigned*>(run)[0] = w0;
            reinterpret_cast<unsigned*>(run)[1] = w1;
        }
    }
    const int g = off / 4, t = off % 4;
    for (int it = tid; it < nh * 16; it += nthr) {         // V: column c of run (g, c)
        const int h = h0 + it / 16;
        const int c = it % 16;
        const float inv = 1.0f / v_scale[h];
        uint8_t* run = blk + (static_cast<int64_t>(h) * 2 + 1) * tile_bytes + (g * 16 + c) * (W / 2);
        const int64_t src = static_cast<int64_t>(h) * D + c;
        // byte 4 j + t of the run: dims 16 (2 j) + c (low nibble) and
        // 16 (2 j + 1) + c (high nibble) of this token
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
            const unsigned lo = quantize_i4(load_in<IN>(v_row, src + 16 * (2 * j)), inv);
            const unsigned hi = quantize_i4(load_in<IN>(v_row, src + 16 * (2 * j + 1)), inv);
            run[4 * j + t] = static_cast<uint8_t>(lo | (hi << 4));
        }
    }
}

template <int KVT, int IN, int D>
__device__ __forceinline__ void write_token(uint8_t* blk, int64_t tile_bytes, int off, const void* k_row,
                                            const void* v_row, int h0, int nh, const float* k_scale,
                                            const float* v_scale, int tid, int nthr) {
    if constexpr (KVT == KV_INT4) {
        write_token_i4<IN, D>(blk, tile_bytes, off, k_row, v_row, h0, nh, k_scale, v_scale, tid, nthr);
        return;
    }
    constexpr int EB = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);
    constexpr int X = 16 / EB;
    constexpr int CH = D / X;
    for (int c = tid; c < nh * CH; c += nthr) {
        const int h = h0 + c / CH;
        const int ch = c % CH;
        uint8_t* dst = blk + static_cast<int64_t>(h) * 2 * tile_bytes + (ch * kBlock + off) * 16;
        const int64_t src = static_cast<int64_t>(h) * D + ch * X;
        if constexpr (kv_scaled<KVT>()) {
            const float inv = 1.0f / k_scale[h];
            unsigned w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned b = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) b |= quantize_code<KVT>(load_in<IN>(k_row, src + 4 * q + e), inv) << (8 * e);
                w[q] = b;
            }
            *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
        } else {
            const uint8_t* s = reinterpret_cast<const uint8_t*>(k_row) + src * EB;
            *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(s);
        }
    }
    for (int e = tid; e < nh * D; e += nthr) {
        const int h = h0 + e / D;
        const int i = e % D;
        uint8_t* dst = blk + (static_cast<int64_t>(h) * 2 + 1) * tile_bytes + (i * kBlock + off) * EB;
        const int64_t src = static_cast<int64_t>(h) * D + i;
        if constexpr (kv_scaled<KVT>()) {
            *dst = static_cast<uint8_t>(quantize_code<KVT>(load_in<IN>(v_row, src), 1.0f / v_scale[h]));
        } else if constexpr (KVT == KV_BF16) {
            *reinterpret_cast<uint16_t*>(dst) = reinterpret_cast<const uint16_t*>(v_row)[src];
        } else {
            *reinterpret_cast<float*>(dst) = reinterpret_cast<const float*>(v_row)[src];
        }
    }
}

}  // namespace pkv
