// Matrix-core operand helpers shared by the decode/verify and the prefill
// attention kernels (gfx950): element conversions, per-lane tile and query
// registers in the layouts the 16x16x32 / 16x16x16 / 16x16x4 MFMAs take, and
// the score product.  Not part of the public ABI.
#pragma once

#include <type_traits>

#include "pkv_device.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// float -> bfloat16 bits, round to nearest even (the gfx950 converter).
__device__ __forceinline__ unsigned f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

// Two floats -> two bf16 (round to nearest even) packed low/high, in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// A vector instruction may read a matrix-core result only some cycles after
// the product issues (the wait states grow with the product's passes).  The
// compiler pads such reads within a basic block, but a read it moved past a
// branch was found unpadded on the branch-taken path (garbage scores in the
// decode kernel).  The decode kernel therefore reads its score tiles in one
// place, the scaling right after the products, and this empty statement,
// which takes the scaled values as its operands, keeps that scaling in the
// products' basic block: the compiler cannot move the reads past it.
__device__ __forceinline__ void pin_after_mfma_reads(f32x4& s) { asm volatile("" : "+v"(s)); }

// Maximum of scores (finite, or -inf where masked): the IEEE maximum, which
// passes NaN through and so needs no quieting of its operands (fmaxf costs
// one canonicalising max per operand in IEEE mode); v_maximum3_f32 takes
// three operands.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum of x over the four lanes l, l^16, l^32, l^48 (the four 16-lane
// rows of the wave), with the gfx950 row-swap permutes (no LDS traffic).
__device__ __forceinline__ float max_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = smax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return smax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Buffer resource over one block's K tile followed by its V tile.  Loads
// through it address the tile with a per-lane 32-bit offset plus an immediate,
// and read 0 beyond the two tiles.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int64_t tile_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0,
                                             static_cast<int>(2 * tile_bytes), 0x00020000);
}

// Partial results pass between work-groups of one launch, which may run on
// different XCDs with separate L2 caches: they are written and read with
// agent-scope accesses, which the hardware keeps coherent across the device.
__device__ __forceinline__ void xwg_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xwg_load(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cache policies of the KV tile loads.  A decode step reads a block that
// one sequence owns once, so its tiles are streamed past the caches
// (non-temporal, "nt"); measured on MI355X (paged_read_floor / read_ceiling
// probes and the decode step itself) this raises the read rate by 10-13%
// over the default policy, random 8 KiB reads from 5.8 to 6.5 TB/s.  A batch
// in which several sequences share blocks (a common prefix) reads those
// blocks once per sequence, and those reads should hit in the caches: its
// launches keep the default policy.  The policy is chosen per launch (a
// template argument), not per block: a per-block branch between the two
// loads made the compiler's wait counts conservative and the pipeline
// shallow.
constexpr int kStreamLoad = 2;
constexpr int kCachedLoad = 0;
// Cache-policy bits of the partial results' vector loads and stores: sc1,
// the bit agent-scope atomic loads and stores of one dword carry (xwg_load,
// xwg_store), so they stay coherent across the XCDs' L2 caches.
constexpr int kCoherent = 16;

// Tile load through a buffer resource with cache policy POL.
template <typename T, int POL>
__device__ __forceinline__ T bload(__amdgpu_buffer_rsrc_t r, int voff, int imm) {
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, imm, POL));
    else if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, voff, imm, POL));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, imm, POL));
}

// Two fp8 E4M3 codes (bytes 0-1, or 2-3 when HI, of w) -> two bf16 values packed in one
// dword, in one gfx950 scaled conversion with scale 1: every E4M3 value
// (3 mantissa bits, exponents 2^-9 .. 2^8) is exactly a bf16 value.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(unsigned, b);
}

// Two int8 codes (bytes 0-1, or 2-3 when HI, of w) -> two bf16 values packed
// in one dword.  |code| <= 127 has at most 8 significant bits, so the float32
// conversion is exact and so is its upper half.
template <bool HI>
__device__ __forceinline__ unsigned i8x2_to_bf16x2(unsigned w) {
    const float f0 = static_cast<float>(static_cast<int8_t>(w >> (HI ? 16 : 0)));
    const float f1 = static_cast<float>(static_cast<int8_t>(w >> (HI ? 24 : 8)));
    return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
}

// Two one-byte codes of type KVT -> two exact bf16 values.
template <int KVT, bool HI>
__device__ __forceinline__ unsigned byte2_to_bf16x2(unsigned w) {
    if constexpr (KVT == KV_INT8) return i8x2_to_bf16x2<HI>(w);
    else return fp8x2_to_bf16x2<HI>(w);
}

// int8 codes for the decode kernel's matrix cores, as fp16: flipping a
// code's sign bit gives the byte u = c + 128, and the fp16 bits 0x6400 | u
// are exactly 1024 + u = c + kI8Bias (fp16 holds every integer up to 2048).
// One byte permute places two codes under the constant high bytes, so four
// codes cost one XOR and two permutes.  The caller takes the bias out:
// kI8Bias times the query row's sum from the scores, times the probability
// sum from the output.
constexpr float kI8Bias = 1152.f;
// Codes b0, b1 (HI: b2, b3) of the sign-flipped dword x -> two fp16.
template <bool HI>
__device__ __forceinline__ unsigned i8x2_to_f16x2(unsigned x) {
    return __builtin_amdgcn_perm(0x64646464u, x, HI ? 0x04030402u : 0x04010400u);
}

// Two fp8 E4M3 codes of w -> bf16 pair, in the decode kernel's K order.
template <int KVT, bool HI>
__device__ __forceinline__ unsigned decode_pair(unsigned w) {
    static_assert(KVT == KV_FP8, "fp8 only");
    return fp8x2_to_bf16x2<HI>(w);
}

// Work-group barrier that orders LDS accesses only.  The plain barrier's
// fence also waits for every global load and store the thread has in flight;
// this one leaves them in flight (for data exchanged through LDS alone).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ tiles
// Per-lane registers of one block's K and V tiles, and their loads.
template <int KVT, int D> struct TileRegs;

template <int D> struct TileRegs<KV_BF16, D> {
    u32x4 k[D / 32];   // 8 bf16: token lane%16, dims of chunk 4s + lane/16
    u32x2 v[D / 16];   // 4 bf16: dim 16m + lane%16, tokens 4*(lane/16) .. +3
    // koff = lane * 16; voff = TILE + (lane % 16) * 32 + (lane / 16) * 8
    template <int POL>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int koff, int voff) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) k[s] = bload<u32x4, POL>(r, koff, 1024 * s);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < D / 16; ++m) v[m] = bload<u32x2, POL>(r, voff, 512 * m);
    }
    static constexpr int kTile = 16 * D * 2;
    __device__ static int v_offset(int lane) { return kTile + (lane & 15) * 32 + (lane >> 4) * 8; }
    // zero V of tokens >= nvalid among this lane's four (tokens 4j .. 4j+3)
    __device__ __forceinline__ void zero_v_from(int nvalid) {
        if (nvalid >= 4) return;
        const unsigned m0 = nvalid <= 0 ? 0u : (nvalid == 1 ? 0x0000ffffu : 0xffffffffu);
        const unsigned m1 = nvalid <= 2 ? 0u : 0x0000ffffu;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) { v[m][0] &= m0; v[m][1] &= m1; }
    }
    // Token o of the tile takes the values staged in LDS at st: its K
    // elements in dim order, then its V elements (the bytes the pool write
    // stores for it).  Only lanes that hold a part of token o change.
    __device__ __forceinline__ void put_token(int o, const uint8_t* st, int lane) {
        const uint16_t* ks = reinterpret_cast<const uint16_t*>(st);
        if ((lane & 15) == o) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s) k[s] = *reinterpret_cast<const u32x4*>(ks + (4 * s + (lane >> 4)) * 8);
        }
        if ((lane >> 4) == (o >> 2)) {
            const int e = o & 3;
            const unsigned sh = 16 * (e & 1);
            const unsigned keep = ~(0xffffu << sh);
#pragma unroll
            for (int m = 0; m < D / 16; ++m) {
                const unsigned x = static_cast<unsigned>(ks[D + 16 * m + (lane & 15)]) << sh;
                if (e < 2) v[m][0] = (v[m][0] & keep) | x;
                else v[m][1] = (v[m][1] & keep) | x;
            }
        }
    }
};

template <int D> struct TileRegs1B {
    u32x4 k[D / 64];   // 16 codes: token lane%16, dims of chunk 4r + lane/16
    unsigned v[D / 16];  // 4 codes: dim 16m + lane%16, tokens 4*(lane/16) .. +3
    // koff = lane * 16; voff = TILE + (lane % 16) * 16 + (lane / 16) * 4
    template <int POL>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int koff, int voff) {
#pragma unroll
        for (int q = 0; q < D / 64; ++q) k[q] = bload<u32x4, POL>(r, koff, 1024 * q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < D / 16; ++m) v[m] = bload<unsigned, POL>(r, voff, 256 * m);
    }
    static constexpr int kTile = 16 * D;
    __device__ static int v_offset(int lane) { return kTile + (lane & 15) * 16 + (lane >> 4) * 4; }
    __device__ __forceinline__ void zero_v_from(int nvalid) {
        if (nvalid >= 4) return;
        const unsigned msk = nvalid <= 0 ? 0u : (0xffffffffu >> (8 * (4 - nvalid)));
#pragma unroll
        for (int m = 0; m < D / 16; ++m) v[m] &= msk;
    }
    // Token o takes the codes staged in LDS at st (K codes in dim order, then
    // V codes); only lanes holding a part of token o change.
    __device__ __forceinline__ void put_token(int o, const uint8_t* st, int lane) {
        if ((lane & 15) == o) {
#pragma unroll
            for (int q = 0; q < D / 64; ++q) k[q] = *reinterpret_cast<const u32x4*>(st + (4 * q + (lane >> 4)) * 16);
        }
        if ((lane >> 4) == (o >> 2)) {
            const unsigned sh = 8 * (o & 3);
            const unsigned keep = ~(0xffu << sh);
#pragma unroll
            for (int m = 0; m < D / 16; ++m)
                v[m] = (v[m] & keep) | (static_cast<unsigned>(st[D + 16 * m + (lane & 15)]) << sh);
        }
    }
};
// fp8 and int8 tiles share the byte layout; only the code conversion differs.
template <int D> struct TileRegs<KV_FP8, D> : TileRegs1B<D> {};
template <int D> struct TileRegs<KV_INT8, D> : TileRegs1B<D> {};

// int4 tiles: each lane reads its own run of D / 4 nibbles from the K and the
// V tile (layout in the library header), so koff = lane * D / 8 and
// voff = TILE + lane * D / 8 with TILE = 8 * D.  K nibble 8 s + e holds dim
// 32 s + 8 (lane / 16) + e of token lane % 16; V byte 4 j + t holds dims
// 16 (2 j) + lane % 16 (low nibble) and 16 (2 j + 1) + lane % 16 (high
// nibble) of token 4 (lane / 16) + t, so V dword j holds two dim tiles for
// the lane's four tokens.
//
// Codes enter the matrix cores biased: flipping a nibble's top bit turns the
// code c into u = c + 8 in [0, 15], and the bf16 bits 0x4300 | u are exactly
// 128 + u = c + kI4Bias.  After the nibbles are split into bytes, two codes
// become one bf16 pair with one byte permute against the constant high
// bytes.  The bias is taken out of the scores (kI4Bias * sum of the query
// row) and of the output (kI4Bias * the row's probability sum) by the caller.
// Every nibble pattern is a finite value, so no V row needs zeroing.
template <int D> struct TileRegs<KV_INT4, D> {
    unsigned k[D / 32];
    unsigned v[D / 32];
    template <int POL>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int koff, int voff) {
        const int kb = (koff >> 4) * (D / 8);   // koff = lane * 16 by the caller's convention
        if constexpr (D == 128) {
            const u32x4 a = bload<u32x4, POL>(r, kb, 0);
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 b = bload<u32x4, POL>(r, voff, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) { k[j] = a[j]; v[j] = b[j]; }
        } else {
            const u32x2 a = bload<u32x2, POL>(r, kb, 0);
            __builtin_amdgcn_sched_barrier(0);
            const u32x2 b = bload<u32x2, POL>(r, voff, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) { k[j] = a[j]; v[j] = b[j]; }
        }
    }
    static constexpr int kTile = 8 * D;
    __device__ static int v_offset(int lane) { return kTile + lane * (D / 8); }
    // probabilities of tokens past the end are 0 and every code is finite
    __device__ __forceinline__ void zero_v_from(int) {}
    // Token o takes the codes staged in LDS at st, one code per byte (low
    // nibble): K codes in dim order, then V codes.  Only lanes holding a part
    // of token o change.
    __device__ __forceinline__ void put_token(int o, const uint8_t* st, int lane) {
        if ((lane & 15) == o) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                unsigned w = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) w |= (static_cast<unsigned>(st[32 * s + 8 * (lane >> 4) + e]) & 0xfu) << (4 * e);
                k[s] = w;
            }
        }
        if ((lane >> 4) == (o >> 2)) {
            // byte o % 4 of every V dword
            const unsigned sh = 8 * (o & 3);
            const unsigned keep = ~(0xffu << sh);
            const int c = lane & 15;
#pragma unroll
            for (int j = 0; j < D / 32; ++j) {
                const unsigned b = (static_cast<unsigned>(st[D + 32 * j + c]) & 0xfu) |
                                   ((static_cast<unsigned>(st[D + 32 * j + 16 + c]) & 0xfu) << 4);
                v[j] = (v[j] & keep) | (b << sh);
            }
        }
    }
};

constexpr float kI4Bias = 136.f;

// Biased nibbles of w split by parity: byte k of `even` holds u of nibble
// 2k, byte k of `odd` that of nibble 2k + 1.
__device__ __forceinline__ void i4_split(unsigned w, unsigned& even, unsigned& odd) {
    // (w ^ 0x88888888) & 0x0f0f0f0f and its shifted twin, each one
    // three-operand bit operation (the shift goes first, so the two do not
    // share an intermediate)
    even = (w ^ 0x88888888u) & 0x0f0f0f0fu;
    odd = ((w >> 4) ^ 0x08888888u) & 0x0f0f0f0fu;
}

// bf16 pair of bytes 2h and 2h + 1 of x (biased nibbles): bits 0x43 | u each.
__device__ __forceinline__ unsigned i4_pair_same(unsigned x, int h) {
    return __builtin_amdgcn_perm(0x43434343u, x, h ? 0x04030402u : 0x04010400u);
}

template <int D> struct TileRegs<KV_F32, D> {
    f32x4 k[D / 16];   // 4 f32: token lane%16, dims of chunk 4r + lane/16
    f32x4 v[D / 16];   // 4 f32: dim 16m + lane%16, tokens 4*(lane/16) .. +3
    // koff = lane * 16; voff = TILE + (lane % 16) * 64 + (lane / 16) * 16
    template <int POL>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int koff, int voff) {
#pragma unroll
        for (int q = 0; q < D / 16; ++q) k[q] = bload<f32x4, POL>(r, koff, 1024 * q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < D / 16; ++m) v[m] = bload<f32x4, POL>(r, voff, 1024 * m);
    }
    static constexpr int kTile = 16 * D * 4;
    __device__ static int v_offset(int lane) { return kTile + (lane & 15) * 64 + (lane >> 4) * 16; }
    __device__ __forceinline__ void zero_v_from(int nvalid) {
        if (nvalid >= 4) return;
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e >= nvalid) v[m][e] = 0.f;
    }
    // Token o takes the values staged in LDS at st (K in dim order, then V);
    // only lanes holding a part of token o change.
    __device__ __forceinline__ void put_token(int o, const uint8_t* st, int lane) {
        const float* fs = reinterpret_cast<const float*>(st);
        if ((lane & 15) == o) {
#pragma unroll
            for (int q = 0; q < D / 16; ++q) k[q] = *reinterpret_cast<const f32x4*>(fs + (4 * q + (lane >> 4)) * 4);
        }
        if ((lane >> 4) == (o >> 2)) {
#pragma unroll
            for (int m = 0; m < D / 16; ++m) {
                const float x = fs[D + 16 * m + (lane & 15)];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e == (o & 3)) v[m][e] = x;
            }
        }
    }
};

// ---------------------------------------------------------- query operand
// B operand of the score MFMA for column tile t: query row 16t + lane%16,
// dims matching the K chunk each lane group holds.
template <int KVT, int D> struct QRegs;

// Sign flip of every 16-bit value in a 16-byte operand register.
template <class V>
__device__ __forceinline__ V flip16(const V& v) {
    return __builtin_bit_cast(V, __builtin_bit_cast(u32x4, v) ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
}

template <int D> struct QRegs<KV_BF16, D> {
    bf16x8 q[D / 32];   // step s: dims (4s + lane/16) * 8 .. +8
    __device__ __forceinline__ void negate() {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) q[s] = flip16(q[s]);
    }
    __device__ __forceinline__ void load(const uint16_t* row, bool valid, int lane) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            u32x4 w = valid ? *reinterpret_cast<const u32x4*>(row + (4 * s + (lane >> 4)) * 8)
                            : u32x4{0u, 0u, 0u, 0u};
            q[s] = __builtin_bit_cast(bf16x8, w);
        }
    }
};

template <int D> struct QRegs1B {
    bf16x8 q[D / 32];   // step 2r + hh: dims (4r + lane/16) * 16 + 8 hh .. +8
    __device__ __forceinline__ void negate() {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) q[s] = flip16(q[s]);
    }
    __device__ __forceinline__ void load(const uint16_t* row, bool valid, int lane) {
#pragma unroll
        for (int st = 0; st < D / 32; ++st) {
            const int dim0 = (4 * (st >> 1) + (lane >> 4)) * 16 + 8 * (st & 1);
            u32x4 w = valid ? *reinterpret_cast<const u32x4*>(row + dim0) : u32x4{0u, 0u, 0u, 0u};
            q[st] = __builtin_bit_cast(bf16x8, w);
        }
    }
};
template <int D> struct QRegs<KV_FP8, D> : QRegs1B<D> {};
template <int D> struct QRegs<KV_INT8, D> : QRegs1B<D> {};
// int4 K runs hold dims 32 s + 8 (lane / 16) + e per step s; the score
// operand takes them as even dims then odd dims (0 2 4 6 1 3 5 7 of each
// eight, the order in which one byte permute per two codes widens them), so
// the query's eight values of a step are loaded in that order.
template <int D> struct QRegs<KV_INT4, D> : QRegs<KV_BF16, D> {
    __device__ __forceinline__ void load(const uint16_t* row, bool valid, int lane) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const u32x4 w = valid ? *reinterpret_cast<const u32x4*>(row + (4 * s + (lane >> 4)) * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
            // w = (q0 q1)(q2 q3)(q4 q5)(q6 q7) -> (q0 q2)(q4 q6)(q1 q3)(q5 q7)
            const u32x4 p = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                             __builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
            this->q[s] = __builtin_bit_cast(bf16x8, p);
        }
    }
};

template <int D> struct QRegs<KV_F32, D> {
    f32x4 q[D / 16];    // r: dims (4r + lane/16) * 4 .. +4, one MFMA per element
    __device__ __forceinline__ void negate() {
#pragma unroll
        for (int r = 0; r < D / 16; ++r) q[r] = -q[r];
    }
    __device__ __forceinline__ void load(const float* row, bool valid, int lane) {
#pragma unroll
        for (int r = 0; r < D / 16; ++r)
            q[r] = valid ? *reinterpret_cast<const f32x4*>(row + (4 * r + (lane >> 4)) * 4)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
};

// S^T tile (tokens x rows) of one block for one column tile.
template <int D>
__device__ __forceinline__ f32x4 scores(const TileRegs<KV_BF16, D>& t, const QRegs<KV_BF16, D>& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[s]), q.q[s], acc, 0, 0, 0);
    return acc;
}

template <int KVT, int D>
__device__ __forceinline__ f32x4 scores_1b(const TileRegs<KVT, D>& t, const QRegs<KVT, D>& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < D / 64; ++r) {
        const u32x4 w = t.k[r];
        auto cv = [](unsigned x, auto hi_half) {
            constexpr bool H = decltype(hi_half)::value;
            return byte2_to_bf16x2<KVT, H>(x);
        };
        using L = std::false_type;
        using H = std::true_type;
        u32x4 lo = {cv(w[0], L{}), cv(w[0], H{}), cv(w[1], L{}), cv(w[1], H{})};
        u32x4 hi = {cv(w[2], L{}), cv(w[2], H{}), cv(w[3], L{}), cv(w[3], H{})};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), q.q[2 * r], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), q.q[2 * r + 1], acc, 0, 0, 0);
    }
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 scores(const TileRegs<KV_FP8, D>& t, const QRegs<KV_FP8, D>& q) {
    return scores_1b<KV_FP8, D>(t, q);
}

template <int D>
__device__ __forceinline__ f32x4 scores(const TileRegs<KV_INT8, D>& t, const QRegs<KV_INT8, D>& q) {
    return scores_1b<KV_INT8, D>(t, q);
}

// Decode-kernel int8 query operand: the bf16 query times 2^-8 as fp16 (in
// QRegs1B's dim order).  A bf16 value keeps its 8 significant bits in fp16
// from 2^-6 to just below 2^24 in magnitude (larger ones overflow);
// below, fp16's subnormal spacing (2^-16 in query units) bounds the error.
// The caller multiplies the scores by 2^8.
constexpr float kI8QScale = 1.f / 256.f;
template <int D> struct QRegsI8 {
    f16x8 q[D / 32];
    __device__ __forceinline__ void negate() {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) q[s] = flip16(q[s]);
    }
    __device__ __forceinline__ void load(const uint16_t* row, bool valid, int lane) {
#pragma unroll
        for (int st = 0; st < D / 32; ++st) {
            const int dim0 = (4 * (st >> 1) + (lane >> 4)) * 16 + 8 * (st & 1);
            const u32x4 w = valid ? *reinterpret_cast<const u32x4*>(row + dim0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = __uint_as_float(w[j] << 16) * kI8QScale;
                const float hi = __uint_as_float(w[j] & 0xffff0000u) * kI8QScale;
                q[st][2 * j] = static_cast<_Float16>(lo);
                q[st][2 * j + 1] = static_cast<_Float16>(hi);
            }
        }
    }
};

// int8 scores for the decode kernel, in units of kI8QScale and biased: the
// caller subtracts kI8Bias times the query row's sum (query_row_sum below).
template <int D>
__device__ __forceinline__ f32x4 scores_i8(const TileRegs<KV_INT8, D>& t, const QRegsI8<D>& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < D / 64; ++r) {
        u32x4 x = t.k[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] ^= 0x80808080u;
        const u32x4 lo = {i8x2_to_f16x2<false>(x[0]), i8x2_to_f16x2<true>(x[0]), i8x2_to_f16x2<false>(x[1]),
                          i8x2_to_f16x2<true>(x[1])};
        const u32x4 hi = {i8x2_to_f16x2<false>(x[2]), i8x2_to_f16x2<true>(x[2]), i8x2_to_f16x2<false>(x[3]),
                          i8x2_to_f16x2<true>(x[3])};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, lo), q.q[2 * r], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, hi), q.q[2 * r + 1], acc, 0, 0, 0);
    }
    return acc;
}

// Biased scores: the caller subtracts kI4Bias times the query row's sum.
template <int D>
__device__ __forceinline__ f32x4 scores(const TileRegs<KV_INT4, D>& t, const QRegs<KV_INT4, D>& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        unsigned ev, od;
        i4_split(t.k[s], ev, od);
        // dims 0 2 4 6 1 3 5 7 (the query's order): bf16 0x43 | u, one
        // permute per pair against the constant high bytes
        const u32x4 kb = {i4_pair_same(ev, 0), i4_pair_same(ev, 1), i4_pair_same(od, 0), i4_pair_same(od, 1)};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), q.q[s], acc, 0, 0, 0);
    }
    return acc;
}

// Sum of a query row over all dims, for every lane of its column: the score
// MFMA against a tile of bf16 ones.
template <int D>
__device__ __forceinline__ f32x4 query_row_sum(const QRegs<KV_BF16, D>& q) {
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), q.q[s], acc, 0, 0, 0);
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 query_row_sum(const QRegsI8<D>& q) {
    const u32x4 ones = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ones), q.q[s], acc, 0, 0, 0);
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 query_row_sum(const QRegs1B<D>& q) {
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), q.q[s], acc, 0, 0, 0);
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 scores(const TileRegs<KV_F32, D>& t, const QRegs<KV_F32, D>& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < D / 16; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(t.k[r][e], q.q[r][e], acc, 0, 0, 0);
    return acc;
}

}  // namespace pkv
