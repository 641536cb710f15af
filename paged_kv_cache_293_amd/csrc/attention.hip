// Paged decode / verify attention for gfx950.
//
// Method (page "KV cache & continuous batching", sections "The core insight"
// and "2. PagedAttention (vLLM)"; page "LLM Serving - KV Cache, Batching,
// Speculative Decoding", section "Hands-on: cache equivalence and scheduling
// oracles"): each query row of a sequence attends with softmax weights over the
// K/V of the positions it may see, K and V being gathered through the
// sequence's block table.  Query heads of one GQA group share the KV head
// (page 1, section "KV cache memory math"); a verify call carries k query rows
// per sequence with causal visibility among them (page 1, section
// "5. Speculative decoding").
//
// Work decomposition.  One work-group of W = 4 wavefronts handles one
// (sequence, partition) unit for one KV head.  Its waves take the partition's
// 16-token blocks round-robin and each keeps an online softmax (running max m,
// running sum l, unnormalised output O) for all query rows of the KV head:
// R = G * k rows, held as NT = ceil(R / 16) column tiles of 16.  The waves are
// merged through LDS at the end (added in wave order, so results are
// deterministic); a sequence with one partition writes its final
// output there, a split sequence writes (O, m, l) partials that
// attn_merge_kernel combines.
//
// Matrix cores.  Per block the scores are S^T[token][row] = K[token][:] .
// Q^T[:][row], a 16 x 16 (tokens x rows) tile per column tile: K is the A
// operand (row = token = lane % 16), Q^T the resident B operand.  The output is
// O^T[dim][row] += V^T[dim][token] . P^T[token][row]: V^T is the A operand
// and the probability tile, which the score MFMA leaves exactly in B-operand
// layout (lane holds tokens 4*(lane/16) .. +3 of column lane % 16), feeds the
// PV MFMA without any lane exchange.  The pool layout (K chunk-major, V
// transposed) makes every operand a plain vector load: each K load instruction
// of a wave reads one contiguous KiB, each V load 16 dims x the tile row.
//   bf16: v_mfma_f32_16x16x32_bf16 (QK), v_mfma_f32_16x16x16_bf16 (PV),
//         probabilities rounded to bf16;
//   fp8 : codes converted to bf16 in registers (exact), then as bf16; the K
//         scale folds into the score scale, the V scale into the final divide;
//   f32 : v_mfma_f32_16x16x4_f32 for both products, probabilities in f32.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

constexpr int kWaves = 4;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// float -> bfloat16 bits, round to nearest even (NaN kept NaN).
__device__ __forceinline__ unsigned f32_to_bf16_rne(float f) {
    unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp8 E4M3 codes (bytes 0-1, or 2-3 when HI, of w) -> two bf16 values packed in one
// dword.  The hardware conversion yields exact float32 values; their upper
// halves are the exact bf16 values (E4M3 has 3 mantissa bits).
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
}

// ------------------------------------------------------------------ tiles
// Per-lane registers of one block's K and V tiles, and their loads.
template <int KVT, int D> struct TileRegs;

template <int D> struct TileRegs<KV_BF16, D> {
    u32x4 k[D / 32];   // 8 bf16: token lane%16, dims of chunk 4s + lane/16
    u32x2 v[D / 16];   // 4 bf16: dim 16m + lane%16, tokens 4*(lane/16) .. +3
    __device__ __forceinline__ void load(const uint8_t* kt, const uint8_t* vt, int lane) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            k[s] = *reinterpret_cast<const u32x4*>(kt + (64 * s + lane) * 16);
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
            v[m] = *reinterpret_cast<const u32x2*>(vt + (16 * m + (lane & 15)) * 32 + 8 * (lane >> 4));
    }
    // zero V of tokens >= nvalid among this lane's four (tokens 4j .. 4j+3)
    __device__ __forceinline__ void zero_v_from(int nvalid) {
        if (nvalid >= 4) return;
        const unsigned m0 = nvalid <= 0 ? 0u : (nvalid == 1 ? 0x0000ffffu : 0xffffffffu);
        const unsigned m1 = nvalid <= 2 ? 0u : 0x0000ffffu;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) { v[m][0] &= m0; v[m][1] &= m1; }
    }
};

template <int D> struct TileRegs<KV_FP8, D> {
    u32x4 k[D / 64];   // 16 codes: token lane%16, dims of chunk 4r + lane/16
    unsigned v[D / 16];  // 4 codes: dim 16m + lane%16, tokens 4*(lane/16) .. +3
    __device__ __forceinline__ void load(const uint8_t* kt, const uint8_t* vt, int lane) {
#pragma unroll
        for (int r = 0; r < D / 64; ++r)
            k[r] = *reinterpret_cast<const u32x4*>(kt + (64 * r + lane) * 16);
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
            v[m] = *reinterpret_cast<const unsigned*>(vt + (16 * m + (lane & 15)) * 16 + 4 * (lane >> 4));
    }
    __device__ __forceinline__ void zero_v_from(int nvalid) {
        if (nvalid >= 4) return;
        const unsigned msk = nvalid <= 0 ? 0u : (0xffffffffu >> (8 * (4 - nvalid)));
#pragma unroll
        for (int m = 0; m < D / 16; ++m) v[m] &= msk;
    }
};

template <int D> struct TileRegs<KV_F32, D> {
    f32x4 k[D / 16];   // 4 f32: token lane%16, dims of chunk 4r + lane/16
    f32x4 v[D / 16];   // 4 f32: dim 16m + lane%16, tokens 4*(lane/16) .. +3
    __device__ __forceinline__ void load(const uint8_t* kt, const uint8_t* vt, int lane) {
#pragma unroll
        for (int r = 0; r < D / 16; ++r)
            k[r] = *reinterpret_cast<const f32x4*>(kt + (64 * r + lane) * 16);
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
            v[m] = *reinterpret_cast<const f32x4*>(vt + (16 * m + (lane & 15)) * 64 + 16 * (lane >> 4));
    }
    __device__ __forceinline__ void zero_v_from(int nvalid) {
        if (nvalid >= 4) return;
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e >= nvalid) v[m][e] = 0.f;
    }
};

// ---------------------------------------------------------- query operand
// B operand of the score MFMA for column tile t: query row 16t + lane%16,
// dims matching the K chunk each lane group holds.
template <int KVT, int D> struct QRegs;

template <int D> struct QRegs<KV_BF16, D> {
    bf16x8 q[D / 32];   // step s: dims (4s + lane/16) * 8 .. +8
    __device__ __forceinline__ void load(const uint16_t* row, bool valid, int lane) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            u32x4 w = valid ? *reinterpret_cast<const u32x4*>(row + (4 * s + (lane >> 4)) * 8)
                            : u32x4{0u, 0u, 0u, 0u};
            q[s] = __builtin_bit_cast(bf16x8, w);
        }
    }
};

template <int D> struct QRegs<KV_FP8, D> {
    bf16x8 q[D / 32];   // step 2r + hh: dims (4r + lane/16) * 16 + 8 hh .. +8
    __device__ __forceinline__ void load(const uint16_t* row, bool valid, int lane) {
#pragma unroll
        for (int st = 0; st < D / 32; ++st) {
            const int dim0 = (4 * (st >> 1) + (lane >> 4)) * 16 + 8 * (st & 1);
            u32x4 w = valid ? *reinterpret_cast<const u32x4*>(row + dim0) : u32x4{0u, 0u, 0u, 0u};
            q[st] = __builtin_bit_cast(bf16x8, w);
        }
    }
};

template <int D> struct QRegs<KV_F32, D> {
    f32x4 q[D / 16];    // r: dims (4r + lane/16) * 4 .. +4, one MFMA per element
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

template <int D>
__device__ __forceinline__ f32x4 scores(const TileRegs<KV_FP8, D>& t, const QRegs<KV_FP8, D>& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < D / 64; ++r) {
        const u32x4 w = t.k[r];
        u32x4 lo = {fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                    fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])};
        u32x4 hi = {fp8x2_to_bf16x2<false>(w[2]), fp8x2_to_bf16x2<true>(w[2]),
                    fp8x2_to_bf16x2<false>(w[3]), fp8x2_to_bf16x2<true>(w[3])};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), q.q[2 * r], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), q.q[2 * r + 1], acc, 0, 0, 0);
    }
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

// O^T[dim tile m] += V^T tile . P^T for one column tile; p holds this lane's
// probabilities of tokens 4*(lane/16) .. +3.
template <int D, int NT>
__device__ __forceinline__ void accumulate_pv(const TileRegs<KV_BF16, D>& t, const f32x4 (&p)[NT],
                                              f32x4 (&o)[NT][D / 16]) {
    s16x4 pb[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const unsigned w0 = f32_to_bf16_rne(p[c][0]) | (f32_to_bf16_rne(p[c][1]) << 16);
        const unsigned w1 = f32_to_bf16_rne(p[c][2]) | (f32_to_bf16_rne(p[c][3]) << 16);
        pb[c] = __builtin_bit_cast(s16x4, u32x2{w0, w1});
    }
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        const s16x4 a = __builtin_bit_cast(s16x4, t.v[m]);
#pragma unroll
        for (int c = 0; c < NT; ++c)
            o[c][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[c], o[c][m], 0, 0, 0);
    }
}

template <int D, int NT>
__device__ __forceinline__ void accumulate_pv(const TileRegs<KV_FP8, D>& t, const f32x4 (&p)[NT],
                                              f32x4 (&o)[NT][D / 16]) {
    s16x4 pb[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const unsigned w0 = f32_to_bf16_rne(p[c][0]) | (f32_to_bf16_rne(p[c][1]) << 16);
        const unsigned w1 = f32_to_bf16_rne(p[c][2]) | (f32_to_bf16_rne(p[c][3]) << 16);
        pb[c] = __builtin_bit_cast(s16x4, u32x2{w0, w1});
    }
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        const u32x2 vb = {fp8x2_to_bf16x2<false>(t.v[m]), fp8x2_to_bf16x2<true>(t.v[m])};
        const s16x4 a = __builtin_bit_cast(s16x4, vb);
#pragma unroll
        for (int c = 0; c < NT; ++c)
            o[c][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[c], o[c][m], 0, 0, 0);
    }
}

template <int D, int NT>
__device__ __forceinline__ void accumulate_pv(const TileRegs<KV_F32, D>& t, const f32x4 (&p)[NT],
                                              f32x4 (&o)[NT][D / 16]) {
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int c = 0; c < NT; ++c)
                o[c][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[m][e], p[c][e], o[c][m], 0, 0, 0);
}

// The probability the normaliser adds up: what the PV product actually used.
template <int KVT>
__device__ __forceinline__ float as_used(float p) {
    if constexpr (KVT == KV_F32) return p;
    else return __uint_as_float(f32_to_bf16_rne(p) << 16);
}

// ------------------------------------------------------- partition kernel
template <int KVT, int D, int NT>
__global__ __launch_bounds__(64 * kWaves) void attn_partition_kernel(AttnArgs a) {
    extern __shared__ float smem[];
    const int R = a.rows;
    float* acc_s = smem;                       // [R][D + 1] merged unnormalised output
    float* m_s = smem + R * (D + 1);           // [W][R]
    float* l_s = m_s + kWaves * R;             // [W][R]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lg = lane >> 4;                  // lane group: tokens 4*lg .. +3
    const int col = lane & 15;                 // column within a row tile
    const int unit = blockIdx.x;
    const int h = blockIdx.y;
    const int seq = a.units[2 * unit];
    const int part = a.units[2 * unit + 1];
    const int n = a.seq_lens[seq];
    const int nblk = (n + kBlock - 1) / kBlock;
    const int b0 = part * a.part_blocks;
    const int b1 = min(b0 + a.part_blocks, nblk);
    const int G = a.group;
    const int kq = a.k_rows;

    for (int e = threadIdx.x; e < R * (D + 1); e += 64 * kWaves) acc_s[e] = 0.f;

    float sscale = a.score_scale;
    float vscale = 1.f;
    if constexpr (KVT == KV_FP8) {
        sscale *= a.k_scale[a.layer * a.num_kv_heads + h];
        vscale = a.v_scale[a.layer * a.num_kv_heads + h];
    }

    // Query operands and per-column visibility limits.
    using QT = QRegs<KVT, D>;
    using ElemQ = typename std::conditional<KVT == KV_F32, float, uint16_t>::type;
    QT qr[NT];
    int lim[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int row = 16 * c + col;
        const bool valid = row < R;
        const int jr = valid ? row / G : 0;
        const int g = valid ? row % G : 0;
        const ElemQ* qrow = reinterpret_cast<const ElemQ*>(a.q) +
            ((static_cast<int64_t>(seq) * kq + jr) * a.num_q_heads + h * G + g) * D;
        qr[c].load(qrow, valid, lane);
        lim[c] = valid ? n - (kq - 1 - jr) : n;
    }
    const int mask_from = n - kq + 1;

    f32x4 o[NT][D / 16];
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        m_run[c] = neg_inf();
        l_run[c] = 0.f;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) o[c][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t* trow = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;
    const int64_t block_stride = static_cast<int64_t>(a.num_kv_heads) * 2 * a.tile_bytes;
    const uint8_t* head_base = a.pool +
        static_cast<int64_t>(a.layer) * a.num_blocks * block_stride + static_cast<int64_t>(h) * 2 * a.tile_bytes;

    auto process = [&](const TileRegs<KVT, D>& tr, int blk) {
        f32x4 s[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            s[c] = scores<D>(tr, qr[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[c][i] *= sscale;
        }
        const int tok0 = blk * kBlock + 4 * lg;
        if (blk * kBlock + kBlock > mask_from) {
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tok0 + i >= lim[c]) s[c][i] = neg_inf();
        }
        TileRegs<KVT, D> tv = tr;
        if (blk * kBlock + kBlock > n) tv.zero_v_from(n - tok0);
        f32x4 p[NT];
        bool rescale = false;
        float alpha[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            float mx = fmaxf(fmaxf(s[c][0], s[c][1]), fmaxf(s[c][2], s[c][3]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m_run[c], mx);
            const float muse = (mnew == neg_inf()) ? 0.f : mnew;
            alpha[c] = fast_exp2(m_run[c] - muse);
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[c][i] = fast_exp2(s[c][i] - muse);
                psum += as_used<KVT>(p[c][i]);
            }
            l_run[c] = l_run[c] * alpha[c] + psum;
            m_run[c] = mnew;
            rescale |= alpha[c] != 1.f;
        }
        if (__ballot(rescale)) {
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int m = 0; m < D / 16; ++m) o[c][m] *= alpha[c];
        }
        accumulate_pv<D, NT>(tv, p, o);
    };

    const int nb = b1 - b0;
    for (int base = wave; base < nb; base += 64 * kWaves) {
        const int cnt = min(64, (nb - base + kWaves - 1) / kWaves);
        int id = lane < cnt ? trow[b0 + base + kWaves * lane] : 0;
        id = min(max(id, 0), a.num_blocks - 1);
        auto ktile = [&](int i) {
            const int pid = __builtin_amdgcn_readlane(id, i);
            return head_base + static_cast<int64_t>(pid) * block_stride;
        };
        TileRegs<KVT, D> ta, tb;
        {
            const uint8_t* t0 = ktile(0);
            ta.load(t0, t0 + a.tile_bytes, lane);
        }
        for (int i = 0; i < cnt; i += 2) {
            if (i + 1 < cnt) {
                const uint8_t* t1 = ktile(i + 1);
                tb.load(t1, t1 + a.tile_bytes, lane);
            }
            process(ta, b0 + base + kWaves * i);
            if (i + 1 >= cnt) break;
            if (i + 2 < cnt) {
                const uint8_t* t2 = ktile(i + 2);
                ta.load(t2, t2 + a.tile_bytes, lane);
            }
            process(tb, b0 + base + kWaves * (i + 1));
        }
    }

    // Merge the waves: publish (m, l), rescale O to the common max, add in LDS.
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        float l = l_run[c];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int row = 16 * c + col;
        if (lg == 0 && row < R) {
            m_s[wave * R + row] = m_run[c];
            l_s[wave * R + row] = l;
        }
    }
    __syncthreads();
    // Waves add their rescaled outputs one after another (fixed order, so the
    // result does not depend on scheduling).
    float f[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int row = 16 * c + col;
        float M = neg_inf();
        if (row < R) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_s[w * R + row]);
        }
        f[c] = (row >= R || M == neg_inf()) ? 0.f : fast_exp2(m_run[c] - M);
    }
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int row = 16 * c + col;
                if (row >= R) continue;
                float* dst = acc_s + row * (D + 1) + 4 * lg;
#pragma unroll
                for (int m = 0; m < D / 16; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[16 * m + i] += o[c][m][i] * f[c];
            }
        }
        __syncthreads();
    }

    const int sbase = a.split_base[seq];
    for (int e = threadIdx.x; e < R * D; e += 64 * kWaves) {
        const int r = e / D;
        const int d = e % D;
        float M = neg_inf();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_s[w * R + r]);
        float L = 0.f;
        if (M != neg_inf()) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) L += l_s[w * R + r] * fast_exp2(m_s[w * R + r] - M);
        }
        const float O = acc_s[r * (D + 1) + d];
        if (sbase < 0) {
            const int jr = r / G;
            const int g = r % G;
            const int64_t oi = ((static_cast<int64_t>(seq) * kq + jr) * a.num_q_heads + h * G + g) * D + d;
            const float val = O / L * vscale;
            if (a.out_bf16)
                reinterpret_cast<uint16_t*>(a.out)[oi] = static_cast<uint16_t>(f32_to_bf16_rne(val));
            else
                reinterpret_cast<float*>(a.out)[oi] = val;
        } else {
            const int64_t slot = static_cast<int64_t>(h) * a.num_split_slots + sbase + part;
            a.part_o[(slot * R + r) * D + d] = O;
            if (d == 0) {
                a.part_m[slot * R + r] = M;
                a.part_l[slot * R + r] = L;
            }
        }
    }
}

// ------------------------------------------------------------ merge kernel
// One work-group per (split sequence, KV head, query row): combines the
// partitions' (O, m, l):  M = max m_p,  L = sum l_p 2^(m_p - M),
// out = sum O_p 2^(m_p - M) / L  (times the V scale of fp8 pools).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int fp8) {
    __shared__ float red[8];
    __shared__ f32x4 part_acc[256];
    const int seq = blockIdx.x;
    const int h = blockIdx.y;
    const int r = blockIdx.z;
    const int sbase = a.split_base[seq];
    if (sbase < 0) return;
    const int R = a.rows;
    const int n = a.seq_lens[seq];
    const int nblk = (n + kBlock - 1) / kBlock;
    const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
    const int64_t slot0 = static_cast<int64_t>(h) * a.num_split_slots + sbase;
    const float* pm = a.part_m + slot0 * R + r;
    const float* pl = a.part_l + slot0 * R + r;
    const float* po = a.part_o + (slot0 * R + r) * D;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    float mx = neg_inf();
    for (int p = tid; p < nparts; p += 256) mx = fmaxf(mx, pm[static_cast<int64_t>(p) * R]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float ls = 0.f;
    for (int p = tid; p < nparts; p += 256) {
        const int64_t i = static_cast<int64_t>(p) * R;
        ls += pl[i] * fast_exp2(pm[i] - M);
    }
    for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
    if (lane == 0) red[4 + wave] = ls;

    constexpr int Q = D / 4;          // float4 columns of one row
    constexpr int GR = 256 / Q;       // partition groups
    const int qd = tid % Q;
    const int grp = tid / Q;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int p = grp;
    for (; p + 3 * GR < nparts; p += 4 * GR) {
        f32x4 v[4];
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t pp = p + u * GR;
            v[u] = *reinterpret_cast<const f32x4*>(po + pp * R * D + 4 * qd);
            w[u] = fast_exp2(pm[pp * R] - M);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += v[u] * w[u];
    }
    for (; p < nparts; p += GR) {
        const int64_t pp = p;
        acc += *reinterpret_cast<const f32x4*>(po + pp * R * D + 4 * qd) * fast_exp2(pm[pp * R] - M);
    }
    part_acc[tid] = acc;
    __syncthreads();
    if (tid < Q) {
        f32x4 sum = part_acc[tid];
        for (int g = 1; g < GR; ++g) sum += part_acc[g * Q + tid];
        const float L = red[4] + red[5] + red[6] + red[7];
        const float vscale = fp8 ? a.v_scale[a.layer * a.num_kv_heads + h] : 1.f;
        const int G = a.group;
        const int jr = r / G;
        const int g = r % G;
        const int64_t oi = ((static_cast<int64_t>(seq) * a.k_rows + jr) * a.num_q_heads + h * G + g) * D + 4 * tid;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float val = sum[i] / L * vscale;
            if (a.out_bf16)
                reinterpret_cast<uint16_t*>(a.out)[oi + i] = static_cast<uint16_t>(f32_to_bf16_rne(val));
            else
                reinterpret_cast<float*>(a.out)[oi + i] = val;
        }
    }
}

template <int KVT, int D, int NT>
hipError_t launch_instance(const AttnArgs& a, int num_units, hipStream_t stream) {
    const size_t lds = (static_cast<size_t>(a.rows) * (D + 1) + 2 * kWaves * a.rows) * sizeof(float);
    dim3 grid(num_units, a.num_kv_heads);
    hipLaunchKernelGGL((attn_partition_kernel<KVT, D, NT>), grid, dim3(64 * kWaves), lds, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.num_split_slots > 0) {
        dim3 g2(a.num_seqs, a.num_kv_heads, a.rows);
        hipLaunchKernelGGL((attn_merge_kernel<D>), g2, dim3(256), 0, stream, a, KVT == KV_FP8 ? 1 : 0);
        err = hipGetLastError();
    }
    return err;
}

template <int KVT, int D>
hipError_t launch_rows(const AttnArgs& a, int num_units, hipStream_t stream) {
    if (a.rows <= 16) return launch_instance<KVT, D, 1>(a, num_units, stream);
    if (a.rows <= 32) return launch_instance<KVT, D, 2>(a, num_units, stream);
    return launch_instance<KVT, D, 4>(a, num_units, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int kv_dtype, int head_dim, int num_units,
                            hipStream_t stream) {
    if (num_units <= 0) return hipSuccess;
    if (kv_dtype == KV_BF16)
        return head_dim == 128 ? launch_rows<KV_BF16, 128>(a, num_units, stream)
                               : launch_rows<KV_BF16, 64>(a, num_units, stream);
    if (kv_dtype == KV_FP8)
        return head_dim == 128 ? launch_rows<KV_FP8, 128>(a, num_units, stream)
                               : launch_rows<KV_FP8, 64>(a, num_units, stream);
    return head_dim == 128 ? launch_rows<KV_F32, 128>(a, num_units, stream)
                           : launch_rows<KV_F32, 64>(a, num_units, stream);
}

}  // namespace pkv
