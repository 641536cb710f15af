// Paged decode / verify attention for gfx950.
//
// Method (page "KV cache & continuous batching", sections "The core insight"
// and "2. PagedAttention (vLLM)"; page "LLM Serving - KV Cache, Batching,
// Speculative Decoding", section "Hands-on: cache equivalence and scheduling
// oracles"): each query row of a sequence attends with softmax weights over the
// K/V of the positions it may see, K and V being gathered through the
// sequence's block table.  Query heads of one GQA group share the KV head
// (page "KV cache & continuous batching", section "KV cache memory math"); a
// verify call carries k query rows per sequence with causal visibility among
// them (same page, section "5. Speculative decoding").
//
// Work decomposition.  An item is one (sequence, partition) unit for one KV
// head.  One work-group of W = 4 wavefronts attends over an item: its waves
// take the partition's 16-token blocks round-robin and each keeps an online
// softmax (running max m, running sum l, unnormalised output O) for all query
// rows of the KV head: R = G * k rows, held as NT = ceil(R / 16) column tiles
// of 16.  The waves are merged through LDS at the end (added in wave order,
// so results are deterministic); a sequence with one partition writes its
// final output there, a split sequence writes (O, m, l) partials that the
// last of its work-groups to finish (or attn_merge_kernel, for many
// partitions) combines.  The grid holds only as many work-groups as fit on
// the device at once; they take further items from a queue as they finish,
// because the memory system serves CUs and XCDs unevenly and equal static
// shares finish far apart.
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
//         probabilities rounded to bf16; their row sums come from one more
//         16x16x16 MFMA against a tile of ones (the values PV used);
//   fp8 : codes converted to bf16 in registers (exact), then as bf16; the K
//         scale folds into the score scale, the V scale into the final divide;
//   int8: codes widened to fp16 with a bias (1152, one byte permute per two
//         codes), queries as fp16 times 2^-8, probabilities as fp16, with
//         v_mfma_f32_16x16x32_f16 (QK) and v_mfma_f32_16x16x16_f16 (PV); the
//         kernel takes the bias out of the scores (bias x the query row's
//         sum) and of the output (bias x the probability sum); scales as fp8;
//   int4: codes widened to bf16 with a bias (136) taken out the same way;
//   f32 : v_mfma_f32_16x16x4_f32 for both products, probabilities in f32.
#include <mutex>

#include "pkv_mfma.h"

namespace pkv {
namespace {

// Partial results (O, m, l) of split sequences for paged_attention_verify_noalloc,
// which takes no workspace argument: one array per device, alive until the
// process ends.  Host code must not pass this name to a kernel (on the host
// it is only a stand-in for the symbol); it uses the device address that
// attention_scratch() looks up per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kWaves = 4;
constexpr float kLazyMax = 8.f;   // exp2 units the running max may lag behind a row's scores

// O^T[dim tile m] += V^T tile . P^T for one column tile; p holds this lane's
// probabilities of tokens 4*(lane/16) .. +3.
template <int D, int NT>
__device__ __forceinline__ void accumulate_pv(const TileRegs<KV_BF16, D>& t, const f32x4 (&p)[NT],
                                              f32x4 (&o)[NT][D / 16]) {
    s16x4 pb[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        pb[c] = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[c][0], p[c][1]), pack_bf16x2(p[c][2], p[c][3])});
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
        pb[c] = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[c][0], p[c][1]), pack_bf16x2(p[c][2], p[c][3])});
    }
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        const u32x2 vb = {decode_pair<KV_FP8, false>(t.v[m]), decode_pair<KV_FP8, true>(t.v[m])};
        const s16x4 a = __builtin_bit_cast(s16x4, vb);
#pragma unroll
        for (int c = 0; c < NT; ++c)
            o[c][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[c], o[c][m], 0, 0, 0);
    }
}

// The probabilities as fp16 (they lie in [0, 2^kLazyMax]), for the int8
// products.
template <int NT>
__device__ __forceinline__ void probs_f16(const f32x4 (&p)[NT], f16x4 (&ph)[NT]) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const f16x2_t a = __builtin_convertvector(f32x2_t{p[c][0], p[c][1]}, f16x2_t);
        const f16x2_t b = __builtin_convertvector(f32x2_t{p[c][2], p[c][3]}, f16x2_t);
        ph[c] = __builtin_bit_cast(f16x4, u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)});
    }
}

// int8: fp16 operands biased by kI8Bias (the caller subtracts kI8Bias times
// the row's probability sum).
template <int D, int NT>
__device__ __forceinline__ void accumulate_pv(const TileRegs<KV_INT8, D>& t, const f32x4 (&p)[NT],
                                              f32x4 (&o)[NT][D / 16]) {
    f16x4 ph[NT];
    probs_f16<NT>(p, ph);
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        const unsigned x = t.v[m] ^ 0x80808080u;
        const f16x4 a = __builtin_bit_cast(f16x4, u32x2{i8x2_to_f16x2<false>(x), i8x2_to_f16x2<true>(x)});
#pragma unroll
        for (int c = 0; c < NT; ++c)
            o[c][m] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, ph[c], o[c][m], 0, 0, 0);
    }
}

// Biased: the caller subtracts kI4Bias times the row's probability sum.
template <int D, int NT>
__device__ __forceinline__ void accumulate_pv(const TileRegs<KV_INT4, D>& t, const f32x4 (&p)[NT],
                                              f32x4 (&o)[NT][D / 16]) {
    s16x4 pb[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        pb[c] = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[c][0], p[c][1]), pack_bf16x2(p[c][2], p[c][3])});
    }
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        // V dword j: byte t holds token 4 (lane / 16) + t at dims 16 (2 j) +
        // lane % 16 (low nibble) and 16 (2 j + 1) + lane % 16 (high nibble)
        unsigned ev, od;
        i4_split(t.v[j], ev, od);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const unsigned src = hh ? od : ev;
            const s16x4 a = __builtin_bit_cast(s16x4, u32x2{i4_pair_same(src, 0), i4_pair_same(src, 1)});
#pragma unroll
            for (int c = 0; c < NT; ++c)
                o[c][2 * j + hh] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[c], o[c][2 * j + hh], 0, 0, 0);
        }
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

// Final output element (row r of KV head h of sequence seq, dim d).
__device__ __forceinline__ void store_out(const AttnArgs& a, int seq, int h, int r, int d, float val) {
    const int G = a.group;
    const int jr = r / G;
    const int g = r % G;
    const int64_t oi = ((static_cast<int64_t>(seq) * a.k_rows + jr) * a.num_q_heads + h * G + g) * a.head_dim + d;
    if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.out)[oi] = static_cast<uint16_t>(f32_to_bf16_rne(val));
    else
        reinterpret_cast<float*>(a.out)[oi] = val;
}

// Bytes one appended token occupies in the LDS staging area: its K then its
// V elements in dim order, in the pool's element encoding (int4: one code per
// byte).
template <int KVT, int D> constexpr int stage_token_bytes() {
    return 2 * D * (KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1));
}

// Floats of the LDS area at the start of the dynamic LDS: the waves' outputs
// (one [rows][d + 1] copy per wave when `copies` = kWaves, one shared copy
// otherwise), or (before the merge) the staged appended tokens followed by
// the ids of the blocks they go to (at most k / 16 + 2 blocks).
__host__ __device__ inline int acc_area_floats(int rows, int d, int k_rows, int stage_bytes, int copies) {
    const int a = copies * rows * (d + 1);
    const int b = k_rows * stage_bytes / 4 + k_rows / 16 + 2;
    return a > b ? a : b;
}

// Output copies of the wave merge: one per wave up to 32 rows (the waves
// write at once), one shared copy beyond (the waves add in turn).
constexpr int wave_copies(int nt) { return nt <= 2 ? kWaves : 1; }

// Dynamic LDS of the partition kernel: the accumulator area, the waves' (m, l),
// the (m, l) of up to kCascadeMaxChunks shared-prefix partials per row and
// the output phase's row factors (8 per row).
__host__ __device__ inline size_t partition_lds_bytes(int rows, int d, int k_rows, int stage_bytes, int copies) {
    return (static_cast<size_t>(acc_area_floats(rows, d, k_rows, stage_bytes, copies)) + 2 * kWaves * rows +
            2 * kCascadeMaxChunks * rows + 8 * rows) * sizeof(float);
}

// ------------------------------------------------------- partition kernel
// One (unit, KV head) item: attend over the unit's blocks with the work-group's
// four waves, merge the waves, then write the output (unsplit sequence) or the
// partial result, merging the sequence's partials when this is the last of
// them to arrive.
template <int KVT, int D, int NT, int POL>
__device__ __forceinline__ void attend_item(const AttnArgs& a, const int unit, const int h, float* smem,
                                            int* ticket_s, int& claimed, const int tid) {
    const int R = a.rows;
    constexpr int STOK = stage_token_bytes<KVT, D>();
    float* acc_s = smem;                       // [R][D + 1] merged unnormalised output
    uint8_t* stage = reinterpret_cast<uint8_t*>(smem);   // appended tokens, during the block walk
    // One-row-tile instances give every wave its own output copy to merge.
    constexpr int kCopies = wave_copies(NT);
    float* m_s = smem + acc_area_floats(R, D, a.k_rows, STOK, kCopies);   // [W][R]
    float* l_s = m_s + kWaves * R;             // [W][R]
    float* pre_s = l_s + kWaves * R;           // [2][kCascadeMaxChunks * R] prefix partials' m, then l

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4;                  // lane group: tokens 4*lg .. +3
    const int col = lane & 15;                 // column within a row tile
    // Unit descriptor (see the plan built by block_table_upload) and, loaded
    // independently of it, this wave's first block ids.
    const int32_t* ud = a.units + static_cast<int64_t>(unit) * kUnitInts;
    const int32_t* uids = a.unit_ids + static_cast<int64_t>(unit) * a.unit_stride;
    int id0 = 0;
    if (wave + kWaves * lane < a.unit_stride) id0 = uids[wave + kWaves * lane];
    const int seq = ud[kUnitSeq];
    const int b0 = ud[kUnitB0];
    const int nb = ud[kUnitNb];
    const int n = ud[kUnitLen];
    const int parts = ud[kUnitParts];
    const int slot = ud[kUnitSlot];
    const int rot = ud[kUnitRot];
    const int part = ud[kUnitPart];
    const int tickets = ud[kUnitTickets];
    const int G = a.group;
    const int kq = a.k_rows;


    float sscale = a.score_scale;
    float vscale = 1.f;
    if constexpr (kv_scaled<KVT>()) {
        sscale *= a.k_scale[a.layer * a.num_kv_heads + h];
        vscale = a.v_scale[a.layer * a.num_kv_heads + h];
    }
    if constexpr (KVT == KV_INT8) sscale *= 1.f / kI8QScale;   // int8 scores come in units of kI8QScale

    // Query operands and per-column visibility limits.
    using QT = typename std::conditional<KVT == KV_INT8, QRegsI8<D>, QRegs<KVT, D>>::type;
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
    // int4 and int8: scores come out biased by the code bias times the sum of
    // the query row
    float qbias[NT];
    float qbs[NT];   // the bias scaled (int4, int8: taken out of the scaled scores; otherwise 0)
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        if constexpr (KVT == KV_INT4) qbias[c] = kI4Bias * query_row_sum<D>(qr[c])[0];
        else if constexpr (KVT == KV_INT8) qbias[c] = kI8Bias * query_row_sum<D>(qr[c])[0];   // units of kI8QScale
        else qbias[c] = 0.f;
        qbs[c] = (KVT == KV_INT4 || KVT == KV_INT8) ? qbias[c] * sscale : 0.f;
    }
    const int mask_from = n - kq + 1;

    // Row sums of the probabilities: float32 pools add them on the VALU per
    // lane (l_run, four tokens per lane group); the others on the matrix
    // cores, with the PV product's bf16 (int8: fp16) operand against a tile of ones
    // (lacc: every element holds the row's sum of the values used).
    f32x4 o[NT][D / 16];
    float m_run[NT], l_run[NT];
    float thr[NT];   // scaled (biased) score above which a column's reference must move
    f32x4 lacc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        m_run[c] = neg_inf();
        thr[c] = neg_inf();
        l_run[c] = 0.f;
        lacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < D / 16; ++m) o[c][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Full row sum of column tile c for this lane's row.
    auto row_sum = [&](int c) {
        if constexpr (KVT == KV_F32) {
            float l = l_run[c];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            return l;
        } else {
            return lacc[c][0];
        }
    };

    const int64_t block_stride = static_cast<int64_t>(a.num_kv_heads) * 2 * a.tile_bytes;
    const uint8_t* head_base = a.pool +
        static_cast<int64_t>(a.layer) * a.num_blocks * block_stride + static_cast<int64_t>(h) * 2 * a.tile_bytes;

    // Appended positions [lo, hi) of this unit (fused append): their K/V are
    // staged in LDS and substituted into the tile registers, so the tiles are
    // read without waiting for the pool write.
    int lo = 0, hi = 0;
    if (a.k_new != nullptr) {
        lo = max(n - kq, b0 * kBlock);
        hi = min(n, (b0 + nb) * kBlock);
    }
    const bool appends = lo < hi;

    const int koff = lane * 16;
    const int voff = TileRegs<KVT, D>::v_offset(lane);
    const int blk_lo = lo / kBlock;
    int* pid_s = reinterpret_cast<int*>(stage + kq * STOK);   // block ids of the appended positions

    auto process = [&](TileRegs<KVT, D>& tr, int blk) {
        if (appends && blk * kBlock + kBlock > lo && blk * kBlock < hi) {
            const int t0 = max(lo, blk * kBlock);
            const int t1 = min(hi, blk * kBlock + kBlock);
            for (int t = t0; t < t1; ++t) tr.put_token(t - blk * kBlock, stage + (t - lo) * STOK, lane);
        }
        // Scaled scores (int4, int8: still biased by qbs).  The scaling is
        // the products' only reader and is pinned to their basic block (see
        // pin_after_mfma_reads).
        f32x4 s[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            if constexpr (KVT == KV_INT8) s[c] = scores_i8<D>(tr, qr[c]);
            else s[c] = scores<D>(tr, qr[c]);
        }
#pragma unroll
        for (int c = 0; c < NT; ++c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s[c][i] *= sscale;
            pin_after_mfma_reads(s[c]);
        }
        const int tok0 = blk * kBlock + 4 * lg;
        if (blk * kBlock + kBlock > mask_from) {
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tok0 + i >= lim[c]) s[c][i] = neg_inf();
        }
        if (blk * kBlock + kBlock > n) tr.zero_v_from(n - tok0);
        f32x4 p[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            // The running max is a lagging reference: it moves only when a
            // score exceeds it by more than kLazyMax, so probabilities stay
            // <= 2^kLazyMax and the accumulators are rescaled on few blocks.
            // O and l share the reference, so O / l does not depend on it.
            // Each lane compares its own 4 scores with the column's threshold
            // (reference + kLazyMax, in the scores' biased units); only when
            // some lane passes it does the wave reduce the column maxima
            // across lanes and move the reference (a row's first finite
            // score always does).
            const float ml = smax(smax(s[c][0], s[c][1]), smax(s[c][2], s[c][3]));
            if (__ballot(ml > thr[c])) {
                const float mx = max_over_rows(ml) - qbs[c];
                if (mx > m_run[c] + kLazyMax) {
                    const float alpha = fast_exp2(m_run[c] - mx);
                    m_run[c] = mx;
                    lacc[c] *= alpha;
                    l_run[c] *= alpha;
#pragma unroll
                    for (int m = 0; m < D / 16; ++m) o[c][m] *= alpha;
                }
                thr[c] = m_run[c] + kLazyMax + qbs[c];
            }
            const float muse = m_run[c] == neg_inf() ? 0.f : m_run[c];
            const float off = qbs[c] + muse;
#pragma unroll
            for (int i = 0; i < 4; ++i) p[c][i] = fast_exp2(s[c][i] - off);
            if constexpr (KVT == KV_F32) {
                float psum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) psum += p[c][i];
                l_run[c] += psum;
            }
        }
        if constexpr (KVT == KV_INT8) {
            // the fp16 probabilities the int8 PV product uses
            const f16x4 ones = __builtin_bit_cast(f16x4, u32x2{0x3c003c00u, 0x3c003c00u});
            f16x4 ph[NT];
            probs_f16<NT>(p, ph);
#pragma unroll
            for (int c = 0; c < NT; ++c) lacc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, ph[c], lacc[c], 0, 0, 0);
        } else if constexpr (KVT != KV_F32) {
            const s16x4 ones = __builtin_bit_cast(s16x4, u32x2{0x3f803f80u, 0x3f803f80u});
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[c][0], p[c][1]),
                                                                 pack_bf16x2(p[c][2], p[c][3])});
                lacc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, lacc[c], 0, 0, 0);
            }
        }
        accumulate_pv<D, NT>(tr, p, o);
    };

    // The unit's ids are stored in walking order j = 0 .. nb-1, which visits
    // logical block b0 + (j + rot) mod nb: sequences that share physical
    // blocks (a common prefix) start their walk at different blocks instead of
    // all reading the same block at the same moment.  A wave walks j = wave,
    // wave + 4, ... in chunks of up to 64 blocks (one block id per lane).
    auto logical = [&](int j) { const int x = j + rot; return b0 + (x >= nb ? x - nb : x); };
    constexpr int NBUF = decode_buffers(KVT, D, NT);   // tiles a wave holds: NBUF - 1 in flight
    int base = wave;
    int cnt = 0;
    int id = 0;
    // The next block's loads are issued unconditionally so the wait counts
    // stay static; past the last block they go through a zero-sized
    // resource (no memory traffic, zeros returned).
    // Block i of the chunk, loaded with the launch's cache policy POL.
    auto issue = [&](TileRegs<KVT, D>& t, int i, bool valid) {
        const int pid = __builtin_amdgcn_readlane(id, min(i, 63));
        t.template load<POL>(tile_rsrc(head_base + static_cast<int64_t>(pid) * block_stride, valid ? a.tile_bytes : 0),
                             koff, voff);
    };
    TileRegs<KVT, D> tr[NBUF];
    // First loads of a chunk: NBUF - 1 blocks in flight.
    // A wave without blocks (cnt = 0) issues them through zero-sized
    // resources, so the first chunk's loads are issued on every path.
    auto begin_chunk = [&]() {
        cnt = min(64, (nb - base + kWaves - 1) / kWaves);
        id = id0;
        if (base != wave) {
            id = 0;
            if (base + kWaves * lane < a.unit_stride) id = uids[base + kWaves * lane];
        }
        id = min(max(id, 0), a.num_blocks - 1);
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b) issue(tr[b], b, cnt > b);
    };
    // Fused append (paged_attention_append): the k newest positions n-k ..
    // n-1 of the sequence are written into the pool, for this KV head, by the
    // work-group whose unit holds them.  Their codes are staged in LDS and
    // take the place of what the tile loads return for those positions, so
    // no tile read waits for a pool write (the writes, issued after the walk,
    // complete by the end of the kernel, before any later call reads the
    // pool).  The inputs, the
    // block ids and the scales are loaded before the first tile loads are
    // issued: vector loads complete in issue order, so loading them later
    // would hold the wave until its first tiles had arrived.
    constexpr int kPre = 8;                       // input elements per thread per batch
    constexpr int kBatch = 64 * kWaves * kPre;    // elements per batch (whole tokens)
    static_assert(kBatch % (2 * D) == 0, "a batch holds whole tokens");
    const int first_new = n - kq;
    const int ib = a.append_in_f32 ? 4 : 2;       // input element bytes
    const int n_elem = (hi - lo) * 2 * D;         // staged elements: K then V of each token
    unsigned xin[kPre];
    float k_sc = 1.f, v_sc = 1.f;                 // scales of code pools
    // Buffer resources over the unit's appended input rows of KV head h (K
    // and V; element (t, i) at ((t - lo) * H_kv * D + i) * ib).  They are
    // zero-sized when nothing is appended, so the loads below are issued on
    // every path, without branches, and read nothing then.
    const int64_t row0 = (static_cast<int64_t>(seq) * kq + (lo - first_new)) * a.num_kv_heads + h;
    const int in_span = appends ? ((hi - lo - 1) * a.num_kv_heads * D + D) * ib : 0;
    const uint8_t* kin = appends ? reinterpret_cast<const uint8_t*>(a.k_new) + row0 * D * ib : a.pool;
    const uint8_t* vin = appends ? reinterpret_cast<const uint8_t*>(a.v_new) + row0 * D * ib : a.pool;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kin), 0, in_span, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vin), 0, in_span, 0x00020000);
    // Element e = e0 + tid + 64 W r of a batch: token lo + e / 2D, element
    // e % 2D of its K (< D) or V row.  2D is a multiple of 64, so K or V is
    // the same for a whole wave.  One dword load per element (a bf16 input
    // takes its half; row lengths are even, so the dword stays in the span);
    // elements past the end lie past the span and read as zero.
    auto load_batch = [&](int e0) {
#pragma unroll
        for (int r = 0; r < kPre; ++r) {
            const int eb = e0 + 64 * kWaves * r + 64 * wave;   // uniform
            const int tt = eb / (2 * D);
            const int iw = eb % (2 * D);
            const bool isv = iw >= D;
            const int off = (tt * a.num_kv_heads * D + (isv ? iw - D : iw) + lane) * ib;
            const unsigned raw = __builtin_amdgcn_raw_buffer_load_b32(isv ? vrs : krs, off & ~3, 0, 0);
            xin[r] = ib == 4 ? raw : ((raw >> ((off & 2) * 8)) & 0xffffu);
        }
    };
    auto stage_batch = [&](int e0) {
        float kinv = 1.f, vinv = 1.f;
        if constexpr (kv_scaled<KVT>()) {
            kinv = 1.0f / k_sc;
            vinv = 1.0f / v_sc;
        }
#pragma unroll
        for (int r = 0; r < kPre; ++r) {
            const int e = e0 + tid + 64 * kWaves * r;
            if (e < n_elem) {
                const int i = e % (2 * D);
                uint8_t* st = stage + (e / (2 * D)) * STOK;
                if constexpr (kv_scaled<KVT>()) {
                    const float x = ib == 4 ? __uint_as_float(xin[r]) : __uint_as_float(xin[r] << 16);
                    st[i] = static_cast<uint8_t>(quantize_code<KVT>(x, i < D ? kinv : vinv));
                } else if constexpr (KVT == KV_BF16) {
                    reinterpret_cast<uint16_t*>(st)[i] = static_cast<uint16_t>(xin[r]);
                } else {
                    reinterpret_cast<unsigned*>(st)[i] = xin[r];
                }
            }
        }
    };
    // Block ids of the appended positions (lanes past them load the last
    // one's; without appended positions, entry 0) and the scales.
    int pid_r;
    {
        int j = appends ? blk_lo + min(tid, (hi - 1) / kBlock - blk_lo) - b0 - rot : 0;
        if (j < 0) j += nb;
        pid_r = uids[j];
    }
    if constexpr (kv_scaled<KVT>()) {
        k_sc = a.k_scale[a.layer * a.num_kv_heads + h];
        v_sc = a.v_scale[a.layer * a.num_kv_heads + h];
    }
    load_batch(0);

    begin_chunk();

    if (appends) {
        stage_batch(0);
        for (int e0 = kBatch; e0 < n_elem; e0 += kBatch) {   // more than a batch: loaded here
            load_batch(e0);
            stage_batch(e0);
        }
        if (tid < (hi - 1) / kBlock - blk_lo + 1) pid_s[tid] = pid_r;   // clamped where it is read
        lds_barrier();   // the tile loads stay in flight
    }

    while (base < nb) {
        // NBUF buffers in rotation: before block i + b is processed, block
        // i + b + NBUF - 1 is issued into the buffer block i + b - 1 left.
        int i = 0;
        for (; i + NBUF - 1 < cnt; i += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                issue(tr[(b + NBUF - 1) % NBUF], i + b + NBUF - 1, b == 0 || i + b + NBUF - 1 < cnt);
                process(tr[b], logical(base + kWaves * (i + b)));
            }
        }
#pragma unroll
        for (int b = 0; b < NBUF - 1; ++b)
            if (i + b < cnt) process(tr[b], logical(base + kWaves * (i + b)));
        base += 64 * kWaves;
        if (base < nb) begin_chunk();
    }

    // Pool writes of the appended positions, from the staged codes (tile
    // layouts in the library header: K in 16-byte chunks of consecutive
    // dims, V transposed).  They are issued after the walk, so no tile load
    // of the walk waits behind them (measured: issued before the walk they
    // cost the c2 step about 2 us more).
    if (appends) {
        for (int t = lo; t < hi; ++t) {
            const int o = t % kBlock;
            const int pid = min(max(pid_s[t / kBlock - blk_lo], 0), a.num_blocks - 1);
            uint8_t* tk = const_cast<uint8_t*>(head_base) + static_cast<int64_t>(pid) * block_stride;
            uint8_t* tv = tk + a.tile_bytes;
            const uint8_t* st = stage + (t - lo) * STOK;
            if constexpr (KVT == KV_INT4) {
                // K: run (g, o) holds dims 32 s + 8 g + e at nibble 8 s + e;
                // V: run (o / 4, c) holds dims 16 (2 j) + c and 16 (2 j + 1) + c
                // of token o in byte 4 j + o % 4 (low, high nibble).
                for (int w = tid; w < 4 + 16; w += 64 * kWaves) {
                    if (w < 4) {
                        unsigned wd[D / 32];
#pragma unroll
                        for (int q = 0; q < D / 32; ++q) {
                            unsigned x = 0;
#pragma unroll
                            for (int e = 0; e < 8; ++e) x |= (static_cast<unsigned>(st[32 * q + 8 * w + e]) & 0xfu) << (4 * e);
                            wd[q] = x;
                        }
                        uint8_t* run = tk + (w * 16 + o) * (D / 8);
                        if constexpr (D == 128) *reinterpret_cast<u32x4*>(run) = u32x4{wd[0], wd[1], wd[2], wd[3]};
                        else *reinterpret_cast<u32x2*>(run) = u32x2{wd[0], wd[1]};
                    } else {
                        const int c = w - 4;
                        uint8_t* run = tv + ((o / 4) * 16 + c) * (D / 8);
#pragma unroll
                        for (int j = 0; j < D / 32; ++j)
                            run[4 * j + o % 4] = static_cast<uint8_t>((st[D + 32 * j + c] & 0xfu) |
                                                                      ((st[D + 32 * j + 16 + c] & 0xfu) << 4));
                    }
                }
            } else {
                constexpr int EB = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);
                constexpr int CH = D * EB / 16;   // 16-byte K chunks per token
                for (int w = tid; w < CH + D; w += 64 * kWaves) {
                    if (w < CH) {
                        *reinterpret_cast<u32x4*>(tk + (w * kBlock + o) * 16) =
                            *reinterpret_cast<const u32x4*>(st + w * 16);
                    } else {
                        const int i = w - CH;
                        uint8_t* dst = tv + (i * kBlock + o) * EB;
                        if constexpr (EB == 4) *reinterpret_cast<unsigned*>(dst) = reinterpret_cast<const unsigned*>(st)[D + i];
                        else if constexpr (EB == 2) *reinterpret_cast<uint16_t*>(dst) = reinterpret_cast<const uint16_t*>(st)[D + i];
                        else *dst = st[D + i];
                    }
                }
            }
        }
    }

    // int4 and int8: the output came out biased by the code bias times the
    // row's probability sum (over all of the wave's tokens).
    if constexpr (KVT == KV_INT4 || KVT == KV_INT8) {
        constexpr float bias = KVT == KV_INT4 ? kI4Bias : kI8Bias;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const float l = row_sum(c);
#pragma unroll
            for (int m = 0; m < D / 16; ++m) o[c][m] -= bias * l;
        }
    }

    // This work-group's blocks are read: claim its next item now, while the
    // waves merge, so work-groups that finish early take more items.
    // (The offset, zero, is hidden from the optimiser: with a visibly uniform
    // address it turns the add into a wave-wide scan whose result it waits
    // for at once, behind every load in flight.)
    if (tid == 0 && a.num_items > static_cast<int>(gridDim.x)) {
        int zero = 0;
        asm volatile("" : "+v"(zero));
        claimed = __hip_atomic_fetch_add(a.queue + zero, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ------------------------------------------------------------ output
    // The output phase works on groups of 4 dims: group q is row q / (D / 4),
    // dims 4 (q % (D / 4)) .. +3.  A sequence with one partition writes its
    // output; a split one its partial result (O, m, l), and the last of its
    // work-groups to take a ticket merges all partials.  A sequence whose
    // only work-group in this launch is this one, its other partials (the
    // slots before this unit's) written by the shared-prefix pass, an
    // earlier launch, is merged here at once, with no partial or ticket of
    // its own; the loads of those partials go out before the waves merge
    // (up to two row tiles), so they travel meanwhile.
    const int lead = parts - 1;
    const bool split = parts > 1;
    const bool direct = split && tickets == 1 && lead <= kCascadeMaxChunks;
    const int64_t first_slot = static_cast<int64_t>(h) * a.num_split_slots + (slot - part);
    constexpr int Q = D / 4;                   // groups per row
    const int groups = R * Q;
    constexpr int kG = 4;                      // groups per thread and batch of prefix loads
    constexpr bool kEarly = NT <= 2;
    f32x4 po[kG][kCascadeMaxChunks];
    // Buffer resources over the sequence's prefix partials (O, then m and l).
    const __amdgpu_buffer_rsrc_t pre_o = __builtin_amdgcn_make_buffer_rsrc(
        direct ? a.part_o + first_slot * R * D : a.part_o, 0, direct ? lead * R * D * 4 : 0, 0x00020000);
    auto load_prefix = [&](int q0) {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int q = min(q0 + 64 * kWaves * u, groups - 1);
            const int r = q / Q;
#pragma unroll
            for (int c = 0; c < kCascadeMaxChunks; ++c)
                po[u][c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    pre_o, ((min(c, lead - 1) * R + r) * D + 4 * (q - r * Q)) * 4, 0, 0));
        }
    };
    float pre_m = 0.f, pre_l = 0.f;
    if (direct) {
        if (tid < lead * R) {
            pre_m = a.part_m[first_slot * R + tid];
            pre_l = a.part_l[first_slot * R + tid];
        }
        if constexpr (kEarly) load_prefix(tid);
    }

    // Merge the waves: publish (m, l), rescale O to the common max, add in LDS.
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const float l = row_sum(c);
        const int row = 16 * c + col;
        if (lg == 0 && row < R) {
            m_s[wave * R + row] = m_run[c];
            l_s[wave * R + row] = l;
        }
    }
    // The merge exchanges data through LDS only; the pool writes of appended
    // tokens stay in flight.
    lds_barrier();
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
    if constexpr (kCopies == kWaves) {
        // Every wave writes its rescaled output to its own copy; the output
        // loop adds the copies in wave order.
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int row = 16 * c + col;
            if (row >= R) continue;
            float* dst = acc_s + (wave * R + row) * (D + 1) + 4 * lg;
#pragma unroll
            for (int m = 0; m < D / 16; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[16 * m + i] = o[c][m][i] * f[c];
        }
        lds_barrier();
    } else {
        for (int w = 0; w < kWaves; ++w) {
            if (wave == w) {
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const int row = 16 * c + col;
                    if (row >= R) continue;
                    float* dst = acc_s + row * (D + 1) + 4 * lg;
                    // wave 0 overwrites (the area held the staged tokens)
#pragma unroll
                    for (int m = 0; m < D / 16; ++m)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            dst[16 * m + i] = (w == 0 ? 0.f : dst[16 * m + i]) + o[c][m][i] * f[c];
                }
            }
            lds_barrier();
        }
    }

    // Row factors, one thread per row: the waves' common max M and sum L
    // (the copies in acc_s are already relative to M); with prefix partials
    // the max over those too, their weights and the final scale.
    float* row_s = pre_s + 2 * kCascadeMaxChunks * R;   // [R][8]
    if (direct) {
        if (tid < lead * R) {
            pre_s[tid] = pre_m;
            pre_s[kCascadeMaxChunks * R + tid] = pre_l;
        }
        lds_barrier();
    }
    if (tid < R) {
        const int r = tid;
        float M = neg_inf();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_s[w * R + r]);
        float L = 0.f;
        if (M != neg_inf()) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) L += l_s[w * R + r] * fast_exp2(m_s[w * R + r] - M);
        }
        if (direct) {
            float Mx = M;
#pragma unroll
            for (int c = 0; c < kCascadeMaxChunks; ++c)
                if (c < lead) Mx = fmaxf(Mx, pre_s[c * R + r]);
            const float so = M == neg_inf() ? 0.f : fast_exp2(M - Mx);
            float Lx = L * so;
            float wc[kCascadeMaxChunks];
#pragma unroll
            for (int c = 0; c < kCascadeMaxChunks; ++c) {
                wc[c] = c < lead ? fast_exp2(pre_s[c * R + r] - Mx) : 0.f;
                if (c < lead) Lx += pre_s[kCascadeMaxChunks * R + c * R + r] * wc[c];
            }
            const float inv = vscale / Lx;
            row_s[8 * r] = so * inv;
#pragma unroll
            for (int c = 0; c < kCascadeMaxChunks; ++c) row_s[8 * r + 1 + c] = wc[c] * inv;
        } else if (!split) {
            row_s[8 * r] = vscale / L;
        } else {
            row_s[8 * r] = M;
            row_s[8 * r + 1] = L;
        }
    }
    lds_barrier();

    // Own output of group (r, dq), summed over the wave copies.
    auto own4 = [&](int r, int dq) {
        const float* src = acc_s + r * (D + 1) + 4 * dq;
        f32x4 O = {src[0], src[1], src[2], src[3]};
        if constexpr (kCopies == kWaves) {
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                const float* sw = acc_s + (w * R + r) * (D + 1) + 4 * dq;
                O += f32x4{sw[0], sw[1], sw[2], sw[3]};
            }
        }
        return O;
    };
    // Final output of group (r, dq): one 8- or 16-byte store when the output
    // array is 16-byte aligned.
    const bool vec_out = (reinterpret_cast<uintptr_t>(a.out) & 15) == 0;
    auto store4 = [&](int r, int dq, const f32x4& v) {
        if (vec_out) {
            const int jr = r / G;
            const int g = r - jr * G;
            const int64_t oi =
                ((static_cast<int64_t>(seq) * kq + jr) * a.num_q_heads + h * G + g) * D + 4 * dq;
            if (a.out_bf16)
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + oi) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            else
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + oi) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) store_out(a, seq, h, r, 4 * dq + i, v[i]);
        }
    };

    if (direct) {
        for (int q0 = tid; q0 < groups; q0 += 64 * kWaves * kG) {
            if (!kEarly || q0 != tid) load_prefix(q0);
#pragma unroll
            for (int u = 0; u < kG; ++u) {
                const int q = q0 + 64 * kWaves * u;
                if (q >= groups) break;
                const int r = q / Q;
                const float* rf = row_s + 8 * r;
                f32x4 O = own4(r, q - r * Q) * rf[0];
#pragma unroll
                for (int c = 0; c < kCascadeMaxChunks; ++c)
                    if (c < lead) O += po[u][c] * rf[1 + c];
                store4(r, q - r * Q, O);
            }
        }
        return;
    }
    if (!split) {
        for (int q = tid; q < groups; q += 64 * kWaves) {
            const int r = q / Q;
            store4(r, q - r * Q, own4(r, q - r * Q) * row_s[8 * r]);
        }
        return;
    }

    // Partial result of this unit: O with agent-coherent (sc1) 16-byte
    // stores, m and l by the row threads.
    {
        const int64_t sl = static_cast<int64_t>(h) * a.num_split_slots + slot;
        const __amdgpu_buffer_rsrc_t po_r =
            __builtin_amdgcn_make_buffer_rsrc(a.part_o + sl * R * D, 0, R * D * 4, 0x00020000);
        for (int q = tid; q < groups; q += 64 * kWaves) {
            const int r = q / Q;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, own4(r, q - r * Q)), po_r,
                                                   (r * D + 4 * (q - r * Q)) * 4, 0, kCoherent);
        }
        if (tid < R) {
            xwg_store(a.part_m + sl * R + tid, row_s[8 * tid]);
            xwg_store(a.part_l + sl * R + tid, row_s[8 * tid + 1]);
        }
    }
    if (parts > a.fuse_max_parts) return;

    // Split-KV merge in the kernel: the last of the sequence's work-groups
    // (for this KV head) to take a ticket combines all partials.  Every thread
    // waits until its partial stores have completed before the work-group
    // takes its ticket; the last one reads the partials only after its ticket.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int32_t* counter = a.counters + static_cast<int64_t>(seq) * a.num_kv_heads + h;
    if (tid == 0)
        *ticket_s = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // (the sequence's first partials may come from an earlier shared-prefix
    // pass: only the work-groups of this launch take tickets)
    if (*ticket_s != tickets - 1) return;
    // The partials' (m, l) go to LDS in one parallel pass (every load in
    // flight at once: these loads travel to the coherent level, so a chain of
    // them would cost a round trip each); acc_s is free now and holds
    // 2 * parts * R <= R * (D + 1) floats for parts <= kFuseMaxParts.
    float* pm = acc_s;                // [parts][R] maxima, then the partition weights
    float* pw = acc_s + parts * R;    // [parts][R] sums
    float* Lr = m_s;                  // [R] common sum of each row
    for (int e = tid; e < parts * R; e += 64 * kWaves) {
        pm[e] = xwg_load(a.part_m + first_slot * R + e);
        pw[e] = xwg_load(a.part_l + first_slot * R + e);
    }
    __syncthreads();
    for (int r = tid; r < R; r += 64 * kWaves) {
        float M = neg_inf();
        for (int q = 0; q < parts; ++q) M = fmaxf(M, pm[q * R + r]);
        float L = 0.f;
        for (int q = 0; q < parts; ++q) {
            const float wq = fast_exp2(pm[q * R + r] - M);
            L += pw[q * R + r] * wq;
            pm[q * R + r] = wq;       // weight of partition q for row r
        }
        Lr[r] = vscale / L;
    }
    __syncthreads();
    // Partials' O: 16-byte coherent loads, 8 partitions in flight per group.
    const __amdgpu_buffer_rsrc_t all_o =
        __builtin_amdgcn_make_buffer_rsrc(a.part_o + first_slot * R * D, 0, parts * R * D * 4, 0x00020000);
    for (int q = tid; q < groups; q += 64 * kWaves) {
        const int r = q / Q;
        const int off = (r * D + 4 * (q - r * Q)) * 4;
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
        for (int p0 = 0; p0 < parts; p0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    all_o, off + min(p0 + u, parts - 1) * R * D * 4, 0, kCoherent));
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (p0 + u < parts) O += v[u] * pm[(p0 + u) * R + r];
        }
        store4(r, q - r * Q, O * Lr[r]);
    }
    if (tid == 0)   // ready for the next call
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Persistent work-groups: work-group b first takes item b, then items
// gridDim.x, gridDim.x + 1, ... in the order they are claimed from the
// queue, until none is left; a work-group claims its next item when it has
// read all blocks of the current one.  Every work-group leaves the loop
// after exactly one claim past the end; the last to leave sets both queue
// counters back to zero for the next call.  When the grid has a work-group
// per item nothing is claimed and the queue is not touched.  No work-group
// ever waits for another.
template <int KVT, int D, int NT, int POL>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(NT == 1 ? decode_wgs_per_cu(KVT, D) : (NT == 2 && KVT != KV_F32 ? 2 : 1))))
void attn_partition_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    __shared__ int ticket;
    __shared__ int next_item;
    const int wave_s = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    int item = blockIdx.x;
    while (item < a.num_items) {
        int claimed = a.num_items;   // thread 0: the next item's place in the queue
        // The arguments are read afresh from the kernel-argument segment for
        // every item (the pointer is made opaque to the optimiser), so values
        // derived from them are not kept live across the whole loop.
#if defined(__HIP_DEVICE_COMPILE__)
        typedef const AttnArgs __attribute__((address_space(4)))* KernargPtr;
        KernargPtr ap = (KernargPtr)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const AttnArgs ia = *ap;
#else
        const AttnArgs ia = a;
#endif
        int unit, h;
        item_coords(item, ia.num_items / ia.num_kv_heads, ia.num_kv_heads, unit, h);
        // The thread index is made opaque per item as well, so lane-derived
        // offsets are computed inside the item instead of held (or spilled)
        // across the whole loop.
        int tid = wave_s * 64 + static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
        asm volatile("" : "+v"(tid));
        attend_item<KVT, D, NT, POL>(ia, unit, h, smem, &ticket, claimed, tid);
        if (tid == 0) next_item = static_cast<int>(gridDim.x) + claimed;
        lds_barrier();   // next_item visible; this item's LDS reads are done
        item = next_item;
    }
    // Thread 0 found again from the wave index and the lane, so the thread
    // index is not held across the loop.
    const bool first_thread =
        wave_s == 0 && __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0;
    if (first_thread && a.num_items > static_cast<int>(gridDim.x)) {
        // The claim that ended the loop has returned before this add is issued,
        // so when the last work-group counts itself no claim is outstanding.
        const int left = __hip_atomic_fetch_add(a.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (left == static_cast<int>(gridDim.x) - 1) {
            __hip_atomic_store(a.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------ merge kernel
// One work-group per (split sequence, KV head, query row): combines the
// partitions' (O, m, l):  M = max m_p,  L = sum l_p 2^(m_p - M),
// out = sum O_p 2^(m_p - M) / L  (times the V scale of fp8 pools).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int scaled) {
    __shared__ float red[8];
    __shared__ f32x4 part_acc[256];
    const int seq = blockIdx.x;
    const int h = blockIdx.y;
    const int r = blockIdx.z;
    const int nparts = a.seq_parts[2 * seq];
    const int sbase = a.seq_parts[2 * seq + 1];
    if (nparts <= a.fuse_max_parts) return;   // merged inside the partition kernel
    const int R = a.rows;
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
        const float vscale = scaled ? a.v_scale[a.layer * a.num_kv_heads + h] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out(a, seq, h, r, 4 * tid + i, sum[i] / L * vscale);
    }
}

// Work-groups of one instance that fit on the device at once (all CUs).
template <int KVT, int D, int NT>
int resident_work_groups() {
    static int per_cu = 0;   // same for every device of one architecture
    if (per_cu == 0) {
        constexpr int rows = 16 * NT;   // at most rows appended tokens per sequence (G = 1)
        const size_t lds_max = partition_lds_bytes(rows, D, rows, stage_token_bytes<KVT, D>(), wave_copies(NT));
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_partition_kernel<KVT, D, NT, kStreamLoad>, 64 * kWaves,
                                                         lds_max) != hipSuccess || n < 1)
            n = 1;
        per_cu = n;
    }
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    return per_cu * cus;
}

template <int KVT, int D, int NT>
hipError_t launch_instance(const AttnArgs& a, int num_units, bool shared_blocks, hipStream_t stream) {
    (void)num_units;
    const size_t lds = partition_lds_bytes(a.rows, D, a.k_rows, stage_token_bytes<KVT, D>(), wave_copies(NT));
    const int grid = std::min(a.num_items, resident_work_groups<KVT, D, NT>());
    // Tiles are streamed (each is read once per step) unless the batch shares
    // blocks between sequences, whose repeated reads should hit the caches.
    if (shared_blocks)
        hipLaunchKernelGGL((attn_partition_kernel<KVT, D, NT, kCachedLoad>), dim3(grid), dim3(64 * kWaves), lds, stream, a);
    else
        hipLaunchKernelGGL((attn_partition_kernel<KVT, D, NT, kStreamLoad>), dim3(grid), dim3(64 * kWaves), lds, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.max_parts > a.fuse_max_parts) {
        dim3 g2(a.num_seqs, a.num_kv_heads, a.rows);
        hipLaunchKernelGGL((attn_merge_kernel<D>), g2, dim3(256), 0, stream, a, kv_scaled<KVT>() ? 1 : 0);
        err = hipGetLastError();
    }
    return err;
}

template <int KVT, int D>
hipError_t launch_rows(const AttnArgs& a, int num_units, bool shared, hipStream_t stream) {
    if (a.rows <= 16) return launch_instance<KVT, D, 1>(a, num_units, shared, stream);
    if (a.rows <= 32) return launch_instance<KVT, D, 2>(a, num_units, shared, stream);
    return launch_instance<KVT, D, 4>(a, num_units, shared, stream);
}

}  // namespace

hipError_t attention_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* address[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (address[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        address[dev] = p;
    }
    *ptr = address[dev];
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, int kv_dtype, int head_dim, int num_units, bool shared_blocks,
                            hipStream_t stream) {
    if (num_units <= 0) return hipSuccess;
    const bool sh = shared_blocks;
    if (kv_dtype == KV_BF16)
        return head_dim == 128 ? launch_rows<KV_BF16, 128>(a, num_units, sh, stream)
                               : launch_rows<KV_BF16, 64>(a, num_units, sh, stream);
    if (kv_dtype == KV_FP8)
        return head_dim == 128 ? launch_rows<KV_FP8, 128>(a, num_units, sh, stream)
                               : launch_rows<KV_FP8, 64>(a, num_units, sh, stream);
    if (kv_dtype == KV_INT8)
        return head_dim == 128 ? launch_rows<KV_INT8, 128>(a, num_units, sh, stream)
                               : launch_rows<KV_INT8, 64>(a, num_units, sh, stream);
    if (kv_dtype == KV_INT4)
        return head_dim == 128 ? launch_rows<KV_INT4, 128>(a, num_units, sh, stream)
                               : launch_rows<KV_INT4, 64>(a, num_units, sh, stream);
    return head_dim == 128 ? launch_rows<KV_F32, 128>(a, num_units, sh, stream)
                           : launch_rows<KV_F32, 64>(a, num_units, sh, stream);
}

}  // namespace pkv
