// Chunked-prefill paged attention for gfx950.
//
// Method (page "KV cache & continuous batching", section "3. Chunked
// prefill": a long prompt is processed in chunks of a few thousand tokens,
// each chunk attending over the cached K/V of everything before it and over
// itself; sections "The core insight" and "2. PagedAttention (vLLM)" for the
// cache and the gather through the block table; page "LLM Inference
// Optimization: KV Cache, Batching, and Speculative Decoding", section
// "Prefill Optimization": prefill is a compute-bound matrix product):
//   row (j, g) of sequence s is chunk token j (position n - C + j) for query
//   head h*G + g; out = softmax(scale * q . K[t]^T over t <= n - C + j) V[t],
//   with K, V of KV head h read through the block table.  It is the verify
//   computation with C rows, at sizes where the matrix cores bound it.
//
// Work decomposition.  One work-group of 4 waves per (sequence, KV head,
// tile of 192 query rows); rows are ordered (token, head of the group), so
// the G heads of one token sit side by side.  Each wave owns 48 rows as three
// 16-row column tiles, with their queries resident in registers; the rest of
// its state fits in 256 VGPRs, so two work-groups share a CU and each SIMD
// has a second wave to issue while one waits (on gfx950 a SIMD's fp32 VALU
// and matrix instructions do not run side by side, so softmax time adds to
// matrix time; within a pair the next column tile's score MFMAs share a
// basic block with the current tile's softmax, so neither waits on the
// other's branch).  The K/V of
// the visible blocks stream through a four-stage LDS ring, two blocks (a
// "pair") per stage, copied straight from the pool into LDS by 16-byte
// buffer loads with the LDS as destination (no register staging; one buffer
// resource per block, loop-invariant lane offsets); each wave issues its
// share of the pair three steps ahead, and one barrier per pair publishes it.
// The block ids are read with scalar loads, a pair ahead of their use.  A
// wave's pairs before the first position one of its rows may not see take a
// step without the mask and tail code.
//
// Matrix cores.  Scores: S^T[token][row] = K[token][:] . Q^T[:][row] with
// v_mfma_f32_16x16x32_bf16 per block (K is the A operand, one 16-byte LDS
// read per lane, as in the decode kernel).  Output: O^T[dim][row] +=
// V^T[dim][32 tokens] . P^T[32 tokens][row] with one v_mfma_f32_16x16x32_bf16
// per 16 dims over the pair, so the contraction runs at the full-rate
// 32-deep instruction; each lane's 8 probabilities come straight from the
// two score tiles.  For bf16 the two score tiles each take half of both
// blocks' tokens, so that a lane group's 8 probabilities are 8 consecutive
// tokens of one block and its V^T operand is one 16-byte read (operand
// order below); for one-byte codes tile 0 is block A and tile 1 block B,
// and a lane group takes tokens 4lg..4lg+3 of each.  fp8 codes are converted to bf16 exactly
// after the LDS read, and so are int8 codes; int4 codes are widened to bf16
// biased by kI4Bias (as in the decode kernel: each lane reads its own run of
// a tile), the bias taken out of the scores (kI4Bias times the query row's
// sum) and of the output (kI4Bias times the row's probability sum).  The K
// scale folds into the score scale, the V scale into the final divide.
//
// Work-group order: groups of 8 (sequence, KV head) pairs x all row tiles,
// the pair fastest; work-groups go to the 8 XCDs round-robin, so each XCD
// serves one pair's row tiles and its L2 holds that pair's K/V for all of
// them.  Row tiles go longest (most visible tokens) first.  Sequences may
// carry chunks of different lengths (query_start): the grid holds the
// longest chunk's row tiles for every sequence, and a work-group whose tile
// lies past its own sequence's chunk returns at once.
#include "pkv_mfma.h"

namespace pkv {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfNT = kPrefillRows / (16 * kPfWaves);   // column tiles per wave (3)
#ifndef PKV_PREFILL_STAGES
#define PKV_PREFILL_STAGES 4
#endif
constexpr int kPfStages = PKV_PREFILL_STAGES;           // LDS ring of block pairs
constexpr int kPfAhead = kPfStages - 1;                 // pairs in flight ahead of the one computed
static_assert(kPfAhead >= 1 && kPfAhead <= 3, "the wait counts cover up to 3 pairs in flight");
constexpr int kPfXcds = 8;
constexpr float kLazyMax = 8.f;                         // exp2 units the running max may lag

template <int KVT, int D> struct PfGeom {
    static constexpr int EB = KVT == KV_BF16 ? 2 : 1;      // bytes per element (int4: 2 codes per byte)
    static constexpr int TILE = KVT == KV_INT4 ? 8 * D : 16 * D * EB;   // one K or V tile
    static constexpr int PAIR = 4 * TILE;                  // K_A, V_A, K_B, V_B
    static constexpr int PIECES = PAIR / 1024;             // 1 KiB wave loads per pair
    // wave loads per wave per pair (int4 at head dim 64: waves 2 and 3 load nothing)
    static constexpr int LOADS = (PIECES + kPfWaves - 1) / kPfWaves;
    static_assert(PIECES >= 1 && (TILE % 1024 == 0 || TILE == 512), "whole 1 KiB pieces per tile pair");
    static constexpr int LDS = kPfStages * PAIR;
};

// s_waitcnt immediate: vector-memory count <= N, no wait on the other counters.
template <int N> constexpr int vmcnt_imm() { return (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14); }

// bf16 operand order over a pair.  The two score tiles of a pair do not
// split it by block: in score tile T (0 or 1), MFMA row t = lane % 16 is
// token 8 ((t & 7) >> 2) + 4T + (t & 3) of block t >> 3.  So lane group g
// (lanes 16g .. 16g+15) of both score outputs holds tokens 8 (g & 1) .. +3
// (tile 0) and +4 .. +7 (tile 1) of block g >> 1: 8 consecutive tokens of
// one block, whose V^T entries are one 16-byte half of a V^T row.  The PV
// operands are then one 16-byte LDS read each and the probabilities stay
// where the score MFMAs leave them.  (One-byte codes keep tile 0 = block A,
// tile 1 = block B, lane group g holding tokens 4g .. 4g+3 of each.)
//
// LDS placement of the bf16 K tiles.  A K tile is 16-byte chunks of 8
// dims, 16 token rows per chunk group (256 bytes).  A score-operand read
// takes, in the lanes t = 0 .. 15 of one lane group, token rows {0..3,
// 8..11} (tile 0) or {4..7, 12..15} (tile 1) of one chunk group of block A
// (t < 8) and the same rows of block B (t >= 8): with both tiles stored as
// in the pool those 16 reads fall on 8 bank groups twice (measured on
// gfx950 with the bank-conflict counter).  Block B's K tile therefore holds
// its token rows o at o ^ 4: LDS chunk c of that tile is the pool's chunk
// c ^ 4, and the 16 reads cover 16 distinct row slots (no conflicts,
// measured).  V tiles, and every tile of one-byte codes, are stored as in
// the pool (their reads do not conflict, measured).
template <int KVT>
__device__ __forceinline__ int pf_k_chunk(int c, int block_b) {
    if constexpr (KVT == KV_BF16) return block_b ? c ^ 4 : c;
    else return c;
}

// Copy one pair (blocks A and B) of this KV head into an LDS stage: this
// wave's share of the 1 KiB pieces, 16 bytes per lane, straight into LDS by
// buffer_load ... lds (the lane's 16 bytes land at LDS offset lane * 16 of
// the piece; K tiles take their chunks in the order pf_k_chunk gives).  A
// piece lies in one block (tiles 0-1 of the pair are block A's K and V, 2-3
// block B's; a piece spans two tiles only when tiles are 512 bytes, int4 at
// head dim 64, and then both are one block's), so each load goes through
// that block's buffer resource with a per-lane offset that is the same for
// every pair: pf_piece_offset, computed once.
template <int KVT, int D>
__device__ __forceinline__ int pf_piece_offset(int k, int wave, int lane) {
    using Gm = PfGeom<KVT, D>;
    const int at = (wave + kPfWaves * k) * 1024 + lane * 16;   // byte of the pair in LDS
    const int tile = at / Gm::TILE;
    const int c = (at - tile * Gm::TILE) / 16;
    return (tile & 1) * Gm::TILE + ((tile & 1) ? c : pf_k_chunk<KVT>(c, tile >> 1)) * 16;
}

template <int KVT, int D>
__device__ __forceinline__ void pf_issue(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, uint8_t* stage,
                                         const int (&voff)[PfGeom<KVT, D>::LOADS], int wave) {
    using Gm = PfGeom<KVT, D>;
#pragma unroll
    for (int k = 0; k < Gm::LOADS; ++k) {
        const int gk = wave + kPfWaves * k;             // 1 KiB piece of the pair's 4 tiles
        if (Gm::PIECES % kPfWaves != 0 && gk >= Gm::PIECES) break;
        const bool in_a = gk * 1024 < 2 * Gm::TILE;
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(in_a ? ra : rb,
                                                 (__attribute__((address_space(3))) void*)(stage + gk * 1024), 16,
                                                 voff[k], 0, 0, 0);
#else
        (void)in_a; (void)ra; (void)rb; (void)stage; (void)voff;
#endif
    }
}

// K operand registers of one block from its LDS tile (same per-lane reads as
// the decode kernel's buffer loads: token lane % 16, 16-byte chunk).
template <int KVT, int D>
__device__ __forceinline__ void pf_k_regs(TileRegs<KVT, D>& t, const uint8_t* tile, int lane) {
    if constexpr (KVT == KV_INT4) {
        // the lane's run of D / 4 nibbles (layout in the library header)
        if constexpr (D == 128) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + lane * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) t.k[j] = w[j];
        } else {
            const u32x2 w = *reinterpret_cast<const u32x2*>(tile + lane * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j) t.k[j] = w[j];
        }
    } else if constexpr (KVT == KV_BF16) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) t.k[s] = *reinterpret_cast<const u32x4*>(tile + lane * 16 + 1024 * s);
    } else {
#pragma unroll
        for (int q = 0; q < D / 64; ++q) t.k[q] = *reinterpret_cast<const u32x4*>(tile + lane * 16 + 1024 * q);
    }
}

// bf16 score operand of tile T of the pair in an LDS stage (operand order
// above): lane (t, lg) reads token row o of block t >> 3, dims 32s + 8lg ..
// +7 for k-step s.
template <int D>
__device__ __forceinline__ void pf_k_regs_bf16(TileRegs<KV_BF16, D>& r, const uint8_t* stage, int T, int lane) {
    using Gm = PfGeom<KV_BF16, D>;
    const int t = lane & 15;
    const int o = 8 * ((t & 7) >> 2) + 4 * T + (t & 3);
    const int b = t >> 3;
    const uint8_t* base = stage + b * 2 * Gm::TILE + (lane >> 4) * 256 + pf_k_chunk<KV_BF16>(o, b) * 16;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) r.k[s] = *reinterpret_cast<const u32x4*>(base + 1024 * s);
}

// Position in the pair of score value i of lane group lg in score tile T.
template <int KVT>
__device__ __forceinline__ int pf_token(int T, int lg, int i) {
    if constexpr (KVT == KV_BF16) return 16 * (lg >> 1) + 8 * (lg & 1) + 4 * T + i;
    else return 16 * T + 4 * lg + i;
}

// V^T operand of dims 16m .. 16m+15 over the pair, this lane's dim 16m +
// lane % 16.  bf16: tokens 8 (lg & 1) .. +7 of block lg >> 1, one 16-byte
// read; one-byte codes: tokens 4lg .. 4lg+3 of block A then of block B, as
// 8 bf16.
template <int KVT, int D>
__device__ __forceinline__ u32x4 pf_v_op(const uint8_t* va, const uint8_t* vb, int m, int col, int lg) {
    if constexpr (KVT == KV_BF16) {
        // half lg & 1 of the row
        const int off = (16 * m + col) * 32 + ((lg & 1) << 4);
        return *reinterpret_cast<const u32x4*>(((lg >> 1) ? vb : va) + off);
    } else {
        const int off = (16 * m + col) * 16 + lg * 4;
        const unsigned x = *reinterpret_cast<const unsigned*>(va + off);
        const unsigned y = *reinterpret_cast<const unsigned*>(vb + off);
        return u32x4{byte2_to_bf16x2<KVT, false>(x), byte2_to_bf16x2<KVT, true>(x), byte2_to_bf16x2<KVT, false>(y),
                     byte2_to_bf16x2<KVT, true>(y)};
    }
}

// int4 V^T operand over a pair.  Lane (col, lg)'s run of a V tile holds,
// in byte 4j + t, token 4lg + t at dims 16 (2j) + col (low nibble) and
// 16 (2j + 1) + col (high nibble) (layout in the library header); its codes,
// biased by 8 (so code + kI4Bias as bf16), split into bytes: ev[b][j] holds
// dim tile 2j, od[b][j] dim tile 2j + 1, tokens 0..3 of block b.
template <int D>
struct PfV4 {
    unsigned ev[2][D / 32], od[2][D / 32];
    __device__ __forceinline__ void load(const uint8_t* va, const uint8_t* vb, int lane) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint8_t* run = (b == 0 ? va : vb) + lane * (D / 8);
            if constexpr (D == 128) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(run);
#pragma unroll
                for (int j = 0; j < 4; ++j) i4_split(w[j], ev[b][j], od[b][j]);
            } else {
                const u32x2 w = *reinterpret_cast<const u32x2*>(run);
#pragma unroll
                for (int j = 0; j < 2; ++j) i4_split(w[j], ev[b][j], od[b][j]);
            }
        }
    }
    // 8 biased bf16: dim 16m + col, tokens 0..3 of A then of B
    __device__ __forceinline__ u32x4 op(int m) const {
        const unsigned a = (m % 2) ? od[0][m / 2] : ev[0][m / 2];
        const unsigned b = (m % 2) ? od[1][m / 2] : ev[1][m / 2];
        return u32x4{i4_pair_same(a, 0), i4_pair_same(a, 1), i4_pair_same(b, 0), i4_pair_same(b, 1)};
    }
};

// Zero, in an LDS stage, the V entries of tokens >= n of both blocks of the
// pair starting at token t0 (bytes past the sequence end, or the second block
// of an odd count, hold no value of this sequence; their probability is 0,
// but 0 times a NaN would not be).  One thread per (block, dim) row of the
// transposed V tiles.
template <int KVT, int D>
__device__ __forceinline__ void pf_zero_v_tail(uint8_t* stage, int t0, int n, int tid) {
    using Gm = PfGeom<KVT, D>;
    for (int r = tid; r < 2 * D; r += 64 * kPfWaves) {
        const int blk = r / D;
        const int dim = r - blk * D;
        const int cut = n - (t0 + 16 * blk);          // tokens of this block below n
        uint8_t* row = stage + (2 * blk + 1) * Gm::TILE + dim * 16 * Gm::EB;
        for (int o = max(cut, 0); o < 16; ++o)
            for (int b = 0; b < Gm::EB; ++b) row[o * Gm::EB + b] = 0;
    }
}

// CASCADE: the shared-prefix pass of a verify or decode call instead of a
// prefill.  Its "chunk" is every query row of the batch (row j of the packed
// [B * k] tokens is row j mod k of sequence j / k), the visible positions are
// one prefix chunk's blocks of the first table row, all of them visible to
// every row, and each row writes its unnormalised partial result (O, m, l) to
// the split-KV slot of that prefix chunk instead of an output.
template <int KVT, int D, bool CASCADE>
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_kernel(PrefillArgs a) {
    using Gm = PfGeom<KVT, D>;
    extern __shared__ __attribute__((aligned(16))) uint8_t pf_smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4;
    const int col = lane & 15;

    // Work-group -> (sequence, KV head, row tile); for the prefix pass
    // (prefix chunk, KV head, row tile).
    const int H = a.num_kv_heads;
    const int RT = a.row_tiles;
    const int pairs_sh = (CASCADE ? a.prefix_chunks : a.num_seqs) * H;
    const int grp = blockIdx.x / (kPfXcds * RT);
    const int r = blockIdx.x - grp * kPfXcds * RT;
    const int in_group = min(kPfXcds, pairs_sh - grp * kPfXcds);
    const int sh = grp * kPfXcds + r % in_group;
    const int rt = RT - 1 - r / in_group;
    const int s = CASCADE ? 0 : sh / H;         // the prefix pass reads the first table row
    const int pc = CASCADE ? sh / H : 0;        // prefix chunk
    const int h = sh - (sh / H) * H;
    const int blk0 = pc * a.prefix_chunk_blocks;   // first block of the prefix chunk

    const int G = a.group;
    int n, q0, C, first;
    if constexpr (CASCADE) {
        n = kBlock * min(a.prefix_blocks - blk0, a.prefix_chunk_blocks);
        q0 = 0;
        C = a.num_seqs * a.chunk;
        first = 0;
    } else {
        n = a.seq_lens[s];
        // The sequence's chunk: C tokens whose queries (and outputs) are rows
        // q0 .. q0 + C - 1 of the packed arrays.
        q0 = a.query_start ? a.query_start[s] : s * a.chunk;
        C = a.query_start ? a.query_start[s + 1] - q0 : a.chunk;
        first = n - C;                          // position of chunk token 0
    }
    const int Rt = C * G;                       // query rows of this (sequence, KV head)
    const int row_wg = rt * kPrefillRows;
    if (row_wg >= Rt) return;                   // a row tile past a shorter chunk (the whole work-group)
    const int last_row = min(Rt, row_wg + kPrefillRows) - 1;
    // blocks the tile's last row sees
    const int nblk = CASCADE ? n / kBlock : (first + last_row / G + kBlock) / kBlock;
    const int npair = (nblk + 1) >> 1;
    const int row_w = row_wg + wave * 16 * kPfNT;
    // fewest positions a row of this wave sees
    const int lim_lo = CASCADE ? n : (row_w < Rt ? first + row_w / G + 1 : 0);

    float sscale = a.score_scale;
    float vscale = 1.f;
    if constexpr (kv_scaled<KVT>()) {
        sscale *= a.k_scale[a.layer * H + h];
        vscale = a.v_scale[a.layer * H + h];
    }
    // Scores are scaled inside the exponent and a row's maximum scaled score
    // comes from its maximum raw score, which needs a positive factor: a
    // negative one moves its sign into the query, a zero one becomes the
    // smallest normal float (scaled scores round to 0 against the offset,
    // masked ones still give -inf).
    const bool qneg = sscale < 0.f;
    sscale = sscale == 0.f ? 1.17549435e-38f : fabsf(sscale);

    QRegs<KVT, D> qr[kPfNT];
    int lim[kPfNT];
#pragma unroll
    for (int c = 0; c < kPfNT; ++c) {
        const int row = row_w + 16 * c + col;
        const bool valid = row < Rt;
        const int j = valid ? row / G : 0;
        const int g = valid ? row - (row / G) * G : 0;
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
            ((static_cast<int64_t>(q0) + j) * a.num_q_heads + h * G + g) * D;
        qr[c].load(qrow, valid, lane);
        if (qneg) qr[c].negate();
        lim[c] = CASCADE ? n : (valid ? first + j + 1 : 0);
    }
    // int4: kI4Bias times each query row's sum (the bias of its scores)
    float qbias[kPfNT], qbs[kPfNT];   // qbs: the bias scaled
#pragma unroll
    for (int c = 0; c < kPfNT; ++c) {
        qbias[c] = KVT == KV_INT4 ? kI4Bias * query_row_sum<D>(qr[c])[0] : 0.f;
        qbs[c] = qbias[c] * sscale;
    }

    // o: unnormalised output per (column tile, 16 dims); ol: the row sums of
    // the bf16 probabilities, accumulated by the matrix cores against a tile
    // of ones (every entry of a column holds that row's sum).
    f32x4 o[kPfNT][D / 16];
    f32x4 ol[kPfNT];
    float m_run[kPfNT];
    float thr[kPfNT];   // raw score above which a column's reference must move
    const float inv_sscale = 1.f / sscale;
#pragma unroll
    for (int c = 0; c < kPfNT; ++c) {
        m_run[c] = neg_inf();
        thr[c] = neg_inf();
        ol[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < D / 16; ++m) o[c][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    const int64_t block_stride = static_cast<int64_t>(H) * 2 * a.tile_bytes;
    const uint8_t* head_base = a.pool + static_cast<int64_t>(a.layer) * a.num_blocks * block_stride +
                               static_cast<int64_t>(h) * 2 * a.tile_bytes;
    const int32_t* trow = a.table + static_cast<int64_t>(s) * a.max_blocks + blk0;

    // Block ids come straight from the table through scalar loads (the row is
    // uniform over the work-group and read-only during the kernel), the ids
    // of the pair after next fetched one iteration before they are needed.
    // Scalar loads leave the vector-memory counter to the LDS copies alone:
    // block ids loaded with vector loads (or staged through LDS) made the
    // compiler wait for every copy in flight before each pair's LDS reads.
    typedef const int32_t __attribute__((address_space(4)))* ConstIds;
    const ConstIds crow = (ConstIds)(trow);
    auto ids_of = [&](int q, int& ia, int& ib) {
        ia = crow[2 * q];
        ib = 2 * q + 1 < nblk ? crow[2 * q + 1] : ia;
    };
    int voff[Gm::LOADS];
#pragma unroll
    for (int k = 0; k < Gm::LOADS; ++k) voff[k] = pf_piece_offset<KVT, D>(k, wave, lane);
    auto block_rsrc = [&](int id) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(head_base) + static_cast<int64_t>(id) * block_stride,
                                                 0, static_cast<int>(2 * Gm::TILE), 0x00020000);
    };
    auto issue = [&](int q, int ia, int ib) {
        pf_issue<KVT, D>(block_rsrc(ia), block_rsrc(ib), pf_smem + (q % kPfStages) * Gm::PAIR, voff, wave);
    };
#pragma unroll
    for (int q = 0; q < kPfAhead; ++q) {
        if (q < npair) {
            int ia, ib;
            ids_of(q, ia, ib);
            issue(q, ia, ib);
        }
    }
    int next_a = 0, next_b = 0;   // ids of pair p + kPfAhead
    if (kPfAhead < npair) ids_of(kPfAhead, next_a, next_b);

    // One pair.  MASKED: the pair may hold positions some row of this wave
    // may not see (causal mask, and positions past the sequence end, whose V
    // entries are zeroed); the pairs before p_split hold none, and their
    // steps carry no mask code.
    auto step = [&](int p, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        // This wave's pieces of pair p have landed (the next pairs may still
        // be in flight); the barrier makes every wave's pieces visible and
        // ensures pair p-1's stage is no longer read.
        const int later = min(kPfAhead - 1, npair - 1 - p);   // pairs issued after p
        if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * Gm::LOADS>());
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm<Gm::LOADS>());
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
        __builtin_amdgcn_s_barrier();
        if (p + kPfAhead < npair) {
            issue(p + kPfAhead, next_a, next_b);
            if (p + kPfAhead + 1 < npair) ids_of(p + kPfAhead + 1, next_a, next_b);
        }

        uint8_t* st = pf_smem + (p % kPfStages) * Gm::PAIR;
        const int t0 = 32 * p;
        if (MASKED && !CASCADE && KVT != KV_INT4 && t0 + 32 > n) {
            // only the last pair reaches past the sequence end; nothing is in
            // flight (every int4 nibble is a finite value: no zeroing needed)
            pf_zero_v_tail<KVT, D>(st, t0, n, tid);
            __syncthreads();
        }
        TileRegs<KVT, D> ka, kb;   // the two score tiles' K operands
        if constexpr (KVT == KV_BF16) {
            pf_k_regs_bf16<D>(ka, st, 0, lane);
            pf_k_regs_bf16<D>(kb, st, 1, lane);
        } else {
            pf_k_regs<KVT, D>(ka, st, lane);
            pf_k_regs<KVT, D>(kb, st + 2 * Gm::TILE, lane);
        }
        // Software pipeline over the wave's column tiles: the score MFMAs of
        // tile c + 1 are issued in the same basic block as tile c's softmax,
        // and the V products of the earlier tiles in the same block as the
        // last tile's, so the matrix cores work while the VALU computes the
        // probabilities.  The probabilities are taken against the current
        // running max before the lazy-max check; the rare case that moves the
        // max computes them again.
        f32x4 sa[kPfNT], sb[kPfNT];
        u32x4 pop[kPfNT];
        u32x4 vop[D / 16];
        auto qk = [&](int c) {
            // raw scores (int4: biased by kI4Bias times the query row's sum,
            // taken out in the exponent's offset and in the maximum)
            sa[c] = scores<D>(ka, qr[c]);
            sb[c] = scores<D>(kb, qr[c]);
        };
        auto probs = [&](int c) {
            // (every score of an unmasked pair is finite, so the max is too)
            const float muse = MASKED && m_run[c] == neg_inf() ? 0.f : m_run[c];
            const float off = -(qbs[c] + muse);
            float pa[4], pb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pa[i] = fast_exp2(__builtin_fmaf(sa[c][i], sscale, off));
                pb[i] = fast_exp2(__builtin_fmaf(sb[c][i], sscale, off));
            }
            pop[c] = u32x4{pack_bf16x2(pa[0], pa[1]), pack_bf16x2(pa[2], pa[3]), pack_bf16x2(pb[0], pb[1]),
                           pack_bf16x2(pb[2], pb[3])};
        };
        auto pv = [&](int c) {
            ol[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, pop[c]), ol[c], 0, 0, 0);
#pragma unroll
            for (int m = 0; m < D / 16; ++m)
                o[c][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[m]),
                                                                  __builtin_bit_cast(bf16x8, pop[c]), o[c][m], 0, 0, 0);
        };
        qk(0);
#pragma unroll
        for (int c = 0; c < kPfNT; ++c) {
            if (c + 1 < kPfNT) {
                qk(c + 1);
            } else {
                // V^T operands of the pair (the K operands are dead by now),
                // then the products of every earlier tile
                const uint8_t* va = st + Gm::TILE;
                const uint8_t* vb = st + 3 * Gm::TILE;
                PfV4<D> v4;
                if constexpr (KVT == KV_INT4) v4.load(va, vb, lane);
#pragma unroll
                for (int m = 0; m < D / 16; ++m) {
                    if constexpr (KVT == KV_INT4) vop[m] = v4.op(m);
                    else vop[m] = pf_v_op<KVT, D>(va, vb, m, col, lg);
                }
#pragma unroll
                for (int e = 0; e < kPfNT - 1; ++e) pv(e);
            }
            if constexpr (MASKED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (t0 + pf_token<KVT>(0, lg, i) >= lim[c]) sa[c][i] = neg_inf();
                    if (t0 + pf_token<KVT>(1, lg, i) >= lim[c]) sb[c][i] = neg_inf();
                }
            }
            // (grouped in threes: four three-input maxima)
            const float m1 = smax(smax(sa[c][0], sa[c][1]), sa[c][2]);
            const float m2 = smax(smax(sa[c][3], sb[c][0]), sb[c][1]);
            const float ml = smax(smax(smax(sb[c][2], sb[c][3]), m1), m2);
            probs(c);
            // Running max in exp2 units, kept stale: it moves (and the
            // accumulators are rescaled) only when a score exceeds it by more
            // than kLazyMax, so probabilities stay <= 2^kLazyMax.  O and its
            // row sum share the same max, so O / sum is unchanged.  Each lane
            // compares its own 8 raw scores with the column's threshold
            // (the reference plus kLazyMax, in raw units); only when some
            // lane exceeds it does the wave reduce the columns' maxima across
            // lanes and move the reference.
            if (__ballot(ml > thr[c])) {
                const float mx = (max_over_rows(ml) - qbias[c]) * sscale;
                if (mx > m_run[c] + kLazyMax) {
                    const float alpha = fast_exp2(m_run[c] - mx);
                    m_run[c] = mx;
                    ol[c] *= alpha;
#pragma unroll
                    for (int m = 0; m < D / 16; ++m) o[c][m] *= alpha;
                }
                thr[c] = m_run[c] == neg_inf() ? neg_inf() : (m_run[c] + kLazyMax) * inv_sscale + qbias[c];
                probs(c);
            }
        }
        pv(kPfNT - 1);
    };
    // Pair p needs the mask iff 32 p + 32 > lim_lo; the waves' splits differ,
    // their barrier counts (one per pair) do not.
    const int p_split = min(npair, lim_lo >= 32 ? (lim_lo - 32) / 32 + 1 : 0);
    for (int p = 0; p < p_split; ++p) step(p, std::false_type{});
    for (int p = p_split; p < npair; ++p) step(p, std::true_type{});

    // Normalise and store: lane holds dims 16m + 4lg .. +3 of row 16c + col.
#pragma unroll
    for (int c = 0; c < kPfNT; ++c) {
        const float l = ol[c][0];
        if constexpr (KVT == KV_INT4) {
            // int4: the output came out biased by kI4Bias times the row's probability sum
#pragma unroll
            for (int m = 0; m < D / 16; ++m) o[c][m] -= kI4Bias * l;
        }
        const int row = row_w + 16 * c + col;
        if (row >= Rt) continue;
        const int j = row / G;
        const int g = row - j * G;
        if constexpr (CASCADE) {
            // partial of row jr * G + g of sequence sq, in the prefix chunk's slot
            const int sq = j / a.chunk;
            const int R = a.chunk * G;
            const int rr = (j - sq * a.chunk) * G + g;
            const int64_t sl = static_cast<int64_t>(h) * a.num_split_slots + a.seq_parts[2 * sq + 1] + pc;
            float* po = a.part_o + (sl * R + rr) * D + 4 * lg;
#pragma unroll
            for (int m = 0; m < D / 16; ++m) *reinterpret_cast<f32x4*>(po + 16 * m) = o[c][m];
            if (lg == 0) {
                a.part_m[sl * R + rr] = m_run[c];
                a.part_l[sl * R + rr] = l;
            }
            continue;
        }
        const float inv = vscale / l;
        const int64_t base = ((static_cast<int64_t>(q0) + j) * a.num_q_heads + h * G + g) * D + 4 * lg;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
            const f32x4 v = o[c][m] * inv;
            if (a.out_bf16) {
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + base + 16 * m) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + base + 16 * m) = v;
            }
        }
    }
}

template <int KVT, int D>
hipError_t launch_pf(const PrefillArgs& a, hipStream_t stream) {
    constexpr size_t lds = PfGeom<KVT, D>::LDS;
    if (a.part_o) {
        const int grid = a.prefix_chunks * a.num_kv_heads * a.row_tiles;
        hipLaunchKernelGGL((attn_prefill_kernel<KVT, D, true>), dim3(grid), dim3(64 * kPfWaves), lds, stream, a);
    } else {
        const int grid = a.num_seqs * a.num_kv_heads * a.row_tiles;
        hipLaunchKernelGGL((attn_prefill_kernel<KVT, D, false>), dim3(grid), dim3(64 * kPfWaves), lds, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, hipStream_t stream) {
    if (kv_dtype == KV_BF16) return head_dim == 128 ? launch_pf<KV_BF16, 128>(a, stream) : launch_pf<KV_BF16, 64>(a, stream);
    if (kv_dtype == KV_INT8) return head_dim == 128 ? launch_pf<KV_INT8, 128>(a, stream) : launch_pf<KV_INT8, 64>(a, stream);
    if (kv_dtype == KV_INT4) return head_dim == 128 ? launch_pf<KV_INT4, 128>(a, stream) : launch_pf<KV_INT4, 64>(a, stream);
    return head_dim == 128 ? launch_pf<KV_FP8, 128>(a, stream) : launch_pf<KV_FP8, 64>(a, stream);
}

}  // namespace pkv
