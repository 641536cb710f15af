// Internal declarations shared by the host API (api.cpp) and the HIP kernel
// files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;       // tokens per physical block
constexpr int kMaxRows = 64;     // query rows per KV head handled by one work-group

// Work-unit descriptor: one (sequence, partition), int32 fields.
constexpr int kUnitSeq = 0;      // sequence index
constexpr int kUnitB0 = 1;       // first logical block of the partition
constexpr int kUnitNb = 2;       // blocks in the partition
constexpr int kUnitLen = 3;      // sequence length (positions visible to its last row)
constexpr int kUnitPart = 4;     // partition index within the sequence
constexpr int kUnitParts = 5;    // partitions of the sequence
constexpr int kUnitSlot = 6;     // partial-result slot (split sequences) or -1
constexpr int kUnitRot = 7;      // walking-order rotation, seq mod nb
constexpr int kUnitTickets = 8;  // work-groups of the sequence (per KV head) that take a merge ticket
constexpr int kUnitInts = 9;

// Shared-prefix ("cascade") plan: when every sequence of a batch starts with
// the same kCascadeMinBlocks or more physical blocks, the prefix is attended
// once for all sequences' query rows (a dense pass over the shared blocks,
// cut into prefix chunks of at least kCascadeChunkBlocks blocks, each writing
// a partial result per row) and the decode kernel walks only each
// sequence's own blocks, merging the prefix partials with its own.
constexpr int kCascadeMinBlocks = 8;
constexpr int kCascadeMinSeqs = 4;
constexpr int kCascadeChunkBlocks = 32;
constexpr int kCascadeMaxChunks = 4;

// Sequences with at most this many partitions are merged inside the
// partition kernel; longer ones by the separate merge kernel.
constexpr int kFuseMaxParts = 32;

// Balanced plan: units sized so the batch gives up to kAutoItemsPerWg
// (unit, KV head) items per resident work-group (decode_wgs_per_cu() per CU), as
// many as keep units at kAutoMinItemBlocks blocks or more, with units of
// kAutoMinBlocks .. kAutoMaxBlocks blocks.  The attention kernel's
// work-groups take items from a queue, so work-groups that drain early (the
// memory system does not serve CUs and XCDs evenly) take more of them.
#ifndef PKV_AUTO_ITEMS_PER_WG
#define PKV_AUTO_ITEMS_PER_WG 3
#endif
#ifndef PKV_AUTO_MIN_ITEM_BLOCKS
#define PKV_AUTO_MIN_ITEM_BLOCKS 96
#endif
// Decode-kernel instances with one row tile (R <= 16), per KV dtype (PKV_*
// code) and head dim: the prefetch depth (tiles a wave has in flight while it
// processes one) and the waves per SIMD it is built for, which is also its
// resident work-groups per CU (a work-group is one wave on each SIMD).  At
// d = 128 a deeper pipeline with two waves per SIMD streams faster than three
// waves with one tile in flight each; int4 (2 KiB per block and KV head, the
// most widening work per byte) runs three waves per SIMD with the deeper
// pipeline too (measured on the Llama-3-8B decode batch: 39.2 -> 35.5 us).
constexpr int decode_depth(int kv, int d) { return kv != 0 && d == 128 ? 2 : 1; }
// Tile buffers a wave of the decode kernel rotates through (NBUF - 1 blocks
// in flight while one is processed): 1 + decode_depth for one row tile,
// overridable per element size for measurements; 2 for more row tiles.
#ifndef PKV_BUFS_1B
#define PKV_BUFS_1B 3
#endif
#ifndef PKV_BUFS_I4
#define PKV_BUFS_I4 3
#endif
#ifndef PKV_BUFS_NT2
#define PKV_BUFS_NT2 2
#endif
constexpr int decode_buffers(int kv, int d, int nt) {
    return nt == 2 && kv >= 2 ? PKV_BUFS_NT2
         : nt != 1 ? 2
         : decode_depth(kv, d) == 1 ? 2
         : kv == 4 ? PKV_BUFS_I4
         : (kv == 2 || kv == 3) ? PKV_BUFS_1B : 3;
}
constexpr int decode_wgs_per_cu(int kv, int d) { return kv == 0 ? 1 : (d == 128 ? (kv == 4 ? 3 : 2) : 3); }
// Work-groups per CU the balanced plan sizes its units for.  The int4
// instance runs three per CU to hide latency, but cutting sequences to give
// that third work-group an item costs more (partials and merges) than it
// balances: on the Llama-3-8B decode batch, whole sequences (64 units) ran
// 31.4-32.1 us against 33.4-34.5 us for 96 units, four runs each.
constexpr int plan_wgs_per_cu(int kv, int d) { return kv == 4 && d == 128 ? 2 : decode_wgs_per_cu(kv, d); }
constexpr int kAutoItemsPerWg = PKV_AUTO_ITEMS_PER_WG;
constexpr int kAutoMinItemBlocks = PKV_AUTO_MIN_ITEM_BLOCKS;
constexpr int kAutoMinBlocks = 8;
constexpr int kAutoMaxBlocks = 256;

// Item i -> (unit, KV head).  Items come in groups of kXcds units x H_kv heads
// (the last group may hold fewer units); within a group the unit is the
// fastest index.  Work-groups are handed to the XCDs round-robin by index, so
// in the first round every head of a unit runs on the same XCD, which then
// reads the unit's blocks whole (all heads of a block are adjacent) and
// touches fewer pages.
constexpr int kXcds = 8;
__host__ __device__ inline void item_coords(int item, int num_units, int hkv, int& unit, int& h) {
    const int group = item / (kXcds * hkv);
    const int r = item - group * kXcds * hkv;
    const int in_group = num_units - group * kXcds < kXcds ? num_units - group * kXcds : kXcds;
    h = r / in_group;
    unit = group * kXcds + (r - h * in_group);
}

// The inverse: the item of (unit, KV head).
__host__ __device__ inline int item_of(int unit, int h, int num_units, int hkv) {
    const int group = unit / kXcds;
    const int in_group = num_units - group * kXcds < kXcds ? num_units - group * kXcds : kXcds;
    return group * kXcds * hkv + h * in_group + (unit - group * kXcds);
}

// Everything the attention kernel reads; built by the host per call.
struct AttnArgs {
    const uint8_t* pool;         // pool base
    const float* k_scale;        // [L][H_kv] (fp8 pools) or null
    const float* v_scale;
    const int32_t* units;        // [U][kUnitInts] work-unit descriptors
    const int32_t* unit_ids;     // [U][unit_stride] physical block ids in walking order
    const int32_t* seq_parts;    // [B][2] = (partitions, first partial slot or -1)
    int32_t* counters;           // [B][H_kv] arrival tickets of the in-kernel merge (zero between calls)
    int32_t* queue;              // [2] items taken beyond the grid, work-groups finished (zero between calls)
    const void* q;               // [B][k][H_q][D]
    void* out;                   // [B][k][H_q][D]
    const void* k_new;           // fused append: [B][k][H_kv][D] K of positions n-k .. n-1, or null
    const void* v_new;           // and V
    float* part_o;               // [H_kv][slots][R][D]
    float* part_m;               // [H_kv][slots][R]
    float* part_l;               // [H_kv][slots][R]
    int64_t tile_bytes;          // 16 * D * elem_bytes
    int32_t layer;
    int32_t num_blocks;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t head_dim;
    int32_t group;               // G = H_q / H_kv
    int32_t rows;                // R = G * k, query rows per KV head
    int32_t k_rows;              // k
    int32_t unit_stride;
    int32_t num_items;           // units * H_kv; item i is unit i / H_kv, KV head i % H_kv
    int32_t num_split_slots;
    int32_t max_parts;
    int32_t fuse_max_parts;
    int32_t out_bf16;            // 1: bf16 output, 0: f32 output
    int32_t append_in_f32;       // fused append input: 1 float32, 0 bfloat16
    float score_scale;           // softmax scale * log2(e)
};

// Size of the per-device static scratch array that holds the split-KV
// partial results of paged_attention_verify_noalloc.
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(64) << 20;

// Device address of this device's scratch array (looked up once per device,
// on the first call with that device current) and its size.
hipError_t attention_scratch(void** ptr, size_t* bytes);

// Launch the attention kernels (partition pass, then the split-KV merge when
// some sequence is split).  kv_dtype / head_dim / rows select the instance;
// shared_blocks (some physical block is named by more than one sequence of
// the batch) selects cached instead of streaming tile loads.
hipError_t launch_attention(const AttnArgs& a, int kv_dtype, int head_dim, int num_units, bool shared_blocks,
                            hipStream_t stream);

// Chunked-prefill attention: every sequence carries `chunk` query tokens at
// positions n-chunk .. n-1 (their K/V already in the pool); row (j, g) sees
// positions t <= n - chunk + j.  One work-group per (sequence, KV head, tile
// of kPrefillRows query rows).
constexpr int kPrefillRows = 192;

struct PrefillArgs {
    const uint8_t* pool;
    const float* k_scale;        // [L][H_kv] (fp8 pools) or null
    const float* v_scale;
    const int32_t* table;        // [B][max_blocks] block table (validated at upload)
    const int32_t* seq_lens;     // [B]
    const void* q;               // [total chunk tokens][H_q][D] bfloat16, sequences in order
    void* out;                   // [total chunk tokens][H_q][D]
    const int32_t* query_start;  // [B + 1] first packed row of each sequence's chunk, or null: s * chunk
    int64_t tile_bytes;
    int32_t layer;
    int32_t num_blocks;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t group;               // G = H_q / H_kv
    int32_t chunk;               // query tokens per sequence (without query_start)
    int32_t max_blocks;          // table row stride
    int32_t row_tiles;           // ceil(longest chunk * G / kPrefillRows)
    int32_t out_bf16;
    float score_scale;           // softmax scale * log2(e)
    // Shared-prefix pass of a verify or decode call (part_o non-null): the
    // k = chunk query rows of every sequence ([B][k][H_q][D] in q) attend to
    // prefix chunk c, blocks c * prefix_chunk_blocks .. (at most
    // prefix_blocks) of the first table row, all positions visible; each row
    // writes its partial (O, m, l) to slot seq_parts[2 s + 1] + c, laid out
    // as the attention kernel's partials.
    float* part_o = nullptr;     // [H_kv][slots][R][D]
    float* part_m = nullptr;     // [H_kv][slots][R]
    float* part_l = nullptr;
    const int32_t* seq_parts = nullptr;
    int32_t num_split_slots = 0;
    int32_t prefix_blocks = 0;
    int32_t prefix_chunk_blocks = 0;
    int32_t prefix_chunks = 0;
};

// Launch the prefill kernel (or, with part_o set, the shared-prefix pass);
// kv_dtype is any pool code but KV_F32, head_dim 64 or 128.
hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, hipStream_t stream);

// Exact speculative acceptance (see speculative.hip).
struct SpecArgs {
    const float* p;              // [B][K+1][V] target probabilities
    const float* q;              // [B][K][V] draft probabilities
    const int32_t* draft;        // [B][K] drafted tokens
    const float* u_accept;       // [B][K] uniforms of the acceptance tests
    const float* u_sample;       // [B] uniform of the emitted draw
    int32_t* num_accepted;       // [B] out
    int32_t* tokens;             // [B][K+1] out: accepted drafts, the draw, then -1
    int64_t seg_len;             // weights per wave segment (speculative_segment_len)
    int32_t num_seqs;
    int32_t k;
    int32_t vocab;
};

hipError_t launch_speculative_accept(const SpecArgs& a, hipStream_t stream);
int64_t speculative_segment_len(int64_t vocab);

struct CacheArgs {
    uint8_t* pool;
    const float* k_scale;
    const float* v_scale;
    const void* k_new;           // [T][H_kv][D]
    const void* v_new;
    const int64_t* slots;        // [T]
    int64_t tile_bytes;
    int64_t num_slots;           // num_blocks * 16
    int32_t layer;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t num_tokens;
};

hipError_t launch_reshape_and_cache(const CacheArgs& a, int kv_dtype, int in_dtype,
                                    hipStream_t stream);

struct SlotArgs {
    const int32_t* block_table;
    const int32_t* seq_ids;
    const int32_t* positions;
    int64_t* slots;
    int32_t num_seqs;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t num_tokens;
};

hipError_t launch_slot_mapping(const SlotArgs& a, hipStream_t stream);

// Whole-block copies for copy-on-write: every layer of block src -> block dst.
struct CopyArgs {
    uint8_t* pool;
    const int32_t* pairs;        // [n][2] (src, dst)
    int64_t block_bytes;         // H_kv * 2 * tile bytes: one block of one layer
    int32_t num_pairs;
    int32_t num_blocks;
    int32_t num_layers;
};

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

}  // namespace pkv
