// Internal declarations shared by the host API (api.cpp) and the HIP kernel
// files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;       // tokens per physical block
constexpr int kMaxRows = 64;     // query rows per KV head handled by one work-group

// Everything the attention kernel reads; built by the host per call.
struct AttnArgs {
    const uint8_t* pool;         // pool base
    const float* k_scale;        // [L][H_kv] (fp8 pools) or null
    const float* v_scale;
    const int32_t* block_table;  // [B][max_blocks]
    const int32_t* seq_lens;     // [B]
    const int32_t* units;        // [U][2] = (sequence, partition)
    const int32_t* split_base;   // [B] first partial slot of a split sequence, -1 otherwise
    const void* q;               // [B][k][H_q][D]
    void* out;                   // [B][k][H_q][D]
    float* part_o;               // [H_kv][slots][R][D]
    float* part_m;               // [H_kv][slots][R]
    float* part_l;               // [H_kv][slots][R]
    int64_t tile_bytes;          // 16 * D * elem_bytes
    int32_t layer;
    int32_t num_blocks;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t group;               // G = H_q / H_kv
    int32_t rows;                // R = G * k, query rows per KV head
    int32_t k_rows;              // k
    int32_t max_blocks;          // table row width
    int32_t part_blocks;         // blocks per partition
    int32_t num_split_slots;
    int32_t out_bf16;            // 1: bf16 output, 0: f32 output
    float score_scale;           // softmax scale * log2(e)
};

// Launch the attention kernels (partition pass, then the split-KV merge when
// some sequence is split).  kv_dtype / head_dim / rows select the instance.
hipError_t launch_attention(const AttnArgs& a, int kv_dtype, int head_dim, int num_units,
                            hipStream_t stream);

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

}  // namespace pkv
