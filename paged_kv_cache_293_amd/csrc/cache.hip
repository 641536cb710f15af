// Slot mapping and the cache append (reshape_and_cache) for gfx950.
//
// Page "KV cache & continuous batching", section "2. PagedAttention (vLLM)":
// position t of a request lives in the physical block its block table names
// for logical block t / 16, at offset t % 16.  Section "The core insight": a
// decode step appends the new token's K and V to the cache.  Page "LLM
// Inference Optimization: KV Cache, Batching, and Speculative Decoding",
// section "Memory Bandwidth Optimization": the cache may hold one byte per
// element (here fp8 E4M3 with a float32 scale per layer and KV head).
//
// One work-group per appended token writes that token's K and V for every KV
// head: K as 16-byte chunks into the chunk-major K tiles, V element by element
// into the transposed V tiles (element (o, i) at i * 16 + o).
#include "pkv_device.h"

namespace pkv {
namespace {

template <int KVT, int IN, int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheArgs a) {
    const int t = blockIdx.x;
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_slots) return;
    const int64_t blk = slot / kBlock;
    const int off = static_cast<int>(slot % kBlock);
    const int H = a.num_kv_heads;
    constexpr int EB = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);
    constexpr int IB = IN == KV_F32 ? 4 : 2;
    uint8_t* bbase = a.pool + (static_cast<int64_t>(a.layer) * a.num_blocks + blk) * H * 2 * a.tile_bytes;
    const int64_t row = static_cast<int64_t>(t) * H * D * (kv_scaled<KVT>() ? IB : EB);
    const float* ks = kv_scaled<KVT>() ? a.k_scale + a.layer * H : nullptr;
    const float* vs = kv_scaled<KVT>() ? a.v_scale + a.layer * H : nullptr;
    write_token<KVT, IN, D>(bbase, a.tile_bytes, off, reinterpret_cast<const uint8_t*>(a.k_new) + row,
                            reinterpret_cast<const uint8_t*>(a.v_new) + row, 0, H, ks, vs,
                            threadIdx.x, blockDim.x);
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(SlotArgs a) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.num_tokens) return;
    const int s = a.seq_ids[t];
    const int pos = a.positions[t];
    int64_t slot = -1;
    if (s >= 0 && s < a.num_seqs && pos >= 0 && pos < a.max_blocks * kBlock) {
        const int id = a.block_table[static_cast<int64_t>(s) * a.max_blocks + pos / kBlock];
        if (id >= 0 && id < a.num_blocks) slot = static_cast<int64_t>(id) * kBlock + pos % kBlock;
    }
    a.slots[t] = slot;
}

// Copy one block of one layer (all KV heads, K and V tiles: one contiguous run
// of block_bytes) for the pair blockIdx.x, layer blockIdx.y.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
    const int src = a.pairs[2 * blockIdx.x];
    const int dst = a.pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) return;
    const int64_t layer_base = static_cast<int64_t>(blockIdx.y) * a.num_blocks * a.block_bytes;
    const uint4* s = reinterpret_cast<const uint4*>(a.pool + layer_base + src * a.block_bytes);
    uint4* d = reinterpret_cast<uint4*>(a.pool + layer_base + dst * a.block_bytes);
    for (int64_t i = threadIdx.x; i < a.block_bytes / 16; i += blockDim.x) d[i] = s[i];
}

template <int KVT, int IN>
hipError_t launch_cache_dim(const CacheArgs& a, hipStream_t stream) {
    if (a.head_dim == 128)
        hipLaunchKernelGGL((reshape_and_cache_kernel<KVT, IN, 128>), dim3(a.num_tokens), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((reshape_and_cache_kernel<KVT, IN, 64>), dim3(a.num_tokens), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheArgs& a, int kv_dtype, int in_dtype, hipStream_t stream) {
    if (a.num_tokens <= 0) return hipSuccess;
    if (kv_dtype == KV_F32) return launch_cache_dim<KV_F32, KV_F32>(a, stream);
    if (kv_dtype == KV_BF16) return launch_cache_dim<KV_BF16, KV_BF16>(a, stream);
    if (kv_dtype == KV_INT8)
        return in_dtype == KV_F32 ? launch_cache_dim<KV_INT8, KV_F32>(a, stream)
                                  : launch_cache_dim<KV_INT8, KV_BF16>(a, stream);
    if (kv_dtype == KV_INT4)
        return in_dtype == KV_F32 ? launch_cache_dim<KV_INT4, KV_F32>(a, stream)
                                  : launch_cache_dim<KV_INT4, KV_BF16>(a, stream);
    if (in_dtype == KV_F32) return launch_cache_dim<KV_FP8, KV_F32>(a, stream);
    return launch_cache_dim<KV_FP8, KV_BF16>(a, stream);
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
    if (a.num_pairs <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, a.num_layers), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_slot_mapping(const SlotArgs& a, hipStream_t stream) {
    if (a.num_tokens <= 0) return hipSuccess;
    hipLaunchKernelGGL(slot_mapping_kernel, dim3((a.num_tokens + 255) / 256), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
