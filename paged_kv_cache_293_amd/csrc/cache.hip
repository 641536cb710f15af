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
#include "pkv_internal.h"

namespace pkv {
namespace {

enum { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// E4M3 code of x * inv: the product is one float32 multiply (round to nearest
// even), saturated to +-448 by comparisons that let NaN through, then
// converted with round-to-nearest-even by the hardware converter.
__device__ __forceinline__ unsigned quantize_e4m3(float x, float inv) {
    float y = __fmul_rn(x, inv);
    y = (y > 448.f) ? 448.f : y;
    y = (y < -448.f) ? -448.f : y;
    return static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false)) & 0xffu;
}

template <int IN>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
    if constexpr (IN == KV_F32) return reinterpret_cast<const float*>(p)[i];
    else return __uint_as_float(static_cast<unsigned>(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

template <int KVT, int IN, int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheArgs a) {
    const int t = blockIdx.x;
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_slots) return;
    const int64_t blk = slot / kBlock;
    const int off = static_cast<int>(slot % kBlock);
    const int H = a.num_kv_heads;
    constexpr int EB = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);
    constexpr int X = 16 / EB;                 // elements per 16-byte K chunk
    constexpr int CH = D / X;                  // K chunks per head
    uint8_t* bbase = a.pool + (static_cast<int64_t>(a.layer) * a.num_blocks + blk) * H * 2 * a.tile_bytes;
    const int64_t in_row = static_cast<int64_t>(t) * H * D;

    // K: one 16-byte chunk per thread-iteration.
    for (int ch = threadIdx.x; ch < H * CH; ch += blockDim.x) {
        const int h = ch / CH;
        const int c = ch % CH;
        uint8_t* dst = bbase + static_cast<int64_t>(h) * 2 * a.tile_bytes + (c * kBlock + off) * 16;
        const int64_t src = in_row + static_cast<int64_t>(h) * D + c * X;
        if constexpr (KVT == KV_FP8) {
            const float inv = 1.0f / a.k_scale[a.layer * H + h];
            unsigned w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned b = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) b |= quantize_e4m3(load_in<IN>(a.k_new, src + 4 * q + e), inv) << (8 * e);
                w[q] = b;
            }
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        } else {
            const uint8_t* s = reinterpret_cast<const uint8_t*>(a.k_new) + src * EB;
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(s);
        }
    }
    // V: transposed tile, one element per thread-iteration.
    for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
        const int h = e / D;
        const int i = e % D;
        uint8_t* dst = bbase + (static_cast<int64_t>(h) * 2 + 1) * a.tile_bytes + (i * kBlock + off) * EB;
        const int64_t src = in_row + e;
        if constexpr (KVT == KV_FP8) {
            const float inv = 1.0f / a.v_scale[a.layer * H + h];
            *dst = static_cast<uint8_t>(quantize_e4m3(load_in<IN>(a.v_new, src), inv));
        } else if constexpr (KVT == KV_BF16) {
            *reinterpret_cast<uint16_t*>(dst) = reinterpret_cast<const uint16_t*>(a.v_new)[src];
        } else {
            *reinterpret_cast<float*>(dst) = reinterpret_cast<const float*>(a.v_new)[src];
        }
    }
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
    if (in_dtype == KV_F32) return launch_cache_dim<KV_FP8, KV_F32>(a, stream);
    return launch_cache_dim<KV_FP8, KV_BF16>(a, stream);
}

hipError_t launch_slot_mapping(const SlotArgs& a, hipStream_t stream) {
    if (a.num_tokens <= 0) return hipSuccess;
    hipLaunchKernelGGL(slot_mapping_kernel, dim3((a.num_tokens + 255) / 256), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
