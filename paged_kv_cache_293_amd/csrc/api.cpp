// Host side of the C ABI declared in include/pagedkv.h: argument validation,
// the pool and block-table handles, the split-KV plan and kernel launches.
// Nothing here allocates device memory; every device buffer is the caller's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

struct pkv_pool {
    pkv_pool_desc desc;
    uint8_t* base;
    size_t bytes;
    const float* k_scale;
    const float* v_scale;
    int64_t tile_bytes;
};

struct pkv_table {
    int32_t num_seqs;
    int32_t max_blocks;
    int32_t num_kv_heads;
    int32_t partition_tokens;
    int32_t num_units;
    int32_t unit_stride;
    int32_t num_split_slots;
    int32_t max_parts;
    int32_t max_seq_len;
    int32_t min_seq_len;
    int32_t max_block_id;
    int32_t pool_blocks;            // block count of the pool validated against
    int32_t* d_table;
    int32_t* d_seq_lens;
    int32_t* d_seq_parts;
    int32_t* d_counters;
    int32_t* d_queue;
    int32_t* d_units;
    int32_t* d_unit_ids;
    std::vector<int32_t> staging;   // source of the asynchronous upload (host image of the buffer)
    size_t seq_lens_offset = 0;     // byte offset of the lengths in that image
    hipEvent_t uploaded;
    // Set when an attention launch on this table returned an error: the
    // launch may have left merge tickets or queue counters non-zero, so the
    // table is refused until uploaded again.
    bool stale = false;
    bool shared_blocks = false;     // some physical block is named by two sequences
    // Shared-prefix plan (prefix_blocks > 0): every sequence starts with the
    // same prefix_blocks physical blocks; its units cover each sequence's
    // own blocks whole, and each sequence has prefix_chunks leading partials.
    int32_t prefix_blocks = 0;
    int32_t prefix_chunks = 0;
    int32_t prefix_chunk_blocks = 0;   // blocks per prefix chunk (the last one may hold fewer)
    int32_t c_num_units = 0;
    int32_t c_unit_stride = 0;
    int32_t c_num_split_slots = 0;
    int32_t c_max_parts = 0;
    bool c_shared_blocks = false;   // blocks shared among the sequences' own blocks
    int32_t* d_cseq_parts = nullptr;
    int32_t* d_cunits = nullptr;
    int32_t* d_cunit_ids = nullptr;
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bits per stored element (0: not a pool element type).
int elem_bits(int32_t dtype) {
    switch (dtype) {
        case PKV_F32: return 32;
        case PKV_BF16: return 16;
        case PKV_FP8_E4M3: return 8;
        case PKV_INT8: return 8;
        case PKV_INT4: return 4;
        default: return 0;
    }
}

// Element types stored as codes with a float32 scale per (layer, KV head).
bool scaled_dtype(int32_t dtype) { return dtype == PKV_FP8_E4M3 || dtype == PKV_INT8 || dtype == PKV_INT4; }

pkv_status check_desc(const pkv_pool_desc* d) {
    if (!d) return PKV_ERR_INVALID;
    if (d->num_layers < 1 || d->num_blocks < 1 || d->num_kv_heads < 1) return PKV_ERR_INVALID;
    if (d->block_size != PKV_BLOCK_SIZE) return PKV_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (elem_bits(d->kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

// Split-KV plan of one batch.  A work unit is one (sequence, partition); the
// attention kernel runs one work-group per (unit, KV head).
struct Plan {
    int32_t num_units = 0;
    int32_t stride = 0;          // block ids stored per unit
    int32_t num_split_slots = 0; // partial-result slots (sequences with > 1 part)
    int32_t max_parts = 0;
    std::vector<int32_t> units;  // [U][kUnitInts]
    std::vector<int32_t> seq_parts;  // [B][2] = (parts, first slot or -1)
};

// Device sub-buffers of an uploaded table, in this order, each 256-byte aligned.
struct TableLayout {
    size_t table, seq_lens, seq_parts, counters, queue, units, unit_ids;
    size_t cseq_parts, cunits, cunit_ids;   // shared-prefix plan (empty without one)
    size_t total;
};

int device_cu_count() {
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cached = n;
        else
            cached = 256;
    }
    return cached;
}

// Blocks per unit for the balanced plan: the smallest unit size whose plan has
// at most wgs_per_cu work-groups per CU over all KV heads (plan_wgs_per_cu),
// kept within
// [kAutoMinBlocks, kAutoMaxBlocks].
int32_t auto_unit_blocks(const std::vector<int32_t>& nblk, int32_t num_kv_heads, int32_t wgs_per_cu) {
    const int64_t slots = static_cast<int64_t>(device_cu_count()) * wgs_per_cu;
    int64_t total = 0;
    for (int32_t b : nblk) total += b;
    total *= std::max(1, num_kv_heads);
    // Items per work-group: as many as keep a unit at kAutoMinItemBlocks or more
    // (a work-group's fixed cost per item is amortised over its blocks), at
    // most kAutoItemsPerWg.
    const int64_t per_slot = total / std::max<int64_t>(1, slots);
    const int64_t items = std::max<int64_t>(1, std::min<int64_t>(pkv::kAutoItemsPerWg, per_slot / pkv::kAutoMinItemBlocks));
    const int64_t target_units = std::max<int64_t>(1, slots * items / std::max(1, num_kv_heads));
    int32_t lo = pkv::kAutoMinBlocks, hi = pkv::kAutoMinBlocks;
    for (int32_t b : nblk) hi = std::max(hi, b);
    auto units_for = [&](int32_t T) {
        int64_t u = 0;
        for (int32_t b : nblk) u += (b + T - 1) / T;
        return u;
    };
    if (units_for(lo) <= target_units) return lo;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        if (units_for(mid) <= target_units) hi = mid; else lo = mid + 1;
    }
    return std::min(hi, pkv::kAutoMaxBlocks);
}

// Unit order for a grid with one work-group per item.  Every work-group is
// then resident from the start, and (measured on MI355X) work-groups w and
// w + C, C the number of CUs, run on the same CU; a CU streams its
// work-groups' blocks at about the same rate whatever their split, so the
// kernel ends when the CU with the most blocks is done.  Units (given longest
// first, sizes from nb(i)) are placed one by one, longest first, at the free
// position whose items' CUs would carry the smallest maximum load: the
// greedy longest-processing-time rule over CUs.  Returns order[position] =
// unit; the identity when the items exceed the resident work-groups (the
// work-groups then take items from the queue, longest first).
template <class NB>
std::vector<int32_t> place_on_cus(size_t num_units, int32_t num_kv_heads, int32_t wgs_per_cu, NB nb) {
    std::vector<int32_t> order(num_units);
    for (size_t i = 0; i < num_units; ++i) order[i] = static_cast<int32_t>(i);
    const int64_t cus = device_cu_count();
    const int64_t items = static_cast<int64_t>(num_units) * num_kv_heads;
    if (num_units < 2 || items > cus * wgs_per_cu) return order;
    const int U = static_cast<int>(num_units);
    std::vector<int64_t> load(static_cast<size_t>(cus), 0);
    std::vector<char> used(num_units, 0);
    std::vector<int32_t> cu_of(num_units * static_cast<size_t>(num_kv_heads));
    for (int p = 0; p < U; ++p)
        for (int h = 0; h < num_kv_heads; ++h)
            cu_of[static_cast<size_t>(p) * num_kv_heads + h] =
                static_cast<int32_t>(pkv::item_of(p, h, U, num_kv_heads) % cus);
    for (int i = 0; i < U; ++i) {
        const int64_t w = nb(static_cast<size_t>(i));
        int best = -1;
        int64_t best_max = 0;
        for (int p = 0; p < U; ++p) {
            if (used[p]) continue;
            int64_t m = 0;
            for (int h = 0; h < num_kv_heads; ++h) m = std::max(m, load[cu_of[static_cast<size_t>(p) * num_kv_heads + h]]);
            if (best < 0 || m < best_max) { best = p; best_max = m; }
        }
        used[best] = 1;
        order[best] = i;
        for (int h = 0; h < num_kv_heads; ++h) load[cu_of[static_cast<size_t>(best) * num_kv_heads + h]] += w;
    }
    return order;
}

// Build the plan.  partition_tokens > 0: fixed partitions of that many tokens
// (the last one of a sequence shorter); 0: one partition per sequence; -1:
// balanced, every sequence cut into near-equal parts of about
// auto_unit_blocks() blocks (no part under 2 * kAutoMinItemBlocks when the
// batch alone fills the device).  Units are ordered longest first, or placed
// by place_on_cus() when the grid has a work-group per item.  wgs_per_cu: the
// work-groups per CU the balanced units are sized for (plan_wgs_per_cu);
// resident_per_cu: those the kernel keeps resident (decode_wgs_per_cu), which
// decide whether every item has its own work-group.
// Shared-prefix plans: the units cover blocks skip .. of every sequence (the
// first `skip` blocks are attended by the prefix pass), and every sequence
// carries `lead` more partial results (the prefix chunks', in its first
// slots), merged with its own.
bool build_plan(const int32_t* seq_lens, int32_t num_seqs, int32_t max_blocks, int32_t partition_tokens,
                int32_t num_kv_heads, int32_t wgs_per_cu, int32_t resident_per_cu, Plan* P, int32_t skip = 0,
                int32_t lead = 0) {
    if (num_seqs < 1 || max_blocks < 1) return false;
    if (partition_tokens < -1 || (partition_tokens > 0 && partition_tokens % PKV_BLOCK_SIZE)) return false;
    std::vector<int32_t> nblk(num_seqs);
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = seq_lens[s];
        if (n < 1 || static_cast<int64_t>(n) > static_cast<int64_t>(max_blocks) * PKV_BLOCK_SIZE) return false;
        nblk[s] = (n + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE - skip;
        if (nblk[s] < 1) return false;
    }
    int32_t unit_blocks;
    int32_t min_part = 1;   // balanced plan: smallest part a sequence is cut into
    if (partition_tokens > 0) unit_blocks = partition_tokens / PKV_BLOCK_SIZE;
    else if (partition_tokens == 0) unit_blocks = max_blocks;
    else {
        unit_blocks = auto_unit_blocks(nblk, num_kv_heads, wgs_per_cu);
        // When whole sequences already give every resident work-group an item,
        // cutting them further only balances the long ones: parts stay at
        // 2 * kAutoMinItemBlocks or more (each part costs a partial result and
        // its merge, more so with many query rows).
        const int64_t slots = static_cast<int64_t>(device_cu_count()) * wgs_per_cu;
        if (static_cast<int64_t>(num_seqs) * num_kv_heads >= slots) min_part = 2 * pkv::kAutoMinItemBlocks;
    }

    struct U { int32_t seq, b0, nb, part, parts, own; };
    std::vector<U> us;
    P->seq_parts.assign(2 * static_cast<size_t>(num_seqs), -1);
    P->num_split_slots = 0;
    P->max_parts = 0;
    P->stride = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t own = std::max(1, std::min((nblk[s] + unit_blocks - 1) / unit_blocks, nblk[s] / min_part));
        const int32_t parts = lead + own;   // partial results merged for the sequence
        P->seq_parts[2 * s] = parts;
        if (parts > 1) {
            P->seq_parts[2 * s + 1] = P->num_split_slots;
            P->num_split_slots += parts;
        }
        P->max_parts = std::max(P->max_parts, parts);
        for (int32_t p = 0; p < own; ++p) {
            int32_t b0, nb;
            if (partition_tokens == -1) {      // near-equal parts
                const int32_t q = nblk[s] / own, r = nblk[s] % own;
                b0 = p * q + std::min(p, r);
                nb = q + (p < r ? 1 : 0);
            } else {
                b0 = p * unit_blocks;
                nb = std::min(unit_blocks, nblk[s] - b0);
            }
            us.push_back({s, skip + b0, nb, lead + p, parts, own});
            P->stride = std::max(P->stride, nb);
        }
    }
    std::stable_sort(us.begin(), us.end(), [](const U& x, const U& y) { return x.nb > y.nb; });
    const std::vector<int32_t> order =
        place_on_cus(us.size(), num_kv_heads, resident_per_cu, [&](size_t i) { return us[i].nb; });
    {
        std::vector<U> placed(us.size());
        for (size_t pos = 0; pos < us.size(); ++pos) placed[pos] = us[order[pos]];
        us.swap(placed);
    }
    P->num_units = static_cast<int32_t>(us.size());
    P->units.assign(static_cast<size_t>(P->num_units) * pkv::kUnitInts, 0);
    for (size_t i = 0; i < us.size(); ++i) {
        int32_t* d = &P->units[i * pkv::kUnitInts];
        const U& u = us[i];
        d[pkv::kUnitSeq] = u.seq;
        d[pkv::kUnitB0] = u.b0;
        d[pkv::kUnitNb] = u.nb;
        d[pkv::kUnitLen] = seq_lens[u.seq];
        d[pkv::kUnitPart] = u.part;
        d[pkv::kUnitParts] = u.parts;
        d[pkv::kUnitSlot] = u.parts > 1 ? P->seq_parts[2 * u.seq + 1] + u.part : -1;
        d[pkv::kUnitRot] = u.seq % u.nb;   // sequences sharing blocks start their walk apart
        d[pkv::kUnitTickets] = u.own;
    }
    return true;
}

TableLayout table_layout(int32_t num_seqs, int32_t max_blocks, int32_t num_kv_heads, const Plan& P,
                         const Plan* C = nullptr) {
    TableLayout L;
    size_t off = 0;
    L.table = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(num_seqs) * max_blocks);
    L.seq_lens = off;
    off = align_up(off + sizeof(int32_t) * num_seqs);
    L.seq_parts = off;
    off = align_up(off + sizeof(int32_t) * 2 * num_seqs);
    L.counters = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(num_seqs) * num_kv_heads);
    L.queue = off;
    off = align_up(off + sizeof(int32_t) * 2);
    L.units = off;
    off = align_up(off + sizeof(int32_t) * pkv::kUnitInts * static_cast<size_t>(P.num_units));
    L.unit_ids = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(P.num_units) * P.stride);
    L.cseq_parts = L.cunits = L.cunit_ids = off;
    if (C) {
        L.cseq_parts = off;
        off = align_up(off + sizeof(int32_t) * 2 * num_seqs);
        L.cunits = off;
        off = align_up(off + sizeof(int32_t) * pkv::kUnitInts * static_cast<size_t>(C->num_units));
        L.cunit_ids = off;
        off = align_up(off + sizeof(int32_t) * static_cast<size_t>(C->num_units) * C->stride);
    }
    L.total = off;
    return L;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// partition_tokens value: the balanced plan, and the shared-prefix plan
// whenever the tables share a prefix (no cost estimate).
constexpr int32_t kForcePrefixPlan = -2;

// The largest shared prefix (in blocks) the lengths allow: every sequence
// keeps at least one position past it.  0 when no shared-prefix plan can
// arise (too few sequences, too short, or a float32 pool, which the prefix
// pass does not take).
int32_t max_prefix_blocks(const pkv_pool* pool, const int32_t* seq_lens, int32_t num_seqs) {
    if (pool->desc.kv_dtype == PKV_F32 || num_seqs < pkv::kCascadeMinSeqs) return 0;
    int32_t m = INT32_MAX;
    for (int32_t s = 0; s < num_seqs; ++s) m = std::min(m, (seq_lens[s] - 1) / PKV_BLOCK_SIZE);
    return m >= pkv::kCascadeMinBlocks ? m : 0;
}

// A shared-prefix plan: each sequence's own blocks (after the prefix) cut
// as the balanced plan cuts whole sequences (one unit when the batch fills
// the device, near-equal parts when few long sequences do not), with
// prefix_chunks leading partials per sequence.
bool build_cascade_plan(const int32_t* seq_lens, int32_t num_seqs, int32_t max_blocks, int32_t num_kv_heads,
                        int32_t wgs_per_cu, int32_t resident_per_cu, int32_t prefix_blocks, int32_t prefix_chunks,
                        Plan* C) {
    return build_plan(seq_lens, num_seqs, max_blocks, -1, num_kv_heads, wgs_per_cu, resident_per_cu, C, prefix_blocks,
                      prefix_chunks);
}

// Prefix chunks: at most kCascadeMaxChunks, each of at least
// kCascadeChunkBlocks blocks (or one chunk of the whole prefix), an even
// number of blocks per chunk but the last.
void prefix_chunking(int32_t prefix_blocks, int32_t* chunk_blocks, int32_t* chunks) {
    const int32_t want = std::max(1, std::min(pkv::kCascadeMaxChunks, prefix_blocks / pkv::kCascadeChunkBlocks));
    const int32_t per = (prefix_blocks + 2 * want - 1) / (2 * want) * 2;
    *chunk_blocks = per;
    *chunks = (prefix_blocks + per - 1) / per;
}

// Whether attending a shared prefix once for all rows should beat reading
// it once per sequence, by a rough model fitted on MI355X: a prefix-pass
// work-group walks one chunk at about 1.5 us per block pair after about
// 5 us of start-up (the pass's work-groups run side by side), while the
// plain walk reads every sequence's reference to the prefix tiles at about
// 12 TB/s (the repeated reads of shared tiles hit the L2 and the Infinity
// Cache).  Measured, prefix plan against plain plan: 128 fp8 verify
// sequences over a 2,048-token prefix 88 against 101 us, 64 bf16 decode
// sequences 44 against 49 us (model: prefix plan); 32 bf16 sequences 36.5
// against 34.9 us, 4 sequences behind a 4,096-token prefix 43 against
// 19 us (model: plain plan).
bool prefix_plan_pays(const pkv_pool* pool, int32_t num_seqs, int32_t prefix_blocks, int32_t chunk_blocks) {
    const double pass_us = 5.0 + 1.5 * (chunk_blocks / 2.0);
    const double plain_us = static_cast<double>(num_seqs) * prefix_blocks * pool->desc.num_kv_heads * 2.0 *
                            static_cast<double>(pool->tile_bytes) / 12.0e6;
    return pass_us < plain_us;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "ok";
        case PKV_ERR_INVALID: return "invalid argument";
        case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
        case PKV_ERR_BLOCK_RANGE: return "block-table entry outside the pool";
        case PKV_ERR_SEQ_LEN: return "sequence length out of range";
        case PKV_ERR_WORKSPACE: return "device buffer or workspace too small";
        case PKV_ERR_HIP: return "HIP runtime error";
        case PKV_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
        case PKV_ERR_TABLE_STALE: return "an earlier attention launch on this table failed; upload it again";
        default: return "unknown status";
    }
}

int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim, int32_t kv_dtype) {
    const int bits = elem_bits(kv_dtype);
    if (num_layers < 1 || num_kv_heads < 1 || head_dim < 1 || bits == 0) return -1;
    return 2LL * num_layers * num_kv_heads * head_dim * bits / 8;
}

int64_t kv_pool_bytes(const pkv_pool_desc* desc) {
    if (check_desc(desc) != PKV_OK) return -1;
    return static_cast<int64_t>(desc->num_blocks) * PKV_BLOCK_SIZE *
           kv_bytes_per_token(desc->num_layers, desc->num_kv_heads, desc->head_dim, desc->kv_dtype);
}

pkv_status kv_pool_create(const pkv_pool_desc* desc, void* dev_base, size_t dev_bytes,
                          const float* dev_k_scale, const float* dev_v_scale, pkv_pool** out) {
    try {
        if (!out) return PKV_ERR_INVALID;
        *out = nullptr;
        const pkv_status st = check_desc(desc);
        if (st != PKV_OK) return st;
        if (!dev_base || reinterpret_cast<uintptr_t>(dev_base) % kAlign) return PKV_ERR_INVALID;
        if (dev_bytes < static_cast<size_t>(kv_pool_bytes(desc))) return PKV_ERR_INVALID;
        const bool scaled = scaled_dtype(desc->kv_dtype);
        if (scaled && (!dev_k_scale || !dev_v_scale)) return PKV_ERR_INVALID;
        pkv_pool* p = new pkv_pool;
        p->desc = *desc;
        p->base = static_cast<uint8_t*>(dev_base);
        p->bytes = dev_bytes;
        p->k_scale = scaled ? dev_k_scale : nullptr;
        p->v_scale = scaled ? dev_v_scale : nullptr;
        p->tile_bytes = static_cast<int64_t>(PKV_BLOCK_SIZE) * desc->head_dim * elem_bits(desc->kv_dtype) / 8;
        *out = p;
        return PKV_OK;
    } catch (...) {
        return PKV_ERR_INVALID;
    }
}

pkv_status kv_pool_destroy(pkv_pool* pool) {
    delete pool;
    return PKV_OK;
}

size_t block_table_device_bytes(const pkv_pool* pool, const int32_t* host_seq_lens, int32_t num_seqs,
                                int32_t max_blocks_per_seq, int32_t partition_tokens) {
    try {
        if (!pool || !host_seq_lens) return 0;
        const bool balanced = partition_tokens == -1 || partition_tokens == kForcePrefixPlan;
        if (partition_tokens == kForcePrefixPlan) partition_tokens = -1;
        Plan P;
        const int32_t wpc = pkv::plan_wgs_per_cu(pool->desc.kv_dtype, pool->desc.head_dim);
        const int32_t rpc = pkv::decode_wgs_per_cu(pool->desc.kv_dtype, pool->desc.head_dim);
        if (!build_plan(host_seq_lens, num_seqs, max_blocks_per_seq, partition_tokens, pool->desc.num_kv_heads, wpc,
                        rpc, &P))
            return 0;
        // Room for a shared-prefix plan if the tables turn out to share one,
        // sized for the smallest prefix (the most own blocks); an upload whose
        // actual prefix plan would not fit keeps the plain plan.
        Plan C;
        const bool maybe = balanced && max_prefix_blocks(pool, host_seq_lens, num_seqs) > 0 &&
                           build_cascade_plan(host_seq_lens, num_seqs, max_blocks_per_seq, pool->desc.num_kv_heads,
                                              wpc, rpc, pkv::kCascadeMinBlocks, 1, &C);
        return table_layout(num_seqs, max_blocks_per_seq, pool->desc.num_kv_heads, P, maybe ? &C : nullptr).total;
    } catch (...) {
        return 0;
    }
}

pkv_status block_table_upload(const pkv_pool* pool, const int32_t* host_block_table, int32_t num_seqs,
                              int32_t max_blocks_per_seq, const int32_t* host_seq_lens,
                              int32_t partition_tokens, void* dev_buffer, size_t dev_buffer_bytes,
                              void* stream, pkv_table** out) {
    try {
        if (!out) return PKV_ERR_INVALID;
        *out = nullptr;
        if (!pool || !host_block_table || !host_seq_lens || !dev_buffer) return PKV_ERR_INVALID;
        if (reinterpret_cast<uintptr_t>(dev_buffer) % kAlign) return PKV_ERR_INVALID;
        if (num_seqs < 1 || max_blocks_per_seq < 1) return PKV_ERR_INVALID;
        if (partition_tokens < kForcePrefixPlan || (partition_tokens > 0 && partition_tokens % PKV_BLOCK_SIZE))
            return PKV_ERR_INVALID;
        const bool force_prefix = partition_tokens == kForcePrefixPlan;
        if (force_prefix) partition_tokens = -1;
        const int32_t nb_pool = pool->desc.num_blocks;
        const int32_t hkv = pool->desc.num_kv_heads;
        const int64_t cap = static_cast<int64_t>(max_blocks_per_seq) * PKV_BLOCK_SIZE;

        int32_t max_len = 0, min_len = INT32_MAX, max_id = -1;
        for (int32_t s = 0; s < num_seqs; ++s) {
            const int32_t n = host_seq_lens[s];
            if (n < 1 || n > cap) return PKV_ERR_SEQ_LEN;
            max_len = std::max(max_len, n);
            min_len = std::min(min_len, n);
            const int32_t used = (n + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
            const int32_t* row = host_block_table + static_cast<int64_t>(s) * max_blocks_per_seq;
            for (int32_t j = 0; j < used; ++j) {
                if (row[j] < 0 || row[j] >= nb_pool) return PKV_ERR_BLOCK_RANGE;
                max_id = std::max(max_id, row[j]);
            }
        }
        Plan P;
        const int32_t wpc = pkv::plan_wgs_per_cu(pool->desc.kv_dtype, pool->desc.head_dim);
        const int32_t rpc = pkv::decode_wgs_per_cu(pool->desc.kv_dtype, pool->desc.head_dim);
        if (!build_plan(host_seq_lens, num_seqs, max_blocks_per_seq, partition_tokens, hkv, wpc, rpc, &P))
            return PKV_ERR_INVALID;
        // Shared prefix (balanced plans only: fixed partitions are kept as
        // asked): the longest run of leading physical blocks that every
        // sequence's table names alike (at most what the lengths allow).
        int32_t prefix = partition_tokens == -1 ? max_prefix_blocks(pool, host_seq_lens, num_seqs) : 0;
        for (int32_t j = 0; j < prefix; ++j) {
            const int32_t id = host_block_table[j];
            for (int32_t s = 1; s < num_seqs; ++s) {
                if (host_block_table[static_cast<int64_t>(s) * max_blocks_per_seq + j] != id) {
                    prefix = j;
                    break;
                }
            }
        }
        if (prefix < pkv::kCascadeMinBlocks) prefix = 0;
        Plan C;
        int32_t chunk_blocks = 0, chunks = 0;
        if (prefix) prefix_chunking(prefix, &chunk_blocks, &chunks);
        if (prefix && !force_prefix && !prefix_plan_pays(pool, num_seqs, prefix, chunk_blocks)) prefix = 0;
        if (prefix && !build_cascade_plan(host_seq_lens, num_seqs, max_blocks_per_seq, hkv, wpc, rpc, prefix, chunks,
                                          &C))
            return PKV_ERR_INVALID;
        TableLayout L = table_layout(num_seqs, max_blocks_per_seq, hkv, P, prefix ? &C : nullptr);
        if (prefix && dev_buffer_bytes < L.total) {
            prefix = 0;
            L = table_layout(num_seqs, max_blocks_per_seq, hkv, P, nullptr);
        }
        if (dev_buffer_bytes < L.total) return PKV_ERR_WORKSPACE;

        pkv_table* t = new pkv_table;
        t->num_seqs = num_seqs;
        t->max_blocks = max_blocks_per_seq;
        t->num_kv_heads = hkv;
        t->partition_tokens = partition_tokens;
        t->num_units = P.num_units;
        t->unit_stride = P.stride;
        t->num_split_slots = P.num_split_slots;
        t->max_parts = P.max_parts;
        t->max_seq_len = max_len;
        t->min_seq_len = min_len;
        t->max_block_id = max_id;
        t->pool_blocks = nb_pool;
        uint8_t* base = static_cast<uint8_t*>(dev_buffer);
        t->d_table = reinterpret_cast<int32_t*>(base + L.table);
        t->d_seq_lens = reinterpret_cast<int32_t*>(base + L.seq_lens);
        t->d_seq_parts = reinterpret_cast<int32_t*>(base + L.seq_parts);
        t->d_counters = reinterpret_cast<int32_t*>(base + L.counters);
        t->d_queue = reinterpret_cast<int32_t*>(base + L.queue);
        t->d_units = reinterpret_cast<int32_t*>(base + L.units);
        t->d_unit_ids = reinterpret_cast<int32_t*>(base + L.unit_ids);
        t->seq_lens_offset = L.seq_lens;
        if (prefix) {
            t->prefix_blocks = prefix;
            t->prefix_chunks = chunks;
            t->prefix_chunk_blocks = chunk_blocks;
            t->c_num_units = C.num_units;
            t->c_unit_stride = C.stride;
            t->c_num_split_slots = C.num_split_slots;
            t->c_max_parts = C.max_parts;
            t->d_cseq_parts = reinterpret_cast<int32_t*>(base + L.cseq_parts);
            t->d_cunits = reinterpret_cast<int32_t*>(base + L.cunits);
            t->d_cunit_ids = reinterpret_cast<int32_t*>(base + L.cunit_ids);
        }

        // One host image of the whole buffer (counters start at zero), copied once.
        t->staging.assign(L.total / sizeof(int32_t), 0);
        int32_t* hs = t->staging.data();
        std::memcpy(hs + L.table / 4, host_block_table,
                    sizeof(int32_t) * static_cast<size_t>(num_seqs) * max_blocks_per_seq);
        std::memcpy(hs + L.seq_lens / 4, host_seq_lens, sizeof(int32_t) * num_seqs);
        std::memcpy(hs + L.seq_parts / 4, P.seq_parts.data(), sizeof(int32_t) * 2 * num_seqs);
        std::memcpy(hs + L.units / 4, P.units.data(), sizeof(int32_t) * P.units.size());
        // Is any physical block named twice among the used entries (from
        // block `from` on)?  Such a batch reads those blocks once per
        // reference, and its attention launches keep the cached tile-load
        // policy instead of streaming.
        auto any_shared = [&](int32_t from) {
            std::vector<uint8_t> seen(static_cast<size_t>(nb_pool), 0);
            for (int32_t s = 0; s < num_seqs; ++s) {
                const int32_t used = (host_seq_lens[s] + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
                const int32_t* row = host_block_table + static_cast<int64_t>(s) * max_blocks_per_seq;
                for (int32_t j = from; j < used; ++j) {
                    if (seen[row[j]]) return true;
                    seen[row[j]] = 1;
                }
            }
            return false;
        };
        t->shared_blocks = any_shared(0);
        if (prefix) t->c_shared_blocks = any_shared(prefix);
        // Unit block ids in walking order: j = 0 .. nb-1 visits logical block
        // b0 + (j + rot) mod nb; the tail of the stride repeats the first id.
        auto write_ids = [&](const Plan& Q, size_t at) {
            for (int32_t u = 0; u < Q.num_units; ++u) {
                const int32_t* d = &Q.units[static_cast<size_t>(u) * pkv::kUnitInts];
                const int32_t* row = host_block_table + static_cast<int64_t>(d[pkv::kUnitSeq]) * max_blocks_per_seq;
                int32_t* ids = hs + at / 4 + static_cast<size_t>(u) * Q.stride;
                const int32_t b0 = d[pkv::kUnitB0], nb = d[pkv::kUnitNb], rot = d[pkv::kUnitRot];
                for (int32_t j = 0; j < Q.stride; ++j) {
                    const int32_t jj = j < nb ? (j + rot) % nb : rot;
                    ids[j] = row[b0 + jj];
                }
            }
        };
        write_ids(P, L.unit_ids);
        if (prefix) {
            std::memcpy(hs + L.cseq_parts / 4, C.seq_parts.data(), sizeof(int32_t) * 2 * num_seqs);
            std::memcpy(hs + L.cunits / 4, C.units.data(), sizeof(int32_t) * C.units.size());
            write_ids(C, L.cunit_ids);
        }
        hipStream_t st = static_cast<hipStream_t>(stream);
        hipError_t e = hipEventCreateWithFlags(&t->uploaded, hipEventDisableTiming);
        if (e != hipSuccess) {
            delete t;
            return PKV_ERR_HIP;
        }
        e = hipMemcpyAsync(dev_buffer, hs, L.total, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipEventRecord(t->uploaded, st);
        if (e != hipSuccess) {
            (void)hipEventDestroy(t->uploaded);
            delete t;
            return PKV_ERR_HIP;
        }
        *out = t;
        return PKV_OK;
    } catch (...) {
        return PKV_ERR_INVALID;
    }
}

pkv_status block_table_destroy(pkv_table* table) {
    if (!table) return PKV_OK;
    pkv_status st = hip_status(hipEventSynchronize(table->uploaded));
    (void)hipEventDestroy(table->uploaded);
    delete table;
    return st;
}

pkv_status block_table_info(const pkv_table* table, int32_t* num_units, int32_t* num_split_slots,
                            int32_t* max_seq_len, int32_t* min_seq_len, int32_t* max_parts) {
    if (!table) return PKV_ERR_INVALID;
    if (num_units) *num_units = table->num_units;
    if (num_split_slots) *num_split_slots = table->num_split_slots;
    if (max_seq_len) *max_seq_len = table->max_seq_len;
    if (min_seq_len) *min_seq_len = table->min_seq_len;
    if (max_parts) *max_parts = table->max_parts;
    return PKV_OK;
}

pkv_status block_table_shared_prefix(const pkv_table* table, int32_t* prefix_blocks, int32_t* prefix_chunks) {
    if (!table) return PKV_ERR_INVALID;
    if (prefix_blocks) *prefix_blocks = table->prefix_blocks;
    if (prefix_chunks) *prefix_chunks = table->prefix_chunks;
    return PKV_OK;
}

pkv_status slot_mapping_compute(const pkv_table* table, const int32_t* dev_seq_ids, const int32_t* dev_positions,
                                int32_t num_tokens, int64_t* dev_slot_mapping, void* stream) {
    if (!table || num_tokens < 0) return PKV_ERR_INVALID;
    if (num_tokens == 0) return PKV_OK;
    if (!dev_seq_ids || !dev_positions || !dev_slot_mapping) return PKV_ERR_INVALID;
    pkv::SlotArgs a;
    a.block_table = table->d_table;
    a.seq_ids = dev_seq_ids;
    a.positions = dev_positions;
    a.slots = dev_slot_mapping;
    a.num_seqs = table->num_seqs;
    a.max_blocks = table->max_blocks;
    a.num_blocks = table->pool_blocks;
    a.num_tokens = num_tokens;
    return hip_status(pkv::launch_slot_mapping(a, static_cast<hipStream_t>(stream)));
}

pkv_status reshape_and_cache(const pkv_pool* pool, int32_t layer, const void* dev_k_new, const void* dev_v_new,
                             int32_t in_dtype, const int64_t* dev_slot_mapping, int32_t num_tokens, void* stream) {
    if (!pool || num_tokens < 0) return PKV_ERR_INVALID;
    if (layer < 0 || layer >= pool->desc.num_layers) return PKV_ERR_INVALID;
    const int32_t kv = pool->desc.kv_dtype;
    const bool ok = (kv == PKV_F32 && in_dtype == PKV_F32) || (kv == PKV_BF16 && in_dtype == PKV_BF16) ||
                    (scaled_dtype(kv) && (in_dtype == PKV_F32 || in_dtype == PKV_BF16));
    if (!ok) return PKV_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PKV_OK;
    if (!dev_k_new || !dev_v_new || !dev_slot_mapping) return PKV_ERR_INVALID;
    pkv::CacheArgs a;
    a.pool = pool->base;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.k_new = dev_k_new;
    a.v_new = dev_v_new;
    a.slots = dev_slot_mapping;
    a.tile_bytes = pool->tile_bytes;
    a.num_slots = static_cast<int64_t>(pool->desc.num_blocks) * PKV_BLOCK_SIZE;
    a.layer = layer;
    a.num_blocks = pool->desc.num_blocks;
    a.num_kv_heads = pool->desc.num_kv_heads;
    a.head_dim = pool->desc.head_dim;
    a.num_tokens = num_tokens;
    return hip_status(pkv::launch_reshape_and_cache(a, kv, in_dtype, static_cast<hipStream_t>(stream)));
}

size_t paged_attention_workspace_bytes(const pkv_pool* pool, const pkv_table* table, int32_t num_q_heads,
                                       int32_t query_rows) {
    if (!pool || !table || num_q_heads < 1 || query_rows < 1) return 0;
    const int32_t hkv = pool->desc.num_kv_heads;
    if (num_q_heads % hkv) return 0;
    const int64_t rows = static_cast<int64_t>(num_q_heads / hkv) * query_rows;
    // room for the partials of either plan (with a shared prefix, the
    // shared-prefix plan's whenever a call can use it)
    const int64_t slots = std::max(table->num_split_slots, table->c_num_split_slots);
    const int64_t entries = static_cast<int64_t>(hkv) * slots * rows;
    if (entries == 0) return 0;
    const size_t o_bytes = align_up(sizeof(float) * static_cast<size_t>(entries) * pool->desc.head_dim);
    const size_t ml_bytes = align_up(sizeof(float) * static_cast<size_t>(entries));
    return o_bytes + 2 * ml_bytes;
}

}  // extern "C"

namespace {

// Attention over the table's units, optionally appending the k newest tokens
// of every sequence first (k_new != NULL).
pkv_status attention_call(const pkv_pool* pool, int32_t layer, const pkv_table* table, const void* k_new,
                          const void* v_new, int32_t in_dtype, const void* dev_q, int32_t q_dtype,
                          int32_t query_rows, int32_t num_q_heads, float scale, void* dev_workspace,
                          size_t workspace_bytes, void* dev_out, int32_t out_dtype, void* stream) {
    if (!pool || !table || !dev_q || !dev_out) return PKV_ERR_INVALID;
    if (table->stale) return PKV_ERR_TABLE_STALE;
    if (layer < 0 || layer >= pool->desc.num_layers) return PKV_ERR_INVALID;
    if (query_rows < 1 || num_q_heads < 1) return PKV_ERR_INVALID;
    if (!std::isfinite(scale)) return PKV_ERR_INVALID;
    const int32_t hkv = pool->desc.num_kv_heads;
    if (num_q_heads % hkv) return PKV_ERR_INVALID;
    const int32_t group = num_q_heads / hkv;
    if (static_cast<int64_t>(group) * query_rows > pkv::kMaxRows) return PKV_ERR_UNSUPPORTED;
    const int32_t kv = pool->desc.kv_dtype;
    const int32_t want_q = kv == PKV_F32 ? PKV_F32 : PKV_BF16;
    if (q_dtype != want_q) return PKV_ERR_UNSUPPORTED;
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
    if (table->min_seq_len < query_rows) return PKV_ERR_SEQ_LEN;
    if (table->max_block_id >= pool->desc.num_blocks) return PKV_ERR_BLOCK_RANGE;
    if (table->num_kv_heads != hkv) return PKV_ERR_INVALID;
    const size_t need = paged_attention_workspace_bytes(pool, table, num_q_heads, query_rows);
    if (need > 0 && (!dev_workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
    if (need > 0 && reinterpret_cast<uintptr_t>(dev_workspace) % kAlign) return PKV_ERR_INVALID;
    if (k_new || v_new) {
        if (!k_new || !v_new) return PKV_ERR_INVALID;
        const bool ok = (kv == PKV_F32 && in_dtype == PKV_F32) || (kv == PKV_BF16 && in_dtype == PKV_BF16) ||
                        (scaled_dtype(kv) && (in_dtype == PKV_F32 || in_dtype == PKV_BF16));
        if (!ok) return PKV_ERR_UNSUPPORTED;
    }

    // The shared-prefix plan applies when every row of every sequence sees
    // the whole prefix (and tokens appended by this call lie past it).
    const bool cascade = table->prefix_blocks > 0 &&
                         static_cast<int64_t>(table->min_seq_len) - query_rows >=
                             static_cast<int64_t>(table->prefix_blocks) * PKV_BLOCK_SIZE;
    const int32_t slots = std::max(table->num_split_slots, table->c_num_split_slots);

    pkv::AttnArgs a;
    a.pool = pool->base;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.units = cascade ? table->d_cunits : table->d_units;
    a.unit_ids = cascade ? table->d_cunit_ids : table->d_unit_ids;
    a.seq_parts = cascade ? table->d_cseq_parts : table->d_seq_parts;
    a.counters = table->d_counters;
    a.queue = table->d_queue;
    a.q = dev_q;
    a.out = dev_out;
    a.k_new = k_new;
    a.v_new = v_new;
    a.append_in_f32 = in_dtype == PKV_F32 ? 1 : 0;
    const int64_t entries = static_cast<int64_t>(hkv) * slots * group * query_rows;
    uint8_t* ws = static_cast<uint8_t*>(dev_workspace);
    const size_t o_bytes = align_up(sizeof(float) * static_cast<size_t>(entries) * pool->desc.head_dim);
    const size_t ml_bytes = align_up(sizeof(float) * static_cast<size_t>(entries));
    a.part_o = need ? reinterpret_cast<float*>(ws) : nullptr;
    a.part_m = need ? reinterpret_cast<float*>(ws + o_bytes) : nullptr;
    a.part_l = need ? reinterpret_cast<float*>(ws + o_bytes + ml_bytes) : nullptr;
    a.tile_bytes = pool->tile_bytes;
    a.layer = layer;
    a.num_blocks = pool->desc.num_blocks;
    a.num_seqs = table->num_seqs;
    a.num_kv_heads = hkv;
    a.num_q_heads = num_q_heads;
    a.group = group;
    a.rows = group * query_rows;
    a.k_rows = query_rows;
    a.head_dim = pool->desc.head_dim;
    a.unit_stride = cascade ? table->c_unit_stride : table->unit_stride;
    const int32_t units = cascade ? table->c_num_units : table->num_units;
    a.num_items = units * hkv;
    a.num_split_slots = slots;
    a.max_parts = cascade ? table->c_max_parts : table->max_parts;
    a.fuse_max_parts = pkv::kFuseMaxParts;
    a.out_bf16 = out_dtype == PKV_BF16 ? 1 : 0;
    a.score_scale = scale * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (cascade) {
        // Shared-prefix pass: every sequence's query rows against the prefix
        // chunks, one partial per (row, chunk) in the sequence's first slots.
        pkv::PrefillArgs pa;
        pa.pool = pool->base;
        pa.k_scale = pool->k_scale;
        pa.v_scale = pool->v_scale;
        pa.table = table->d_table;
        pa.seq_lens = table->d_seq_lens;
        pa.q = dev_q;
        pa.out = nullptr;
        pa.query_start = nullptr;
        pa.tile_bytes = pool->tile_bytes;
        pa.layer = layer;
        pa.num_blocks = pool->desc.num_blocks;
        pa.num_seqs = table->num_seqs;
        pa.num_kv_heads = hkv;
        pa.num_q_heads = num_q_heads;
        pa.group = group;
        pa.chunk = query_rows;
        pa.max_blocks = table->max_blocks;
        const int64_t tiles = (static_cast<int64_t>(table->num_seqs) * query_rows * group + pkv::kPrefillRows - 1) /
                              pkv::kPrefillRows;
        if (tiles * hkv * table->prefix_chunks > INT32_MAX) return PKV_ERR_UNSUPPORTED;
        pa.row_tiles = static_cast<int32_t>(tiles);
        pa.out_bf16 = 0;
        pa.score_scale = a.score_scale;
        pa.part_o = a.part_o;
        pa.part_m = a.part_m;
        pa.part_l = a.part_l;
        pa.seq_parts = table->d_cseq_parts;
        pa.num_split_slots = slots;
        pa.prefix_blocks = table->prefix_blocks;
        pa.prefix_chunk_blocks = table->prefix_chunk_blocks;
        pa.prefix_chunks = table->prefix_chunks;
        const hipError_t e = pkv::launch_prefill(pa, kv, pool->desc.head_dim, st);
        if (e != hipSuccess) return PKV_ERR_HIP;
    }
    const hipError_t err = pkv::launch_attention(a, kv, pool->desc.head_dim, units,
                                                 cascade ? table->c_shared_blocks : table->shared_blocks, st);
    if (err != hipSuccess) const_cast<pkv_table*>(table)->stale = true;
    return hip_status(err);
}

// Chunked-prefill attention: every sequence's chunk is chunk_tokens long
// (host_query_start NULL) or host_query_start[s + 1] - host_query_start[s]
// long, its rows packed from host_query_start[s] (the device copy is what the
// kernel reads).
pkv_status prefill_call(const pkv_pool* pool, int32_t layer, const pkv_table* table, const void* dev_q,
                        int32_t q_dtype, int32_t chunk_tokens, const int32_t* host_query_start,
                        const int32_t* dev_query_start, int32_t num_q_heads, float scale, void* dev_out,
                        int32_t out_dtype, void* stream) {
    if (!pool || !table) return PKV_ERR_INVALID;
    if (layer < 0 || layer >= pool->desc.num_layers) return PKV_ERR_INVALID;
    if (num_q_heads < 1 || !std::isfinite(scale)) return PKV_ERR_INVALID;
    const int32_t hkv = pool->desc.num_kv_heads;
    if (num_q_heads % hkv || table->num_kv_heads != hkv) return PKV_ERR_INVALID;
    const int32_t kv = pool->desc.kv_dtype;
    if (kv == PKV_F32) return PKV_ERR_UNSUPPORTED;
    if (q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
    if (table->max_block_id >= pool->desc.num_blocks) return PKV_ERR_BLOCK_RANGE;
    const int32_t group = num_q_heads / hkv;
    int64_t longest = chunk_tokens;
    if (host_query_start) {
        // chunks: non-negative lengths, each within its sequence, rows packed in order
        if (host_query_start[0] != 0) return PKV_ERR_INVALID;
        const int32_t* lens = table->staging.data() + table->seq_lens_offset / 4;
        longest = 0;
        for (int32_t s = 0; s < table->num_seqs; ++s) {
            const int64_t c = static_cast<int64_t>(host_query_start[s + 1]) - host_query_start[s];
            if (c < 0) return PKV_ERR_INVALID;
            if (c > lens[s]) return PKV_ERR_SEQ_LEN;
            longest = std::max(longest, c);
        }
        if (static_cast<int64_t>(host_query_start[table->num_seqs]) * num_q_heads > INT32_MAX)
            return PKV_ERR_UNSUPPORTED;
    } else {
        if (table->min_seq_len < chunk_tokens) return PKV_ERR_SEQ_LEN;
        if (static_cast<int64_t>(chunk_tokens) * table->num_seqs * num_q_heads > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    }
    const int64_t tiles = (longest * group + pkv::kPrefillRows - 1) / pkv::kPrefillRows;
    if (tiles == 0) return PKV_OK;   // no chunk token in the batch (q and out may be NULL)
    if (!dev_q || !dev_out) return PKV_ERR_INVALID;
    if (tiles * table->num_seqs * hkv > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    pkv::PrefillArgs a;
    a.pool = pool->base;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.table = table->d_table;
    a.seq_lens = table->d_seq_lens;
    a.q = dev_q;
    a.out = dev_out;
    a.query_start = dev_query_start;
    a.tile_bytes = pool->tile_bytes;
    a.layer = layer;
    a.num_blocks = pool->desc.num_blocks;
    a.num_seqs = table->num_seqs;
    a.num_kv_heads = hkv;
    a.num_q_heads = num_q_heads;
    a.group = group;
    a.chunk = chunk_tokens;
    a.max_blocks = table->max_blocks;
    a.row_tiles = static_cast<int32_t>(tiles);
    a.out_bf16 = out_dtype == PKV_BF16 ? 1 : 0;
    a.score_scale = scale * 1.4426950408889634f;
    const int32_t kvt = kv;   // PKV_* element codes equal the kernels' KV_* codes
    return hip_status(pkv::launch_prefill(a, kvt, pool->desc.head_dim, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pkv_status paged_attention_verify(const pkv_pool* pool, int32_t layer, const pkv_table* table, const void* dev_q,
                                  int32_t q_dtype, int32_t query_rows, int32_t num_q_heads, float scale,
                                  void* dev_workspace, size_t workspace_bytes, void* dev_out, int32_t out_dtype,
                                  void* stream) {
    return attention_call(pool, layer, table, nullptr, nullptr, 0, dev_q, q_dtype, query_rows, num_q_heads, scale,
                          dev_workspace, workspace_bytes, dev_out, out_dtype, stream);
}

static_assert(PKV_NOALLOC_SCRATCH_BYTES == pkv::kNoAllocScratchBytes, "scratch size");

pkv_status paged_attention_verify_noalloc(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                          const void* dev_q, int32_t q_dtype, int32_t query_rows,
                                          int32_t num_q_heads, float scale, void* dev_out, int32_t out_dtype,
                                          void* stream) {
    if (!pool || !table) return PKV_ERR_INVALID;
    const size_t need = paged_attention_workspace_bytes(pool, table, num_q_heads, query_rows);
    if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    if (pkv::attention_scratch(&scratch, &scratch_bytes) != hipSuccess) return PKV_ERR_HIP;
    return attention_call(pool, layer, table, nullptr, nullptr, 0, dev_q, q_dtype, query_rows, num_q_heads, scale,
                          scratch, scratch_bytes, dev_out, out_dtype, stream);
}

pkv_status paged_attention_append(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                  const void* dev_k_new, const void* dev_v_new, int32_t in_dtype,
                                  const void* dev_q, int32_t q_dtype, int32_t query_rows, int32_t num_q_heads,
                                  float scale, void* dev_workspace, size_t workspace_bytes, void* dev_out,
                                  int32_t out_dtype, void* stream) {
    if (!dev_k_new || !dev_v_new) return PKV_ERR_INVALID;
    return attention_call(pool, layer, table, dev_k_new, dev_v_new, in_dtype, dev_q, q_dtype, query_rows,
                          num_q_heads, scale, dev_workspace, workspace_bytes, dev_out, out_dtype, stream);
}

pkv_status paged_attention_prefill(const pkv_pool* pool, int32_t layer, const pkv_table* table, const void* dev_q,
                                   int32_t q_dtype, int32_t chunk_tokens, int32_t num_q_heads, float scale,
                                   void* dev_out, int32_t out_dtype, void* stream) {
    if (!table) return PKV_ERR_INVALID;
    if (chunk_tokens < 1) return PKV_ERR_INVALID;
    return prefill_call(pool, layer, table, dev_q, q_dtype, chunk_tokens, nullptr, nullptr, num_q_heads, scale,
                        dev_out, out_dtype, stream);
}

pkv_status paged_attention_prefill_varlen(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                          const void* dev_q, int32_t q_dtype, const int32_t* host_query_start,
                                          const int32_t* dev_query_start, int32_t num_q_heads, float scale,
                                          void* dev_out, int32_t out_dtype, void* stream) {
    if (!table || !host_query_start || !dev_query_start) return PKV_ERR_INVALID;
    return prefill_call(pool, layer, table, dev_q, q_dtype, 0, host_query_start, dev_query_start, num_q_heads, scale,
                        dev_out, out_dtype, stream);
}

pkv_status kv_copy_blocks(const pkv_pool* pool, const int32_t* dev_pairs, int32_t num_pairs, void* stream) {
    if (!pool || num_pairs < 0) return PKV_ERR_INVALID;
    if (num_pairs == 0) return PKV_OK;
    if (!dev_pairs) return PKV_ERR_INVALID;
    pkv::CopyArgs a;
    a.pool = pool->base;
    a.pairs = dev_pairs;
    a.num_pairs = num_pairs;
    a.num_blocks = pool->desc.num_blocks;
    a.num_layers = pool->desc.num_layers;
    a.block_bytes = static_cast<int64_t>(pool->desc.num_kv_heads) * 2 * pool->tile_bytes;
    return hip_status(pkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

pkv_status speculative_accept(const float* dev_p, const float* dev_q, const int32_t* dev_draft,
                              const float* dev_u_accept, const float* dev_u_sample, int32_t num_seqs,
                              int32_t draft_tokens, int32_t vocab, int32_t* dev_num_accepted, int32_t* dev_tokens,
                              void* stream) {
    if (num_seqs < 0 || draft_tokens < 1 || vocab < 1) return PKV_ERR_INVALID;
    if (num_seqs == 0) return PKV_OK;
    if (!dev_p || !dev_q || !dev_draft || !dev_u_accept || !dev_u_sample || !dev_num_accepted || !dev_tokens)
        return PKV_ERR_INVALID;
    if (draft_tokens > 1024) return PKV_ERR_UNSUPPORTED;
    // float4 reads of the rows need 16-byte aligned rows
    if (reinterpret_cast<uintptr_t>(dev_p) % 16 || reinterpret_cast<uintptr_t>(dev_q) % 16) return PKV_ERR_INVALID;
    pkv::SpecArgs a;
    a.p = dev_p;
    a.q = dev_q;
    a.draft = dev_draft;
    a.u_accept = dev_u_accept;
    a.u_sample = dev_u_sample;
    a.num_accepted = dev_num_accepted;
    a.tokens = dev_tokens;
    a.seg_len = pkv::speculative_segment_len(vocab);
    a.num_seqs = num_seqs;
    a.k = draft_tokens;
    a.vocab = vocab;
    return hip_status(pkv::launch_speculative_accept(a, static_cast<hipStream_t>(stream)));
}

pkv_status paged_attention_decode(const pkv_pool* pool, int32_t layer, const pkv_table* table, const void* dev_q,
                                  int32_t q_dtype, int32_t num_q_heads, float scale, void* dev_workspace,
                                  size_t workspace_bytes, void* dev_out, int32_t out_dtype, void* stream) {
    return paged_attention_verify(pool, layer, table, dev_q, q_dtype, 1, num_q_heads, scale, dev_workspace,
                                  workspace_bytes, dev_out, out_dtype, stream);
}

}  // extern "C"
