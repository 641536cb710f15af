// Host-side KV block manager: on-demand block allocation, free on finish,
// reference-counted sharing of prefix blocks with hash-keyed lookup, forks
// with copy-on-write of a shared partial block.
//
// Method (page "KV cache & continuous batching", section "Visual: the
// lifecycle of a request in continuous batching": the cache is handed out in
// 16-token blocks, a finished request frees its blocks at once; section
// "2. PagedAttention (vLLM)": a block table per request maps logical blocks to
// physical blocks allocated on demand; section "4. Prefix caching / prompt
// caching": prefix blocks are hashed and reused across requests that share
// the prefix; page "LLM Serving - KV Cache, Batching, Speculative Decoding",
// section "KV memory, paging and prefix identity": physical blocks may be
// shared, reuse needs the exact token prefix, and a salt keeps tenants apart).
//
// Policy (readings recorded in the design notes):
//  * only full blocks are registered for reuse, under the chain key
//    (key of the previous block, salt, the block's 16 token ids); a lookup
//    also compares the stored token ids and previous key, so a match is an
//    exact prefix match, never a hash collision;
//  * a request reuses the longest run of leading full blocks found, but always
//    computes its last prompt token itself (at most len-1 tokens are cached);
//  * a block whose reference count drops to 0 goes to the tail of the free
//    list; if registered it stays findable until it is handed out again;
//    allocation takes the head (the least recently freed block), which then
//    leaves the registry;
//  * an append into a block another sequence also references first moves the
//    appending sequence to a fresh copy of that block (copy-on-write); the
//    caller copies the K/V with kv_copy_blocks before writing.
// Not thread-safe: one manager is driven by one host thread.
#include <algorithm>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int kB = PKV_BLOCK_SIZE;

// 64-bit mixing (splitmix64 finaliser) for the chain key.
inline uint64_t mix64(uint64_t x) {
    x += 0x9e3779b97f4a7c15ull;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
    return x ^ (x >> 31);
}

uint64_t chain_key(uint64_t prev, uint64_t salt, const int32_t* tokens) {
    uint64_t h = mix64(prev ^ 0x6a09e667f3bcc909ull);
    h = mix64(h ^ salt);
    for (int i = 0; i < kB; ++i) h = mix64(h ^ static_cast<uint32_t>(tokens[i]));
    return h == 0 ? 1 : h;   // 0 marks "not registered"
}

struct Seq {
    std::vector<int32_t> blocks;
    std::vector<int32_t> tokens;   // every token id of the sequence
    uint64_t salt = 0;
    uint64_t last_key = 0;         // chain key of the last full block (0: none)
};

}  // namespace

struct pkv_block_manager {
    int32_t num_blocks = 0;
    std::vector<int32_t> refs;
    std::vector<uint64_t> key;                 // registered chain key, 0 if none
    std::vector<uint64_t> prev_key;            // previous block's key (for exact match)
    std::vector<int32_t> block_tokens;         // [num_blocks][16] token ids of registered blocks
    std::list<int32_t> free_list;              // head: least recently freed
    std::vector<std::list<int32_t>::iterator> free_pos;
    std::vector<uint8_t> is_free;
    std::unordered_map<uint64_t, int32_t> registry;
    std::unordered_map<int64_t, Seq> seqs;

    void push_free(int32_t b) {
        free_pos[b] = free_list.insert(free_list.end(), b);
        is_free[b] = 1;
    }
    void take_free(int32_t b) {
        free_list.erase(free_pos[b]);
        is_free[b] = 0;
    }
    void unregister(int32_t b) {
        if (key[b]) {
            auto it = registry.find(key[b]);
            if (it != registry.end() && it->second == b) registry.erase(it);
            key[b] = 0;
        }
    }
    int32_t allocate() {   // caller has checked that a free block exists
        const int32_t b = free_list.front();
        take_free(b);
        unregister(b);
        refs[b] = 1;
        return b;
    }
    void release(int32_t b) {
        if (--refs[b] == 0) push_free(b);
    }
    // Registered block holding exactly (prev, salt, tokens), or -1.
    int32_t lookup(uint64_t k, uint64_t prev, const int32_t* tokens) const {
        auto it = registry.find(k);
        if (it == registry.end()) return -1;
        const int32_t b = it->second;
        if (prev_key[b] != prev) return -1;
        if (std::memcmp(&block_tokens[static_cast<size_t>(b) * kB], tokens, sizeof(int32_t) * kB)) return -1;
        return b;
    }
    void register_block(int32_t b, uint64_t k, uint64_t prev, const int32_t* tokens) {
        if (registry.count(k)) return;     // an identical block is registered already
        key[b] = k;
        prev_key[b] = prev;
        std::memcpy(&block_tokens[static_cast<size_t>(b) * kB], tokens, sizeof(int32_t) * kB);
        registry[k] = b;
    }
};

extern "C" {

pkv_status block_manager_create(int32_t num_blocks, pkv_block_manager** out) {
    if (!out) return PKV_ERR_INVALID;
    *out = nullptr;
    if (num_blocks < 1) return PKV_ERR_INVALID;
    try {
        auto* m = new pkv_block_manager;
        m->num_blocks = num_blocks;
        m->refs.assign(num_blocks, 0);
        m->key.assign(num_blocks, 0);
        m->prev_key.assign(num_blocks, 0);
        m->block_tokens.assign(static_cast<size_t>(num_blocks) * kB, 0);
        m->free_pos.resize(num_blocks);
        m->is_free.assign(num_blocks, 0);
        for (int32_t b = 0; b < num_blocks; ++b) m->push_free(b);
        *out = m;
        return PKV_OK;
    } catch (...) {
        return PKV_ERR_INVALID;
    }
}

pkv_status block_manager_destroy(pkv_block_manager* m) {
    delete m;
    return PKV_OK;
}

int32_t block_manager_free_blocks(const pkv_block_manager* m) {
    return m ? static_cast<int32_t>(m->free_list.size()) : -1;
}

pkv_status block_manager_add(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                             uint64_t salt, int32_t* out_cached_tokens, int64_t* out_slots) {
    if (!m || num_tokens < 1 || !tokens || !out_cached_tokens || !out_slots) return PKV_ERR_INVALID;
    try {
        if (m->seqs.count(seq_id)) return PKV_ERR_INVALID;
        const int32_t nblk = (num_tokens + kB - 1) / kB;
        // leading full blocks found registered (the last prompt token is always computed)
        const int32_t reusable = (num_tokens - 1) / kB;
        std::vector<int32_t> hits;
        std::vector<uint64_t> keys;
        uint64_t prev = 0;
        for (int32_t i = 0; i < reusable; ++i) {
            const uint64_t k = chain_key(prev, salt, tokens + static_cast<int64_t>(i) * kB);
            const int32_t b = m->lookup(k, prev, tokens + static_cast<int64_t>(i) * kB);
            if (b < 0) break;
            hits.push_back(b);
            keys.push_back(k);
            prev = k;
        }
        // free blocks consumed: every miss, and every hit lying in the free list
        int64_t need = nblk - static_cast<int64_t>(hits.size());
        for (int32_t b : hits) need += m->is_free[b] ? 1 : 0;
        if (need > static_cast<int64_t>(m->free_list.size())) return PKV_ERR_OUT_OF_BLOCKS;

        Seq s;
        s.salt = salt;
        s.tokens.assign(tokens, tokens + num_tokens);
        for (int32_t b : hits) {
            if (m->is_free[b]) {
                m->take_free(b);
                m->refs[b] = 1;
            } else {
                ++m->refs[b];
            }
            s.blocks.push_back(b);
        }
        for (int32_t i = static_cast<int32_t>(hits.size()); i < nblk; ++i) s.blocks.push_back(m->allocate());
        // register the newly filled full blocks (their K/V is written by the caller next)
        for (int32_t i = 0; i < num_tokens / kB; ++i) {
            const int32_t* t = tokens + static_cast<int64_t>(i) * kB;
            const uint64_t k = i < static_cast<int32_t>(keys.size()) ? keys[i] : chain_key(prev, salt, t);
            if (i >= static_cast<int32_t>(keys.size())) {
                m->register_block(s.blocks[i], k, prev, t);
                prev = k;
            }
            s.last_key = k;
        }
        const int32_t cached = static_cast<int32_t>(hits.size()) * kB;
        for (int32_t t = cached; t < num_tokens; ++t)
            out_slots[t - cached] = static_cast<int64_t>(s.blocks[t / kB]) * kB + t % kB;
        *out_cached_tokens = cached;
        m->seqs.emplace(seq_id, std::move(s));
        return PKV_OK;
    } catch (...) {
        return PKV_ERR_INVALID;
    }
}

pkv_status block_manager_append(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                                int64_t* out_slots, int32_t* out_copies, int32_t* out_num_copies) {
    if (!m || num_tokens < 0 || (num_tokens > 0 && (!tokens || !out_slots)) || !out_num_copies)
        return PKV_ERR_INVALID;
    try {
        auto it = m->seqs.find(seq_id);
        if (it == m->seqs.end()) return PKV_ERR_INVALID;
        Seq& s = it->second;
        *out_num_copies = 0;
        if (num_tokens == 0) return PKV_OK;
        int32_t len = static_cast<int32_t>(s.tokens.size());
        // blocks needed: a copy of a shared partial last block, and new blocks
        int64_t need = 0;
        if (len % kB && m->refs[s.blocks.back()] > 1) ++need;
        need += (len + num_tokens + kB - 1) / kB - (len + kB - 1) / kB;
        if (need > static_cast<int64_t>(m->free_list.size())) return PKV_ERR_OUT_OF_BLOCKS;
        if (need > 0 && len % kB && m->refs[s.blocks.back()] > 1 && !out_copies) return PKV_ERR_INVALID;
        for (int32_t j = 0; j < num_tokens; ++j) {
            const int32_t off = len % kB;
            if (off == 0) {
                s.blocks.push_back(m->allocate());
            } else if (m->refs[s.blocks.back()] > 1) {
                // copy-on-write: this sequence moves to a private copy
                const int32_t src = s.blocks.back();
                const int32_t dst = m->allocate();
                m->release(src);
                s.blocks.back() = dst;
                out_copies[2 * *out_num_copies] = src;
                out_copies[2 * *out_num_copies + 1] = dst;
                ++*out_num_copies;
            }
            out_slots[j] = static_cast<int64_t>(s.blocks.back()) * kB + off;
            s.tokens.push_back(tokens[j]);
            ++len;
            if (len % kB == 0) {   // the block is full: register it for reuse
                const int32_t* t = s.tokens.data() + (len - kB);
                const uint64_t k = chain_key(s.last_key, s.salt, t);
                m->register_block(s.blocks.back(), k, s.last_key, t);
                s.last_key = k;
            }
        }
        return PKV_OK;
    } catch (...) {
        return PKV_ERR_INVALID;
    }
}

pkv_status block_manager_fork(pkv_block_manager* m, int64_t parent_id, int64_t child_id) {
    if (!m) return PKV_ERR_INVALID;
    try {
        auto it = m->seqs.find(parent_id);
        if (it == m->seqs.end() || m->seqs.count(child_id)) return PKV_ERR_INVALID;
        Seq c = it->second;
        for (int32_t b : c.blocks) ++m->refs[b];
        m->seqs.emplace(child_id, std::move(c));
        return PKV_OK;
    } catch (...) {
        return PKV_ERR_INVALID;
    }
}

pkv_status block_manager_free(pkv_block_manager* m, int64_t seq_id) {
    if (!m) return PKV_ERR_INVALID;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_ERR_INVALID;
    // release from the last block backwards, so a sequence's prefix blocks are
    // the last of its blocks to be handed out again
    const std::vector<int32_t>& blocks = it->second.blocks;
    for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) m->release(*b);
    m->seqs.erase(it);
    return PKV_OK;
}

pkv_status block_manager_table(const pkv_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t* out_table, int32_t* out_seq_lens) {
    if (!m || !seq_ids || num_seqs < 1 || max_blocks_per_seq < 1 || !out_table || !out_seq_lens)
        return PKV_ERR_INVALID;
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = m->seqs.find(seq_ids[i]);
        if (it == m->seqs.end()) return PKV_ERR_INVALID;
        if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks_per_seq) return PKV_ERR_SEQ_LEN;
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const Seq& s = m->seqs.find(seq_ids[i])->second;
        int32_t* row = out_table + static_cast<int64_t>(i) * max_blocks_per_seq;
        std::fill(row, row + max_blocks_per_seq, -1);
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        out_seq_lens[i] = static_cast<int32_t>(s.tokens.size());
    }
    return PKV_OK;
}

int32_t block_manager_refcount(const pkv_block_manager* m, int32_t block) {
    if (!m || block < 0 || block >= m->num_blocks) return -1;
    return m->refs[block];
}

}  // extern "C"
