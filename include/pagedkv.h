/*
 * pagedkv.h - C ABI of a paged KV-cache decode-attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (the pages this library follows):
 *
 *  - Page "KV cache & continuous batching" (docs.masst.dev), section "The core
 *    insight": a decode step computes the query of the new token only and
 *    attends over the cached keys and values of every earlier token.  Section
 *    "KV cache memory math": the cache holds K and V per layer, per KV head and
 *    per token; grouped-query attention lets several query heads share one KV
 *    head.  Section "Visual: the lifecycle of a request in continuous
 *    batching": the cache is handed out in blocks of 16 tokens.  Section
 *    "2. PagedAttention (vLLM)": each request has a block table mapping its
 *    logical blocks to physical blocks that need not be contiguous, and the
 *    attention kernel gathers K and V through that list of blocks.  Section
 *    "5. Speculative decoding": the target model checks K drafted tokens in one
 *    forward pass at length current + K.
 *  - Page "LLM Serving - KV Cache, Batching, Speculative Decoding"
 *    (dineshblog.com), section "KV memory, paging and prefix identity": logical
 *    blocks map to physical blocks, which several sequences may share.
 *  - Page "LLM Inference Optimization: KV Cache, Batching, and Speculative
 *    Decoding" (adaptiverecall.com), section "Memory Bandwidth Optimization":
 *    decode reads the entire cache for each new token, and storing the cache in
 *    one byte per element halves those reads.
 *
 * Conventions shared by every call
 *  - Device pointers ("dev_") point to memory the caller allocated on the GPU
 *    the call runs on; host pointers ("host_") to ordinary host memory read
 *    only during the call.  The library never allocates device memory.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Work is enqueued asynchronously on it; order between calls is the
 *    caller's, by using one stream.
 *  - Every call returns a pkv_status: 0 on success, a negative code on error.
 *    On an error nothing has been enqueued (except PKV_ERR_HIP, which reports
 *    a failure of the HIP runtime while enqueuing).  No call throws.
 *  - Handles (pkv_pool, pkv_table) are immutable after creation and hold
 *    non-owning pointers; destroying a handle frees only the handle.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16
#define PKV_ABI_VERSION 1

typedef int32_t pkv_status;
#define PKV_OK               0
#define PKV_ERR_INVALID     (-1) /* null pointer, bad count or size, bad layer  */
#define PKV_ERR_UNSUPPORTED (-2) /* dtype combination, head_dim, block size    */
#define PKV_ERR_BLOCK_RANGE (-3) /* a used block-table entry outside the pool  */
#define PKV_ERR_SEQ_LEN     (-4) /* seq_len < 1, > table capacity, or < rows   */
#define PKV_ERR_WORKSPACE   (-5) /* device buffer or workspace too small       */
#define PKV_ERR_HIP         (-6) /* the HIP runtime reported an error          */
#define PKV_ERR_OUT_OF_BLOCKS (-7) /* block manager: not enough free blocks     */
#define PKV_ERR_TABLE_STALE (-8) /* an earlier attention launch on this table
                                    failed; its merge counters may not be zero:
                                    upload the table again                      */

/* Element types. */
#define PKV_F32      0  /* IEEE binary32                                        */
#define PKV_BF16     1  /* bfloat16 (upper half of a binary32)                  */
#define PKV_FP8_E4M3 2  /* OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, NaN S.1111.111,
                           no infinities) times a float32 scale per (layer, KV head) */
#define PKV_INT8     3  /* symmetric int8 code in [-127, 127] times a float32 scale per
                           (layer, KV head); written as sat127(round-half-even(
                           f32(x) * f32(1 / scale))), NaN written as 0 (page "KV cache &
                           continuous batching", section "KV cache memory math": one
                           byte per element for fp8 or int8) */
#define PKV_INT4     4  /* symmetric int4 code in [-7, 7] times a float32 scale per
                           (layer, KV head); written as sat7(round-half-even(
                           f32(x) * f32(1 / scale))), NaN written as 0; two codes per
                           byte, low nibble first, two's complement (page "LLM
                           Inference Optimization: KV Cache, Batching, and
                           Speculative Decoding", section "Memory Bandwidth
                           Optimization": int4 KV at half a byte per element) */

/*
 * Pool geometry.
 *
 * The pool is one caller-owned device buffer of kv_pool_bytes(desc) bytes,
 * i.e. num_blocks * 16 token slots times the per-token size
 * 2 * num_layers * num_kv_heads * head_dim * b (b = 4, 2, 1, 1/2 bytes), which is
 * the per-token formula of page "KV cache & continuous batching", section "KV
 * cache memory math", applied to the pool's capacity.
 *
 * Byte layout.  The buffer is an array of tiles, one per
 * (layer l, physical block p, KV head h, kv in {K = 0, V = 1}); tile
 * (l, p, h, kv) starts at byte
 *        ((((l * num_blocks + p) * num_kv_heads + h) * 2 + kv) * TILE,
 *        TILE = 16 * head_dim * b.
 * Inside a K tile, element (token offset o in [0,16), dim i) is element number
 *        ((i / X) * 16 + o) * X + (i % X),   X = 16 / b,
 * i.e. 16-byte chunks of X consecutive dims, chunk-major then token.  Inside a
 * V tile, element (o, i) is element number  i * 16 + o  (V stored transposed).
 * PKV_INT4 tiles are instead nibble arrays (nibble N = byte N / 2, low nibble
 * when N is even), laid out so that no byte holds codes of two tokens and each
 * of the attention kernel's 64 lanes reads one contiguous run; with
 * W = head_dim / 4 nibbles per run:
 *   K (o, i), i = 32 s + 8 g + e (e < 8, g < 4):   N = (g * 16 + o) * W + 8 s + e
 *   V (o, i), o = 4 g + t, i = 16 m + c (c < 16):  N = (g * 16 + c) * W + 8 (m / 2) + 2 t + (m % 2)
 * (a V run's byte 4 j + t holds token 4 g + t at dims 16 (2 j) + c, low
 * nibble, and 16 (2 j + 1) + c, high nibble).
 * Token position t of a sequence with block table row `bt` lives at block
 * bt[t / 16], offset t % 16; its flat slot is bt[t / 16] * 16 + t % 16.
 * For PKV_FP8_E4M3, PKV_INT8 and PKV_INT4 the stored code c of head h in layer l stands for the value
 * decode(c) * scale[l][h], with separate K and V scale arrays.
 */
typedef struct pkv_pool_desc {
    int32_t num_layers;    /* >= 1                                    */
    int32_t num_blocks;    /* >= 1 physical blocks per layer          */
    int32_t num_kv_heads;  /* >= 1                                    */
    int32_t head_dim;      /* 64 or 128                               */
    int32_t block_size;    /* must be PKV_BLOCK_SIZE (16)             */
    int32_t kv_dtype;      /* PKV_F32, PKV_BF16, PKV_FP8_E4M3, PKV_INT8, PKV_INT4 */
} pkv_pool_desc;

typedef struct pkv_pool pkv_pool;
typedef struct pkv_table pkv_table;

/* ABI version (PKV_ABI_VERSION of the built library). */
int32_t pkv_abi_version(void);

/* Static description of a status code; never NULL. */
const char* pkv_status_string(pkv_status status);

/*
 * Bytes one token adds to the cache across all layers: 2 * L * H_kv * d * b
 * (page "KV cache & continuous batching", section "KV cache memory math";
 * page "LLM Serving - KV Cache, Batching, Speculative Decoding", section "KV
 * memory, paging and prefix identity").  Returns -1 for invalid arguments.
 */
int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                           int32_t kv_dtype);

/* Bytes of the pool described by desc (layout above); -1 if desc is invalid. */
int64_t kv_pool_bytes(const pkv_pool_desc* desc);

/*
 * Wrap a caller-allocated pool buffer in a handle: the physical blocks the
 * block tables name (page "KV cache & continuous batching", section
 * "2. PagedAttention (vLLM)": the cache is split into fixed-size physical
 * blocks that need not be contiguous, handed to requests on demand; section
 * "KV cache memory math" for the bytes per token; page "LLM Serving - KV
 * Cache, Batching, Speculative Decoding", section "KV memory, paging and
 * prefix identity": physical blocks may be shared by several sequences).
 *   dev_base   device buffer of at least kv_pool_bytes(desc) bytes, 256-byte aligned.
 *   dev_k_scale, dev_v_scale  float32 [num_layers][num_kv_heads] device arrays;
 *              required (non-NULL) for PKV_FP8_E4M3, PKV_INT8 and PKV_INT4, ignored otherwise.
 * Errors: PKV_ERR_INVALID (null, short or misaligned buffer, bad counts),
 *         PKV_ERR_UNSUPPORTED (block_size != 16, head_dim not 64/128, dtype).
 * The buffer contents are not touched.
 */
pkv_status kv_pool_create(const pkv_pool_desc* desc, void* dev_base, size_t dev_bytes,
                          const float* dev_k_scale, const float* dev_v_scale,
                          pkv_pool** out);
pkv_status kv_pool_destroy(pkv_pool* pool);

/*
 * Device bytes block_table_upload needs for this batch: the tables, the
 * lengths and the split-KV plan (which depends on the lengths, the pool's KV
 * head count and, for partition_tokens = -1 or -2, the device's CU count).  Same
 * arguments as block_table_upload.  0 for invalid arguments.
 */
size_t block_table_device_bytes(const pkv_pool* pool, const int32_t* host_seq_lens, int32_t num_seqs,
                                int32_t max_blocks_per_seq, int32_t partition_tokens);

/*
 * Validate a batch of block tables, plan its split-KV partitions and copy
 * both to the device (page "KV cache & continuous batching", section
 * "2. PagedAttention (vLLM)": one table per request, logical block -> physical
 * block).
 *   host_block_table  int32 [num_seqs][max_blocks_per_seq], row-major.  Entry
 *                     j of row s is used iff j < ceil(seq_len[s] / 16); every
 *                     used entry must lie in [0, pool num_blocks).  Unused
 *                     entries are ignored (any value).  Rows may share entries.
 *   host_seq_lens     int32 [num_seqs]: positions visible to the last query row
 *                     of each sequence, counting tokens appended this step;
 *                     1 <= seq_len <= max_blocks_per_seq * 16.
 *   partition_tokens  split-KV plan: a positive multiple of 16 cuts every
 *                     sequence into partitions of that many tokens (the last
 *                     one shorter); 0 keeps each sequence whole; -1 cuts each
 *                     sequence into near-equal partitions sized so the whole
 *                     batch gives about one wave of work-groups on the device
 *                     (balanced plan).  A split sequence's partitions are
 *                     attended independently and their partial results
 *                     merged (inside the attention kernel for up to 32
 *                     partitions, by a second kernel beyond that).
 *                     With -1 or -2 the upload also looks for a shared prefix (page
 *                     "KV cache & continuous batching", section "4. Prefix
 *                     caching / prompt caching": requests with a common
 *                     prefix reuse its cached K/V; page "LLM Serving - KV
 *                     Cache, Batching, Speculative Decoding", section "KV
 *                     memory, paging and prefix identity"): the longest run
 *                     of leading physical blocks that every row names alike,
 *                     kept when it holds 8 or more blocks, the batch has 4 or
 *                     more sequences, the pool is not PKV_F32 and every
 *                     sequence has a position past it.  An attention call on
 *                     such a table whose rows all see the whole prefix
 *                     (shortest seq_len - query_rows >= 16 * prefix blocks)
 *                     attends to the prefix once for all sequences' query
 *                     rows (a dense pass over the shared blocks, in up to 4
 *                     chunks, each giving a partial result per row) and
 *                     walks only each sequence's own blocks, merged with
 *                     the prefix partials: the
 *                     same softmax, split at the prefix end.  With -1 the
 *                     prefix plan is kept only when a rough cost model
 *                     (the prefix pass's chunk walk against every
 *                     sequence reading the prefix) favours it; -2 keeps it
 *                     whenever a prefix is found.  Each sequence's own
 *                     blocks are cut as the balanced plan cuts sequences.
 *   dev_buffer        device buffer of >= block_table_device_bytes(...) bytes;
 *                     it must stay valid and unmodified while the table is in use.
 * The host arrays are copied into the handle before returning; the copy to
 * dev_buffer is enqueued on `stream`.  Destroying the handle waits for that
 * copy.  The buffer also holds the arrival counters of the in-kernel merge,
 * which every attention launch that completes leaves at zero: attention calls
 * that use one table must not overlap (issue them on one stream).  A table
 * whose attention launch returned PKV_ERR_HIP is marked stale and refused by
 * later attention calls (PKV_ERR_TABLE_STALE) until it is uploaded again.
 * Errors: PKV_ERR_INVALID, PKV_ERR_BLOCK_RANGE, PKV_ERR_SEQ_LEN,
 * PKV_ERR_WORKSPACE (dev_buffer too small), PKV_ERR_HIP.
 */
pkv_status block_table_upload(const pkv_pool* pool, const int32_t* host_block_table,
                              int32_t num_seqs, int32_t max_blocks_per_seq,
                              const int32_t* host_seq_lens, int32_t partition_tokens,
                              void* dev_buffer, size_t dev_buffer_bytes, void* stream,
                              pkv_table** out);
pkv_status block_table_destroy(pkv_table* table);

/*
 * Facts of an uploaded table (any output pointer may be NULL): number of
 * (sequence, partition) work units, partial-result slots of split sequences,
 * the longest and shortest sequence, and the most partitions of one sequence
 * (above 32, attention calls launch the separate merge kernel).
 */
pkv_status block_table_info(const pkv_table* table, int32_t* num_units, int32_t* num_split_slots,
                            int32_t* max_seq_len, int32_t* min_seq_len, int32_t* max_parts);

/*
 * The table's shared prefix (see block_table_upload, partition_tokens = -1, -2):
 * its length in blocks and the chunks the prefix pass cuts it into; both 0
 * when the table has none.  Either output pointer may be NULL.
 */
pkv_status block_table_shared_prefix(const pkv_table* table, int32_t* prefix_blocks, int32_t* prefix_chunks);

/*
 * Slot of each (sequence, position) pair through the uploaded tables:
 *   slot = table[seq][pos / 16] * 16 + pos % 16
 * (page "KV cache & continuous batching", section "2. PagedAttention (vLLM)").
 *   dev_seq_ids, dev_positions  int32 [num_tokens]; dev_slot_mapping int64 [num_tokens] out.
 * A pair whose sequence is outside the batch, whose position is negative or
 * beyond the row's capacity (max_blocks_per_seq * 16), or whose table entry is
 * outside the pool gets slot -1.  num_tokens == 0 enqueues nothing.
 */
pkv_status slot_mapping_compute(const pkv_table* table, const int32_t* dev_seq_ids,
                                const int32_t* dev_positions, int32_t num_tokens,
                                int64_t* dev_slot_mapping, void* stream);

/*
 * Append new tokens' K and V to the pool through a slot mapping (the decode
 * step extends the cache before attending: page "KV cache & continuous
 * batching", section "The core insight"; page "LLM Serving - KV Cache,
 * Batching, Speculative Decoding", section "Hands-on: cache equivalence and
 * scheduling oracles").
 *   dev_k_new, dev_v_new  [num_tokens][num_kv_heads][head_dim], element type in_dtype.
 *   in_dtype     PKV_F32 for an F32 pool, PKV_BF16 for a BF16 pool, PKV_F32 or
 *                PKV_BF16 for an FP8, INT8 or INT4 pool.
 *   dev_slot_mapping  int64 [num_tokens]; a slot outside [0, num_blocks * 16)
 *                (e.g. -1) skips its token.  Two tokens with the same slot race.
 * F32 and BF16 pools store the input bits unchanged.  FP8 pools store
 *   e4m3( sat448( f32(x) * f32(1 / scale[layer][h]) ) )
 * with round-to-nearest-even, saturation to +-448 and NaN kept NaN; INT8 and
 * INT4 pools the codes their element types define.
 */
pkv_status reshape_and_cache(const pkv_pool* pool, int32_t layer, const void* dev_k_new,
                             const void* dev_v_new, int32_t in_dtype,
                             const int64_t* dev_slot_mapping, int32_t num_tokens,
                             void* stream);

/*
 * Workspace bytes paged_attention_decode (query_rows = 1) or
 * paged_attention_verify needs with this pool and table: the split-KV partial
 * results (float32 output, max and sum per partition, query row and KV head),
 * with a shared prefix also those of the prefix chunks.
 * 0 when no sequence is split.  Returns 0 for invalid arguments as well.
 */
size_t paged_attention_workspace_bytes(const pkv_pool* pool, const pkv_table* table,
                                       int32_t num_q_heads, int32_t query_rows);

/*
 * Decode attention, one query token per sequence (page "KV cache & continuous
 * batching", section "The core insight": the new token's query attends over
 * the cached K and V of every earlier token and its own; section
 * "2. PagedAttention (vLLM)": K and V are gathered through the sequence's list
 * of blocks; section "KV cache memory math": query heads of a group share a KV
 * head; page "LLM Serving - KV Cache, Batching, Speculative Decoding", section
 * "Hands-on: cache equivalence and scheduling oracles": the cached result is
 * softmax attention over the visible rows):
 *   out[s][g] = softmax( scale * q[s][g] . K_s[t][h]^T, t < seq_len[s] ) V_s[t][h],
 *   h = g / (num_q_heads / num_kv_heads)          (grouped-query sharing)
 * with K_s, V_s read from `layer` of the pool through the table's block list.
 *   dev_q    [num_seqs][num_q_heads][head_dim], q_dtype.
 *   dev_out  [num_seqs][num_q_heads][head_dim], out_dtype.
 *   q_dtype  PKV_F32 with an F32 pool; PKV_BF16 with BF16, FP8, INT8 and INT4 pools.
 *   out_dtype  PKV_F32 or PKV_BF16 (round to nearest even).
 *   scale    softmax scale (typically 1/sqrt(head_dim)).
 *   dev_workspace  >= paged_attention_workspace_bytes(pool, table, num_q_heads, 1)
 *            bytes (may be NULL when that is 0); no initial contents needed.
 * num_q_heads must be a multiple of num_kv_heads with at most 64 query heads
 * per KV head.  Accumulation is float32; bf16 operands (fp8, int8 and int4
 * codes convert to bf16 exactly) go through the matrix cores with float32
 * accumulation, probabilities rounded to bfloat16.
 * Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_BLOCK_RANGE (the table's
 * entries do not fit this pool), PKV_ERR_WORKSPACE, PKV_ERR_HIP (the table is
 * then marked stale), PKV_ERR_TABLE_STALE (an earlier launch on this table
 * failed: upload it again).
 */
pkv_status paged_attention_decode(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                  const void* dev_q, int32_t q_dtype, int32_t num_q_heads,
                                  float scale, void* dev_workspace, size_t workspace_bytes,
                                  void* dev_out, int32_t out_dtype, void* stream);

/*
 * Speculative verify attention, query_rows (= k) query tokens per sequence
 * (page "KV cache & continuous batching", section "5. Speculative decoding";
 * page "LLM Inference Optimization: KV Cache, Batching, and Speculative
 * Decoding", section "Speculative Decoding").  The k rows of sequence s are
 * positions n-k .. n-1 (n = seq_len[s]) whose K/V were appended beforehand;
 * row j attends causally to positions t <= n - k + j.
 *   dev_q, dev_out  [num_seqs][k][num_q_heads][head_dim].
 * (query rows per KV head) = k * num_q_heads / num_kv_heads must be <= 64,
 * and every seq_len >= k (else PKV_ERR_SEQ_LEN).  Otherwise as decode, which is
 * this call with k = 1.
 */
pkv_status paged_attention_verify(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                  const void* dev_q, int32_t q_dtype, int32_t query_rows,
                                  int32_t num_q_heads, float scale, void* dev_workspace,
                                  size_t workspace_bytes, void* dev_out, int32_t out_dtype,
                                  void* stream);

/*
 * paged_attention_verify without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split-KV partial results go to a
 * static device array of PKV_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends (its address is looked
 * up on the first call on that device; the call allocates nothing).  A table
 * whose partials need more (paged_attention_workspace_bytes(...) >
 * PKV_NOALLOC_SCRATCH_BYTES) is refused with PKV_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares its array: calls that
 * may overlap on one GPU (other streams, other host threads) race and must
 * be serialised by the caller.  Nothing in the array needs clearing between
 * calls: each call writes every partial it reads.  Arguments, results and
 * other errors as paged_attention_verify (decode when query_rows = 1).
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pkv_status paged_attention_verify_noalloc(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                          const void* dev_q, int32_t q_dtype, int32_t query_rows,
                                          int32_t num_q_heads, float scale, void* dev_out,
                                          int32_t out_dtype, void* stream);

/*
 * One decode (or verify) step in one launch: append the K and V of every
 * sequence's k newest tokens to the pool, then attend.  Equivalent to
 * slot_mapping_compute for positions n-k .. n-1 of each sequence, then
 * reshape_and_cache, then paged_attention_verify (decode when k = 1), and
 * writes the same pool bytes and outputs (page "KV cache & continuous
 * batching", section "The core insight": a step extends the cache with the
 * new token and attends over it; section "2. PagedAttention (vLLM)" for the
 * slot rule).
 *   dev_k_new, dev_v_new  [num_seqs][query_rows][num_kv_heads][head_dim] in
 *                 in_dtype (as reshape_and_cache): row j of sequence s is the
 *                 token at position seq_len[s] - query_rows + j.
 *   other arguments as paged_attention_verify.
 * The work-group that attends over a token's block writes the token; its own
 * attention takes the token's K/V codes from on-chip memory, so the write
 * completes by the end of the call but is not waited for before the blocks
 * are read.  Errors as paged_attention_verify, plus
 * PKV_ERR_INVALID for null token pointers and PKV_ERR_UNSUPPORTED for an
 * in_dtype the pool does not take.
 */
pkv_status paged_attention_append(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                  const void* dev_k_new, const void* dev_v_new, int32_t in_dtype,
                                  const void* dev_q, int32_t q_dtype, int32_t query_rows,
                                  int32_t num_q_heads, float scale, void* dev_workspace,
                                  size_t workspace_bytes, void* dev_out, int32_t out_dtype,
                                  void* stream);

/*
 * Chunked-prefill attention (page "KV cache & continuous batching", section
 * "3. Chunked prefill": a long prompt is fed in chunks of a few thousand
 * tokens, each attending over the cache of all earlier positions and over
 * itself; page "LLM Inference Optimization: KV Cache, Batching, and
 * Speculative Decoding", section "Prefill Optimization").  Every sequence
 * carries chunk_tokens (= C) query tokens at positions n-C .. n-1 (n =
 * seq_len[s]) whose K/V were appended beforehand (reshape_and_cache); row j
 * attends causally to positions t <= n - C + j:
 *   out[s][j][g] = softmax( scale * q[s][j][g] . K_s[t][h]^T, t <= n-C+j ) V_s[t][h],
 *   h = g / (num_q_heads / num_kv_heads).
 * It is the computation of paged_attention_verify with C rows, for any C:
 * the kernel keeps each work-group's 192 query rows resident and streams the
 * visible K/V blocks through LDS, bound by the matrix cores.
 *   dev_q    [num_seqs][C][num_q_heads][head_dim] bfloat16.
 *   dev_out  [num_seqs][C][num_q_heads][head_dim], out_dtype PKV_BF16 or PKV_F32.
 *   Pools: PKV_BF16, PKV_FP8_E4M3, PKV_INT8 or PKV_INT4 (PKV_F32 pools:
 *   PKV_ERR_UNSUPPORTED).
 * No workspace.  The table's split-KV plan is not used (any partition_tokens).
 * Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_SEQ_LEN (a sequence
 * shorter than C), PKV_ERR_BLOCK_RANGE, PKV_ERR_HIP.
 */
pkv_status paged_attention_prefill(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                   const void* dev_q, int32_t q_dtype, int32_t chunk_tokens,
                                   int32_t num_q_heads, float scale, void* dev_out, int32_t out_dtype,
                                   void* stream);

/*
 * Chunked-prefill attention with a chunk length per sequence (page "KV cache
 * & continuous batching", section "3. Chunked prefill": prompts of any length
 * are cut into chunks, so one batch carries a full chunk of one prompt and the
 * shorter last chunk of another).  Sequence s carries C_s =
 * host_query_start[s + 1] - host_query_start[s] query tokens (0 allowed) at
 * positions n-C_s .. n-1 of its sequence, their K/V appended beforehand; row
 * j attends causally to positions t <= n - C_s + j, as
 * paged_attention_prefill computes for a uniform C.
 *   dev_q, dev_out  [host_query_start[num_seqs]][num_q_heads][head_dim]: the
 *            chunks' rows packed in sequence order (sequence s from row
 *            host_query_start[s]).
 *   host_query_start  int32 [num_seqs + 1] host array, read during the call:
 *            0 = qs[0] <= qs[1] <= ... and qs[s + 1] - qs[s] <= seq_len[s].
 *   dev_query_start   the same values in a device array, read by the kernel
 *            (the caller keeps the two equal).
 * Other arguments, pools and errors as paged_attention_prefill; PKV_ERR_INVALID
 * for a decreasing or non-zero-based host_query_start, PKV_ERR_SEQ_LEN for a
 * chunk longer than its sequence.  A batch with no chunk token enqueues nothing.
 */
pkv_status paged_attention_prefill_varlen(const pkv_pool* pool, int32_t layer, const pkv_table* table,
                                          const void* dev_q, int32_t q_dtype, const int32_t* host_query_start,
                                          const int32_t* dev_query_start, int32_t num_q_heads, float scale,
                                          void* dev_out, int32_t out_dtype, void* stream);

/*
 * Exact speculative acceptance (page "LLM Serving - KV Cache, Batching,
 * Speculative Decoding", section "Speculative decoding: distribution and
 * break-even"; page "KV cache & continuous batching", section "5. Speculative
 * decoding").  For each sequence the draft proposed K = draft_tokens tokens
 * x_0..x_{K-1} from its distributions q_0..q_{K-1}, and one target pass (the
 * verify attention above) gave p_0..p_K.  Position i accepts x_i with
 * probability min(1, p_i(x_i) / q_i(x_i)), decided as the float32 test
 * u_accept[i] * q_i(x_i) < p_i(x_i); a draft token outside [0, vocab) is
 * rejected.  The first rejected position a emits a token drawn from
 * max(p_a - q_a, 0) (p_a itself if that has no mass); a fully accepted block
 * (a = K) emits a bonus token drawn from p_K.  Drawing from weights w with u:
 * the smallest j with w_0 + .. + w_j > u * sum(w), sums in float32.  The
 * emitted tokens follow the target's distribution.
 *   dev_p         float32 [num_seqs][K+1][vocab] target probabilities
 *   dev_q         float32 [num_seqs][K][vocab] draft probabilities
 *                 (both 16-byte aligned; rows need not sum to exactly 1)
 *   dev_draft     int32 [num_seqs][K]
 *   dev_u_accept  float32 [num_seqs][K] uniforms in [0, 1)
 *   dev_u_sample  float32 [num_seqs] uniforms in [0, 1)
 *   dev_num_accepted  int32 [num_seqs] out: a
 *   dev_tokens    int32 [num_seqs][K+1] out: x_0..x_{a-1}, the drawn token, then -1
 * One work-group per sequence reads the K tested entries and one row (two
 * for a residual).  Errors: PKV_ERR_INVALID (null or misaligned pointer,
 * draft_tokens < 1, vocab < 1), PKV_ERR_UNSUPPORTED (draft_tokens > 1024),
 * PKV_ERR_HIP.
 */
pkv_status speculative_accept(const float* dev_p, const float* dev_q, const int32_t* dev_draft,
                              const float* dev_u_accept, const float* dev_u_sample, int32_t num_seqs,
                              int32_t draft_tokens, int32_t vocab, int32_t* dev_num_accepted,
                              int32_t* dev_tokens, void* stream);

/*
 * Block copies for copy-on-write (see the block manager below): for each pair
 * (src, dst) of dev_pairs (int32 [num_pairs][2]), every layer's K and V tiles
 * of physical block src, all KV heads, are copied to block dst.  Pairs with
 * an id outside [0, num_blocks) or src == dst are skipped.  Pairs must not
 * overlap (no block both written and read by the call).
 */
pkv_status kv_copy_blocks(const pkv_pool* pool, const int32_t* dev_pairs, int32_t num_pairs, void* stream);

/*
 * Block manager (host only, no device memory): hands out the pool's physical
 * blocks (page "KV cache & continuous batching", section "Visual: the
 * lifecycle of a request in continuous batching": 16-token blocks, a finished
 * request frees its blocks at once; section "2. PagedAttention (vLLM)":
 * blocks allocated on demand, one table per request; section "4. Prefix
 * caching / prompt caching": prefix blocks hashed and reused across requests;
 * page "LLM Serving - KV Cache, Batching, Speculative Decoding", section "KV
 * memory, paging and prefix identity": shared physical blocks, reuse only for
 * the exact token prefix, a salt separates tenants).
 *   Reuse: a full block is registered under the chain of (previous block,
 *   salt, its 16 token ids); a new request takes the longest run of leading
 *   registered blocks that match exactly (token ids compared), but at most
 *   len-1 tokens (its last prompt token is always computed).  Freed blocks
 *   stay findable until handed out again; allocation takes the least
 *   recently freed block first.
 *   Forks share every block; an append into a partial block that another
 *   sequence also holds moves the appending sequence to a fresh block first
 *   and reports the (src, dst) pair for kv_copy_blocks, which the caller runs
 *   before writing the new tokens.
 * A manager is driven from one host thread.  Sequence ids are the caller's.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks blocks (all free).  Errors: PKV_ERR_INVALID. */
pkv_status block_manager_create(int32_t num_blocks, pkv_block_manager** out);
pkv_status block_manager_destroy(pkv_block_manager* manager);

/* Free blocks (registered or not), or -1 for a NULL manager. */
int32_t block_manager_free_blocks(const pkv_block_manager* manager);

/* Reference count of a physical block (sequences holding it), or -1. */
int32_t block_manager_refcount(const pkv_block_manager* manager, int32_t block);

/*
 * A new sequence with its prompt tokens host_tokens[num_tokens] (token ids).
 *   *out_cached_tokens  leading tokens whose K/V is already in the pool
 *                       (a multiple of 16, < num_tokens);
 *   out_slots           int64 [num_tokens - cached]: slots of the remaining
 *                       tokens, for reshape_and_cache.
 * Errors: PKV_ERR_INVALID (NULL, num_tokens < 1, seq_id in use),
 * PKV_ERR_OUT_OF_BLOCKS (nothing changed).
 */
pkv_status block_manager_add(pkv_block_manager* manager, int64_t seq_id, const int32_t* host_tokens,
                             int32_t num_tokens, uint64_t salt, int32_t* out_cached_tokens,
                             int64_t* out_slots);

/*
 * Append num_tokens generated tokens: out_slots int64 [num_tokens]; if the
 * sequence's partial last block is shared, *out_num_copies = 1 and
 * out_copies[0..1] = (src, dst) (out_copies may be NULL only when no copy
 * can arise); else *out_num_copies = 0.  Errors: PKV_ERR_INVALID,
 * PKV_ERR_OUT_OF_BLOCKS (nothing changed).
 */
pkv_status block_manager_append(pkv_block_manager* manager, int64_t seq_id, const int32_t* host_tokens,
                                int32_t num_tokens, int64_t* out_slots, int32_t* out_copies,
                                int32_t* out_num_copies);

/* A new sequence child_id sharing every block of parent_id. */
pkv_status block_manager_fork(pkv_block_manager* manager, int64_t parent_id, int64_t child_id);

/* Finish a sequence: its blocks' reference counts drop, blocks at 0 are free. */
pkv_status block_manager_free(pkv_block_manager* manager, int64_t seq_id);

/*
 * The block-table batch of the given sequences, for block_table_upload:
 * out_table int32 [num_seqs][max_blocks_per_seq] (unused entries -1),
 * out_seq_lens int32 [num_seqs].  Errors: PKV_ERR_INVALID (unknown id),
 * PKV_ERR_SEQ_LEN (a sequence needs more than max_blocks_per_seq blocks).
 */
pkv_status block_manager_table(const pkv_block_manager* manager, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t* out_table, int32_t* out_seq_lens);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
