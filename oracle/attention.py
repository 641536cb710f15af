"""Float64 softmax attention over a paged cache (oracle, test infrastructure only).

Definition followed:

* page "KV cache & continuous batching", section "The core insight": at a
  decode step only the new token's query is computed, and it attends over the
  cached K and V of every earlier token (and, as the cache is appended before
  attending, its own);
* page "LLM Serving - KV Cache, Batching, Speculative Decoding", section
  "Hands-on: cache equivalence and scheduling oracles": the cached result is
  softmax(q K^T * scale) V over the visible rows, which equals the last row of
  full causal attention;
* same page, section "KV memory, paging and prefix identity", and page "KV
  cache & continuous batching", section "KV cache memory math": GQA query heads
  share KV heads; query head g reads KV head g // G with G = H_q / H_kv (the
  pages give only the head counts; consecutive grouping is the reading taken);
* page "KV cache & continuous batching", section "5. Speculative decoding", and
  page "LLM Inference Optimization: KV Cache, Batching, and Speculative
  Decoding", section "Speculative Decoding": the target checks the drafted
  tokens in one pass at length current + K.  Reading taken: the k query rows of
  a sequence sit at positions n-k .. n-1 (their K/V already appended) and row j
  sees positions t <= n-k+j (causal among the k rows).

Everything is float64: the score row is scaled, its maximum subtracted, it is
exponentiated, normalised to sum 1, and multiplied into V.
"""

import numpy as np

from .pool import gather_kv


def softmax_attention(q, K, V, scale, visible):
    """out[r] = softmax(scale * q[r] . K[:visible[r]]^T) V[:visible[r]].

    q: [R][d]; K, V: [n][d]; visible: R counts, each in 1..n.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    out = np.zeros((q.shape[0], V.shape[1]), dtype=np.float64)
    for r in range(q.shape[0]):
        c = int(visible[r])
        if c < 1 or c > K.shape[0]:
            raise ValueError("visible count out of range")
        s = (K[:c] @ q[r]) * np.float64(scale)
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum()
        out[r] = p @ V[:c]
    return out


def attention_probs(q_row, K, scale, visible):
    """The probability row of one query (used by the sum-to-one pin)."""
    s = (np.asarray(K[:visible], dtype=np.float64) @ np.asarray(q_row, np.float64)) * scale
    s = s - s.max()
    p = np.exp(s)
    return p / p.sum()


def verify(desc, pool_u8, layer, block_tables, seq_lens, q, k_rows, scale,
           k_scale=None, v_scale=None, seqs=None):
    """k-row verify attention for every (or each selected) sequence.

    q: float64-convertible [B][k][H_q][d].  Returns float64 [B][k][H_q][d]
    (rows of unselected sequences are left zero).  Row j of sequence s sees
    positions 0 .. n_s - k + j.
    """
    q = np.asarray(q, dtype=np.float64)
    B, k, Hq, d = q.shape
    assert k == k_rows
    Hkv = desc.num_kv_heads
    G = Hq // Hkv
    assert G * Hkv == Hq
    out = np.zeros_like(q)
    chosen = range(B) if seqs is None else seqs
    for s in chosen:
        n = int(seq_lens[s])
        if n < k:
            raise ValueError("sequence shorter than its query rows")
        for h in range(Hkv):
            K, V = gather_kv(desc, pool_u8, layer, block_tables[s], n, h, k_scale, v_scale)
            for g in range(h * G, (h + 1) * G):
                rows = q[s, :, g, :]
                visible = [n - k + j + 1 for j in range(k)]
                out[s, :, g, :] = softmax_attention(rows, K, V, scale, visible)
    return out


def decode(desc, pool_u8, layer, block_tables, seq_lens, q, scale,
           k_scale=None, v_scale=None, seqs=None):
    """One-query decode attention: q [B][H_q][d] -> float64 [B][H_q][d].

    Decode is the verify computation with a single query row per sequence,
    which sees all n_s cached positions.
    """
    q = np.asarray(q, dtype=np.float64)
    return verify(desc, pool_u8, layer, block_tables, seq_lens, q[:, None], 1, scale,
                  k_scale, v_scale, seqs)[:, 0]


def prefill(desc, pool_u8, layer, block_tables, seq_lens, q, chunk, scale,
            k_scale=None, v_scale=None, seqs=None, rows=None):
    """Chunked-prefill attention (page "KV cache & continuous batching",
    section "3. Chunked prefill": a prompt is fed in chunks, each attending
    over the cache of all earlier positions and over itself).

    q: [B][C][H_q][d] for the C = chunk tokens of each sequence, at positions
    n_s - C .. n_s - 1 with their K/V already in the pool; row j sees
    positions t <= n_s - C + j.  That is the k-row computation of ``verify``
    with k = C.  ``rows`` (chunk indices) limits the work to those rows of the
    selected sequences; the others are left zero.
    """
    if rows is None:
        return verify(desc, pool_u8, layer, block_tables, seq_lens, q, chunk, scale,
                      k_scale, v_scale, seqs)
    q = np.asarray(q, dtype=np.float64)
    B, C, Hq, d = q.shape
    assert C == chunk
    Hkv = desc.num_kv_heads
    G = Hq // Hkv
    out = np.zeros_like(q)
    rows = [int(j) for j in rows]
    for s in (range(B) if seqs is None else seqs):
        n = int(seq_lens[s])
        if n < C:
            raise ValueError("sequence shorter than its chunk")
        visible = [n - C + j + 1 for j in rows]
        for h in range(Hkv):
            K, V = gather_kv(desc, pool_u8, layer, block_tables[s], n, h, k_scale, v_scale)
            for g in range(h * G, (h + 1) * G):
                out[s, rows, g, :] = softmax_attention(q[s, rows, g, :], K, V, scale, visible)
    return out
