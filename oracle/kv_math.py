"""Byte and block arithmetic of the KV cache (oracle, test infrastructure only).

Page "KV cache & continuous batching", section "KV cache memory math": the
cache holds one K and one V vector per layer, per KV head and per cached token,
so its size is the product 2 x layers x kv_heads x head_dim x seq_len x batch x
bytes-per-element.  GQA and MQA shrink it through the KV head count, never the
query head count (same page, "Pitfall 4").  Page "LLM Serving - KV Cache,
Batching, Speculative Decoding", section "KV memory, paging and prefix
identity", names the same symbols (L, B, T, H_KV, d_h, b).

Page "KV cache & continuous batching", section "Visual: the lifecycle of a
request in continuous batching": memory is handed out in blocks of 16 tokens,
so a request of n tokens holds ceil(n / 16) blocks.  Section "2. PagedAttention
(vLLM)": a per-request block table maps logical block j to a physical block.

Bytes per element may be fractional (int4 = 1/2 byte on the same page), so the
formula is evaluated with exact rationals and returned as an int when whole.
"""

from fractions import Fraction
import math

BLOCK_SIZE = 16


def _exact(x):
    x = Fraction(x)
    return int(x) if x.denominator == 1 else x


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes):
    """2 * L * H_kv * d_h * b: cache bytes one token adds across all layers."""
    return _exact(2 * num_layers * num_kv_heads * head_dim * Fraction(dtype_bytes))


def kv_cache_bytes(num_layers, num_kv_heads, head_dim, seq_len, batch, dtype_bytes):
    """The page's full formula: per-token bytes times seq_len times batch."""
    return _exact(kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes)
                  * seq_len * batch)


def blocks_for_tokens(n_tokens, block_size=BLOCK_SIZE):
    """Blocks a request of n_tokens occupies: ceil(n / block_size); 0 for n = 0."""
    if n_tokens < 0:
        raise ValueError("negative token count")
    return math.ceil(n_tokens / block_size)


def block_capacity(n_blocks, block_size=BLOCK_SIZE):
    """Tokens a list of n_blocks blocks can hold (the page's '4 blocks x 16 = 64')."""
    return n_blocks * block_size


def slot_of(table_row, position, block_size=BLOCK_SIZE):
    """Flat slot of logical position `position` through one block-table row.

    Logical block position // block_size is looked up in the row; the slot is
    that physical block's first slot plus the offset position % block_size.
    """
    if position < 0:
        raise ValueError("negative position")
    return int(table_row[position // block_size]) * block_size + position % block_size


def pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, dtype_bytes,
               block_size=BLOCK_SIZE):
    """Bytes of a pool of num_blocks physical blocks: its token capacity
    (num_blocks * block_size) times the per-token formula."""
    return _exact(num_blocks * block_size
                  * kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes))
