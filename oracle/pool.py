"""Host model of the paged KV pool (oracle, test infrastructure only).

What the pages fix (page "KV cache & continuous batching", section
"2. PagedAttention (vLLM)"; section "Visual: the lifecycle of a request in
continuous batching"; page "LLM Serving - KV Cache, Batching, Speculative
Decoding", section "KV memory, paging and prefix identity"):

* the cache is cut into fixed physical blocks of 16 token positions;
* each request owns a block table: logical block j of the request lives in
  physical block table[j]; blocks need not be contiguous and two requests may
  name the same physical block (shared prefix);
* token position t of a request is therefore found in physical block
  table[t // 16] at offset t % 16 ("slot" = block * 16 + offset).

What the pages leave open and this build defines (the byte layout of the
pool, documented in the library header ``include/pagedkv.h`` and restated here
so the oracle reads the pool from the definition, not from library code):

* pool = num_layers x num_blocks x num_kv_heads x {K tile, V tile};
  the tile for (layer l, block p, head h, kv) starts at byte
  ((((l * NB + p) * H_kv + h) * 2 + kv) * TILE, TILE = 16 * d * b, kv = 0 for K;
* inside a K tile, element (token o, dim i) is element number
  ((i // X) * 16 + o) * X + i % X with X = 16 // b (16-byte chunks of
  consecutive dims, chunk-major, token-minor);
* inside a V tile, element (token o, dim i) is element number i * 16 + o
  (dim-major: the V tile is stored transposed);
* b = 4 (float32), 2 (bfloat16) or 1 (fp8 E4M3, or symmetric int8, with a
  float32 scale per (layer, KV head), separately for K and V; value = code *
  scale);
* int4 (b = 1/2, same scales) instead numbers the nibbles of a tile
  (nibble N is byte N // 2, the low half when N is even) so that no byte
  holds two tokens; with W = d // 4:
  K (token o, dim i = 32 s + 8 g + e):  N = (g * 16 + o) * W + 8 s + e,
  V (token o = 4 g + t, dim i = 16 m + c):  N = (g * 16 + c) * W + 8 * (m // 2) + 2 * t + m % 2.

Pins: the layout formula is checked against hand-computed offsets stored in
``tests/golden/pool_layout.txt``; the slot rule against the block-table
example (``tests/golden/page1_block_tables.txt``); the cache write and the
gather against each other and against brute-force loops in the tests.
"""

import numpy as np

from . import fp8 as _fp8
from . import int4 as _int4
from . import int8 as _int8
from .kv_math import BLOCK_SIZE, slot_of

DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1, "int4": 0.5}


class PoolDesc:
    """Geometry of a pool (plain record)."""

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, kv_dtype):
        if kv_dtype not in DTYPE_BYTES:
            raise ValueError(kv_dtype)
        self.num_layers = int(num_layers)
        self.num_blocks = int(num_blocks)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.kv_dtype = kv_dtype

    @property
    def elem_bytes(self):
        return DTYPE_BYTES[self.kv_dtype]

    @property
    def tile_bytes(self):
        return int(BLOCK_SIZE * self.head_dim * self.elem_bytes)

    @property
    def total_bytes(self):
        return (self.num_layers * self.num_blocks * self.num_kv_heads * 2
                * self.tile_bytes)


def tile_byte_offset(desc, layer, block, head, kv):
    """Byte offset of the (layer, block, head, kv) tile; kv = 0 for K, 1 for V."""
    return ((((layer * desc.num_blocks + block) * desc.num_kv_heads + head) * 2 + kv)
            * desc.tile_bytes)


def k_element_in_tile(desc, token, dim):
    """Element number of K(token, dim) inside its tile (chunk-major, token-minor)."""
    x = 16 // desc.elem_bytes
    return ((dim // x) * BLOCK_SIZE + token) * x + dim % x


def v_element_in_tile(desc, token, dim):
    """Element number of V(token, dim) inside its tile (dim-major: transposed)."""
    return dim * BLOCK_SIZE + token


def k_nibble_in_tile(desc, token, dim):
    """int4: nibble number of K(token, dim) inside its tile."""
    w = desc.head_dim // 4
    s, g, e = dim // 32, (dim // 8) % 4, dim % 8
    return (g * BLOCK_SIZE + token) * w + 8 * s + e


def v_nibble_in_tile(desc, token, dim):
    """int4: nibble number of V(token, dim) inside its tile."""
    w = desc.head_dim // 4
    g, t = token // 4, token % 4
    m, c = dim // 16, dim % 16
    return (g * BLOCK_SIZE + c) * w + 8 * (m // 2) + 2 * t + m % 2


def element_nibble_offset(desc, layer, block, head, kv, token, dim):
    """int4: nibble number of one K or V element in the pool."""
    inner = (k_nibble_in_tile(desc, token, dim) if kv == 0
             else v_nibble_in_tile(desc, token, dim))
    return 2 * tile_byte_offset(desc, layer, block, head, kv) + inner


def element_byte_offset(desc, layer, block, head, kv, token, dim):
    """Byte offset of one K or V element in the pool (byte element types)."""
    inner = (k_element_in_tile(desc, token, dim) if kv == 0
             else v_element_in_tile(desc, token, dim))
    return tile_byte_offset(desc, layer, block, head, kv) + inner * desc.elem_bytes


def empty_pool(desc, fill_byte=0xFF):
    """Host pool image. 0xFF bytes read as NaN in every supported dtype."""
    return np.full(desc.total_bytes, fill_byte, dtype=np.uint8)


# ----------------------------------------------------------------- slots

def slot_mapping(block_tables, seq_ids, positions, num_blocks):
    """Slot of each (sequence, position) pair; -1 where the pair is invalid.

    Invalid: sequence id outside the table, position < 0, position beyond the
    table row's capacity, or a table entry outside [0, num_blocks).
    """
    tables = np.asarray(block_tables)
    out = np.full(len(seq_ids), -1, dtype=np.int64)
    for t, (s, pos) in enumerate(zip(seq_ids, positions)):
        s = int(s)
        pos = int(pos)
        if s < 0 or s >= tables.shape[0]:
            continue
        if pos < 0 or pos >= tables.shape[1] * BLOCK_SIZE:
            continue
        blk = int(tables[s, pos // BLOCK_SIZE])
        if blk < 0 or blk >= num_blocks:
            continue
        out[t] = slot_of(tables[s], pos)
    return out


# ------------------------------------------------------------ decoding

def _raw_view(desc, pool_u8):
    if desc.kv_dtype == "f32":
        return pool_u8.view(np.float32)
    if desc.kv_dtype == "bf16":
        return pool_u8.view(np.uint16)
    return pool_u8


def bf16_bits_to_float(bits):
    """bfloat16 bit pattern -> exact float64 (it is the top half of a float32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _decode_raw(desc, raw, scale):
    if desc.kv_dtype == "f32":
        return raw.astype(np.float64)
    if desc.kv_dtype == "bf16":
        return bf16_bits_to_float(raw)
    if desc.kv_dtype == "int8":
        return _int8.decode(raw.view(np.int8), scale)
    return _fp8.decode(raw) * np.float64(np.float32(scale))


def gather_kv(desc, pool_u8, layer, table_row, n_tokens, head,
              k_scale=None, v_scale=None):
    """Contiguous float64 K[n][d] and V[n][d] of one sequence and KV head.

    For every logical position t < n the physical block table_row[t // 16] and
    offset t % 16 are located, and each element is read at its layout offset
    and decoded exactly (code types: code value times the float32 scale of
    (layer, head)).
    """
    d = desc.head_dim
    t = np.arange(n_tokens)
    blocks = np.asarray(table_row, dtype=np.int64)[t // BLOCK_SIZE]
    offs = t % BLOCK_SIZE
    dims = np.arange(d)
    ks = None if k_scale is None else k_scale[layer][head]
    vs = None if v_scale is None else v_scale[layer][head]
    if desc.kv_dtype == "int4":
        bb, oo, ii = blocks[:, None], offs[:, None], dims[None, :]
        k_nib = element_nibble_offset(desc, layer, bb, head, 0, oo, ii)
        v_nib = element_nibble_offset(desc, layer, bb, head, 1, oo, ii)
        return (_int4.decode(_read_nibbles(pool_u8, k_nib), ks),
                _int4.decode(_read_nibbles(pool_u8, v_nib), vs))
    eb = desc.elem_bytes
    raw = _raw_view(desc, pool_u8)
    k_base = np.array([tile_byte_offset(desc, layer, int(b), head, 0) for b in blocks],
                      dtype=np.int64)
    v_base = np.array([tile_byte_offset(desc, layer, int(b), head, 1) for b in blocks],
                      dtype=np.int64)
    k_idx = (k_base[:, None] // eb) + k_element_in_tile(desc, offs[:, None], dims[None, :])
    v_idx = (v_base[:, None] // eb) + v_element_in_tile(desc, offs[:, None], dims[None, :])
    K = _decode_raw(desc, raw[k_idx], ks)
    V = _decode_raw(desc, raw[v_idx], vs)
    return K, V


def _read_nibbles(pool_u8, nib):
    """Signed codes of the nibbles numbered `nib` (low half of byte N // 2 when N is even)."""
    b = pool_u8[nib // 2].astype(np.int64)
    n = np.where(nib % 2 == 0, b & 0xF, b >> 4)
    return _int4.code_of(n)


def _write_nibbles(pool_u8, nib, codes):
    """Store codes into the nibbles numbered `nib` (all distinct) of a uint8
    image, in place: first every low half, then every high half, so the two
    halves of one byte never overwrite each other."""
    nib = np.ravel(nib).astype(np.int64)
    c = np.ravel(_int4.nibble_of(codes)).astype(np.uint8)
    lo = nib % 2 == 0
    b = nib[lo] // 2
    pool_u8[b] = (pool_u8[b] & np.uint8(0xF0)) | c[lo]
    b = nib[~lo] // 2
    pool_u8[b] = (pool_u8[b] & np.uint8(0x0F)) | (c[~lo] << np.uint8(4))


# ----------------------------------------------------------- cache write

def cache_write(desc, pool_u8, layer, k_new, v_new, in_dtype, slots,
                k_scale=None, v_scale=None):
    """Pool image after writing each new token's K and V at its slot.

    k_new, v_new: [T][H_kv][d] raw input values; in_dtype "f32" (float32
    array) or "bf16" (uint16 bit patterns).  A slot < 0 skips its token.
    f32 and bf16 pools store the input bits unchanged (the input dtype must
    equal the pool dtype); fp8 pools store fp8.quantize(x, scale[layer][h]),
    int8 pools int8.quantize(x, scale[layer][h]), int4 pools the nibbles of
    int4.quantize(x, scale[layer][h]).
    Returns a new array; the input image is not modified.
    """
    pool = pool_u8.copy()
    raw = _raw_view(desc, pool)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    T, H, d = k_new.shape
    assert H == desc.num_kv_heads and d == desc.head_dim
    if desc.kv_dtype in ("f32", "bf16") and in_dtype != desc.kv_dtype:
        raise ValueError("f32/bf16 pools take inputs of their own dtype")
    eb = desc.elem_bytes
    dims = np.arange(d)
    for t in range(T):
        slot = int(slots[t])
        if slot < 0:
            continue
        blk, off = slot // BLOCK_SIZE, slot % BLOCK_SIZE
        for h in range(H):
            if desc.kv_dtype == "int4":
                kx = _input_to_f32(k_new[t, h], in_dtype)
                vx = _input_to_f32(v_new[t, h], in_dtype)
                k_nib = element_nibble_offset(desc, layer, blk, h, 0, off, dims)
                v_nib = element_nibble_offset(desc, layer, blk, h, 1, off, dims)
                _write_nibbles(pool, k_nib, _int4.quantize(kx, k_scale[layer][h]))
                _write_nibbles(pool, v_nib, _int4.quantize(vx, v_scale[layer][h]))
                continue
            k_at = (tile_byte_offset(desc, layer, blk, h, 0) // eb
                    + k_element_in_tile(desc, off, dims))
            v_at = (tile_byte_offset(desc, layer, blk, h, 1) // eb
                    + v_element_in_tile(desc, off, dims))
            if desc.kv_dtype == "fp8":
                kx = _input_to_f32(k_new[t, h], in_dtype)
                vx = _input_to_f32(v_new[t, h], in_dtype)
                raw[k_at] = _fp8.quantize(kx, k_scale[layer][h])
                raw[v_at] = _fp8.quantize(vx, v_scale[layer][h])
            elif desc.kv_dtype == "int8":
                kx = _input_to_f32(k_new[t, h], in_dtype)
                vx = _input_to_f32(v_new[t, h], in_dtype)
                raw[k_at] = _int8.quantize(kx, k_scale[layer][h]).view(np.uint8)
                raw[v_at] = _int8.quantize(vx, v_scale[layer][h]).view(np.uint8)
            else:
                raw[k_at] = k_new[t, h]
                raw[v_at] = v_new[t, h]
    return pool


def _input_to_f32(x, in_dtype):
    if in_dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    return bf16_bits_to_float(x).astype(np.float32)
