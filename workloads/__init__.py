"""Seeded synthetic inputs for the paged decode-attention path.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``; consumed
identically by the CPU oracle and by the HIP library.  This module holds none
of the method's arithmetic: it draws sequence lengths, a physical block
placement and N(0, 1) values, and casts values to the stored dtype with
torch's own conversions.  It imports neither the oracle nor the library.

Workload shapes (one transformer layer each; block size 16):

=====  ==========================================================================
c1     8 query / 2 KV heads, d 64, float32 KV; 4 sequences of 17, 100, 250, 513
       visible tokens; pool of 128 blocks; 1 query token per sequence.
c2     Llama-3-8B-shaped layer: 32 / 8 heads, d 128, bfloat16 KV; 64 sequences,
       lengths uniform in [512, 4096]; pool = 1.25 x blocks in use.
c3     Llama-3-70B-shaped layer: 64 / 8 heads, d 128, bfloat16 KV; 256 sequences,
       179 with lengths uniform in [128, 1024] and 77 uniform in [4096, 32768],
       in seeded random order.
c4     Long context: 32 / 8 heads, d 128, bfloat16 KV; 4 sequences of 131072
       tokens (8192 blocks each), split into 512-token partitions.
c5     Speculative verify over a shared prefix: 32 / 8 heads, d 128, fp8 E4M3 KV
       with float32 scales per (layer, KV head); 128 sequences whose first 128
       table entries name the same 128 physical blocks (a 2048-token prefix),
       then a private suffix of uniform [64, 1024] cached tokens, then 5 query
       positions (4 draft + 1 bonus) at the end.
pf     Chunked prefill, Llama-3-8B-shaped layer (32 / 8 heads, d 128, bf16):
       8 sequences, each a cached prefix of uniform [0, 14336] tokens followed
       by a chunk of 2048 query tokens.
pfv    Chunked prefill with a chunk length per sequence: as pf, chunks uniform
       in [1, 2048] (make_ragged_prefill; pfvs is its reduced variant).
=====  ==========================================================================

Reduced variants (``c2s`` ... ``c5s``) keep the head shapes and the length mix
at sizes the float64 oracle finishes in seconds while still spanning several
blocks, partitions and a ragged last block.

Conventions (readings recorded in the design notes):

* ``seq_lens[s]`` counts the positions visible to the sequence's last query
  row, including the tokens appended this step; the ``new_tokens_per_seq``
  newest positions (n-1 for decode; n-5 .. n-1 for c5) are the tokens written
  through the slot mapping this step, the rest are the prefilled cache;
* lengths "uniform in [a, b]" are integers with both ends included;
* block placement is ``rng.permutation(num_blocks)`` consumed in order,
  sequence-major and logical-block-minor (c5: the prefix takes the first 128);
* unused table entries are -1;
* draw order: lengths, placement, Q, prefill K/V (materialised workloads
  only), new-token K/V;
* softmax scale 1/sqrt(d);
* fp8 / int8 / int4 scales: materialised workloads use amax/448 (amax/127
  for int8, amax/7 for int4) of each head's prefilled values (K and V
  separately); full-size workloads whose pool is filled on the device use
  (4/448) * (1 + h/8) (int8: (4/127) * (1 + h/8), int4: (4/7) * (1 + h/8))
  for head h with codes drawn as e4m3(x*448/4) (int8: round(x*127/4)
  saturated to +-127; int4: round(x*7/4) saturated to +-7, two per byte).

Seeds: 293000 + config number (c1 -> 293001, ...; pf, pfs -> 293006; pfv,
pfvs -> 293008).
"""

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK = 16
SEED_BASE = 293000


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str                 # "f32" | "bf16" | "fp8" | "int8" | "int4"
    q_dtype: str                  # "f32" | "bf16"
    out_dtype: str                # "f32" | "bf16"
    k_rows: int                   # query rows per sequence (1 = decode)
    num_blocks: int
    seq_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray      # int32 [B][max_blocks], -1 unused
    q: np.ndarray                 # raw [B][k][H_q][d] (float32 or uint16 bf16 bits)
    new_seq_ids: np.ndarray       # int32 [T]
    new_positions: np.ndarray     # int32 [T]
    k_new: np.ndarray             # raw [T][H_kv][d] in in_dtype
    v_new: np.ndarray
    in_dtype: str                 # dtype of k_new/v_new and prefill values
    partition_tokens: int = 512
    num_layers: int = 1
    layer: int = 0
    materialized: bool = True
    pre_seq_ids: Optional[np.ndarray] = None
    pre_positions: Optional[np.ndarray] = None
    k_pre: Optional[np.ndarray] = None
    v_pre: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None   # float32 [L][H_kv] (fp8, int8 and int4 only)
    v_scale: Optional[np.ndarray] = None
    shared_prefix_tokens: int = 0
    chunk_lens: Optional[np.ndarray] = None   # int32 [B]: ragged chunked prefill (q packed [T][H_q][d])
    info: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    @property
    def query_start(self):
        """Ragged prefill: first packed query row of each sequence's chunk (B + 1 entries)."""
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int32)


# ------------------------------------------------------------------ casts

def to_bf16_bits(x):
    """float32 array -> bfloat16 bit patterns (torch's round-to-nearest-even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 (torch conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def _cast(x, dtype):
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def values_f32(raw, dtype):
    """Stored input values as float32 (for amax and for the tests' use)."""
    return np.asarray(raw, np.float32) if dtype == "f32" else bf16_bits_to_f32(raw)


# ---------------------------------------------------------------- builder

def build(name, seed, rng, seq_lens, *, num_q_heads, num_kv_heads, head_dim, kv_dtype,
          k_rows=1, shared_prefix_tokens=0, num_blocks=None, materialize=True,
          partition_tokens=512, out_dtype=None):
    """Assemble a workload from already-drawn lengths, continuing the same rng."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = seq_lens.shape[0]
    blocks_per_seq = [-(-int(n) // BLOCK) for n in seq_lens]
    prefix_blocks = shared_prefix_tokens // BLOCK
    assert prefix_blocks * BLOCK == shared_prefix_tokens
    used = prefix_blocks + sum(nb - prefix_blocks for nb in blocks_per_seq)
    if num_blocks is None:
        num_blocks = math.ceil(1.25 * used)
    assert num_blocks >= used
    max_blocks = max(blocks_per_seq)

    # placement: a seeded permutation consumed in order
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    cursor = prefix_blocks
    for s in range(B):
        tables[s, :prefix_blocks] = perm[:prefix_blocks]
        npriv = blocks_per_seq[s] - prefix_blocks
        tables[s, prefix_blocks:blocks_per_seq[s]] = perm[cursor:cursor + npriv]
        cursor += npriv

    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    in_dtype = q_dtype
    if out_dtype is None:
        out_dtype = "f32" if kv_dtype == "f32" else "bf16"
    Hq, Hkv, d = num_q_heads, num_kv_heads, head_dim
    q = _cast(rng.standard_normal((B, k_rows, Hq, d), dtype=np.float32), q_dtype)

    n_new = k_rows
    pre_seq_ids = pre_positions = k_pre = v_pre = None
    if materialize:
        ids, pos = [], []
        for s in range(B):
            n = int(seq_lens[s])
            start = 0 if s == 0 else shared_prefix_tokens
            for t in range(start, n - n_new):
                ids.append(s)
                pos.append(t)
        pre_seq_ids = np.asarray(ids, dtype=np.int32)
        pre_positions = np.asarray(pos, dtype=np.int32)
        T_pre = len(ids)
        k_pre = _cast(rng.standard_normal((T_pre, Hkv, d), dtype=np.float32), in_dtype)
        v_pre = _cast(rng.standard_normal((T_pre, Hkv, d), dtype=np.float32), in_dtype)

    new_ids = np.repeat(np.arange(B, dtype=np.int32), n_new)
    new_pos = np.concatenate([np.arange(int(n) - n_new, int(n), dtype=np.int32)
                              for n in seq_lens]) if B else np.zeros(0, np.int32)
    T_new = new_ids.shape[0]
    k_new = _cast(rng.standard_normal((T_new, Hkv, d), dtype=np.float32), in_dtype)
    v_new = _cast(rng.standard_normal((T_new, Hkv, d), dtype=np.float32), in_dtype)

    k_scale = v_scale = None
    if kv_dtype in ("fp8", "int8", "int4"):
        qmax = np.float32({"fp8": 448.0, "int8": 127.0, "int4": 7.0}[kv_dtype])
        if materialize:
            kv = values_f32(k_pre, in_dtype) if k_pre.shape[0] else np.ones((1, Hkv, d), np.float32)
            vv = values_f32(v_pre, in_dtype) if v_pre.shape[0] else np.ones((1, Hkv, d), np.float32)
            k_amax = np.abs(kv).max(axis=(0, 2))
            v_amax = np.abs(vv).max(axis=(0, 2))
            k_scale = (k_amax / qmax).astype(np.float32)[None, :]
            v_scale = (v_amax / qmax).astype(np.float32)[None, :]
        else:
            base = np.float32(4.0) / qmax
            per_head = (base * (1.0 + np.arange(Hkv, dtype=np.float32) / 8.0)).astype(np.float32)
            k_scale = per_head[None, :].copy()
            v_scale = per_head[None, :].copy()

    return Workload(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        kv_dtype=kv_dtype, q_dtype=q_dtype, out_dtype=out_dtype, k_rows=k_rows,
        num_blocks=int(num_blocks), seq_lens=seq_lens.astype(np.int32),
        block_tables=tables, q=q, new_seq_ids=new_ids, new_positions=new_pos,
        k_new=k_new, v_new=v_new, in_dtype=in_dtype,
        partition_tokens=partition_tokens, materialized=materialize,
        pre_seq_ids=pre_seq_ids, pre_positions=pre_positions, k_pre=k_pre, v_pre=v_pre,
        k_scale=k_scale, v_scale=v_scale, shared_prefix_tokens=shared_prefix_tokens,
        info={"blocks_used": int(used)})


# ------------------------------------------------------------- the configs

def _uniform(rng, lo, hi, size):
    return rng.integers(lo, hi, size=size, endpoint=True)


def make(name, materialize=None, seed=None, kv_dtype=None):
    """Build workload `name` (c1..c5 full size, c2s..c5s reduced; pf / pfs:
    chunked prefill, full size / reduced; a trailing "i8" (c2i8, c5si8, ...)
    or "i4" keeps the config but stores the KV cache as int8 or int4)."""
    if name in ("pf", "pfs"):
        return _make_prefill(name, materialize, seed)
    if name.endswith("i8") or name.endswith("i4"):
        # int8 / int4 KV variant of a config: same seed, lengths and placement
        return make(name[:-2], materialize, seed, kv_dtype="int8" if name.endswith("i8") else "int4")
    num = int(name[1])
    seed = SEED_BASE + num if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    small = name.endswith("s") or name == "c1"
    if materialize is None:
        materialize = small
    if name == "c1":
        lens = np.array([17, 100, 250, 513])
        return build(name, seed, rng, lens, num_q_heads=8, num_kv_heads=2, head_dim=64,
                     kv_dtype="f32", num_blocks=128, materialize=materialize,
                     partition_tokens=64)
    if name == "c2":
        lens = _uniform(rng, 512, 4096, 64)
        return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "bf16", materialize=materialize, partition_tokens=512)
    if name == "c2s":
        lens = _uniform(rng, 17, 700, 6)
        return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "bf16", materialize=materialize, partition_tokens=128)
    if name == "c3":
        lens = np.concatenate([_uniform(rng, 128, 1024, 179), _uniform(rng, 4096, 32768, 77)])
        lens = lens[rng.permutation(lens.shape[0])]
        return build(name, seed, rng, lens, num_q_heads=64, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "bf16", materialize=materialize, partition_tokens=512)
    if name == "c3s":
        lens = np.concatenate([_uniform(rng, 16, 200, 7), _uniform(rng, 600, 1500, 3)])
        lens = lens[rng.permutation(lens.shape[0])]
        return build(name, seed, rng, lens, num_q_heads=64, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "bf16", materialize=materialize, partition_tokens=256)
    if name == "c4":
        lens = np.full(4, 131072)
        return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "bf16", materialize=materialize, partition_tokens=512)
    if name == "c4s":
        lens = np.full(2, 4100)
        return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "bf16", materialize=materialize, partition_tokens=512)
    if name == "c5":
        suffix = _uniform(rng, 64, 1024, 128)
        lens = 2048 + suffix + 5
        return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "fp8", k_rows=5, shared_prefix_tokens=2048,
                     materialize=materialize, partition_tokens=512)
    if name == "c5s":
        suffix = _uniform(rng, 5, 100, 6)
        lens = 256 + suffix + 5
        return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     kv_dtype=kv_dtype or "fp8", k_rows=5, shared_prefix_tokens=256,
                     materialize=materialize, partition_tokens=128)
    raise ValueError(name)


def _make_prefill(name, materialize, seed):
    """Chunked prefill on the Llama-3-8B-shaped layer (32 / 8 heads, d 128,
    bf16 KV): every sequence has a cached prefix of uniform [0, P] tokens and
    a chunk of C query tokens after it (their K/V appended before attention).
    pf: 8 sequences, C = 2048, P = 14336 (contexts up to 16K);
    pfs: 3 sequences, C = 200, P = 300 (a ragged chunk spanning several
    256-row tiles and partial blocks)."""
    seed = SEED_BASE + 6 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    small = name == "pfs"
    if materialize is None:
        materialize = small
    B, C, P = (3, 200, 300) if small else (8, 2048, 14336)
    lens = _uniform(rng, 0, P, B) + C
    return build(name, seed, rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype="bf16",
                 k_rows=C, materialize=materialize, partition_tokens=0)


def build_ragged(name, seed, rng, prefix_lens, chunk_lens, *, num_q_heads, num_kv_heads, head_dim, kv_dtype,
                 materialize=True):
    """A chunked-prefill batch whose sequences carry chunks of different
    lengths: sequence s has prefix_lens[s] cached tokens followed by
    chunk_lens[s] chunk tokens (their K/V appended this step).  Queries and
    outputs are packed [sum of chunks][H_q][d] in sequence order.  Draw order
    as ``build``: placement, Q, prefill K/V (materialised only), chunk K/V."""
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int64)
    seq_lens = prefix_lens + chunk_lens
    B = seq_lens.shape[0]
    blocks_per_seq = [-(-int(n) // BLOCK) for n in seq_lens]
    used = sum(blocks_per_seq)
    num_blocks = max(1, math.ceil(1.25 * used))
    max_blocks = max(1, max(blocks_per_seq))
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for s in range(B):
        tables[s, :blocks_per_seq[s]] = perm[cursor:cursor + blocks_per_seq[s]]
        cursor += blocks_per_seq[s]
    q_dtype = in_dtype = "bf16"
    Hq, Hkv, d = num_q_heads, num_kv_heads, head_dim
    T = int(chunk_lens.sum())
    q = _cast(rng.standard_normal((T, Hq, d), dtype=np.float32), q_dtype)
    pre_seq_ids = pre_positions = k_pre = v_pre = None
    if materialize:
        pre_seq_ids = np.concatenate([np.full(int(p), s, np.int32) for s, p in enumerate(prefix_lens)] +
                                     [np.zeros(0, np.int32)])
        pre_positions = np.concatenate([np.arange(int(p), dtype=np.int32) for p in prefix_lens] +
                                       [np.zeros(0, np.int32)])
        k_pre = _cast(rng.standard_normal((pre_seq_ids.shape[0], Hkv, d), dtype=np.float32), in_dtype)
        v_pre = _cast(rng.standard_normal((pre_seq_ids.shape[0], Hkv, d), dtype=np.float32), in_dtype)
    new_ids = np.concatenate([np.full(int(c), s, np.int32) for s, c in enumerate(chunk_lens)] + [np.zeros(0, np.int32)])
    new_pos = np.concatenate([np.arange(int(p), int(p + c), dtype=np.int32) for p, c in zip(prefix_lens, chunk_lens)]
                             + [np.zeros(0, np.int32)])
    k_new = _cast(rng.standard_normal((T, Hkv, d), dtype=np.float32), in_dtype)
    v_new = _cast(rng.standard_normal((T, Hkv, d), dtype=np.float32), in_dtype)
    k_scale = v_scale = None
    if kv_dtype in ("fp8", "int8", "int4"):
        qmax = np.float32({"fp8": 448.0, "int8": 127.0, "int4": 7.0}[kv_dtype])
        base = np.float32(4.0) / qmax
        if materialize and k_pre.shape[0]:
            k_scale = (np.abs(values_f32(k_pre, in_dtype)).max(axis=(0, 2)) / qmax).astype(np.float32)[None, :]
            v_scale = (np.abs(values_f32(v_pre, in_dtype)).max(axis=(0, 2)) / qmax).astype(np.float32)[None, :]
        else:
            per_head = (base * (1.0 + np.arange(Hkv, dtype=np.float32) / 8.0)).astype(np.float32)
            k_scale = per_head[None, :].copy()
            v_scale = per_head[None, :].copy()
    return Workload(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=kv_dtype, q_dtype=q_dtype,
        out_dtype="bf16", k_rows=0, num_blocks=int(num_blocks), seq_lens=seq_lens.astype(np.int32),
        block_tables=tables, q=q, new_seq_ids=new_ids, new_positions=new_pos, k_new=k_new, v_new=v_new,
        in_dtype=in_dtype, partition_tokens=0, materialized=materialize, pre_seq_ids=pre_seq_ids,
        pre_positions=pre_positions, k_pre=k_pre, v_pre=v_pre, k_scale=k_scale, v_scale=v_scale,
        chunk_lens=chunk_lens.astype(np.int32), info={"blocks_used": int(used)})


def make_ragged_prefill(name, materialize=None, seed=None, kv_dtype="bf16"):
    """Chunked prefill with a chunk length per sequence, Llama-3-8B-shaped
    layer (32 / 8 heads, d 128):
    pfv:  8 sequences, cached prefixes uniform [0, 14336], chunks uniform
          [1, 2048] (the last chunks of prompts of any length);
    pfvs: 5 sequences, prefixes uniform [0, 300], chunks {0, 1, 17, uniform
          [40, 250] twice} in seeded order (an empty chunk, a one-token chunk,
          ragged tiles)."""
    seed = SEED_BASE + 8 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    small = name == "pfvs"
    if materialize is None:
        materialize = small
    if small:
        prefix = _uniform(rng, 0, 300, 5)
        chunks = np.concatenate([[0, 1, 17], _uniform(rng, 40, 250, 2)])
        chunks = chunks[rng.permutation(5)]
        prefix = np.maximum(prefix, 1)   # every sequence holds at least one token
    else:
        prefix = _uniform(rng, 0, 14336, 8)
        chunks = _uniform(rng, 1, 2048, 8)
    return build_ragged(name, seed, rng, prefix, chunks, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        kv_dtype=kv_dtype, materialize=materialize)


def custom(seed, seq_lens, **kw):
    """A workload with explicit lengths and shapes (edge cases in the tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return build("custom", seed, rng, np.asarray(seq_lens), **kw)


# ------------------------------------------------- device-side random pools

def fill_pool_random(pool_u8, kv_dtype, seed, num_kv_heads=None):
    """Fill a device pool tensor (torch uint8) with seeded N(0, 1) values.

    bf16/f32 pools get N(0, 1) in every element.  fp8 pools get
    e4m3(x * 448 / 4) codes of N(0, 1) draws, i.e. values x * scale / (4/448)
    under the per-head scales ``build`` assigns to unmaterialised workloads;
    int8 pools get round(x * 127 / 4) saturated to +-127, int4 pools
    round(x * 7 / 4) saturated to +-7, two codes per byte.
    Used for full-size workloads whose prefilled cache is too large to draw on
    the host; the oracle reads the filled pool back.
    """
    import torch
    g = torch.Generator(device=pool_u8.device)
    g.manual_seed(int(seed))
    if kv_dtype == "f32":
        pool_u8.view(torch.float32).normal_(generator=g)
    elif kv_dtype == "bf16":
        pool_u8.view(torch.bfloat16).normal_(generator=g)
    elif kv_dtype == "int8":
        chunk = 1 << 26
        flat = pool_u8.view(-1)
        for start in range(0, flat.numel(), chunk):
            part = flat[start:start + chunk]
            x = torch.randn(part.numel(), generator=g, device=pool_u8.device,
                            dtype=torch.float32) * (127.0 / 4.0)
            x = torch.round(x).clamp(-127.0, 127.0)
            part.copy_(x.to(torch.int8).view(torch.uint8))
    elif kv_dtype == "int4":
        chunk = 1 << 26
        flat = pool_u8.view(-1)
        for start in range(0, flat.numel(), chunk):
            part = flat[start:start + chunk]
            x = torch.randn(2 * part.numel(), generator=g, device=pool_u8.device,
                            dtype=torch.float32) * (7.0 / 4.0)
            c = torch.round(x).clamp(-7.0, 7.0).to(torch.int32) & 0xF
            part.copy_((c[0::2] | (c[1::2] << 4)).to(torch.uint8))
    elif kv_dtype == "fp8":
        chunk = 1 << 26
        flat = pool_u8.view(-1)
        for start in range(0, flat.numel(), chunk):
            part = flat[start:start + chunk]
            x = torch.randn(part.numel(), generator=g, device=pool_u8.device,
                            dtype=torch.float32) * (448.0 / 4.0)
            x = x.clamp(-448.0, 448.0)
            part.copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
    else:
        raise ValueError(kv_dtype)


# ------------------------------------------------- speculative acceptance

@dataclass
class SpecWorkload:
    """Inputs of one exact speculative-acceptance step (no method arithmetic:
    seeded logits, their softmax, draft tokens drawn from q, and uniforms)."""
    name: str
    seed: int
    p: np.ndarray          # float32 [B][K+1][V]
    q: np.ndarray          # float32 [B][K][V]
    draft: np.ndarray      # int32 [B][K]
    u_accept: np.ndarray   # float32 [B][K]
    u_sample: np.ndarray   # float32 [B]

    @property
    def batch(self):
        return int(self.draft.shape[0])

    @property
    def k(self):
        return int(self.draft.shape[1])

    @property
    def vocab(self):
        return int(self.p.shape[2])


def _softmax32(logits):
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def make_spec(name, seed=None, batch=None, k=None, vocab=None):
    """sp: 128 sequences, 4 drafted tokens (+ the bonus row), Llama-3's
    128,256-token vocabulary; sps: 7 sequences, vocabulary 1000.  Target
    logits are N(0, 3^2); the draft's are the target's plus N(0, 0.7^2) noise,
    so a drafted token is accepted about 70% of the time (page "LLM Inference
    Optimization: KV Cache, Batching, and Speculative Decoding", section
    "Speculative Decoding", puts good drafts at 60-80%).  Draft tokens are drawn
    from q with the generator (an input of the step, not part of it)."""
    seed = SEED_BASE + 7 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    B, K, V = (128, 4, 128256) if name == "sp" else (7, 4, 1000)
    B = batch or B
    K = k or K
    V = vocab or V
    lp = rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(3.0)
    lq = lp[:, :K] + rng.standard_normal((B, K, V), dtype=np.float32) * np.float32(0.7)
    p = _softmax32(lp)
    q = _softmax32(lq)
    cq = np.cumsum(q.astype(np.float64), axis=-1)
    r = rng.random((B, K))
    draft = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        for i in range(K):
            draft[b, i] = min(int(np.searchsorted(cq[b, i], r[b, i] * cq[b, i, -1], side="right")), V - 1)
    u_accept = rng.random((B, K), dtype=np.float32)
    u_sample = rng.random(B, dtype=np.float32)
    return SpecWorkload(name, seed, p, q, draft, u_accept, u_sample)
