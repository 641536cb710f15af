"""torch-facing wrappers with the C ABI's names.

Each wrapper checks tensor shapes/dtypes/devices, takes raw pointers and the
current HIP stream, and calls the library; a non-zero status raises
``PagedKVError``.  Allocation of outputs and workspaces that the caller did
not pass is done with torch (the library itself never allocates).
"""

import ctypes
import math

import numpy as np
import torch

from ._lib import BF16, BLOCK_SIZE, F32, FP8_E4M3, INT4, INT8, PagedKVError, PoolDesc, lib

_KV_DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "int8": INT8, "int4": INT4, F32: F32, BF16: BF16,
              FP8_E4M3: FP8_E4M3, INT8: INT8, INT4: INT4}
_TORCH_CODE = {torch.float32: F32, torch.bfloat16: BF16}
_CODE_TORCH = {F32: torch.float32, BF16: torch.bfloat16}


def _check(call, status):
    if status != 0:
        raise PagedKVError(call, status)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _desc(num_layers, num_blocks, num_kv_heads, head_dim, kv_dtype):
    return PoolDesc(int(num_layers), int(num_blocks), int(num_kv_heads), int(head_dim),
                    BLOCK_SIZE, _KV_DTYPES[kv_dtype])


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, kv_dtype):
    """2 * L * H_kv * d * b (int); -1 if the arguments are invalid."""
    return int(lib.kv_bytes_per_token(int(num_layers), int(num_kv_heads), int(head_dim),
                                      _KV_DTYPES[kv_dtype]))


def kv_pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, kv_dtype):
    d = _desc(num_layers, num_blocks, num_kv_heads, head_dim, kv_dtype)
    return int(lib.kv_pool_bytes(ctypes.byref(d)))


class KVPool:
    """A pool handle plus the tensors it points into (kept alive here)."""

    def __init__(self, handle, storage, k_scale, v_scale, desc):
        self._handle = handle
        self.storage = storage
        self.k_scale = k_scale
        self.v_scale = v_scale
        self.num_layers = desc.num_layers
        self.num_blocks = desc.num_blocks
        self.num_kv_heads = desc.num_kv_heads
        self.head_dim = desc.head_dim
        self.kv_dtype = desc.kv_dtype

    @property
    def handle(self):
        return self._handle

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h:
            lib.kv_pool_destroy(h)
            self._handle = None


def kv_pool_create(num_layers, num_blocks, num_kv_heads, head_dim, kv_dtype, storage=None,
                   k_scale=None, v_scale=None, device="cuda"):
    """Wrap (or allocate, when storage is None) a device pool buffer.

    storage: uint8 CUDA tensor of at least kv_pool_bytes(...) bytes.
    k_scale, v_scale: float32 CUDA tensors [num_layers][num_kv_heads] (fp8, int8 and int4 only).
    """
    desc = _desc(num_layers, num_blocks, num_kv_heads, head_dim, kv_dtype)
    nbytes = int(lib.kv_pool_bytes(ctypes.byref(desc)))
    if nbytes < 0:
        _check("kv_pool_bytes", -2)
    if storage is None:
        storage = torch.empty(nbytes, dtype=torch.uint8, device=device)
    assert storage.dtype == torch.uint8 and storage.is_cuda and storage.is_contiguous()
    for s in (k_scale, v_scale):
        if s is not None:
            assert s.dtype == torch.float32 and s.is_cuda and s.is_contiguous()
            assert s.numel() == num_layers * num_kv_heads
    out = ctypes.c_void_p()
    _check("kv_pool_create", lib.kv_pool_create(ctypes.byref(desc), _ptr(storage), storage.numel(),
                                                _ptr(k_scale), _ptr(v_scale), ctypes.byref(out)))
    return KVPool(out.value, storage, k_scale, v_scale, desc)


class BlockTable:
    """An uploaded, validated block table and its device buffer."""

    def __init__(self, handle, buffer, num_seqs, max_blocks):
        self._handle = handle
        self.buffer = buffer
        self.num_seqs = num_seqs
        self.max_blocks = max_blocks

    @property
    def handle(self):
        return self._handle

    def info(self):
        vals = [ctypes.c_int32() for _ in range(5)]
        _check("block_table_info", lib.block_table_info(self._handle, *[ctypes.byref(v) for v in vals]))
        keys = ("num_units", "num_split_slots", "max_seq_len", "min_seq_len", "max_parts")
        return dict(zip(keys, (v.value for v in vals)))

    def shared_prefix(self):
        """(prefix blocks, prefix chunks) of the table's shared prefix, (0, 0) without one."""
        pb, pc = ctypes.c_int32(), ctypes.c_int32()
        _check("block_table_shared_prefix",
               lib.block_table_shared_prefix(self._handle, ctypes.byref(pb), ctypes.byref(pc)))
        return pb.value, pc.value

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h:
            lib.block_table_destroy(h)
            self._handle = None


def block_table_upload(pool, block_tables, seq_lens, partition_tokens=-1, device="cuda"):
    """Validate and upload host block tables ([B][max_blocks] int32) and lengths ([B]).

    partition_tokens: a multiple of 16 for fixed split-KV partitions, 0 for
    none, -1 (default) for the balanced plan (with the shared-prefix plan
    when the tables share a prefix and a cost estimate favours it), -2 for
    the balanced plan with the shared-prefix plan whenever a prefix is found.
    """
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert bt.ndim == 2 and sl.ndim == 1 and sl.shape[0] == bt.shape[0]
    B, mb = bt.shape
    nbytes = int(lib.block_table_device_bytes(pool.handle, sl.ctypes.data_as(ctypes.c_void_p), B, mb,
                                              int(partition_tokens)))
    if nbytes == 0:
        _check("block_table_device_bytes", -1)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    out = ctypes.c_void_p()
    _check("block_table_upload", lib.block_table_upload(
        pool.handle, bt.ctypes.data_as(ctypes.c_void_p), B, mb, sl.ctypes.data_as(ctypes.c_void_p),
        int(partition_tokens), _ptr(buf), nbytes, _stream(buf.device), ctypes.byref(out)))
    return BlockTable(out.value, buf, B, mb)


def slot_mapping_compute(table, seq_ids, positions, out=None):
    """int64 slots of (sequence, position) pairs; -1 where invalid."""
    assert seq_ids.dtype == torch.int32 and positions.dtype == torch.int32
    assert seq_ids.is_cuda and seq_ids.shape == positions.shape and seq_ids.dim() == 1
    T = seq_ids.numel()
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=seq_ids.device)
    assert out.dtype == torch.int64 and out.numel() == T
    _check("slot_mapping_compute", lib.slot_mapping_compute(
        table.handle, _ptr(seq_ids.contiguous()), _ptr(positions.contiguous()), T, _ptr(out),
        _stream(seq_ids.device)))
    return out


def reshape_and_cache(pool, layer, k_new, v_new, slot_mapping):
    """Write new tokens' K/V ([T][H_kv][d], float32 or bfloat16) at their slots."""
    assert k_new.shape == v_new.shape and k_new.dtype == v_new.dtype
    assert k_new.dim() == 3 and k_new.shape[1:] == (pool.num_kv_heads, pool.head_dim)
    assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.is_cuda
    assert slot_mapping.dtype == torch.int64 and slot_mapping.numel() == k_new.shape[0]
    _check("reshape_and_cache", lib.reshape_and_cache(
        pool.handle, int(layer), _ptr(k_new), _ptr(v_new), _TORCH_CODE[k_new.dtype],
        _ptr(slot_mapping.contiguous()), int(k_new.shape[0]), _stream(k_new.device)))


def paged_attention_workspace_bytes(pool, table, num_q_heads, query_rows=1):
    return int(lib.paged_attention_workspace_bytes(pool.handle, table.handle, int(num_q_heads),
                                                   int(query_rows)))


def _attention(pool, layer, table, q, query_rows, scale, workspace, out, out_dtype):
    assert q.is_cuda and q.is_contiguous() and q.dtype in _TORCH_CODE
    Hq = q.shape[-2]
    if out_dtype is None:
        out_dtype = torch.float32 if pool.kv_dtype == F32 else torch.bfloat16
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    assert out.shape == q.shape and out.is_contiguous() and out.dtype in _TORCH_CODE
    need = paged_attention_workspace_bytes(pool, table, Hq, query_rows)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    return out, workspace, ws_bytes, float(scale), Hq


def paged_attention_decode(pool, layer, table, q, scale=None, workspace=None, out=None, out_dtype=None):
    """Decode attention: q [B][H_q][d] -> out [B][H_q][d]."""
    assert q.dim() == 3 and q.shape[0] == table.num_seqs
    out, workspace, ws_bytes, scale, Hq = _attention(pool, layer, table, q, 1, scale, workspace, out, out_dtype)
    _check("paged_attention_decode", lib.paged_attention_decode(
        pool.handle, int(layer), table.handle, _ptr(q), _TORCH_CODE[q.dtype], Hq, scale,
        _ptr(workspace), ws_bytes, _ptr(out), _TORCH_CODE[out.dtype], _stream(q.device)))
    return out


def paged_attention_verify(pool, layer, table, q, scale=None, workspace=None, out=None, out_dtype=None):
    """k-row verify attention: q [B][k][H_q][d] -> out [B][k][H_q][d]."""
    assert q.dim() == 4 and q.shape[0] == table.num_seqs
    k = q.shape[1]
    out, workspace, ws_bytes, scale, Hq = _attention(pool, layer, table, q, k, scale, workspace, out, out_dtype)
    _check("paged_attention_verify", lib.paged_attention_verify(
        pool.handle, int(layer), table.handle, _ptr(q), _TORCH_CODE[q.dtype], int(k), Hq, scale,
        _ptr(workspace), ws_bytes, _ptr(out), _TORCH_CODE[out.dtype], _stream(q.device)))
    return out


def paged_attention_verify_noalloc(pool, layer, table, q, scale=None, out=None, out_dtype=None):
    """paged_attention_verify with the partial results in the library's static
    per-device scratch (no workspace): q [B][k][H_q][d] -> out [B][k][H_q][d]."""
    assert q.dim() == 4 and q.shape[0] == table.num_seqs
    k = q.shape[1]
    assert q.is_cuda and q.is_contiguous() and q.dtype in _TORCH_CODE
    Hq = q.shape[-2]
    if out_dtype is None:
        out_dtype = torch.float32 if pool.kv_dtype == F32 else torch.bfloat16
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    assert out.shape == q.shape and out.is_contiguous() and out.dtype in _TORCH_CODE
    scale = 1.0 / math.sqrt(pool.head_dim) if scale is None else float(scale)
    _check("paged_attention_verify_noalloc", lib.paged_attention_verify_noalloc(
        pool.handle, int(layer), table.handle, _ptr(q), _TORCH_CODE[q.dtype], int(k), Hq, scale,
        _ptr(out), _TORCH_CODE[out.dtype], _stream(q.device)))
    return out


def paged_attention_append(pool, layer, table, k_new, v_new, q, scale=None, workspace=None, out=None,
                           out_dtype=None):
    """Append then attend in one launch.

    q: [B][H_q][d] (decode) or [B][k][H_q][d] (verify); k_new, v_new:
    [B][k][H_kv][d] (k = 1 may be given as [B][H_kv][d]), the K/V of each
    sequence's k newest positions.  Returns out shaped like q.
    """
    decode = q.dim() == 3
    k = 1 if decode else q.shape[1]
    assert q.shape[0] == table.num_seqs
    assert k_new.shape == v_new.shape and k_new.dtype == v_new.dtype and k_new.is_cuda
    assert k_new.is_contiguous() and v_new.is_contiguous()
    assert k_new.numel() == table.num_seqs * k * pool.num_kv_heads * pool.head_dim
    out, workspace, ws_bytes, scale, Hq = _attention(pool, layer, table, q, k, scale, workspace, out, out_dtype)
    _check("paged_attention_append", lib.paged_attention_append(
        pool.handle, int(layer), table.handle, _ptr(k_new), _ptr(v_new), _TORCH_CODE[k_new.dtype],
        _ptr(q), _TORCH_CODE[q.dtype], int(k), Hq, scale, _ptr(workspace), ws_bytes, _ptr(out),
        _TORCH_CODE[out.dtype], _stream(q.device)))
    return out


def paged_attention_prefill(pool, layer, table, q, scale=None, out=None, out_dtype=None):
    """Chunked-prefill attention: q [B][C][H_q][d] bf16 -> out [B][C][H_q][d].

    Row j of sequence s is position seq_len[s] - C + j (its K/V already
    appended) and sees positions t <= seq_len[s] - C + j.
    """
    assert q.dim() == 4 and q.shape[0] == table.num_seqs
    assert q.is_cuda and q.is_contiguous() and q.dtype == torch.bfloat16
    C, Hq = q.shape[1], q.shape[2]
    if out_dtype is None:
        out_dtype = torch.bfloat16
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    assert out.shape == q.shape and out.is_contiguous() and out.dtype in _TORCH_CODE
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    _check("paged_attention_prefill", lib.paged_attention_prefill(
        pool.handle, int(layer), table.handle, _ptr(q), BF16, int(C), int(Hq), float(scale),
        _ptr(out), _TORCH_CODE[out.dtype], _stream(q.device)))
    return out


def paged_attention_prefill_varlen(pool, layer, table, q, query_start, scale=None, out=None, out_dtype=None):
    """Chunked prefill with a chunk per sequence: q [T][H_q][d] bfloat16, the
    chunks' rows packed in sequence order, query_start the B + 1 row offsets
    (host ints; copied to the device here) -> out [T][H_q][d]."""
    qs = np.ascontiguousarray(np.asarray(query_start, dtype=np.int32))
    assert qs.ndim == 1 and qs.shape[0] == table.num_seqs + 1
    assert q.dim() == 3 and q.is_cuda and q.is_contiguous() and q.dtype == torch.bfloat16
    assert q.shape[0] == int(qs[-1])
    Hq = q.shape[1]
    if out_dtype is None:
        out_dtype = torch.bfloat16
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    assert out.shape == q.shape and out.is_contiguous() and out.dtype in _TORCH_CODE
    dev_qs = torch.from_numpy(qs).to(q.device)
    scale = 1.0 / math.sqrt(pool.head_dim) if scale is None else float(scale)
    _check("paged_attention_prefill_varlen", lib.paged_attention_prefill_varlen(
        pool.handle, int(layer), table.handle, _ptr(q), BF16, qs.ctypes.data_as(ctypes.c_void_p), _ptr(dev_qs),
        Hq, scale, _ptr(out), _TORCH_CODE[out.dtype], _stream(q.device)))
    return out


def speculative_accept(p, q, draft, u_accept, u_sample, num_accepted=None, tokens=None):
    """Exact speculative acceptance: p [B][K+1][V], q [B][K][V] float32,
    draft [B][K] int32, u_accept [B][K], u_sample [B] float32 uniforms in
    [0, 1).  Returns (num_accepted [B], tokens [B][K+1]) int32 tensors."""
    B, K1, V = p.shape
    K = K1 - 1
    assert q.shape == (B, K, V) and draft.shape == (B, K) and u_accept.shape == (B, K)
    assert u_sample.shape == (B,)
    for t, dt in ((p, torch.float32), (q, torch.float32), (u_accept, torch.float32), (u_sample, torch.float32),
                  (draft, torch.int32)):
        assert t.is_cuda and t.is_contiguous() and t.dtype == dt
    if num_accepted is None:
        num_accepted = torch.empty(B, dtype=torch.int32, device=p.device)
    if tokens is None:
        tokens = torch.empty(B, K + 1, dtype=torch.int32, device=p.device)
    _check("speculative_accept", lib.speculative_accept(
        _ptr(p), _ptr(q), _ptr(draft), _ptr(u_accept), _ptr(u_sample), int(B), int(K), int(V),
        _ptr(num_accepted), _ptr(tokens), _stream(p.device)))
    return num_accepted, tokens


def kv_copy_blocks(pool, pairs):
    """Copy blocks (all layers, heads, K and V): pairs int32 CUDA tensor [n][2] of (src, dst)."""
    assert pairs.is_cuda and pairs.dtype == torch.int32 and pairs.is_contiguous()
    n = pairs.numel() // 2
    _check("kv_copy_blocks", lib.kv_copy_blocks(pool.handle, _ptr(pairs), int(n), _stream(pairs.device)))


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """Host block manager of a pool's physical blocks (see the C header for
    the policy).  Token ids are int32; sequence ids are the caller's."""

    def __init__(self, num_blocks):
        h = ctypes.c_void_p()
        _check("block_manager_create", lib.block_manager_create(int(num_blocks), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib.block_manager_destroy(h)
            self._h = None

    @property
    def free_blocks(self):
        return int(lib.block_manager_free_blocks(self._h))

    def refcount(self, block):
        return int(lib.block_manager_refcount(self._h, int(block)))

    def add(self, seq_id, tokens, salt=0):
        """New sequence with its prompt; returns (cached_tokens, slots of the uncached tokens)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(t.size, dtype=np.int64)
        cached = ctypes.c_int32()
        _check("block_manager_add", lib.block_manager_add(self._h, int(seq_id), _np_ptr(t), int(t.size),
                                                          ctypes.c_uint64(int(salt)), ctypes.byref(cached),
                                                          _np_ptr(slots)))
        return int(cached.value), slots[:t.size - cached.value].copy()

    def append(self, seq_id, tokens):
        """Append tokens; returns (slots, copies) with copies a list of (src, dst) block pairs."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(t.size, 1), dtype=np.int64)
        copies = np.empty(2, dtype=np.int32)
        nc = ctypes.c_int32()
        _check("block_manager_append", lib.block_manager_append(self._h, int(seq_id), _np_ptr(t), int(t.size),
                                                                _np_ptr(slots), _np_ptr(copies), ctypes.byref(nc)))
        return slots[:t.size].copy(), [tuple(int(x) for x in copies[2 * i:2 * i + 2]) for i in range(nc.value)]

    def fork(self, parent_id, child_id):
        _check("block_manager_fork", lib.block_manager_fork(self._h, int(parent_id), int(child_id)))

    def free(self, seq_id):
        _check("block_manager_free", lib.block_manager_free(self._h, int(seq_id)))

    def table(self, seq_ids, max_blocks):
        """(table int32 [n][max_blocks], seq_lens int32 [n]) for block_table_upload."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tab = np.empty((ids.size, int(max_blocks)), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _check("block_manager_table", lib.block_manager_table(self._h, _np_ptr(ids), int(ids.size), int(max_blocks),
                                                              _np_ptr(tab), _np_ptr(lens)))
        return tab, lens
