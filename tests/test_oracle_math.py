"""Pins for the oracle's byte, block, slot and layout arithmetic (CPU only)."""

import math

import numpy as np
import pytest

from conftest import golden_lines
from oracle import kv_math, pool as opool


def test_kv_sizes_match_pages():
    rows = golden_lines("kv_sizes.txt")
    assert len(rows) >= 10
    for L, H, d, b, T, B, expected, check in rows:
        got = kv_math.kv_cache_bytes(int(L), int(H), int(d), int(T), int(B), int(b))
        if check == "eq":
            assert got == int(expected)
        elif check == "floorGB":
            assert math.floor(got / 1e9) == int(expected)
        elif check == "GiB":
            assert got == int(expected) * 2 ** 30
        else:
            raise AssertionError(check)


def test_per_layer_bytes_of_the_shapes_streamed():
    # per layer, per token: the 70B and 8B figures divided by their layer counts
    assert kv_math.kv_bytes_per_token(80, 8, 128, 2) // 80 == 4096
    assert kv_math.kv_bytes_per_token(32, 8, 128, 2) // 32 == 4096
    assert kv_math.kv_bytes_per_token(1, 8, 128, 2) == 4096
    # one byte per element halves it (fp8), half a byte quarters it (int4)
    assert kv_math.kv_bytes_per_token(1, 8, 128, 1) == 2048
    assert kv_math.kv_bytes_per_token(1, 8, 128, 0.5) == 1024
    # GQA: the formula takes KV heads; 64 query heads with 8 KV heads is 8x less
    assert kv_math.kv_bytes_per_token(80, 64, 128, 2) == 8 * kv_math.kv_bytes_per_token(80, 8, 128, 2)


def test_block_counts_match_pages():
    rows = golden_lines("block_counts.txt")
    for n, expected in rows:
        assert kv_math.blocks_for_tokens(int(n)) == int(expected)
    assert kv_math.blocks_for_tokens(0) == 0
    assert kv_math.blocks_for_tokens(16) == 1
    assert kv_math.blocks_for_tokens(17) == 2


def _page1_tables():
    tables, slots = {}, []
    for row in golden_lines("page1_block_tables.txt"):
        if row[0] == "SLOT":
            slots.append((row[1], int(row[2]), int(row[3])))
        else:
            name, n, cap = row[0], int(row[1]), int(row[2])
            tables[name] = (n, cap, [int(x) for x in row[3:]])
    return tables, slots


def test_page1_tables_capacity_and_slots():
    tables, slots = _page1_tables()
    for name, (n, cap, ids) in tables.items():
        assert kv_math.blocks_for_tokens(n) == len(ids)
        assert kv_math.block_capacity(len(ids)) == cap
    assert len(slots) == 6
    for name, pos, expected in slots:
        assert kv_math.slot_of(tables[name][2], pos) == expected


def test_slot_mapping_validity_rules():
    tables, _ = _page1_tables()
    width = 9
    tab = np.full((2, width), -1, dtype=np.int32)
    tab[0, :4] = tables["A"][2]
    tab[1, :9] = tables["B"][2]
    seq = [0, 0, 1, 1, 0, 2, -1, 0]
    pos = [0, 49, 129, 143, 64, 0, 0, -1]
    got = opool.slot_mapping(tab, seq, pos, num_blocks=29)
    # A pos 64 -> logical block 4, an unused (-1) entry; seq 2 and -1 do not exist
    assert got.tolist() == [192, 65, 145, 9 * 16 + 15, -1, -1, -1, -1]
    # a table entry beyond the pool is refused
    assert opool.slot_mapping(tab, [1], [0], num_blocks=3).tolist() == [-1]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_pool_layout_hand_offsets(dtype):
    rows = golden_lines("pool_layout.txt")
    desc = opool.PoolDesc(num_layers=2, num_blocks=3, num_kv_heads=2, head_dim=64, kv_dtype=dtype)
    seen = 0
    for row in rows:
        if row[0] == "SIZE":
            if row[1] == dtype:
                assert desc.total_bytes == int(row[2])
                assert desc.total_bytes == kv_math.pool_bytes(2, 3, 2, 64, opool.DTYPE_BYTES[dtype])
            continue
        dt, kv, layer, block, head, tok, dim, expected = row
        if dt != dtype:
            continue
        seen += 1
        got = opool.element_byte_offset(desc, int(layer), int(block), int(head),
                                        0 if kv == "K" else 1, int(tok), int(dim))
        assert got == int(expected)
    assert seen == 2


def test_int4_pool_layout_hand_offsets():
    rows = golden_lines("pool_layout.txt")
    desc = opool.PoolDesc(num_layers=2, num_blocks=3, num_kv_heads=2, head_dim=64, kv_dtype="int4")
    seen = 0
    for row in rows:
        if row[0] == "SIZE":
            if row[1] == "int4":
                assert desc.total_bytes == int(row[2])
                assert desc.total_bytes == kv_math.pool_bytes(2, 3, 2, 64, opool.DTYPE_BYTES["int4"])
            continue
        dt, kv, layer, block, head, tok, dim, expected = row
        if dt != "int4":
            continue
        seen += 1
        got = opool.element_nibble_offset(desc, int(layer), int(block), int(head),
                                          0 if kv == "K" else 1, int(tok), int(dim))
        assert got == int(expected)
    assert seen == 5


@pytest.mark.parametrize("d", [64, 128])
def test_int4_layout_is_a_bijection_and_keeps_tokens_apart(d):
    # every element gets its own nibble, and the two nibbles of a byte always
    # belong to the same token (so tokens can be written independently)
    desc = opool.PoolDesc(num_layers=1, num_blocks=2, num_kv_heads=2, head_dim=d, kv_dtype="int4")
    owner = np.full(2 * desc.total_bytes, -1, dtype=np.int64)
    for blk in range(2):
        for h in range(2):
            for kv in range(2):
                for t in range(16):
                    for i in range(d):
                        n = opool.element_nibble_offset(desc, 0, blk, h, kv, t, i)
                        assert owner[n] == -1
                        owner[n] = ((blk * 2 + h) * 2 + kv) * 16 + t
    assert (owner >= 0).all()
    assert np.array_equal(owner[0::2], owner[1::2])


def test_int4_cache_write_then_gather_round_trips():
    rng = np.random.default_rng(11)
    desc = opool.PoolDesc(1, 6, 2, 64, "int4")
    table = rng.permutation(6)[:4].astype(np.int32)[None, :]
    n = 53
    k = (rng.standard_normal((n, 2, 64)) * 3).astype(np.float32)
    v = (rng.standard_normal((n, 2, 64)) * 3).astype(np.float32)
    ks = np.array([[0.5, 0.75]], np.float32)
    vs = np.array([[1.0, 0.25]], np.float32)
    slots = opool.slot_mapping(table, [0] * n, list(range(n)), 6)
    img = opool.cache_write(desc, opool.empty_pool(desc, 0), 0, k, v, "f32", slots, ks, vs)
    for h in range(2):
        K, V = opool.gather_kv(desc, img, 0, table[0], n, h, ks, vs)
        from oracle import int4
        assert np.array_equal(K, int4.decode(int4.quantize(k[:, h], ks[0][h]), ks[0][h]))
        assert np.array_equal(V, int4.decode(int4.quantize(v[:, h], vs[0][h]), vs[0][h]))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_pool_layout_is_a_bijection(dtype):
    # every (layer, block, head, kv, token, dim) element gets its own byte range
    desc = opool.PoolDesc(num_layers=2, num_blocks=3, num_kv_heads=2, head_dim=64, kv_dtype=dtype)
    eb = desc.elem_bytes
    seen = np.zeros(desc.total_bytes, dtype=np.int32)
    for layer in range(2):
        for blk in range(3):
            for h in range(2):
                for kv in range(2):
                    for t in range(16):
                        for i in range(64):
                            off = opool.element_byte_offset(desc, layer, blk, h, kv, t, i)
                            seen[off:off + eb] += 1
    assert (seen == 1).all()


def test_cache_write_then_gather_round_trips_exactly():
    rng = np.random.default_rng(7)
    desc = opool.PoolDesc(1, 10, 2, 32, "f32")
    table = rng.permutation(10)[:5].astype(np.int32)[None, :]
    n = 70
    k = rng.standard_normal((n, 2, 32)).astype(np.float32)
    v = rng.standard_normal((n, 2, 32)).astype(np.float32)
    slots = opool.slot_mapping(table, [0] * n, list(range(n)), 10)
    img = opool.cache_write(desc, opool.empty_pool(desc), 0, k, v, "f32", slots)
    for h in range(2):
        K, V = opool.gather_kv(desc, img, 0, table[0], n, h)
        assert np.array_equal(K, k[:, h].astype(np.float64))
        assert np.array_equal(V, v[:, h].astype(np.float64))
    # untouched blocks keep the fill (NaN in every dtype)
    untouched = [b for b in range(10) if b not in table[0]]
    off = opool.tile_byte_offset(desc, 0, untouched[0], 0, 0)
    assert (img[off:off + desc.tile_bytes] == 0xFF).all()
