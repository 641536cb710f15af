"""Pins for the oracle's attention (CPU only).

Each test ties the float64 oracle to something other than itself: the cached
== uncached identity of page "LLM Serving - KV Cache, Batching, Speculative
Decoding" (section "Hands-on: cache equivalence and scheduling oracles"),
closed forms, invariances, and a pure-Python brute force that reads the
logical K/V directly (not through the pool).
"""

import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import pool as opool

BS = 16


def _fill(desc, table, seqs_kv):
    """Write logical K/V ([n][H][d] float32 per sequence) into a fresh pool."""
    img = opool.empty_pool(desc)
    for s, (k, v) in enumerate(seqs_kv):
        n = k.shape[0]
        slots = opool.slot_mapping(table, [s] * n, list(range(n)), desc.num_blocks)
        img = opool.cache_write(desc, img, 0, k, v, "f32", slots)
    return img


def _placement(rng, lens, nb):
    perm = rng.permutation(nb)
    width = max(-(-n // BS) for n in lens)
    tab = np.full((len(lens), width), -1, dtype=np.int32)
    c = 0
    for s, n in enumerate(lens):
        m = -(-n // BS)
        tab[s, :m] = perm[c:c + m]
        c += m
    return tab


def _brute(q, K, V, scale, visible):
    """Pure-Python softmax attention on lists of floats."""
    out = []
    for r, qr in enumerate(q):
        c = visible[r]
        scores = [scale * sum(a * b for a, b in zip(qr, K[t])) for t in range(c)]
        m = max(scores)
        w = [math.exp(x - m) for x in scores]
        z = sum(w)
        out.append([sum(w[t] * V[t][i] for t in range(c)) / z for i in range(len(V[0]))])
    return out


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 1), (3, 3)])  # GQA, MQA, MHA
def test_decode_against_brute_force(Hq, Hkv):
    rng = np.random.default_rng(100 + Hq * 10 + Hkv)
    d = 4
    lens = [1, 16, 17, 40]
    desc = opool.PoolDesc(1, 12, Hkv, d, "f32")
    tab = _placement(rng, lens, 12)
    kv = [(rng.standard_normal((n, Hkv, d)).astype(np.float32),
           rng.standard_normal((n, Hkv, d)).astype(np.float32)) for n in lens]
    img = _fill(desc, tab, kv)
    q = rng.standard_normal((len(lens), Hq, d))
    scale = 0.7
    got = oatt.decode(desc, img, 0, tab, np.array(lens), q, scale)
    G = Hq // Hkv
    for s, n in enumerate(lens):
        for g in range(Hq):
            h = g // G
            K = kv[s][0][:, h].astype(np.float64).tolist()
            V = kv[s][1][:, h].astype(np.float64).tolist()
            ref = _brute([q[s, g].tolist()], K, V, scale, [n])[0]
            assert np.allclose(got[s, g], ref, rtol=0, atol=1e-12)


def test_verify_rows_against_brute_force_and_sequential_decode():
    rng = np.random.default_rng(5)
    Hq, Hkv, d, k = 4, 2, 4, 3
    lens = [3, 20, 33]
    desc = opool.PoolDesc(1, 10, Hkv, d, "f32")
    tab = _placement(rng, lens, 10)
    kv = [(rng.standard_normal((n, Hkv, d)).astype(np.float32),
           rng.standard_normal((n, Hkv, d)).astype(np.float32)) for n in lens]
    img = _fill(desc, tab, kv)
    q = rng.standard_normal((len(lens), k, Hq, d))
    got = oatt.verify(desc, img, 0, tab, np.array(lens), q, k, 0.5)
    for s, n in enumerate(lens):
        for g in range(Hq):
            h = g // (Hq // Hkv)
            K = kv[s][0][:, h].astype(np.float64).tolist()
            V = kv[s][1][:, h].astype(np.float64).tolist()
            ref = _brute([q[s, j, g].tolist() for j in range(k)], K, V, 0.5,
                         [n - k + j + 1 for j in range(k)])
            assert np.allclose(got[s, :, g], ref, rtol=0, atol=1e-12)
        # row j of verify == a decode whose sequence ends at n - k + j + 1
        for j in range(k):
            lens_j = np.array(lens)
            lens_j[s] = n - k + j + 1
            dec = oatt.decode(desc, img, 0, tab, lens_j, q[:, j], 0.5, seqs=[s])
            assert np.array_equal(dec[s], got[s, j])


def test_cached_equals_uncached_causal_attention():
    # A 7-token, width-4 toy in float64 as on page "LLM Serving - KV Cache,
    # Batching, Speculative Decoding" (section "Hands-on: cache equivalence
    # and scheduling oracles"): decoding with the cache at every prefix equals
    # the last row of full causal attention.
    rng = np.random.default_rng(124)
    x = rng.standard_normal((7, 4))
    Wq, Wk, Wv = (rng.standard_normal((4, 4)) for _ in range(3))
    # K/V are stored in a float32 pool, so round them to float32 once and use
    # the same rounded values for the uncached reference.
    Kall = (x @ Wk).astype(np.float32)
    Vall = (x @ Wv).astype(np.float32)
    Q = x @ Wq
    scale = 1.0 / math.sqrt(4)

    def full_causal(n):
        S = (Q[:n] @ Kall[:n].astype(np.float64).T) * scale
        S = S + np.triu(np.full((n, n), -np.inf), 1)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P = P / P.sum(axis=1, keepdims=True)
        return P @ Vall[:n].astype(np.float64)

    desc = opool.PoolDesc(1, 6, 1, 4, "f32")
    tab = np.array([[4, 1]], dtype=np.int32)   # two blocks, out of order
    img = opool.empty_pool(desc)
    for t in range(7):
        slot = opool.slot_mapping(tab, [0], [t], 6)
        img = opool.cache_write(desc, img, 0, Kall[t:t + 1, None], Vall[t:t + 1, None], "f32", slot)
        dec = oatt.decode(desc, img, 0, tab, np.array([t + 1]), Q[t:t + 1, None], scale)
        assert np.allclose(dec[0, 0], full_causal(t + 1)[-1], rtol=0, atol=1e-12)
    # negative control: wrong prefix values (V + 1 in one block) break the identity
    bad = img.copy()
    raw = bad.view(np.float32)
    base = opool.tile_byte_offset(desc, 0, 4, 0, 1) // 4
    raw[base:base + desc.tile_bytes // 4] += 1.0
    dec = oatt.decode(desc, bad, 0, tab, np.array([7]), Q[6:7, None], scale)
    assert not np.allclose(dec[0, 0], full_causal(7)[-1], rtol=0, atol=1e-6)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 1)])
def test_chunked_prefill_equals_full_causal_attention(Hq, Hkv):
    # Page "KV cache & continuous batching", section "3. Chunked prefill": a
    # prompt fed in chunks, each appended to the cache and then attended,
    # gives the rows of full causal attention over the whole prompt.  The
    # reference is the textbook dense form: one masked score matrix per query
    # head, softmax along rows, times V.
    rng = np.random.default_rng(303 + Hq)
    n, d = 37, 8
    G = Hq // Hkv
    K = rng.standard_normal((n, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((n, Hkv, d)).astype(np.float32)
    Q = rng.standard_normal((n, Hq, d))
    scale = 1.0 / math.sqrt(d)
    full = np.zeros((n, Hq, d))
    mask = np.triu(np.full((n, n), -np.inf), 1)
    for g in range(Hq):
        h = g // G
        S = (Q[:, g] @ K[:, h].astype(np.float64).T) * scale + mask
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P = P / P.sum(axis=1, keepdims=True)
        full[:, g] = P @ V[:, h].astype(np.float64)
    desc = opool.PoolDesc(1, 6, Hkv, d, "f32")
    tab = np.array([[4, 0, 5]], dtype=np.int32)          # three blocks, out of order
    img = opool.empty_pool(desc)
    pos = 0
    for C in (5, 16, 1, 15):
        slots = opool.slot_mapping(tab, [0] * C, list(range(pos, pos + C)), desc.num_blocks)
        img = opool.cache_write(desc, img, 0, K[pos:pos + C], V[pos:pos + C], "f32", slots)
        got = oatt.prefill(desc, img, 0, tab, np.array([pos + C]), Q[None, pos:pos + C], C, scale)
        assert np.allclose(got[0], full[pos:pos + C], rtol=0, atol=1e-12)
        some = oatt.prefill(desc, img, 0, tab, np.array([pos + C]), Q[None, pos:pos + C], C, scale,
                            rows=[C - 1, 0])
        assert np.array_equal(some[0, [C - 1, 0]], got[0, [C - 1, 0]])
        pos += C
    # negative control: rows that also see the next position break the identity
    C = 15
    wrong = oatt.prefill(desc, img, 0, tab, np.array([n]), Q[None, n - C - 1:n - 1], C, scale)
    assert not np.allclose(wrong[0], full[n - C - 1:n - 1], rtol=0, atol=1e-6)


def test_softmax_rows_sum_to_one_and_ones_in_ones_out():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((300, 8)) * 3
    for c in (1, 7, 300):
        p = oatt.attention_probs(rng.standard_normal(8), K, 0.9, c)
        assert abs(p.sum() - 1.0) < 1e-12 and (p >= 0).all()
    out = oatt.softmax_attention(rng.standard_normal((3, 8)), K, np.ones((300, 5)), 0.9, [1, 50, 300])
    assert np.allclose(out, 1.0, rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(10)
    K = rng.standard_normal((40, 8))
    V = rng.standard_normal((40, 6))
    q = rng.standard_normal((1, 8))
    # one visible token: the output is that token's V exactly
    assert np.array_equal(oatt.softmax_attention(q, K, V, 1.3, [1])[0], V[0])
    # scale 0 (or all keys equal): the mean of the visible V rows
    assert np.allclose(oatt.softmax_attention(q, K, V, 0.0, [25])[0], V[:25].mean(axis=0), atol=1e-14)
    Keq = np.tile(K[:1], (40, 1))
    assert np.allclose(oatt.softmax_attention(q, Keq, V, 2.0, [40])[0], V.mean(axis=0), atol=1e-14)
    # a needle: one key with a score gap of ~180 makes the softmax one-hot
    Kn = np.zeros((40, 8))
    Kn[23, 0] = 128.0
    qn = np.zeros((1, 8))
    qn[0, 0] = 16.0
    out = oatt.softmax_attention(qn, Kn, V, 1 / math.sqrt(128), [40])[0]
    assert np.array_equal(out, V[23])


def test_output_is_invariant_to_physical_placement():
    rng = np.random.default_rng(12)
    lens = [5, 33, 64]
    desc = opool.PoolDesc(1, 20, 2, 8, "f32")
    kv = [(rng.standard_normal((n, 2, 8)).astype(np.float32),
           rng.standard_normal((n, 2, 8)).astype(np.float32)) for n in lens]
    q = rng.standard_normal((3, 4, 8))
    outs = []
    for seed in (1, 2, 3):
        tab = _placement(np.random.default_rng(seed), lens, 20)
        img = _fill(desc, tab, kv)
        outs.append(oatt.decode(desc, img, 0, tab, np.array(lens), q, 0.35))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_physical_blocks_read_the_same_prefix():
    # two sequences whose tables name the same first physical block see the
    # same prefix: with only the prefix visible their outputs coincide.
    rng = np.random.default_rng(13)
    desc = opool.PoolDesc(1, 8, 1, 8, "f32")
    tab = np.array([[5, 2], [5, 7]], dtype=np.int32)
    k = rng.standard_normal((16, 1, 8)).astype(np.float32)
    v = rng.standard_normal((16, 1, 8)).astype(np.float32)
    img = opool.cache_write(desc, opool.empty_pool(desc), 0, k, v, "f32",
                            opool.slot_mapping(tab, [0] * 16, list(range(16)), 8))
    q = np.tile(rng.standard_normal((1, 1, 8)), (2, 1, 1))
    out = oatt.decode(desc, img, 0, tab, np.array([16, 16]), q, 0.4)
    assert np.array_equal(out[0], out[1])


def test_bf16_and_fp8_pools_decode_exactly():
    rng = np.random.default_rng(14)
    from oracle import fp8
    # bf16: the stored bit pattern is the top half of a float32
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80], dtype=np.uint16)
    vals = opool.bf16_bits_to_float(bits)
    assert vals[:5].tolist() == [1.0, -1.0, 3.140625, 0.0, -0.0] and np.isinf(vals[5])
    # fp8: gather returns code value * float32 scale
    desc = opool.PoolDesc(1, 2, 1, 16, "fp8")
    x = rng.standard_normal((16, 1, 16)).astype(np.float32)
    ks = np.array([[0.01]], dtype=np.float32)
    vs = np.array([[0.02]], dtype=np.float32)
    tab = np.array([[1]], dtype=np.int32)
    xb = np.ascontiguousarray(x)
    import workloads
    img = opool.cache_write(desc, opool.empty_pool(desc), 0, workloads.to_bf16_bits(xb),
                            workloads.to_bf16_bits(xb), "bf16",
                            opool.slot_mapping(tab, [0] * 16, list(range(16)), 2), ks, vs)
    K, V = opool.gather_kv(desc, img, 0, tab[0], 16, 0, ks, vs)
    xr = workloads.values_f32(workloads.to_bf16_bits(xb), "bf16")[:, 0]
    assert np.array_equal(K, fp8.decode(fp8.quantize(xr, ks[0, 0])) * np.float64(ks[0, 0]))
    assert np.array_equal(V, fp8.decode(fp8.quantize(xr, vs[0, 0])) * np.float64(vs[0, 0]))
    assert np.abs(K - xr).max() < 0.07 * np.abs(xr).max()
