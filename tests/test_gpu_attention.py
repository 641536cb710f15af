"""GPU: paged decode / verify attention against the float64 oracle.

Tolerances (max-abs error on unit-scale outputs): 1e-5 for float32 KV, 1e-2
for bf16 and fp8 KV, scaled by |ref| above 1.  Bit-exact cases: one-hot
(needle) softmax, one visible token, placement permutations.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from gpu_setup import DEV, Setup, assert_close, log, out_values, to_device
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu


def _pk():
    import paged_kv_cache_293_amd as pk
    return pk


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s", "c5s"])
def test_parity_reduced_configs(name):
    log(f"parity {name}")
    w = workloads.make(name)
    s = Setup(w)
    got = out_values(s.run())
    ref = s.oracle()
    err = assert_close(got, ref, w.kv_dtype, name)
    log(f"  {name}: max abs err {err:.3e}; units {s.table.info()}")


@pytest.mark.parametrize("P", [16, 64, 512, 0, -1])
def test_partition_sizes_agree(P):
    log(f"partition {P}")
    w = workloads.make("c2s")
    s = Setup(w, partition_tokens=P)
    got = out_values(s.run())
    assert_close(got, s.oracle(), w.kv_dtype, f"c2s P={P}")


def test_f32_output_dtype_and_c1_append_then_attend():
    log("c1 f32 / bf16 outputs")
    w = workloads.make("c1")
    s = Setup(w)
    ref = s.oracle()
    assert_close(out_values(s.run(out_dtype="f32")), ref, "f32", "c1 f32 out")
    w2 = workloads.make("c2s")
    s2 = Setup(w2)
    assert_close(out_values(s2.run(out_dtype="f32")), s2.oracle(), "bf16", "c2s f32 out")


@pytest.mark.parametrize("kv,Hq,Hkv,d", [("bf16", 8, 1, 128), ("bf16", 4, 4, 128), ("bf16", 16, 2, 64),
                                          ("f32", 4, 4, 64), ("f32", 8, 2, 128), ("fp8", 12, 2, 64)])
def test_head_shapes(kv, Hq, Hkv, d):
    log(f"heads {kv} {Hq}/{Hkv} d{d}")
    lens = [1, 15, 16, 17, 33, 200, 513]
    w = workloads.custom(77 + Hq + d, lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=kv,
                         partition_tokens=64)
    s = Setup(w)
    assert_close(out_values(s.run()), s.oracle(), kv, f"{kv} {Hq}/{Hkv} d{d}")


@pytest.mark.parametrize("k,Hq,Hkv", [(2, 8, 2), (5, 32, 8), (8, 8, 1), (3, 16, 2)])
def test_verify_shapes(k, Hq, Hkv):
    log(f"verify k={k} {Hq}/{Hkv}")
    lens = [k, k + 1, 16, 40, 300]
    w = workloads.custom(900 + k, lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, kv_dtype="bf16",
                         k_rows=k, partition_tokens=32)
    s = Setup(w)
    assert_close(out_values(s.run()), s.oracle(), "bf16", f"verify k={k}")


def _needle_setup(kv, n_list, k_rows=1, P=64, d=128, needle_positions=None, Hq=4, Hkv=1):
    """Workload whose softmax is one-hot: q = 16 e_0, K[:, 0] = 0 except 128 at the needle."""
    w = workloads.custom(31, n_list, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=kv,
                         k_rows=k_rows, partition_tokens=P)
    qf = np.zeros(w.q.shape, dtype=np.float32)
    qf[..., 0] = 16.0
    w.q = workloads._cast(qf, w.q_dtype)
    vals_pre = workloads.values_f32(w.k_pre, w.in_dtype).copy()
    vals_new = workloads.values_f32(w.k_new, w.in_dtype).copy()
    vals_pre[..., 0] = 0.0
    vals_new[..., 0] = 0.0
    for s, t in enumerate(needle_positions):
        hit = np.flatnonzero((w.pre_seq_ids == s) & (w.pre_positions == t))
        if hit.size:
            vals_pre[hit[0], :, 0] = 128.0
        hit = np.flatnonzero((w.new_seq_ids == s) & (w.new_positions == t))
        if hit.size:
            vals_new[hit[0], :, 0] = 128.0
    w.k_pre = workloads._cast(vals_pre, w.in_dtype)
    w.k_new = workloads._cast(vals_new, w.in_dtype)
    if kv == "fp8":
        w.k_scale = np.ones_like(w.k_scale)
        w.v_scale = np.ones_like(w.v_scale)
    return w


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_needle_is_bit_exact(kv):
    log(f"needle {kv}")
    lens = [1, 16, 17, 130, 200, 513, 700]
    needles = [0, 15, 16, 129, 63, 64, 383]       # first/last of blocks, partition edges (P=64)
    d = 64 if kv == "f32" else 128
    w = _needle_setup(kv, lens, needle_positions=needles, d=d)
    s = Setup(w)
    got = out_values(s.run(out_dtype="f32"))
    ref = s.oracle()
    # the float64 oracle keeps exp(-181)-sized weights that float32 flushes to
    # zero; rounded to float32 it is exactly V[needle], which the kernel must
    # reproduce bit for bit
    ref32 = ref.astype(np.float32).astype(np.float64)
    assert np.array_equal(got, ref32), f"max diff {np.abs(got - ref32).max()}"


def test_verify_needle_beyond_row_is_invisible():
    log("verify causal needle")
    k = 4
    lens = [40, 64, 100]
    # needle at the last position: visible only to the last query row
    w = _needle_setup("bf16", lens, k_rows=k, P=32, needle_positions=[n - 1 for n in lens])
    s = Setup(w)
    got = out_values(s.run(out_dtype="f32"))
    ref = s.oracle()
    assert_close(got, ref, "bf16", "verify needle")
    assert np.array_equal(got[:, k - 1], ref[:, k - 1].astype(np.float32).astype(np.float64))


def test_placement_permutation_is_bitwise_invariant():
    log("placement invariance")
    a = workloads.make("c2s")
    b = workloads.make("c2s")
    rng = np.random.default_rng(5)
    relabel = rng.permutation(a.num_blocks).astype(np.int32)
    b.block_tables = np.where(a.block_tables >= 0, relabel[np.maximum(a.block_tables, 0)], -1).astype(np.int32)
    ga = out_values(Setup(a).run())
    gb = out_values(Setup(b).run())
    assert np.array_equal(ga, gb)


def test_single_visible_token_and_ones():
    log("closed forms")
    pk = _pk()
    w = workloads.custom(3, [1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype="bf16")
    s = Setup(w)
    got = s.run()
    # one visible token: the output is that token's V, exactly (bf16 in, bf16 out)
    v = workloads.values_f32(w.v_new, "bf16")               # [B][H_kv][d]
    expect = np.repeat(v, 4, axis=1)
    assert np.array_equal(out_values(got), expect.astype(np.float64))
    # V = 1 everywhere: every output is 1
    w2 = workloads.custom(4, [5, 300, 1000], num_q_heads=8, num_kv_heads=2, head_dim=128,
                          kv_dtype="bf16", partition_tokens=128)
    w2.v_pre = workloads._cast(np.ones(w2.v_pre.shape, np.float32), "bf16")
    w2.v_new = workloads._cast(np.ones(w2.v_new.shape, np.float32), "bf16")
    out = out_values(Setup(w2).run())
    assert (out == 1.0).all()
    del pk


def test_fp8_every_code_decodes_exactly():
    log("fp8 codes through attention")
    pk = _pk()
    d, H = 128, 1
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    tiles = np.zeros((2, d), dtype=np.uint8)
    tiles.reshape(-1)[:codes.size] = codes
    # pool with one block: K makes token t one-hot for query row t; V holds the codes
    from oracle import pool as opool
    desc = opool.PoolDesc(1, 1, H, d, "fp8")
    img = np.zeros(desc.total_bytes, dtype=np.uint8)
    K1 = ofp8.encode(np.array([1.0]))[0]
    for t in range(16):
        for i in range(d):
            if t < 2:
                img[opool.element_byte_offset(desc, 0, 0, 0, 1, t, i)] = tiles[t, i]
        img[opool.element_byte_offset(desc, 0, 0, 0, 0, t, t)] = K1
    storage = torch.from_numpy(img).to(DEV)
    ones = torch.ones(1, H, dtype=torch.float32, device=DEV)
    pool = pk.kv_pool_create(1, 1, H, d, "fp8", storage=storage, k_scale=ones, v_scale=ones.clone())
    table = pk.block_table_upload(pool, np.zeros((1, 1), np.int32), [2], 0)
    q = torch.zeros(1, 2, d, dtype=torch.float32)
    q[0, 0, 0] = 400.0
    q[0, 1, 1] = 400.0
    out = pk.paged_attention_decode(pool, 0, table, q.to(torch.bfloat16).to(DEV), 1.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got[0], ofp8.decode(tiles))


def test_verify_rows_equal_sequential_decodes():
    log("verify == sequential decode")
    k = 3
    w = workloads.custom(8, [20, 77, 300], num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype="bf16",
                         k_rows=k, partition_tokens=64)
    s = Setup(w)
    ver = out_values(s.run())
    pk = _pk()
    for j in range(k):
        lens = w.seq_lens - (k - 1 - j)
        t = pk.block_table_upload(s.pool, w.block_tables, lens, 64)
        q = to_device(w.q[:, j], w.q_dtype)
        dec = out_values(pk.paged_attention_decode(s.pool, 0, t, q, w.scale))
        assert_close(dec, ver[:, j], "bf16", f"row {j}")


def test_repeated_calls_are_deterministic():
    log("determinism")
    w = workloads.make("c4s")
    s = Setup(w)
    a = out_values(s.run())
    b = out_values(s.run())
    assert np.array_equal(a, b)


@pytest.mark.parametrize("P", [16, -1])
def test_work_queue_many_items(P):
    """Far more (unit, KV head) items than resident work-groups: the
    work-groups take the rest from the table's queue.  Three calls in a row
    give bitwise-identical outputs that match the oracle, and leave the
    table's device buffer (merge tickets, queue counters) exactly as uploaded."""
    log(f"work queue P={P}")
    rng = np.random.default_rng(2930)
    lens = rng.integers(700, 2600, size=48).tolist() + [1, 16, 17]
    w = workloads.custom(41, lens, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype="bf16",
                         partition_tokens=P)
    s = Setup(w)
    torch.cuda.synchronize()
    before = s.table.buffer.cpu().numpy().copy()
    info = s.table.info()
    log(f"  units {info}")
    if P == 16:
        assert info["num_units"] * w.num_kv_heads > 4 * 768
    outs = [out_values(s.run()) for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    after = s.table.buffer.cpu().numpy()
    assert np.array_equal(before, after), "queue counters or merge tickets not back at zero"
    assert_close(outs[0], s.oracle(), "bf16", f"queue P={P}")
