"""GPU: paged_attention_append (append + attend in one launch) equals the
separate slot_mapping_compute + reshape_and_cache + attention calls, bit for
bit in the pool and in the outputs."""

import numpy as np
import pytest
import torch

import workloads
from gpu_setup import Setup, assert_close, log, out_values, to_device

pytestmark = pytest.mark.gpu


def _both_routes(w, P=None, poison=True):
    import paged_kv_cache_293_amd as pk
    s = Setup(w, partition_tokens=P, poison=poison, write_new=False)
    fused_store = s.pool.storage.clone()
    fused_pool = pk.kv_pool_create(w.num_layers, w.num_blocks, w.num_kv_heads, w.head_dim, w.kv_dtype,
                                   storage=fused_store, k_scale=s.pool.k_scale, v_scale=s.pool.v_scale)
    # separate calls
    s._write(w.new_seq_ids, w.new_positions, w.k_new, w.v_new)
    ref = s.run()
    # fused call: new tokens arrive as [B][k][H_kv][d] in sequence order
    k_new = to_device(w.k_new, w.in_dtype)
    v_new = to_device(w.v_new, w.in_dtype)
    got = pk.paged_attention_append(fused_pool, w.layer, s.table, k_new, v_new, s.q, w.scale)
    torch.cuda.synchronize()
    return s, ref, got, fused_store


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s", "c5s"])
def test_append_equals_separate_calls(name):
    log(f"append {name}")
    w = workloads.make(name)
    s, ref, got, fused_store = _both_routes(w)
    assert torch.equal(fused_store, s.pool.storage), "pool bytes differ"
    assert torch.equal(got, ref), "outputs differ"
    assert_close(out_values(got), s.oracle(), w.kv_dtype, f"append {name}")


def test_append_fp8_from_float32_inputs():
    log("append fp8 from f32")
    w = workloads.make("c5s")
    for attr in ("k_pre", "v_pre", "k_new", "v_new"):
        setattr(w, attr, workloads.values_f32(getattr(w, attr), "bf16"))
    w.in_dtype = "f32"
    s, ref, got, fused_store = _both_routes(w)
    assert torch.equal(fused_store, s.pool.storage)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_append_full_size_bench_configuration(name):
    log(f"append full size {name}")
    w = workloads.make(name, materialize=False)
    s, ref, got, fused_store = _both_routes(w, P=-1, poison=True)
    assert torch.equal(fused_store, s.pool.storage)
    assert torch.equal(got, ref)


# Appends spanning several blocks and unit boundaries, every pool type, and
# row counts on both sides of 32 (up to 32 rows the appended positions fall in
# each wave's first tile; beyond, any tile may hold them).  Sequence lengths
# put the first appended position at offsets 0, 1, 15 of a block, and the
# 32-token partitions cut several sequences into units.
@pytest.mark.parametrize("kv,k,Hq,Hkv,d", [
    ("bf16", 1, 8, 2, 128), ("bf16", 8, 16, 4, 128), ("bf16", 9, 32, 8, 128),
    ("bf16", 33, 8, 8, 64), ("fp8", 17, 8, 4, 128), ("int8", 12, 32, 8, 64),
    ("f32", 6, 8, 2, 128), ("f32", 20, 4, 2, 64), ("int4", 17, 8, 4, 128), ("int4", 33, 8, 8, 64),
])
def test_append_multi_block_rows(kv, k, Hq, Hkv, d):
    log(f"append multi-block kv={kv} k={k} {Hq}/{Hkv} d{d}")
    lens = [k, k + 1, k + 15, 16 + k, 17 + k, 47 + k, 200, 321]
    w = workloads.custom(4100 + 7 * k + d, lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=kv,
                         k_rows=k, partition_tokens=32)
    for P in (32, -1, 0):
        s, ref, got, fused_store = _both_routes(w, P=P)
        assert torch.equal(fused_store, s.pool.storage), f"pool bytes differ (P={P})"
        assert torch.equal(got, ref), f"outputs differ (P={P})"
    assert_close(out_values(got), s.oracle(), kv, f"append multi-block {kv} k={k}")
