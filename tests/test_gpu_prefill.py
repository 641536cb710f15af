"""GPU: chunked-prefill paged attention against the float64 oracle.

Every sequence carries C query tokens at positions n-C .. n-1 (their K/V
appended through the library first); row j sees positions t <= n-C+j.
Tolerance as for decode: 1e-2 max-abs for bf16 / fp8 KV on unit-scale
outputs.  Covered: the reduced and full-size chunked-prefill workloads,
GQA / MQA / MHA heads, head_dim 64 and 128, bf16 and fp8 pools, chunks that
do not fill the last 256-row tile or the last block, a chunk that is the whole
sequence, a causal needle, and agreement with the verify kernel where both
apply.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_setup import Setup, assert_close, log, out_values, to_device

pytestmark = pytest.mark.gpu


def test_prefill_reduced_workload():
    log("prefill pfs")
    w = workloads.make("pfs")
    s = Setup(w)
    got = out_values(s.run_prefill())
    err = assert_close(got, s.oracle_prefill(), "bf16", "pfs")
    log(f"  pfs: max abs err {err:.3e}")


@pytest.mark.parametrize("kv,Hq,Hkv,d,C,lens", [
    ("bf16", 32, 8, 128, 64, [64, 65, 300, 1000]),      # GQA G=4; chunk == whole first sequence
    ("bf16", 64, 8, 128, 48, [48, 200, 529]),           # G=8 (Llama-3-70B heads)
    ("bf16", 8, 1, 128, 40, [40, 77]),                  # MQA
    ("bf16", 4, 4, 64, 100, [100, 131, 260]),           # MHA, d=64
    ("fp8", 32, 8, 128, 70, [70, 150, 333]),
    ("fp8", 16, 2, 64, 33, [33, 100]),
])
def test_prefill_shapes(kv, Hq, Hkv, d, C, lens):
    log(f"prefill {kv} {Hq}/{Hkv} d{d} C={C}")
    w = workloads.custom(500 + C + Hq, lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, kv_dtype=kv,
                         k_rows=C, partition_tokens=0)
    s = Setup(w)
    got = out_values(s.run_prefill())
    assert np.isfinite(got).all()
    err = assert_close(got, s.oracle_prefill(), kv, f"{kv} {Hq}/{Hkv} d{d} C={C}")
    log(f"  max abs err {err:.3e}")
    f32 = out_values(s.run_prefill(out_dtype="f32"))
    assert_close(f32, s.oracle_prefill(), kv, "f32 output")


def test_prefill_matches_verify_kernel():
    """Where both calls apply (G * k <= 64 rows), the prefill and verify
    kernels compute the same rows."""
    log("prefill == verify")
    w = workloads.custom(77, [16, 90, 400], num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype="bf16",
                         k_rows=12, partition_tokens=64)
    s = Setup(w)
    pre = out_values(s.run_prefill())
    ver = out_values(s.run())
    assert_close(pre, ver, "bf16", "prefill vs verify")
    assert_close(pre, s.oracle(), "bf16", "prefill vs oracle")


def test_prefill_causal_needle():
    """A needle key at chunk token j* is seen by rows j >= j* only: with
    q = 16 e_0 and K[:, 0] = 128 at the needle (0 elsewhere) rows at or after
    it return V[needle] exactly, rows before it do not see it."""
    log("prefill causal needle")
    C = 50
    lens = [C + 30, C]
    needle = [30 + 20, 17]          # positions: chunk token 20 of seq 0, chunk token 17 of seq 1
    w = workloads.custom(12, lens, num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype="bf16",
                         k_rows=C, partition_tokens=0)
    qf = np.zeros(w.q.shape, dtype=np.float32)
    qf[..., 0] = 16.0
    w.q = workloads._cast(qf, "bf16")
    kp = workloads.values_f32(w.k_pre, "bf16").copy()
    kn = workloads.values_f32(w.k_new, "bf16").copy()
    kp[..., 0] = 0.0
    kn[..., 0] = 0.0
    for sq, t in enumerate(needle):
        hit = np.flatnonzero((w.new_seq_ids == sq) & (w.new_positions == t))
        kn[hit[0], :, 0] = 128.0
    w.k_pre = workloads._cast(kp, "bf16")
    w.k_new = workloads._cast(kn, "bf16")
    s = Setup(w)
    got = out_values(s.run_prefill(out_dtype="f32"))
    ref = s.oracle_prefill()
    assert_close(got, ref, "bf16", "needle")
    for sq, t in enumerate(needle):
        j = t - (lens[sq] - C)
        after = ref[sq, j:].astype(np.float32).astype(np.float64)
        assert np.array_equal(got[sq, j:], after), f"seq {sq}: rows from the needle on are not one-hot"


@pytest.mark.parametrize("seqs,rows", [([0, 5], [0, 1, 255, 256, 1023, 2046, 2047]), ([7], [100, 1500])])
def test_prefill_full_size_sampled(seqs, rows):
    """The full chunked-prefill workload (8 sequences, 2048-token chunks,
    contexts to 16K) in the configuration bench.py times; sampled rows of
    sampled sequences against the oracle reading the device pool back (blocks
    no table names hold NaN)."""
    log(f"prefill full size seqs {seqs} rows {rows}")
    w = workloads.make("pf")
    s = Setup(w, poison=True)
    got = out_values(s.run_prefill())
    assert np.isfinite(got).all()
    ref = s.oracle_prefill(seqs=seqs, rows=rows)
    err = assert_close(got[np.ix_(seqs, rows)], ref[np.ix_(seqs, rows)], "bf16", "pf sampled")
    log(f"  max abs err {err:.3e}")
