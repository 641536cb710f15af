"""GPU: the sign and the zero of the softmax scale factor.

The kernels scale scores inside the exponent and take a row's largest scaled
score from its largest raw score, which holds only for a positive factor; a
negative factor has its sign moved into the query, a zero factor is replaced
by the smallest normal float.  Checked against the float64 oracle (which
applies the factor as given): a zero factor (every visible position weighs
the same: the mean of the visible V rows), negative factors, and a positive
one for contrast, for decode and verify rows (causal masks inside the last
blocks) over every pool type, split and unsplit sequences, and the chunked
prefill kernel over its pool types; plus the shared-prefix plan, whose prefix
pass runs the prefill kernel with the verify call's factor.
"""

import numpy as np
import pytest

import workloads
from gpu_setup import Setup, assert_close, log, out_values

pytestmark = pytest.mark.gpu

FACTORS = [0.0, -1.0, -0.3, 1.0]   # times 1 / sqrt(head_dim)


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "int8", "int4"])
@pytest.mark.parametrize("k,part", [(1, 0), (5, 64)])
def test_decode_verify_scale_sign(kv, k, part):
    w = workloads.custom(7100 + k, [37, 200, 517], num_q_heads=8, num_kv_heads=2, head_dim=64, kv_dtype=kv,
                         k_rows=k, partition_tokens=part)
    s = Setup(w)
    for f in FACTORS:
        scale = f * w.scale
        log(f"{kv} k={k} partitions {part}: scale {scale:+.4f}")
        got = out_values(s.run(scale=scale))
        assert np.isfinite(got).all()
        assert_close(got, s.oracle(scale=scale), kv, f"{kv} k={k} scale {scale:+.4f}")


def test_zero_scale_is_the_mean():
    """A zero factor: each row's output is the mean of the V rows it sees."""
    w = workloads.custom(7110, [3, 40, 129], num_q_heads=4, num_kv_heads=1, head_dim=64, kv_dtype="f32",
                         k_rows=2, partition_tokens=0)
    s = Setup(w)
    got = out_values(s.run(scale=0.0))
    ref = s.oracle(scale=0.0)
    assert_close(got, ref, "f32", "zero scale")
    # every weight is exactly 1, so the query heads of the one KV head agree bit for bit
    for g in range(1, 4):
        assert np.array_equal(got[:, :, g], got[:, :, 0])


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8", "int4"])
def test_prefill_scale_sign(kv):
    w = workloads.custom(7120, [60, 97, 300], num_q_heads=8, num_kv_heads=2, head_dim=64, kv_dtype=kv,
                         k_rows=60, partition_tokens=0)
    s = Setup(w)
    for f in FACTORS:
        scale = f * w.scale
        log(f"prefill {kv}: scale {scale:+.4f}")
        got = out_values(s.run_prefill(scale=scale))
        assert np.isfinite(got).all()
        assert_close(got, s.oracle_prefill(scale=scale), kv, f"prefill {kv} scale {scale:+.4f}")


def test_shared_prefix_scale_sign():
    rng = np.random.Generator(np.random.PCG64(7130))
    lens = 16 * 20 + rng.integers(5, 60, size=5, endpoint=True)
    w = workloads.build("prefix-scale", 7130, rng, lens, num_q_heads=8, num_kv_heads=2, head_dim=64,
                        kv_dtype="fp8", k_rows=5, shared_prefix_tokens=16 * 20, materialize=True,
                        partition_tokens=-2)
    s = Setup(w, partition_tokens=-2)
    assert s.table.shared_prefix()[0] == 20
    for f in FACTORS:
        scale = f * w.scale
        log(f"shared prefix fp8: scale {scale:+.4f}")
        got = out_values(s.run(scale=scale))
        assert np.isfinite(got).all()
        assert_close(got, s.oracle(scale=scale), "fp8", f"shared prefix scale {scale:+.4f}")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8", "int4"])
def test_prefill_large_scale_factors(kv):
    """Peaky softmax: 2, 4 and 8 times 1/sqrt(d).  The scale is applied to
    float32 scores, so the error does not grow with the scores' size (a
    query rounded to bf16 after scaling gave 2e-2 at 4x and 4e-2 at 8x)."""
    w = workloads.custom(7125, [60, 97, 300], num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype=kv,
                         k_rows=60, partition_tokens=0)
    s = Setup(w)
    for f in [2.0, 4.0, 8.0]:
        scale = f * w.scale
        got = out_values(s.run_prefill(scale=scale, out_dtype="f32"))
        err = assert_close(got, s.oracle_prefill(scale=scale), kv, f"prefill {kv} scale x{f}")
        log(f"prefill {kv} x{f}: max abs err {err:.3e}")


@pytest.mark.parametrize("kv", ["bf16", "int4"])
def test_verify_large_scale_factors(kv):
    w = workloads.custom(7126, [37, 200, 517], num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype=kv,
                         k_rows=5, partition_tokens=64)
    s = Setup(w)
    for f in [4.0, 8.0]:
        scale = f * w.scale
        got = out_values(s.run(scale=scale))
        err = assert_close(got, s.oracle(scale=scale), kv, f"verify {kv} scale x{f}")
        log(f"verify {kv} x{f}: max abs err {err:.3e}")
