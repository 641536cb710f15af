"""GPU: the full-size workloads, every sequence against the float64 oracle.

Each pool is filled by the seeded device RNG over the blocks the tables name;
every other block holds the poison byte (NaN, or a code the cache write never
stores), so a read outside a sequence's own blocks shows in its output.  The
oracle reads the device pool back and runs over all sequences (spread over
host threads).  Each workload runs in the launch configuration bench.py times
(its default partition plan) and at the config's other plan: c4 at its stated
512-token partitions (merged by the separate merge kernel) and at the balanced
plan, the others at the balanced plan and at 512-token partitions.  Every
output must be finite and meet the plain max-abs bound where |ref| <= 1 (and
the bound scaled by |ref| above 1); the errors are logged per workload and plan.
"""

import time

import numpy as np
import pytest

import workloads
from gpu_setup import Setup, assert_close, error_stats, log, out_values

pytestmark = pytest.mark.gpu

CASES = [("c2", -1), ("c2", 512), ("c3", -1), ("c3", 512), ("c4", 512), ("c4", -1),
         ("c5", -1), ("c5", 512), ("c2i8", -1), ("c2i8", 512), ("c2i4", -1), ("c2i4", 512)]

_cache = {}


def _standing(name):
    """The workload on the device and the oracle's output over every
    sequence; one workload is kept at a time (c3's pool is 7.8 GB)."""
    if name not in _cache:
        _cache.clear()
        w = workloads.make(name, materialize=False)
        t0 = time.perf_counter()
        s = Setup(w, partition_tokens=-1, poison=True)
        ref = s.oracle_all()
        log(f"  {name}: oracle over {w.batch} sequences ({int(w.seq_lens.sum())} tokens) "
            f"in {time.perf_counter() - t0:.1f} s")
        _cache[name] = (w, s, ref)
    return _cache[name]


@pytest.mark.parametrize("name,P", CASES)
def test_full_size_every_sequence(name, P):
    log(f"full size {name} P={P}")
    w, s, ref = _standing(name)
    table = s.table if P == -1 else s.upload(P)
    got = out_values(s.run(table=table))
    err = assert_close(got, ref, w.kv_dtype, f"{name} P={P}")
    e_unit, r_big, n_big = error_stats(got, ref)
    log(f"  {name} P={P}: {w.batch} sequences, max abs err {err:.3e} (|ref| <= 1), "
        f"max rel err {r_big:.3e} over {n_big} outputs with |ref| > 1; {table.info()}")
    assert e_unit == err
    if name == "c4" and P == 512:
        assert table.info()["max_parts"] == 256   # 131072 / 512: the separate merge kernel runs
    if name == "c5":
        # the balanced upload keeps the shared-prefix plan (its cost estimate
        # favours it at 128 sequences); fixed partitions do not
        assert table.shared_prefix() == ((128, 4) if P == -1 else (0, 0))
