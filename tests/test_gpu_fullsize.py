"""GPU: full-size workloads in the launch configuration bench.py times, checked
on sampled sequences against the float64 oracle (which reads the device pool
back: at these sizes the prefilled cache comes from the seeded device RNG)."""

import numpy as np
import pytest

import workloads
from gpu_setup import Setup, assert_close, log, out_values

pytestmark = pytest.mark.gpu


def _sample(w, k_extra, seed):
    lens = w.seq_lens
    rng = np.random.default_rng(seed)
    picks = {int(np.argmax(lens)), int(np.argmin(lens))}
    picks.update(int(x) for x in rng.choice(w.batch, size=min(k_extra, w.batch), replace=False))
    return sorted(picks)


# P = -1 is the balanced plan bench.py times; the other value is the config's
# own partition length (c4: 512-token partitions and a separate merge kernel).
@pytest.mark.parametrize("name,extra,P", [("c2", 4, -1), ("c2", 4, 512), ("c3", 4, -1), ("c3", 4, 512),
                                          ("c4", 1, 512), ("c4", 1, -1), ("c5", 4, -1), ("c5", 4, 512)])
def test_full_size_sampled(name, extra, P):
    log(f"full size {name} P={P}")
    w = workloads.make(name, materialize=False)
    s = Setup(w, partition_tokens=P, poison=False)
    got = out_values(s.run())
    seqs = _sample(w, extra, 11)
    ref = s.oracle(seqs=seqs)
    err = assert_close(got[seqs], ref[seqs], w.kv_dtype, name)
    log(f"  {name} P={P}: seqs {seqs} max abs err {err:.3e}; {s.table.info()}")
    assert np.isfinite(got).all()
