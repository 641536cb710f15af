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


@pytest.mark.parametrize("name,extra", [("c2", 4), ("c3", 4), ("c4", 1), ("c5", 4)])
def test_full_size_sampled(name, extra):
    log(f"full size {name}")
    w = workloads.make(name, materialize=False)
    s = Setup(w, poison=False)
    got = out_values(s.run())
    seqs = _sample(w, extra, 11)
    ref = s.oracle(seqs=seqs)
    err = assert_close(got[seqs], ref[seqs], w.kv_dtype, name)
    log(f"  {name}: seqs {seqs} max abs err {err:.3e}; {s.table.info()}")
    assert np.isfinite(got).all()
