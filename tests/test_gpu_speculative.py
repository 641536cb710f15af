"""GPU: exact speculative acceptance against the oracle.

The number accepted and the accepted draft tokens are integers decided by
the same float32 test on both sides: they must match exactly.  The drawn
token is the first index whose running sum of weights exceeds u * sum; the
kernel sums in float32, the oracle in float64, so where u * sum falls within
rounding of a running-sum boundary either neighbour is correct: the test
requires the kernel's token to equal the oracle's, or to be a valid draw
within that rounding.  Also: the scalar path (vocabulary not a multiple of
4), one and many drafted tokens, special cases, and the emitted token's
distribution over many uniforms equalling the target's.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_setup import DEV, log
from oracle import speculative as osp

pytestmark = pytest.mark.gpu


def _run(w):
    import paged_kv_cache_293_amd as pk
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    a, toks = pk.speculative_accept(t(w.p), t(w.q), t(w.draft), t(w.u_accept), t(w.u_sample))
    torch.cuda.synchronize()
    return a.cpu().numpy(), toks.cpu().numpy()


def _check(w, a, toks, tol=2e-6):
    ra, rt = osp.accept_batch(w.p, w.q, w.draft, w.u_accept, w.u_sample)
    assert np.array_equal(a, ra), f"accepted counts differ: {a} vs {ra}"
    ambiguous = 0
    for b in range(w.batch):
        n = int(ra[b])
        assert np.array_equal(toks[b, :n], rt[b, :n])
        assert (toks[b, n + 1:] == -1).all()
        if toks[b, n] == rt[b, n]:
            continue
        # a different draw must sit on a rounding boundary of the weights' running sum
        if n < w.k:
            wts = osp.residual(w.p[b, n], w.q[b, n])
            if wts.sum() == 0:
                wts = w.p[b, n].astype(np.float64)
        else:
            wts = w.p[b, w.k].astype(np.float64)
        c = np.cumsum(wts)
        T = float(w.u_sample[b]) * c[-1]
        j = int(toks[b, n])
        assert 0 <= j < w.vocab and wts[j] > 0, f"seq {b}: drew a zero-weight token {j}"
        lo = c[j - 1] if j > 0 else 0.0
        assert lo - tol * c[-1] <= T <= c[j] + tol * c[-1], f"seq {b}: token {j} is not a valid draw"
        ambiguous += 1
    return ambiguous


def test_reduced_workload():
    log("speculative sps")
    w = workloads.make_spec("sps")
    a, toks = _run(w)
    _check(w, a, toks)


@pytest.mark.parametrize("B,K,V", [(33, 1, 4097), (9, 7, 1003), (20, 4, 256), (5, 3, 70000)])
def test_shapes(B, K, V):
    log(f"speculative B={B} K={K} V={V}")
    w = workloads.make_spec("sps", seed=77 + V, batch=B, k=K, vocab=V)
    a, toks = _run(w)
    _check(w, a, toks)


def test_special_cases():
    log("speculative special cases")
    w = workloads.make_spec("sps", seed=5, batch=6, k=4, vocab=300)
    w.q[0] = w.p[0, :4]                    # identical distributions: everything accepted
    w.u_accept[0] = 0.999
    w.p[1] = 0.0
    w.p[1, :, 17] = 1.0                    # one-hot target on a token the draft did not pick
    w.draft[1] = [3, 17, 17, 17]
    w.draft[2, 0] = 300                    # out of range: rejected
    w.u_sample[3] = 0.0                    # draws the first weighted index
    w.q[4, 0] = w.p[4, 0]                  # zero residual mass at the first position
    w.u_accept[4, 0] = 0.999999            # ... while the test still rejects
    w.p[4, 0, w.draft[4, 0]] = 0.0
    a, toks = _run(w)
    _check(w, a, toks)
    assert a[0] == 4 and a[1] == 0 and toks[1, 0] == 17 and a[2] == 0


def test_emitted_tokens_follow_the_target_distribution():
    """The page's 3-token example, 65536 sequences with fresh uniforms: the
    frequency of each first emitted token is p within statistical error."""
    log("speculative distribution")
    n = 65536
    rng = np.random.default_rng(424)
    p = np.array([0.2, 0.5, 0.3], np.float32)
    q = np.array([0.6, 0.3, 0.1], np.float32)
    draft = np.searchsorted(np.cumsum(q), rng.random(n) * q.sum(), side="right").astype(np.int32)[:, None]
    w = workloads.SpecWorkload("dist", 0, np.tile(p, (n, 2, 1)).copy(), np.tile(q, (n, 1, 1)).copy(),
                               np.minimum(draft, 2), rng.random((n, 1), dtype=np.float32),
                               rng.random(n, dtype=np.float32))
    a, toks = _run(w)
    _check(w, a, toks)
    freq = np.bincount(toks[:, 0], minlength=3) / n
    sigma = np.sqrt(p * (1 - p) / n)
    assert (np.abs(freq - p) < 5 * sigma).all(), (freq, p)


def test_full_size_vocabulary():
    log("speculative sp full size")
    w = workloads.make_spec("sp")
    a, toks = _run(w)
    amb = _check(w, a, toks)
    log(f"  mean accepted {a.mean():.2f}; boundary-ambiguous draws {amb}")


def test_draw_near_the_end_of_the_row():
    """u just below 1 at Llama-3's vocabulary, with the rows' last 2,256
    weights zero (the last wave's trailing tiles carry no weight): every draw
    must still be a weighted token, the last one or within rounding of the
    row's end, for a residual (rejection at position 0) and a bonus draw."""
    log("speculative u near 1")
    w = workloads.make_spec("sps", seed=31, batch=4, k=4, vocab=128256)
    w.p[:, :, 126000:] = 0.0
    w.q[:, :, 126000:] = 0.0
    w.q[0] = w.p[0, :4]                       # identical: all accepted, the bonus row is drawn
    w.draft[0] = np.argmax(w.p[0, :4], axis=1)
    w.u_accept[0] = 0.5
    w.u_accept[1, 0] = 0.999999               # position 0 rejects: a residual draw
    w.draft[1, 0] = int(np.argmax(w.q[1, 0] - w.p[1, 0]))
    w.u_sample[:] = np.float32(1.0) - np.float32(2.0 ** -24)
    a, toks = _run(w)
    _check(w, a, toks)
    assert a[0] == 4 and a[1] == 0
    assert (toks[np.arange(4), a] >= 0).all() and (toks[np.arange(4), a] < 126000).all()
