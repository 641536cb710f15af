"""Pins for the oracle's exact speculative sampling (CPU only)."""

import numpy as np

from conftest import golden_lines
from oracle import speculative as osp


def _example():
    rows = {r[0]: np.array([float(x) for x in r[1:]]) for r in golden_lines("speculative_example.txt")}
    return rows


def test_page_worked_example_masses():
    ex = _example()
    p, q = ex["p"], ex["q"]
    assert np.allclose(np.minimum(p, q), ex["accepted"], atol=1e-15)
    assert np.allclose(osp.residual(p, q), ex["residual"], atol=1e-15)
    assert np.allclose(np.minimum(p, q) + osp.residual(p, q), p, atol=1e-15)
    # acceptance probability of a proposed token is min(1, p/q): token 0 is
    # accepted for u < 1/3, tokens 1 and 2 always
    assert osp.accept_position(p.astype(np.float32), q.astype(np.float32), 0, 0.33)
    assert not osp.accept_position(p.astype(np.float32), q.astype(np.float32), 0, 0.34)
    for t in (1, 2):
        assert osp.accept_position(p.astype(np.float32), q.astype(np.float32), t, 0.999)


def test_emitted_token_follows_the_target_distribution():
    """Integrate over the draft token (weight q(x)) and a fine grid of both
    uniforms: the probability that the first emitted token is j is p(j)."""
    ex = _example()
    p = ex["p"].astype(np.float32)[None]
    q = ex["q"].astype(np.float32)[None]
    n = 400
    grid = (np.arange(n) + 0.5) / n
    prob = np.zeros(3)
    for x in range(3):
        for ua in grid:
            for us in grid[::4]:
                a, toks = osp.accept_sequence(np.vstack([p, p]), q, np.array([x]), np.array([ua]), us)
                prob[toks[0]] += q[0, x] / (n * (n // 4))
    assert np.allclose(prob, ex["p"], atol=5e-3), prob


def test_special_cases():
    rng = np.random.default_rng(5)
    V, K = 11, 4
    p = rng.dirichlet(np.ones(V), size=K + 1).astype(np.float32)
    draft = rng.integers(0, V, size=K)
    # identical draft and target: every position accepts, the bonus comes from p_{K+1}
    a, toks = osp.accept_sequence(p, p[:K], draft, np.full(K, 0.999), 0.0)
    assert a == K and toks[:K] == list(draft)
    assert toks[K] == int(np.argmax(p[K] > 0))
    # target one-hot on a token the draft did not propose: rejected at once, emits it
    onehot = np.zeros((K + 1, V), np.float32)
    onehot[:, 3] = 1.0
    q = np.full((K, V), 1.0 / V, np.float32)
    a, toks = osp.accept_sequence(onehot, q, np.array([5, 3, 3, 3]), np.zeros(K), 0.7)
    assert a == 0 and toks == [3]
    # out-of-range draft token is rejected
    a, toks = osp.accept_sequence(p, p[:K], np.array([V, 0, 0, 0]), np.zeros(K), 0.5)
    assert a == 0
    # draw: smallest j whose running sum exceeds u * total; zero weights never drawn
    w = np.array([0.0, 0.25, 0.0, 0.25, 0.5])
    assert [osp.draw(w, u) for u in (0.0, 0.24, 0.25, 0.49, 0.5, 0.99)] == [1, 1, 3, 3, 4, 4]
