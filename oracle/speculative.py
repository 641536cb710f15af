"""Exact speculative sampling (oracle, test infrastructure only).

Method (page "LLM Serving - KV Cache, Batching, Speculative Decoding",
section "Speculative decoding: distribution and break-even"; page "KV cache
& continuous batching", section "5. Speculative decoding"): a draft model
proposes tokens x_1..x_K drawn from its distributions q_1..q_K; one target
pass gives p_1..p_{K+1}.  Position i accepts x_i with probability
min(1, p_i(x_i) / q_i(x_i)); the first rejected position emits a token drawn
from the normalised positive residual (p_i - q_i)+ and ends the block; when
all K are accepted, a bonus token is drawn from p_{K+1}.  The accepted mass
min(p, q) plus the residual (p - q)+ is p, so the emitted tokens follow the
target's distribution.

Readings taken where the pages leave the step open (recorded in the design
notes):

* random draws are inputs: u_accept[i] in [0, 1) per position and one
  u_sample in [0, 1) for the emitted draw;
* accepting x_i is the float32 test  u_accept[i] * q_i(x_i) < p_i(x_i)
  (the ratio test without a division; q_i(x_i) = 0 accepts iff p_i(x_i) > 0);
  a draft token outside [0, V) is rejected;
* drawing from weights w with u: the smallest j whose running sum
  w_0 + .. + w_j exceeds u * sum(w) (inverse CDF; zero-weight tokens are never
  drawn); a residual with no mass falls back to p_i itself.

The oracle evaluates sums in float64 (exactly, for float32 inputs, up to
float64 rounding); the acceptance decision is the float32 comparison above.
Pins: tests/test_oracle_speculative.py (the page's 3-token worked example,
the mass identity, distribution preservation by exhaustive integration over
u, special cases).
"""

import numpy as np


def accept_position(p_row, q_row, token, u):
    """Whether the draft token passes position i's test (float32, as stated above)."""
    V = p_row.shape[0]
    if token < 0 or token >= V:
        return False
    pu = np.float32(p_row[token])
    qu = np.float32(q_row[token])
    return bool(np.float32(np.float32(u) * qu) < pu)


def residual(p_row, q_row):
    """(p - q)+ as float64."""
    return np.maximum(np.asarray(p_row, np.float64) - np.asarray(q_row, np.float64), 0.0)


def draw(weights, u):
    """Smallest j with w_0 + ... + w_j > u * sum(w) (float64)."""
    w = np.asarray(weights, np.float64)
    c = np.cumsum(w)
    target = float(u) * c[-1]
    return int(np.argmax(c > target))


def accept_sequence(p, q, draft, u_accept, u_sample):
    """One sequence: p [K+1][V], q [K][V], draft [K], u_accept [K], u_sample.

    Returns (number accepted a, emitted tokens: the a accepted drafts then
    the residual or bonus draw, a + 1 tokens).
    """
    K = q.shape[0]
    for i in range(K):
        if not accept_position(p[i], q[i], int(draft[i]), u_accept[i]):
            r = residual(p[i], q[i])
            w = r if r.sum() > 0 else np.asarray(p[i], np.float64)
            return i, [int(t) for t in draft[:i]] + [draw(w, u_sample)]
    return K, [int(t) for t in draft] + [draw(p[K], u_sample)]


def accept_batch(p, q, draft, u_accept, u_sample):
    """Batched: p [B][K+1][V], q [B][K][V], draft [B][K] -> (a [B], tokens [B][K+1], -1 padded)."""
    B, K = draft.shape
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, K + 1), -1, dtype=np.int32)
    for b in range(B):
        a, toks = accept_sequence(p[b], q[b], draft[b], u_accept[b], u_sample[b])
        acc[b] = a
        out[b, :len(toks)] = toks
    return acc, out
