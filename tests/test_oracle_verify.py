"""Pins of the oracle's verification against what the method guarantees.

* greedy: the accepted length is the longest matching prefix, and running
  rounds of draft + verify commits exactly the tokens that plain token-by-token
  argmax decoding of the same target commits, whatever the drafts are;
* rejection sampling: on a tiny vocabulary, exact enumeration with rational
  arithmetic over every draft, accept and draw outcome shows that the
  committed tokens follow the target's autoregressive distribution (the
  lossless property of speculative sampling), for drafts that disagree with
  the target, including zero-probability tokens on either side.
"""
import itertools
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import dmtp
from oracle.dmtp import verify_greedy, verify_rejection, verify_target_only


def test_verify_greedy_longest_prefix_bruteforce():
    rng = np.random.default_rng(0)
    for _ in range(3000):
        K = int(rng.integers(1, 9))
        y = rng.integers(0, 3, size=K + 1)
        d = rng.integers(0, 3, size=K)
        L, toks = verify_greedy(d, y)
        # brute force: largest L with d[:L] == y[:L]
        best = max(l for l in range(K + 1) if all(d[i] == y[i] for i in range(l)))
        assert L == best
        assert toks == list(d[:L]) + [int(y[L])]
        assert len(toks) == L + 1


def _toy_logits(prefix, V=11, H=6, seed=3):
    """A deterministic toy target: logits are a fixed random map of a prefix hash."""
    h = np.random.default_rng([seed] + [int(t) + 1 for t in prefix]).standard_normal(H)
    W = np.random.default_rng([seed, 999]).standard_normal((V, H))
    return W @ h


def test_greedy_rounds_commit_plain_greedy_decoding():
    rng = np.random.default_rng(1)
    prompt = [2, 5]
    n_tokens = 60
    # plain decoding, one argmax at a time
    plain = list(prompt)
    while len(plain) < len(prompt) + n_tokens:
        plain.append(int(np.argmax(_toy_logits(plain))))
    for K in (1, 3, 7):
        seq = list(prompt)
        while len(seq) < len(prompt) + n_tokens:
            # drafts: the true continuation with some corruption
            truth, tmp = [], list(seq)
            for _ in range(K):
                t = int(np.argmax(_toy_logits(tmp)))
                truth.append(t)
                tmp.append(t)
            drafts = [t if rng.random() < 0.7 else int(rng.integers(0, 11)) for t in truth]
            # target rows: row i sees the prefix plus drafts[:i]
            y = [int(np.argmax(_toy_logits(seq + drafts[:i]))) for i in range(K + 1)]
            L, toks = verify_greedy(drafts, y)
            seq += toks
        assert seq[: len(plain)] == plain, K


class ExactOps:
    @staticmethod
    def ratio(p_row, q_row, tok):
        return p_row[tok] / q_row[tok]

    @staticmethod
    def residual(p_row, q_row):
        return [max(Fr(0), a - b) for a, b in zip(p_row, q_row)]

    @staticmethod
    def total(w):
        return sum(w, Fr(0))


class _Path:
    """Replays a fixed list of choices and records the probability of the path."""

    def __init__(self, choices):
        self.choices = list(choices)
        self.pos = 0
        self.prob = Fr(1)
        self.branch_points = []     # (position, number of options)

    def _choose(self, probs):
        opts = [i for i, p in enumerate(probs) if p > 0]
        if self.pos >= len(self.choices):
            self.branch_points.append((self.pos, len(opts)))
            self.choices.append(0)
        c = opts[self.choices[self.pos]]
        self.pos += 1
        self.prob *= probs[c]
        return c

    def accept(self, i, ratio):
        a = min(Fr(1), ratio)
        return self._choose([a, 1 - a]) == 0

    def draw(self, i, w):
        tot = sum(w, Fr(0))
        return self._choose([x / tot for x in w])


def _enumerate(run):
    out = []
    stack = [[]]
    while stack:
        prefix = stack.pop()
        path = _Path(prefix)
        res = run(path)
        out.append((path.prob, res))
        for pos, n in path.branch_points:
            for alt in range(1, n):
                stack.append(path.choices[:pos] + [alt])
    return out


def _toy_dist(prefix, V, salt):
    """Rational toy distribution with some zero entries; depends on the prefix."""
    h = 7 if salt == "p" else 13
    for t in prefix:
        h = (h * 31 + t + 1) % 1000003
    w = [Fr(((h * 17 + t * 29 + h // 7) % 4)) for t in range(V)]
    if sum(w) == 0:
        w[len(prefix) % V] = Fr(1)
    s = sum(w)
    return [x / s for x in w]


@pytest.mark.parametrize("V,K,N", [(3, 2, 3), (4, 1, 3), (3, 3, 2)])
def test_rejection_sampling_is_lossless_exact_enumeration(V, K, N):
    p = lambda pre: _toy_dist(pre, V, "p")  # noqa: E731
    q = lambda pre: _toy_dist(pre, V, "q")  # noqa: E731

    def run(path):
        seq = []
        while len(seq) < N:
            drafts = []
            for i in range(K):
                drafts.append(path.draw(-1, q(seq + drafts)))
            p_rows = [p(seq + drafts[:i]) for i in range(K + 1)]
            q_rows = [q(seq + drafts[:i]) for i in range(K)]
            # a draft drawn from q never has q = 0 at its own token
            L, toks = verify_rejection(drafts, p_rows, q_rows, path.accept, path.draw, ops=ExactOps)
            seq += toks
        return tuple(seq[:N])

    dist = {}
    for prob, s in _enumerate(run):
        dist[s] = dist.get(s, Fr(0)) + prob
    assert sum(dist.values()) == 1
    for s in itertools.product(range(V), repeat=N):
        want = Fr(1)
        for t in range(N):
            want *= p(list(s[:t]))[s[t]]
        assert dist.get(s, Fr(0)) == want, (s, dist.get(s), want)


def test_rejection_special_cases():
    V = 5
    p = [Fr(1, 5)] * V
    # q == p: every candidate is accepted, the bonus comes from p_K
    for d in itertools.product(range(V), repeat=2):
        res = _enumerate(lambda path: verify_rejection(list(d), [p] * 3, [p] * 2, path.accept,
                                                       path.draw, ops=ExactOps)[0])
        assert all(L == 2 for _, L in res)
    # q one-hot on a token that p gives zero: always rejected, correction from p
    p0 = [Fr(0), Fr(1, 2), Fr(1, 4), Fr(1, 4), Fr(0)]
    q0 = [Fr(1), Fr(0), Fr(0), Fr(0), Fr(0)]
    res = _enumerate(lambda path: verify_rejection([0], [p0, p0], [q0], path.accept, path.draw,
                                                   ops=ExactOps))
    dist = {}
    for prob, (L, toks) in res:
        assert L == 0
        dist[toks[0]] = dist.get(toks[0], Fr(0)) + prob
    assert dist == {1: Fr(1, 2), 2: Fr(1, 4), 3: Fr(1, 4)}


def test_float_ops_agree_with_exact_ops():
    rng = np.random.default_rng(2)
    p = rng.random(7)
    p /= p.sum()
    q = rng.random(7)
    q /= q.sum()
    r = dmtp.VerifyOps.residual(p, q)
    re = ExactOps.residual([Fr(x) for x in p], [Fr(x) for x in q])
    np.testing.assert_allclose(r, [float(x) for x in re], rtol=0, atol=1e-16)
    assert dmtp.VerifyOps.ratio(p, q, 3) == pytest.approx(p[3] / q[3])


def test_enumeration_detects_a_planted_mistake():
    """Sensitivity: a wrong residual (max(0, q - p)) breaks the lossless identity."""
    class WrongOps(ExactOps):
        @staticmethod
        def residual(p_row, q_row):
            return [max(Fr(0), b - a) for a, b in zip(p_row, q_row)]

    V, K = 3, 1
    p = lambda pre: _toy_dist(pre, V, "p")  # noqa: E731
    q = lambda pre: _toy_dist(pre, V, "q")  # noqa: E731

    def run(path):
        d = [path.draw(-1, q([]))]
        L, toks = verify_rejection(d, [p([]), p(d)], [q([])], path.accept, path.draw, ops=WrongOps)
        return toks[0]

    dist = {}
    for prob, t in _enumerate(run):
        dist[t] = dist.get(t, Fr(0)) + prob
    assert any(dist.get(t, Fr(0)) != p([])[t] for t in range(V))


# ---------------------------------------------------------------------------
# target-only verification
# ---------------------------------------------------------------------------


def test_target_only_with_argmax_picks_is_greedy():
    rng = np.random.default_rng(4)
    for _ in range(3000):
        K = int(rng.integers(1, 9))
        y = rng.integers(0, 3, size=K + 1)
        d = rng.integers(0, 3, size=K)
        called = []

        def pick(i):
            called.append(i)
            return int(y[i])

        assert verify_target_only(d, pick) == verify_greedy(d, y)
        # picks are taken in order and stop at the first mismatch (or the bonus row)
        assert called == list(range(len(called)))
        assert len(called) == verify_greedy(d, y)[0] + 1


def _target_only_committed(V, K, N, p, q, commit_rejected_draft=False):
    """Distribution of the first N committed tokens of repeated target-only rounds."""

    def run(path):
        seq = []
        while len(seq) < N:
            drafts = []
            for _ in range(K):
                drafts.append(path.draw(-1, q(seq + drafts)))

            def pick(i, seq=seq, drafts=drafts):
                return path.draw(i, p(seq + drafts[:i]))

            L, toks = verify_target_only(drafts, pick)
            if commit_rejected_draft and L < K:
                toks[L] = drafts[L]
            seq += toks
        return tuple(seq[:N])

    dist = {}
    for prob, s in _enumerate(run):
        dist[s] = dist.get(s, Fr(0)) + prob
    return dist


@pytest.mark.parametrize("V,K,N", [(3, 2, 3), (4, 1, 3), (3, 3, 2)])
def test_target_only_is_lossless_exact_enumeration(V, K, N):
    p = lambda pre: _toy_dist(pre, V, "p")  # noqa: E731
    q = lambda pre: _toy_dist(pre, V, "q")  # noqa: E731
    dist = _target_only_committed(V, K, N, p, q)
    assert sum(dist.values()) == 1
    for s in itertools.product(range(V), repeat=N):
        want = Fr(1)
        for t in range(N):
            want *= p(list(s[:t]))[s[t]]
        assert dist.get(s, Fr(0)) == want, (s, dist.get(s), want)


def test_target_only_acceptance_closed_form():
    """For fixed drafts, P(L >= k) = prod_{i<k} p_i(d_i) with p_i after d_0..d_{i-1}."""
    V, K = 4, 3
    p = lambda pre: _toy_dist(pre, V, "p")  # noqa: E731
    for d in itertools.product(range(V), repeat=K):
        d = list(d)

        def run(path):
            return verify_target_only(d, lambda i: path.draw(i, p(d[:i])))[0]

        hist = {}
        for prob, L in _enumerate(run):
            hist[L] = hist.get(L, Fr(0)) + prob
        for k in range(K + 1):
            want = Fr(1)
            for i in range(k):
                want *= p(d[:i])[d[i]]
            got = sum((v for L, v in hist.items() if L >= k), Fr(0))
            assert got == want, (d, k, got, want)


def test_target_only_enumeration_detects_a_planted_mistake():
    """Sensitivity: committing the rejected draft instead of the target's pick is not lossless."""
    V, K, N = 3, 2, 2
    p = lambda pre: _toy_dist(pre, V, "p")  # noqa: E731
    q = lambda pre: _toy_dist(pre, V, "q")  # noqa: E731
    dist = _target_only_committed(V, K, N, p, q, commit_rejected_draft=True)
    wrong = 0
    for s in itertools.product(range(V), repeat=N):
        want = Fr(1)
        for t in range(N):
            want *= p(list(s[:t]))[s[t]]
        wrong += dist.get(s, Fr(0)) != want
    assert wrong > 0
