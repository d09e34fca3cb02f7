"""Philox4x64-10 and the Gumbel noise drawn from it -- oracle side.

Philox is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  One call maps a
256-bit counter and a 128-bit key to 256 random bits through 10 rounds.  A
round multiplies counter words 0 and 2 by two fixed odd constants, keeps
both halves of each 128-bit product, and mixes them with the other two
words and the round key; the key is bumped by two Weyl constants between
rounds.  This module is written from that definition; the tests pin it
against NumPy's independent ``numpy.random.Philox``.

Draw layout (shared definition with the HIP sampler, each side implementing
it on its own): a draw is named by ``(seed, draw_key)``; the 32-bit word for
index j of noise level L comes from counter ``(j >> 3, draw_key, L, 0)`` under
key ``(seed, 0)``, output word ``(j & 7) >> 1``, low half when ``j & 1 == 0``.
Level 0 indexes vocabulary entries, level 1 blocks of entries.

Gumbel variate of word x: t = (x + 1/2) / 2^32, E = -log(1 - t) (an Exp(1)
variate), g = -log(E).  Taking E through log1p keeps full relative precision
for the small E that decide the maximum.  Sampling index j with probability
proportional to w_j is then argmax_j (log w_j + g_j) (the Gumbel-max
identity).

A draw over a vocabulary is taken in two levels (grouped_gumbel_argmax):
first a block of DRAW_BLOCK consecutive entries by Gumbel-max over the
blocks' log masses (level-1 noise), then an entry of that block by
Gumbel-max over its log weights (level-0 noise).  The two noises are
independent, so P(j) = P(block of j) P(j | block) = (Z_b / Z)(w_j / Z_b) =
w_j / Z: the same distribution as one Gumbel-max over all entries.  Test
infrastructure only.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
DRAW_BLOCK = 128
_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: int, b: np.ndarray):
    """High and low 64-bit halves of the 128-bit product a * b (b a uint64 array)."""
    a0 = np.uint64(a & 0xFFFFFFFF)
    a1 = np.uint64(a >> 32)
    b0 = b & _M32
    b1 = b >> _S32
    p00 = a0 * b0
    p01 = a0 * b1
    p10 = a1 * b0
    p11 = a1 * b1
    mid = (p00 >> _S32) + (p01 & _M32) + (p10 & _M32)
    lo = (p00 & _M32) | ((mid & _M32) << _S32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x64 with 10 rounds on arrays of counters; returns 4 uint64 arrays."""
    c = [np.asarray(v, dtype=np.uint64).copy() for v in np.broadcast_arrays(c0, c1, c2, c3)]
    mask = (1 << 64) - 1
    ka, kb = k0 & mask, k1 & mask
    for r in range(10):
        if r > 0:
            ka = (ka + W0) & mask
            kb = (kb + W1) & mask
        hi0, lo0 = _mulhilo(M0, c[0])
        hi1, lo1 = _mulhilo(M1, c[2])
        c = [hi1 ^ c[1] ^ np.uint64(ka), lo1, hi0 ^ c[3] ^ np.uint64(kb), lo0]
    return c


def words32(seed: int, draw_key: int, n: int, level: int = 0) -> np.ndarray:
    """The n 32-bit words of noise level `level` of draw (seed, draw_key),
    index j = 0..n-1 (uint64)."""
    j = np.arange(n, dtype=np.uint64)
    blocks = np.arange((n + 7) // 8, dtype=np.uint64)
    out = philox4x64_10(blocks, np.uint64(draw_key), np.uint64(level), 0, int(seed), 0)
    o = np.stack(out, axis=1)                 # [n_blocks, 4]
    w = j & np.uint64(7)
    word64 = o[(j >> np.uint64(3)).astype(np.int64), (w >> np.uint64(1)).astype(np.int64)]
    half = (w & np.uint64(1)).astype(bool)
    return np.where(half, word64 >> _S32, word64 & _M32)


def gumbel(seed: int, draw_key: int, n: int, level: int = 0) -> np.ndarray:
    """Gumbel(0, 1) noise of draw (seed, draw_key), level `level`, for indices 0..n-1."""
    x = words32(seed, draw_key, n, level).astype(np.float64)
    t = (x + 0.5) * 2.0 ** -32
    e = -np.log1p(-t)
    return -np.log(e)


def _argmax_gap(s: np.ndarray):
    """Index of the maximum (lowest among equals) and the top-2 gap."""
    j = int(np.argmax(s))
    if s.shape[-1] < 2:
        return j, np.inf
    part = np.partition(s, -2)
    return j, float(part[-1] - part[-2])


def gumbel_argmax(log_w: np.ndarray, seed: int, draw_key: int, level: int = 0):
    """Sample index j with probability exp(log_w_j) / sum exp(log_w) (Gumbel max)
    with the noise of level `level`.

    Entries with log_w = -inf never win.  Returns (index, margin) where the
    margin is the gap between the best and second-best perturbed score.
    """
    lw = np.asarray(log_w, dtype=np.float64)
    return _argmax_gap(lw + gumbel(seed, draw_key, lw.shape[-1], level))


def grouped_gumbel_argmax(log_w: np.ndarray, seed: int, draw_key: int, block: int = DRAW_BLOCK):
    """Sample index j with probability w_j / sum(w), w = exp(log_w), in two levels.

    The entries are cut into blocks of `block` consecutive indices (the last
    one may be shorter).  Level 1: block b = argmax_b (log Z_b + g1_b), Z_b
    the block's mass and g1 the level-1 noise of the draw, indexed by block.
    Level 2: j = argmax over the entries of block b of (log_w_j + g0_j), g0 the
    level-0 noise indexed by entry.  Blocks of zero mass, and entries with
    log_w = -inf, never win.  Returns (index, margin): the margin is the
    smaller of the two levels' top-2 score gaps, so a decision whose margin is
    large stays the same under a small change of any weight.
    """
    lw = np.asarray(log_w, dtype=np.float64)
    V = lw.shape[-1]
    top = np.max(lw)
    w = np.exp(lw - top)                       # the common shift leaves both levels unchanged
    starts = np.arange(0, V, block)
    Z = np.add.reduceat(w, starts)
    with np.errstate(divide="ignore"):
        logZ = np.log(Z)
    b, gap1 = _argmax_gap(logZ + gumbel(seed, draw_key, len(starts), level=1))
    lo, hi = b * block, min(V, (b + 1) * block)
    j, gap2 = _argmax_gap(lw[lo:hi] + gumbel(seed, draw_key, V, level=0)[lo:hi])
    return lo + j, min(gap1, gap2)
