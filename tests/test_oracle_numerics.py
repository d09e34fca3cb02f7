"""Pins of the oracle's elementary definitions against libraries and closed forms.

Each test checks the oracle against something other than its own code: a
library routine (PyTorch, SciPy, NumPy's Philox), a closed form, or an
invariant that a plausible slip (dropped gain, wrong sign, swapped halves,
off-by-one exponent) would break.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import numerics as nm
from oracle import philox


def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38]),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = nm.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_bf16_ties_go_to_even():
    # spacing of bf16 in [1, 2) is 2^-7
    assert nm.round_bf16(1.0 + 2.0 ** -8) == 1.0                    # tie, even below
    assert nm.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie, even above
    assert nm.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    # subnormal range: spacing 2^-133
    assert nm.round_bf16(1.5 * 2.0 ** -133) == 2.0 ** -132
    assert nm.round_bf16(2.5 * 2.0 ** -133) == 2.0 ** -132
    # a float64 value that float32 would round first (double rounding trap):
    # 1 + 2^-8 + 2^-30 is above the tie, so the correct bf16 is 1 + 2^-7,
    # while rounding to float32 first gives 1 + 2^-8 exactly and then 1.
    assert nm.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


def test_rmsnorm_matches_torch_and_closed_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    g = 1.0 + 0.1 * rng.standard_normal(64)
    want = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(nm.rmsnorm(x, g, 1e-6), want, rtol=1e-13, atol=0)
    c = np.full((1, 64), -3.0)
    np.testing.assert_allclose(nm.rmsnorm(c, g, 1e-6), -g[None] * 3.0 / math.sqrt(9.0 + 1e-6),
                               rtol=1e-14)


def test_softmax_and_logsumexp_match_scipy():
    rng = np.random.default_rng(3)
    x = 5.0 * rng.standard_normal((4, 1000))
    np.testing.assert_allclose(nm.logsumexp(x), scipy.special.logsumexp(x, axis=-1), rtol=1e-14)
    np.testing.assert_allclose(nm.softmax(x), scipy.special.softmax(x, axis=-1), rtol=1e-12)


def test_rope_preserves_norm_and_depends_on_relative_position():
    rng = np.random.default_rng(4)
    d = 64
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    base = 1e6

    def rot(v, p):
        return nm.rope(v[None, :], np.array([p]), base)[0]

    for p in (0, 3, 1000, 32790):
        assert np.isclose(np.linalg.norm(rot(q, p)), np.linalg.norm(q), rtol=1e-13)
    s1 = rot(q, 137) @ rot(k, 100)
    s2 = rot(q, 5037) @ rot(k, 5000)
    s3 = rot(q, 37) @ rot(k, 0)
    assert np.isclose(s1, s2, rtol=1e-9) and np.isclose(s1, s3, rtol=1e-9)
    assert not np.isclose(s1, rot(q, 36) @ rot(k, 0), rtol=1e-6)
    # position 0 is the identity
    np.testing.assert_array_equal(rot(q, 0), q)
    # dimension 0 pairs with d/2 and turns by exactly the position (inverse frequency 1)
    e0 = np.zeros(d)
    e0[0] = 1.0
    r = rot(e0, 2)
    assert np.isclose(r[0], math.cos(2.0)) and np.isclose(r[d // 2], math.sin(2.0))


def test_attention_matches_torch_sdpa_and_special_cases():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((8, 32))
    k = rng.standard_normal((50, 32))
    v = rng.standard_normal((50, 32))
    want = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
                                          torch.from_numpy(v)[None, None]).numpy()[0, 0]
    np.testing.assert_allclose(nm.attention(q, k, v), want, rtol=1e-12, atol=1e-13)
    # a single key returns its value whatever the query
    np.testing.assert_allclose(nm.attention(q, k[:1], v[:1]), np.repeat(v[:1], 8, 0), rtol=1e-14)
    # a zero query averages the values
    np.testing.assert_allclose(nm.attention(np.zeros((1, 32)), k, v)[0], v.mean(0), rtol=1e-12)


def test_philox4x64_matches_numpy():
    key = (0x0123456789ABCDEF, 0x0F1E2D3C4B5A6978)
    ctr = (0xFFFFFFFFFFFFFFF0, 7, 11, 0xDEADBEEF)
    gen = np.random.Philox(key=np.array(key, dtype=np.uint64),
                           counter=np.array(ctr, dtype=np.uint64))
    raw = gen.random_raw(4 * 6)      # numpy bumps the counter before each block
    for blk in range(6):
        c0 = (ctr[0] + blk + 1) & ((1 << 64) - 1)
        c1 = ctr[1] + (1 if ctr[0] + blk + 1 >= (1 << 64) else 0)
        out = philox.philox4x64_10(np.uint64(c0), np.uint64(c1), np.uint64(ctr[2]),
                                   np.uint64(ctr[3]), key[0], key[1])
        np.testing.assert_array_equal(np.array([int(o) for o in out], dtype=np.uint64),
                                      raw[4 * blk: 4 * blk + 4])


def test_words32_layout():
    seed, dk = 99, (1 << 32) | 5
    for level in (0, 1):
        w = philox.words32(seed, dk, 20, level)
        for j in (0, 1, 7, 8, 13, 19):
            o = philox.philox4x64_10(np.uint64(j >> 3), np.uint64(dk), np.uint64(level), 0, seed, 0)
            v = int(o[(j & 7) >> 1])
            assert int(w[j]) == ((v >> 32) if (j & 1) else (v & 0xFFFFFFFF))
    # the two levels are different streams
    assert not np.array_equal(philox.words32(seed, dk, 64, 0), philox.words32(seed, dk, 64, 1))


def test_gumbel_moments_and_gumbel_max_frequencies():
    g = philox.gumbel(7, 3, 400000)
    assert abs(g.mean() - np.euler_gamma) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    w = np.arange(1, 17, dtype=np.float64)
    counts = np.zeros(16)
    n = 16000
    for key in range(n):
        j, _ = philox.gumbel_argmax(np.log(w), 11, key)
        counts[j] += 1
    expect = n * w / w.sum()
    chi2 = ((counts - expect) ** 2 / expect).sum()
    # 15 degrees of freedom: P(chi2 > 37.7) = 1e-3
    assert chi2 < 37.7, chi2
    # -inf weights never win
    lw = np.log(np.array([0.0, 1.0, 0.0, 2.0]))
    for key in range(200):
        assert philox.gumbel_argmax(lw, 5, key)[0] in (1, 3)


# ------------------------------------------------- two-level Gumbel-max draw


def _chi2(counts, expect):
    return float(((counts - expect) ** 2 / expect).sum())


@pytest.mark.parametrize("block", [4, 5, 16])
def test_grouped_draw_frequencies_match_the_weights(block):
    # 16 entries in blocks of 4 (even), 5 (ragged last block) and 16 (one block)
    w = np.arange(1, 17, dtype=np.float64)
    w[3] = 0.0                                  # a zero weight never wins
    counts = np.zeros(16)
    n = 16000
    for key in range(n):
        j, _ = philox.grouped_gumbel_argmax(np.log(np.where(w > 0, w, 1.0)) + np.where(w > 0, 0, -np.inf),
                                            11, key, block=block)
        counts[j] += 1
    assert counts[3] == 0
    keep = w > 0
    expect = n * w[keep] / w.sum()
    # 14 degrees of freedom: P(chi2 > 36.1) = 1e-3
    assert _chi2(counts[keep], expect) < 36.1


def test_grouped_draw_with_one_block_is_the_level0_gumbel_max():
    r = np.random.default_rng(21)
    for key in range(50):
        lw = r.standard_normal(37) * 2
        assert philox.grouped_gumbel_argmax(lw, 7, key, block=64) == philox.gumbel_argmax(lw, 7, key, 0)


def test_grouped_draw_with_unit_blocks_is_the_level1_gumbel_max():
    r = np.random.default_rng(22)
    for key in range(50):
        lw = r.standard_normal(29)
        j, m = philox.grouped_gumbel_argmax(lw, 5, key, block=1)
        j1, m1 = philox.gumbel_argmax(lw, 5, key, 1)
        assert j == j1 and math.isclose(m, m1, rel_tol=1e-9, abs_tol=1e-12)


def test_grouped_draw_block_choice_follows_block_masses():
    # two blocks of two entries; block masses 1 : 3 -> P(block 1) = 3/4, and
    # within block 1 entries in ratio 1 : 2
    lw = np.log(np.array([0.5, 0.5, 1.0, 2.0]))
    n = 12000
    counts = np.zeros(4)
    for key in range(n):
        counts[philox.grouped_gumbel_argmax(lw, 3, key, block=2)[0]] += 1
    expect = n * np.array([0.125, 0.125, 0.25, 0.5])
    assert _chi2(counts, expect) < 16.3    # 3 degrees of freedom, P = 1e-3


def test_grouped_draw_ignores_empty_blocks_and_reports_the_smaller_gap():
    lw = np.full(12, -np.inf)
    lw[9] = 0.0
    for key in range(100):
        assert philox.grouped_gumbel_argmax(lw, 1, key, block=4)[0] == 9
    # margin: the smaller of the block-level and entry-level gaps
    r = np.random.default_rng(23)
    lw = r.standard_normal(10)
    seed, key, blk = 4, 77, 4
    j, m = philox.grouped_gumbel_argmax(lw, seed, key, block=blk)
    Z = np.add.reduceat(np.exp(lw), np.arange(0, 10, blk))
    s1 = np.log(Z) + philox.gumbel(seed, key, len(Z), level=1)
    b = int(np.argmax(s1))
    s2 = lw[b * blk:(b + 1) * blk] + philox.gumbel(seed, key, 10, level=0)[b * blk:(b + 1) * blk]
    gaps = [np.sort(s1)[-1] - np.sort(s1)[-2], np.sort(s2)[-1] - np.sort(s2)[-2]]
    assert j == b * blk + int(np.argmax(s2)) and math.isclose(m, min(gaps), rel_tol=1e-12)
