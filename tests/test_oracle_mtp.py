"""Pins of the oracle's MTP decoder block: causal visibility, the KV-cache
identity (rows processed one at a time, each appending its K/V to the cache,
equal the causal call over all of them), the single-row case, the identity
with zero output projections, and its place in the round."""
import numpy as np
import pytest

import dmtp_synth as synth
from oracle import dmtp

Hq, Hkv, d, H, F = 4, 2, 16, 64, 96


def _layer(seed, zero_out=False):
    r = np.random.default_rng(seed)
    wo = np.zeros((H, Hq * d)) if zero_out else 0.2 * r.standard_normal((H, Hq * d))
    wd = np.zeros((H, F)) if zero_out else 0.2 * r.standard_normal((H, F))
    return dmtp.Layer64(g_attn=1 + 0.1 * r.standard_normal(H),
                        wqkv=0.2 * r.standard_normal(((Hq + 2 * Hkv) * d, H)), wo=wo,
                        g_ffn=1 + 0.1 * r.standard_normal(H),
                        wg=0.2 * r.standard_normal((F, H)), wu=0.2 * r.standard_normal((F, H)), wd=wd)


def _cache(seed, lens):
    r = np.random.default_rng(seed)
    return ([r.standard_normal((L, Hkv, d)) for L in lens],
            [r.standard_normal((L, Hkv, d)) for L in lens])


KW = dict(Hq=Hq, Hkv=Hkv, d=d, eps=1e-6, rope_base=1e4)


def test_one_row_causal_equals_unmasked():
    r = np.random.default_rng(0)
    X = r.standard_normal((3, 1, H))
    lens = [5, 0, 9]
    pos = np.array(lens)[:, None]
    ck, cv = _cache(1, lens)
    lw = _layer(2)
    a = dmtp.decoder_layer(X, pos, lw, ck, cv, causal=True, **KW)
    b = dmtp.decoder_layer(X, pos, lw, ck, cv, causal=False, **KW)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_causal_rows_do_not_see_later_rows():
    r = np.random.default_rng(3)
    S = 4
    X = r.standard_normal((2, S, H))
    lens = [6, 3]
    pos = np.array(lens)[:, None] + np.arange(S)
    ck, cv = _cache(4, lens)
    lw = _layer(5)
    base = dmtp.decoder_layer(X, pos, lw, ck, cv, causal=True, **KW)[0]
    for j in range(S):
        X2 = X.copy()
        X2[:, j] += 0.5 * r.standard_normal((2, H))
        out = dmtp.decoder_layer(X2, pos, lw, ck, cv, causal=True, **KW)[0]
        np.testing.assert_array_equal(out[:, :j], base[:, :j])            # earlier rows
        assert np.all(np.abs(out[:, j:] - base[:, j:]).max(axis=-1) > 1e-6)  # this and later
    # without the mask an earlier row does see a later one
    X2 = X.copy()
    X2[:, S - 1] += 1.0
    full = dmtp.decoder_layer(X, pos, lw, ck, cv, causal=False, **KW)[0]
    full2 = dmtp.decoder_layer(X2, pos, lw, ck, cv, causal=False, **KW)[0]
    assert np.abs(full2[:, 0] - full[:, 0]).max() > 1e-6


def test_rows_one_at_a_time_with_cache_appends_equal_the_causal_call():
    """The KV-cache identity: a cache that appends each row's (k, v) and then
    serves the next row gives exactly what the S-row causal call gives."""
    r = np.random.default_rng(6)
    S, lens = 3, [4, 0]
    X = r.standard_normal((2, S, H))
    pos = np.array(lens)[:, None] + np.arange(S)
    layers = [_layer(7), _layer(8)]
    ck = [_cache(9, lens)[0], _cache(10, lens)[0]]
    cv = [_cache(9, lens)[1], _cache(10, lens)[1]]
    out, kv = dmtp.mtp_block(X, pos, layers, ck, cv, **KW)
    ck2 = [[c.copy() for c in l] for l in ck]
    cv2 = [[c.copy() for c in l] for l in cv]
    for j in range(S):
        o1, kv1 = dmtp.mtp_block(X[:, j: j + 1], pos[:, j: j + 1], layers, ck2, cv2, **KW)
        np.testing.assert_allclose(o1[:, 0], out[:, j], rtol=1e-12, atol=1e-12)
        for l in range(2):
            np.testing.assert_allclose(kv1[l][0][:, 0], kv[l][0][:, j], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(kv1[l][1][:, 0], kv[l][1][:, j], rtol=1e-12, atol=1e-12)
            for i in range(2):
                ck2[l][i] = np.concatenate([ck2[l][i], kv1[l][0][i]], axis=0)
                cv2[l][i] = np.concatenate([cv2[l][i], kv1[l][1][i]], axis=0)


def test_zero_output_projections_give_the_identity():
    r = np.random.default_rng(11)
    X = r.standard_normal((2, 2, H))
    lens = [3, 5]
    pos = np.array(lens)[:, None] + np.arange(2)
    ck, cv = _cache(12, lens)
    out, kv = dmtp.mtp_block(X, pos, [_layer(13, zero_out=True)], [ck], [cv], **KW)
    np.testing.assert_array_equal(out, X)
    assert kv[0][0].shape == (2, 2, Hkv, d)


def test_round_with_an_identity_mtp_block_is_the_plain_round():
    cfg = synth.CONFIGS["tiny_greedy_f32"].with_(B=2, ctx_min=10, ctx_max=40, seed=21)
    plain = dmtp.run_round(synth.make_inputs(cfg))
    inp = synth.make_inputs(cfg.with_(mtp_block=True))
    for lw in inp.mtp_layers:
        lw.wo[...] = 0.0
        lw.wd[...] = 0.0
    res = dmtp.run_round(inp)
    np.testing.assert_array_equal(res.h_mtp, res.h_fused)
    for name in ("h_mtp", "t1", "x_t1", "drafts", "accept_len", "out_tokens"):
        np.testing.assert_array_equal(getattr(res, name), getattr(plain, name))
    # a real block changes the MTP hidden, and with it the T1 row
    res2 = dmtp.run_round(synth.make_inputs(cfg.with_(mtp_block=True)))
    assert np.abs(res2.h_mtp - res2.h_fused).max() > 1e-3
    assert res2.mtp_kv[0][0].shape == (2, 1, cfg.Hkv, cfg.d)
