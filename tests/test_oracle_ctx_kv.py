"""Pins of the oracle's context-K/V producer (KV injection of target features
into every drafter layer's cache): a drafter that reads the produced cache
equals one that carries the context rows as extra block rows; the projection
selects streams as its weights say; RMSNorm makes the cache rows invariant to
the scale of the projection; and RoPE puts a row's position into its key."""
import numpy as np

from oracle import dmtp

Hq, Hkv, d, H, F, NF = 4, 2, 16, 64, 96, 5
KW = dict(Hq=Hq, Hkv=Hkv, d=d, eps=1e-6, rope_base=1e4)


def _layer(seed):
    r = np.random.default_rng(seed)
    return dmtp.Layer64(g_attn=1 + 0.1 * r.standard_normal(H),
                        wqkv=0.2 * r.standard_normal(((Hq + 2 * Hkv) * d, H)),
                        wo=0.2 * r.standard_normal((H, Hq * d)),
                        g_ffn=1 + 0.1 * r.standard_normal(H),
                        wg=0.2 * r.standard_normal((F, H)), wu=0.2 * r.standard_normal((F, H)),
                        wd=0.2 * r.standard_normal((H, F)))


def test_produced_cache_equals_context_rows_carried_as_block_rows():
    r = np.random.default_rng(0)
    n_ctx, S = 6, 3
    feats = r.standard_normal((n_ctx, NF, H))
    w_fc = 0.1 * r.standard_normal((H, NF * H))
    lw = _layer(1)
    pos_c = np.arange(n_ctx)
    c, kv = dmtp.ctx_kv(feats, pos_c, w_fc, [lw], **KW)
    X = r.standard_normal((1, S, H))
    pos_x = (n_ctx + np.arange(S))[None]
    # path A: block rows over the produced cache
    out_a = dmtp.decoder_layer(X, pos_x, lw, [kv[0][0]], [kv[0][1]], **KW)[0]
    # path B: context rows as extra rows of the same (unmasked) layer, no cache
    XB = np.concatenate([c[None], X], axis=1)
    pos_b = np.concatenate([pos_c, pos_x[0]])[None]
    out_b, kb, vb = dmtp.decoder_layer(XB, pos_b, lw, [np.zeros((0, Hkv, d))], [np.zeros((0, Hkv, d))], **KW)
    np.testing.assert_allclose(out_a, out_b[:, n_ctx:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kv[0][0], kb[0, :n_ctx], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kv[0][1], vb[0, :n_ctx], rtol=1e-12, atol=1e-12)


def test_projection_selects_a_stream():
    r = np.random.default_rng(2)
    feats = r.standard_normal((4, NF, H))
    for s in range(NF):
        sel = np.zeros((H, NF * H))
        sel[:, s * H:(s + 1) * H] = np.eye(H)
        c, _ = dmtp.ctx_kv(feats, np.arange(4), sel, [_layer(3)], **KW)
        np.testing.assert_array_equal(c, feats[:, s])


def test_cache_rows_are_invariant_to_the_projection_scale():
    r = np.random.default_rng(4)
    feats = r.standard_normal((5, NF, H))
    w_fc = 0.1 * r.standard_normal((H, NF * H))
    lw = _layer(5)
    _, a = dmtp.ctx_kv(feats, np.arange(5), w_fc, [lw], **dict(KW, eps=0.0))
    _, b = dmtp.ctx_kv(feats, np.arange(5), 7.5 * w_fc, [lw], **dict(KW, eps=0.0))
    np.testing.assert_allclose(a[0][0], b[0][0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a[0][1], b[0][1], rtol=1e-12, atol=1e-12)


def test_key_rotation_follows_the_position_values_do_not():
    r = np.random.default_rng(6)
    feats = np.repeat(r.standard_normal((1, NF, H)), 3, axis=0)   # one row at three positions
    w_fc = 0.1 * r.standard_normal((H, NF * H))
    _, kv = dmtp.ctx_kv(feats, np.array([0, 5, 900]), w_fc, [_layer(7)], **KW)
    k, v = kv[0]
    np.testing.assert_array_equal(v[0], v[1])
    assert np.abs(k[1] - k[0]).max() > 1e-6 and np.abs(k[2] - k[1]).max() > 1e-6
    nk = np.linalg.norm(k, axis=-1)
    np.testing.assert_allclose(nk, np.broadcast_to(nk[0], nk.shape), rtol=1e-12)   # rotations keep norms
