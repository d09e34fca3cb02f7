"""Pins of the oracle's SwiGLU feed-forward, RoPE frequency schedule and top-2 gap.

The pages define neither the drafter's feed-forward network nor its rotary
embedding ("DFlash vs MTP", "DFlash: Block Diffusion as a Draft Model": the
drafter is a stack of Transformer layers; DMTP blog section 6.5: projections,
normalisation and a feed-forward network), so these parts follow the standard
forms named in the oracle and are pinned by the mathematics:

  * silu against torch's implementation and its closed form x / (1 + e^-x);
  * the gated product silu(x Wg^T) * (x Wu^T) on selector weights, where
    swapping the gate and up projections, or gating with the sigmoid instead of
    silu, gives a different closed-form value;
  * a whole pre-norm decoder layer against one assembled here from torch's
    own RMSNorm, scaled-dot-product attention and silu, with RoPE taken as a
    complex rotation of the (i, i + d/2) pairs;
  * the rotation of every basis vector e_i and e_{i+d/2} against
    cos / sin(p base^(-2i/d)), for every pair i up to d/2 - 1;
  * top2_gap against a brute-force sort, ties and one- and two-entry rows included.

Each pin is also shown to fail on a planted slip of the oracle (on the CPU).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dmtp, numerics as nm


def _rng(i):
    return np.random.default_rng(7000 + i)


# ------------------------------------------------------------------ silu


def test_silu_matches_torch_and_closed_form():
    x = np.concatenate([np.linspace(-30, 30, 2001), [0.0, -1e-300, 1e-300, 700.0, -700.0]])
    want = F.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(nm.silu(x), want, rtol=1e-14, atol=1e-300)
    for v in (-3.0, -0.5, 0.25, 1.0, 4.0):
        assert math.isclose(float(nm.silu(np.array(v))), v / (1.0 + math.exp(-v)), rel_tol=1e-15)


# ------------------------------------------------ gated feed-forward order

H_SEL = 8


def _ffn_only_layer(alpha, beta, i_out, j_in, H=H_SEL, F_=3):
    """A layer whose attention branch is zero (wo = 0) and whose feed-forward
    network reads input feature j_in through one gate row (weight alpha) and
    one up row (weight beta) and writes output feature i_out."""
    wg = np.zeros((F_, H))
    wu = np.zeros((F_, H))
    wd = np.zeros((H, F_))
    wg[1, j_in] = alpha
    wu[1, j_in] = beta
    wd[i_out, 1] = 1.0
    d = 4
    return dmtp.Layer64(g_attn=np.ones(H), wqkv=np.zeros((3 * d, H)), wo=np.zeros((H, d)),
                        g_ffn=np.ones(H), wg=wg, wu=wu, wd=wd)


def _run_ffn_layer(lw, X):
    out, _, _ = dmtp.decoder_layer(X[None], np.arange(X.shape[0])[None], lw,
                                   [np.zeros((0, 1, 4))], [np.zeros((0, 1, 4))],
                                   Hq=1, Hkv=1, d=4, eps=0.0, rope_base=1e6)
    return out[0]


def _swiglu_closed_form_value(alpha, beta, c):
    # a constant row c normalises to sign(c) (eps = 0, unit gains): the
    # selected feature is s = sign(c); gate silu(alpha s) times up (beta s)
    s = math.copysign(1.0, c)
    return c + (alpha * s / (1.0 + math.exp(-alpha * s))) * (beta * s)


@pytest.mark.parametrize("alpha,beta,c", [(2.0, 0.5, 3.0), (-1.5, 0.75, -2.0), (0.3, 4.0, 1.0)])
def test_swiglu_gate_and_up_order_closed_form(alpha, beta, c):
    X = np.full((1, H_SEL), c)
    lw = _ffn_only_layer(alpha, beta, i_out=5, j_in=2)
    out = _run_ffn_layer(lw, X)
    want = np.full(H_SEL, c)
    want[5] = _swiglu_closed_form_value(alpha, beta, c)
    np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=1e-15)
    # the slips this pins give other values: gate and up swapped, sigmoid gate
    s = math.copysign(1.0, c)
    swapped = c + (beta * s / (1.0 + math.exp(-beta * s))) * (alpha * s)
    sigmoid_gate = c + (1.0 / (1.0 + math.exp(-alpha * s))) * (beta * s)
    assert abs(out[0, 5] - swapped) > 1e-3 and abs(out[0, 5] - sigmoid_gate) > 1e-3


def test_swiglu_pin_detects_planted_slips(monkeypatch):
    X = np.full((1, H_SEL), 3.0)
    want = _swiglu_closed_form_value(2.0, 0.5, 3.0)
    # silu replaced by the sigmoid
    monkeypatch.setattr(nm, "silu", lambda x: 1.0 / (1.0 + np.exp(-x)))
    got = _run_ffn_layer(_ffn_only_layer(2.0, 0.5, 5, 2), X)[0, 5]
    assert abs(got - want) > 1e-3
    monkeypatch.undo()
    # gate and up projections exchanged
    lw = _ffn_only_layer(2.0, 0.5, 5, 2)
    lw_swapped = dmtp.Layer64(lw.g_attn, lw.wqkv, lw.wo, lw.g_ffn, lw.wu, lw.wg, lw.wd)
    got = _run_ffn_layer(lw_swapped, X)[0, 5]
    assert abs(got - want) > 1e-3


def test_ffn_matches_torch_expression_with_random_weights():
    # attention branch zero: X2 = X + (silu(x^ Wg^T) * (x^ Wu^T)) Wd^T, x^ = RMSNorm(X; g_ffn)
    r = _rng(1)
    H, F_, d = 32, 48, 8
    X = r.standard_normal((5, H))
    lw = dmtp.Layer64(g_attn=1 + 0.1 * r.standard_normal(H), wqkv=0.1 * r.standard_normal((3 * d, H)),
                      wo=np.zeros((H, d)), g_ffn=1 + 0.1 * r.standard_normal(H),
                      wg=0.2 * r.standard_normal((F_, H)), wu=0.2 * r.standard_normal((F_, H)),
                      wd=0.2 * r.standard_normal((H, F_)))
    out, _, _ = dmtp.decoder_layer(X[None], np.arange(5)[None], lw, [np.zeros((0, 1, d))],
                                   [np.zeros((0, 1, d))], Hq=1, Hkv=1, d=d, eps=1e-6, rope_base=1e4)
    t = torch.from_numpy
    x = F.rms_norm(t(X), (H,), t(lw.g_ffn), eps=1e-6)
    want = t(X) + (F.silu(x @ t(lw.wg).T) * (x @ t(lw.wu).T)) @ t(lw.wd).T
    np.testing.assert_allclose(out[0], want.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------- whole layer against torch parts


def _torch_layer(X, pos, lw, ck, cv, Hq, Hkv, d, eps, base, causal=False):
    """A pre-norm decoder layer assembled from torch primitives (float64),
    with RoPE written as a complex rotation of the pairs (i, i + d/2)."""
    t = torch.from_numpy
    S, H = X.shape
    Xt = t(X)
    xh = F.rms_norm(Xt, (H,), t(lw.g_attn), eps=eps)
    qkv = xh @ t(np.asarray(lw.wqkv, dtype=np.float64)).T
    q = qkv[:, : Hq * d].reshape(S, Hq, d)
    k = qkv[:, Hq * d: (Hq + Hkv) * d].reshape(S, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(S, Hkv, d)
    half = d // 2
    freq = torch.tensor([base ** (-2.0 * i / d) for i in range(half)], dtype=torch.float64)
    ang = torch.from_numpy(np.asarray(pos, dtype=np.float64))[:, None] * freq[None]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]       # [S, 1, d/2]

    def rope(x):
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    keys = torch.cat([t(ck), k], 0)             # [n_ctx + S, Hkv, d]
    vals = torch.cat([t(cv), v], 0)
    n_ctx = ck.shape[0]
    G = Hq // Hkv
    kk = keys.repeat_interleave(G, dim=1).permute(1, 0, 2)   # [Hq, n_k, d]
    vv = vals.repeat_interleave(G, dim=1).permute(1, 0, 2)
    mask = torch.ones(S, n_ctx + S, dtype=torch.bool)
    if causal:
        mask[:, n_ctx:] = torch.tril(torch.ones(S, S, dtype=torch.bool))
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2), kk, vv, attn_mask=mask)
    X1 = Xt + o.permute(1, 0, 2).reshape(S, Hq * d) @ t(lw.wo).T
    x2 = F.rms_norm(X1, (H,), t(lw.g_ffn), eps=eps)
    return (X1 + (F.silu(x2 @ t(lw.wg).T) * (x2 @ t(lw.wu).T)) @ t(lw.wd).T).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_decoder_layer_matches_torch_assembled_layer(causal):
    r = _rng(2)
    H, Hq, Hkv, d, F_, S, n_ctx = 64, 4, 2, 16, 96, 5, 11
    X = r.standard_normal((S, H))
    lw = dmtp.Layer64(g_attn=1 + 0.1 * r.standard_normal(H),
                      wqkv=0.15 * r.standard_normal(((Hq + 2 * Hkv) * d, H)),
                      wo=0.1 * r.standard_normal((H, Hq * d)), g_ffn=1 + 0.1 * r.standard_normal(H),
                      wg=0.1 * r.standard_normal((F_, H)), wu=0.1 * r.standard_normal((F_, H)),
                      wd=0.1 * r.standard_normal((H, F_)))
    ck, cv = r.standard_normal((n_ctx, Hkv, d)), r.standard_normal((n_ctx, Hkv, d))
    pos = n_ctx + np.arange(S)
    got, _, _ = dmtp.decoder_layer(X[None], pos[None], lw, [ck], [cv], Hq=Hq, Hkv=Hkv, d=d,
                                   eps=1e-6, rope_base=500.0, causal=causal)
    want = _torch_layer(X, pos, lw, ck, cv, Hq, Hkv, d, 1e-6, 500.0, causal=causal)
    np.testing.assert_allclose(got[0], want, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- RoPE


@pytest.mark.parametrize("d,base", [(8, 1e6), (64, 1e4), (128, 1e6)])
def test_rope_rotates_every_pair_by_its_frequency(d, base):
    half = d // 2
    for p in (1, 7, 4095, 32790):
        for i in sorted({0, 1, 2, half // 2, half - 2, half - 1}):
            theta = p * base ** (-2.0 * i / d)
            ei = np.zeros(d)
            ei[i] = 1.0
            r = nm.rope(ei[None], np.array([p]), base)[0]
            want = np.zeros(d)
            want[i], want[i + half] = math.cos(theta), math.sin(theta)
            # theta is rounded once on each side: allow a few ulp of p
            np.testing.assert_allclose(r, want, rtol=0, atol=4e-16 * max(1, p))
            ej = np.zeros(d)
            ej[i + half] = 1.0
            r = nm.rope(ej[None], np.array([p]), base)[0]
            want = np.zeros(d)
            want[i], want[i + half] = -math.sin(theta), math.cos(theta)
            np.testing.assert_allclose(r, want, rtol=0, atol=4e-16 * max(1, p))


def test_rope_pin_detects_planted_frequency_slip(monkeypatch):
    d, base, p, i = 64, 1e4, 100, 5
    theta = p * base ** (-2.0 * i / d)

    def wrong_angles(positions, d_, base_):
        ii = np.arange(d_ // 2, dtype=np.float64)
        return np.asarray(positions, dtype=np.float64)[:, None] * (base_ ** (-ii / d_))[None, :]

    monkeypatch.setattr(nm, "rope_angles", wrong_angles)
    ei = np.zeros(d)
    ei[i] = 1.0
    r = nm.rope(ei[None], np.array([p]), base)[0]
    assert abs(r[i] - math.cos(theta)) > 1e-3 or abs(r[i + d // 2] - math.sin(theta)) > 1e-3


# ------------------------------------------------------------- top-2 gap


def _gap_by_sort(row):
    if len(row) < 2:
        return math.inf
    s = sorted(row, reverse=True)
    return s[0] - s[1]


def test_top2_gap_matches_brute_force_sort():
    r = _rng(3)
    rows = [r.standard_normal(n) for n in (2, 3, 17, 1000)]
    rows += [np.array([1.0, 1.0, 0.5]), np.array([0.5, 2.0, 2.0, -1.0]),   # tied maxima: gap 0
             np.array([3.0, -np.inf]), np.array([-np.inf, 2.0, -5.0]), np.array([5.0, 5.0])]
    for row in rows:
        assert nm.top2_gap(row) == _gap_by_sort(list(row))
    assert nm.top2_gap(np.array([4.0])) == math.inf
    batch = r.standard_normal((6, 40))
    batch[2, 7] = batch[2, 30] = batch[2].max() + 1.0
    np.testing.assert_array_equal(nm.top2_gap(batch), [_gap_by_sort(list(b)) for b in batch])


def test_top2_gap_pin_detects_planted_slip(monkeypatch):
    monkeypatch.setattr(nm, "top2_gap", lambda x: np.max(x, -1) - np.min(x, -1))
    row = np.array([0.1, 3.0, 2.5, -4.0])
    assert nm.top2_gap(row) != _gap_by_sort(list(row))


def test_argmax_first_takes_lowest_index_of_equal_maxima():
    assert int(nm.argmax_first(np.array([1.0, 3.0, 2.0, 3.0]))) == 1
    assert int(nm.argmax_first(np.array([-np.inf, -np.inf]))) == 0
    rows = np.array([[0.0, 5.0, 5.0], [7.0, 7.0, 7.0], [1.0, 2.0, 3.0]])
    np.testing.assert_array_equal(nm.argmax_first(rows), [1, 0, 2])
