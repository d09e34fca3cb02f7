"""Pins of the oracle's fusion, drafter and round against closed forms and invariants."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dmtp_synth as synth
from oracle import dmtp, numerics as nm

TINY = synth.CONFIGS["tiny_greedy_f32"]


def _rng(i):
    return np.random.default_rng(1000 + i)


# ----------------------------------------------------------------- fusion


def test_fuse_zero_projection_returns_residual_bitwise():
    r = _rng(0)
    x1, x2 = r.standard_normal((3, 32)), r.standard_normal((3, 32))
    res = r.standard_normal((3, 32))
    out = dmtp.fuse(x1, x2, np.ones(32), np.ones(32), np.zeros((32, 64)), 1e-6, res=res)
    np.testing.assert_array_equal(out, res)


def test_fuse_selector_projections_give_each_normalised_stream():
    r = _rng(1)
    h, e = r.standard_normal((4, 16)), 0.02 * r.standard_normal((4, 16))
    gh, ge = 1 + 0.1 * r.standard_normal(16), 1 + 0.1 * r.standard_normal(16)
    I, Z = np.eye(16), np.zeros((16, 16))
    out_h = dmtp.fuse(h, e, gh, ge, np.concatenate([I, Z], 1), 1e-6)
    out_e = dmtp.fuse(h, e, gh, ge, np.concatenate([Z, I], 1), 1e-6)
    want_h = F.rms_norm(torch.from_numpy(h), (16,), torch.from_numpy(gh), 1e-6).numpy()
    want_e = F.rms_norm(torch.from_numpy(e), (16,), torch.from_numpy(ge), 1e-6).numpy()
    np.testing.assert_allclose(out_h, want_h, rtol=1e-13)
    np.testing.assert_allclose(out_e, want_e, rtol=1e-13)


def test_fuse_is_linear_in_the_projection():
    r = _rng(2)
    x1, x2, res = (r.standard_normal((2, 8)) for _ in range(3))
    W1, W2 = r.standard_normal((8, 16)), r.standard_normal((8, 16))
    g = np.ones(8)
    a = dmtp.fuse(x1, x2, g, g, W1 + 2 * W2, 1e-6, res=res) - res
    b = (dmtp.fuse(x1, x2, g, g, W1, 1e-6) + 2 * dmtp.fuse(x1, x2, g, g, W2, 1e-6))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- drafter

def _layer(r, H, Hq, Hkv, d, F_, scale=0.05, zero=()):
    def w(shape, name):
        return np.zeros(shape) if name in zero else scale * r.standard_normal(shape)
    return dmtp.Layer64(g_attn=1 + 0.1 * r.standard_normal(H),
                        wqkv=w(((Hq + 2 * Hkv) * d, H), "wqkv"), wo=w((H, Hq * d), "wo"),
                        g_ffn=1 + 0.1 * r.standard_normal(H), wg=w((F_, H), "wg"),
                        wu=w((F_, H), "wu"), wd=w((H, F_), "wd"))


KW = dict(Hq=4, Hkv=2, d=8, eps=1e-6, rope_base=1e6)


def _layer1(X, pos, lw, ck, cv, **kw):
    """draft_layer on one sequence."""
    return dmtp.draft_layer(X[None], np.asarray(pos)[None], lw, [ck], [cv], **kw)[0]


def test_draft_layer_with_zero_output_projections_is_identity():
    r = _rng(3)
    X = r.standard_normal((5, 32))
    lw = _layer(r, 32, 4, 2, 8, 48, zero=("wo", "wd"))
    ck, cv = r.standard_normal((9, 2, 8)), r.standard_normal((9, 2, 8))
    np.testing.assert_array_equal(_layer1(X, 9 + np.arange(5), lw, ck, cv, **KW), X)


def test_draft_layer_single_slot_no_context_closed_form():
    # one slot and no context: attention returns the slot's own value vector
    r = _rng(4)
    X = r.standard_normal((1, 32))
    lw = _layer(r, 32, 4, 2, 8, 48, zero=("wg", "wu"))
    out = _layer1(X, np.array([0]), lw, np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), **KW)
    xh = nm.rmsnorm(X, lw.g_attn, 1e-6)
    v = (xh @ lw.wqkv.T)[:, (4 + 2) * 8:].reshape(1, 2, 8)
    o = np.repeat(v, 2, axis=1).reshape(1, 32)       # q heads 0,1 -> kv 0; 2,3 -> kv 1
    np.testing.assert_allclose(out, X + o @ lw.wo.T, rtol=1e-12, atol=1e-14)


def test_draft_attention_is_bidirectional_inside_the_block():
    r = _rng(5)
    X = r.standard_normal((6, 32))
    lw = _layer(r, 32, 4, 2, 8, 48)
    ck, cv = r.standard_normal((7, 2, 8)), r.standard_normal((7, 2, 8))
    pos = 7 + np.arange(6)
    a = _layer1(X, pos, lw, ck, cv, **KW)
    X2 = X.copy()
    X2[5] += 1.0                       # perturb the last slot only
    b = _layer1(X2, pos, lw, ck, cv, **KW)
    assert np.all(np.abs(a[0] - b[0]) > 0)   # the first slot sees the last one


def test_draft_gqa_equals_mha_with_repeated_kv_heads():
    r = _rng(6)
    H, d = 32, 8
    X = r.standard_normal((4, H))
    g = _layer(r, H, 4, 2, d, 40)
    ck, cv = r.standard_normal((5, 2, d)), r.standard_normal((5, 2, d))
    # build the equivalent 4-kv-head layer: kv head j of the GQA layer serves q heads 2j, 2j+1
    q_rows = g.wqkv[: 4 * d]
    k_rows = g.wqkv[4 * d: 6 * d].reshape(2, d, H)
    v_rows = g.wqkv[6 * d:].reshape(2, d, H)
    rep = lambda a: np.repeat(a, 2, axis=0).reshape(4 * d, H)  # noqa: E731
    m = dmtp.Layer64(g.g_attn, np.concatenate([q_rows, rep(k_rows), rep(v_rows)]), g.wo, g.g_ffn,
                     g.wg, g.wu, g.wd)
    pos = 5 + np.arange(4)
    a = _layer1(X, pos, g, ck, cv, **KW)
    b = _layer1(X, pos, m, np.repeat(ck, 2, 1), np.repeat(cv, 2, 1),
                         **{**KW, "Hkv": 4})
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_draft_window_keeps_the_last_positions():
    r = _rng(7)
    X = r.standard_normal((3, 32))
    lw = _layer(r, 32, 4, 2, 8, 48)
    ck, cv = r.standard_normal((20, 2, 8)), r.standard_normal((20, 2, 8))
    pos = 20 + np.arange(3)
    a = _layer1(X, pos, lw, ck, cv, window=6, **KW)
    b = _layer1(X, pos, lw, ck[-6:], cv[-6:], **KW)
    c = _layer1(X, pos, lw, ck, cv, window=20, **KW)
    d = _layer1(X, pos, lw, ck, cv, **KW)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(c, d)
    assert not np.allclose(a, d)


# ----------------------------------------------------------------- round


@pytest.fixture(scope="module")
def tiny_inputs():
    return synth.make_inputs(TINY.with_(gain_std=0.1))


def test_round_zero_residual_reproduces_the_unfused_draft(tiny_inputs):
    inp = synth.make_inputs(TINY.with_(gain_std=0.1, w_zero=True))
    res = dmtp.run_round(inp)
    t1 = res.t1
    np.testing.assert_array_equal(res.x_t1, inp.emb[t1].astype(np.float64))
    # the unfused block [E(A), E(T1), MASK...] through the same drafter
    slots = [np.stack([inp.emb[inp.anchor[0]], inp.emb[t1[0]]] +
                      [inp.emb[TINY.mask_id]] * (TINY.K - 1)).astype(np.float64)]
    hd = dmtp.block_draft(slots, inp.ctx_len, [dmtp.layer64(l) for l in inp.layers],
                          [l.ctx_k for l in inp.layers], [l.ctx_v for l in inp.layers],
                          inp.cu_ctx, [0], inp.g_final, nm.round_f32, Hq=TINY.Hq, Hkv=TINY.Hkv,
                          d=TINY.d, eps=TINY.eps, rope_base=TINY.rope_base)
    np.testing.assert_array_equal(res.hd[0], hd[0])


def test_round_outputs_are_consistent(tiny_inputs):
    res = dmtp.run_round(tiny_inputs)
    K = TINY.K
    for r in range(len(res.seqs)):
        L = int(res.accept_len[r])
        d, y = res.drafts[r], res.target_argmax[r]
        assert all(d[i] == y[i] for i in range(L)) and (L == K or d[L] != y[L])
        assert res.n_out[r] == L + 1
        np.testing.assert_array_equal(res.out_tokens[r, :L], d[:L])
        assert res.out_tokens[r, L] == y[L] and np.all(res.out_tokens[r, L + 1:] == -1)
    # T1 is the argmax of the MTP row
    assert res.t1[0] == np.argmax(nm.round_f32(nm.rmsnorm(res.h_mtp[0], tiny_inputs.g_f, TINY.eps))
                                  @ tiny_inputs.w_head.astype(np.float64).T)


def test_round_rows_are_independent():
    cfg = TINY.with_(B=4, ctx_min=5, ctx_max=40, gain_std=0.1, tau_mode="mixed")
    inp = synth.make_inputs(cfg)
    full = dmtp.run_round(inp)
    part = dmtp.run_round(inp, seqs=[2, 0])
    for r, b in enumerate([2, 0]):
        np.testing.assert_allclose(part.hd[r], full.hd[b], rtol=1e-12)
        np.testing.assert_array_equal(part.out_tokens[r], full.out_tokens[b])
        np.testing.assert_array_equal(part.drafts[r], full.drafts[b])


def test_planted_rows_accept_their_first_candidate():
    cfg = TINY.with_(B=6, plant_frac=0.5, ctx_min=3, ctx_max=30)
    inp = synth.make_inputs(cfg)
    res = dmtp.run_round(inp)
    assert inp.plant.any() and not inp.plant.all()
    for r in range(cfg.B):
        if inp.plant[r]:
            assert res.t1[r] == res.target_argmax[r, 0] and res.accept_len[r] >= 1


def test_overrides_force_decisions(tiny_inputs):
    base = dmtp.run_round(tiny_inputs)
    forced_t1 = (int(base.t1[0]) + 1) % TINY.V
    res = dmtp.run_round(tiny_inputs, overrides={("T1", 0): forced_t1})
    assert res.t1[0] == forced_t1 and res.drafts[0, 0] == forced_t1
    assert not np.allclose(res.x_t1, base.x_t1)


def test_sampled_round_uses_draws_and_accept_tests():
    cfg = TINY.with_(B=3, tau_mode="sample", seed=77)
    inp = synth.make_inputs(cfg)
    res = dmtp.run_round(inp)
    kinds = {k[0] for k, _, _ in res.decisions}
    assert {"T1", "draft", "accept", "final"} <= kinds
    # a larger temperature flattens the rows: lse(l / tau) falls toward log V
    hot = synth.make_inputs(cfg)
    hot.tau[:] = 4.0
    res_hot = dmtp.run_round(hot)
    assert np.all(res_hot.p_lse < res.p_lse)
    assert np.all(res_hot.p_lse > np.log(cfg.V) - 0.05)


def test_target_only_round_at_tau_zero_is_the_greedy_round():
    cfg = TINY.with_(B=3, ctx_min=20, ctx_max=60, seed=91)
    a = dmtp.run_round(synth.make_inputs(cfg))
    b = dmtp.run_round(synth.make_inputs(cfg.with_(verify="target_only")))
    for name in ("t1", "drafts", "target_argmax", "accept_len", "out_tokens", "n_out"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))


def test_target_only_sampled_round_commits_the_target_picks():
    cfg = TINY.with_(B=4, tau_mode="sample", verify="target_only", ctx_min=20, ctx_max=60, seed=92)
    inp = synth.make_inputs(cfg)
    res = dmtp.run_round(inp)
    kinds = {k[0] for k, _, _ in res.decisions}
    assert "accept" not in kinds and "final" not in kinds     # no accept tests, no residual draws
    from oracle.philox import grouped_gumbel_argmax
    full = dmtp.run_round(inp, keep_logits=True)
    for r in range(cfg.B):
        y = res.target_argmax[r]
        # every pick is the two-level Gumbel-max draw of its row at the row's temperature
        for i in range(cfg.K + 1):
            want, _ = grouped_gumbel_argmax(full.p_logits[r, i] / inp.tau[r], int(inp.philox_seed),
                                            int(inp.target_keys[r, i]))
            assert y[i] == want
        L = int(res.accept_len[r])
        assert np.array_equal(res.drafts[r, :L], y[:L])
        assert L == cfg.K or res.drafts[r, L] != y[L]
        assert res.out_tokens[r, L] == y[L] and np.all(res.out_tokens[r, L + 1:] == -1)
    # the picks are draws, not the argmax: at tau = 1 over V = 1024 some differ
    assert np.any(res.target_argmax != np.argmax(full.p_logits, axis=-1))


def test_single_anchor_layout():
    cfg = TINY.with_(n_anchor=1)
    inp = synth.make_inputs(cfg)
    res = dmtp.run_round(inp)
    assert res.hd.shape[1] == cfg.K       # [T1, MASK x (K-1)]
    assert res.drafts.shape[1] == cfg.K


def test_acceptance_stats_formulas():
    # hist = [2, 1, 0, 3] over K = 3
    acc = [0, 0, 1, 3, 3, 3]
    st = dmtp.acceptance_stats(acc, 3)
    assert st["hist"] == [2, 1, 0, 3]
    assert st["per_verify"] == pytest.approx(1 + (1 * 1 + 3 * 3) / 6)
    assert st["first_candidate"] == pytest.approx(1 - 2 / 6)
    assert st["cumulative"] == pytest.approx([4 / 6, 3 / 6, 3 / 6])


def test_acceptance_stats_reproduce_the_pages_conditional_table():
    """Golden: rebuild a histogram from the printed conditional rates and counts.

    The printed per-position conditional acceptances (two decimals) and the
    verify-round count fix the histogram up to rounding; the statistics must
    give back the printed conditional rates, and the first-candidate rate must
    equal the first conditional (the text states the same number for it).
    """
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "conditional_acceptance.json")) as f:
        gold = json.load(f)
    for name, row in gold["rows"].items():
        N = row["verify_rounds"]
        c = np.array(row["conditional_pct"]) / 100.0
        K = len(c)
        surv = np.concatenate([[1.0], np.cumprod(c)])           # P(L >= k), k = 0..K
        n_geq = np.round(N * surv).astype(np.int64)            # rounds with L >= k
        counts = n_geq - np.append(n_geq[1:], 0)               # hist[0..K], sums to N
        acc = np.repeat(np.arange(K + 1), counts)
        st = dmtp.acceptance_stats(acc, K)
        assert sum(st["hist"]) == N
        np.testing.assert_allclose(np.array(st["conditional"]) * 100, row["conditional_pct"], atol=0.01)
        assert st["first_candidate"] * 100 == pytest.approx(row["first_token_pct_in_text"], abs=0.01)
        # per-verify length is 1 + sum_k P(L >= k)
        assert st["per_verify"] == pytest.approx(1 + float(np.sum(st["cumulative"])), rel=1e-12)
