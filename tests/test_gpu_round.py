"""Whole-round parity of the HIP path with the oracle on the five workloads.

Tokens, accepted lengths and drawn indices must equal the oracle's, except
at near-ties of the oracle's own decision margins (below 1e-3 in logit
units), where the oracle is replayed with the GPU's decision; hidden states
and logit statistics must match to 2e-2 max relative error.  The full-size
workloads run the whole batch on the GPU and compare a subset of sequences
(rows of a round are independent).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import dmtp_synth as synth  # noqa: E402

from tests._harness import compare_round, correlated_targets, max_rel, record  # noqa: E402


@pytest.fixture(scope="module")
def rnd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mtp_block_draft_amd.round import Round
    return Round


def _run(Round, inp, h_target=None):
    R = Round(inp, h_target=h_target)
    R.run()
    return R, R.results()


def _report(name, rep):
    """Print and record the comparison; an exemption is only ever granted for a
    near-tie of the oracle, so there are never more of them than near-ties."""
    record(name, rep)
    assert len(rep["exempt"]) <= rep["near_ties"], (name, rep["exempt"], rep["near_ties"])


@pytest.mark.parametrize("w_zero", [False, True])
@pytest.mark.parametrize("gain_std", [0.0, 0.1])
def test_tiny_greedy_f32(rnd, w_zero, gain_std):
    cfg = synth.CONFIGS["tiny_greedy_f32"].with_(w_zero=w_zero, gain_std=gain_std)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g)
    _report(cfg.name, rep)
    if w_zero:
        # zero residual projection: the T1 slot is E(T1) exactly
        np.testing.assert_array_equal(g["x_t1"], inp.emb[g["t1"]].astype(np.float32))


def test_tiny_sampled_f32(rnd):
    cfg = synth.CONFIGS["tiny_sampled_f32"]
    for seed in (303, 304, 305, 306):
        inp = synth.make_inputs(cfg.with_(seed=seed))
        ht = correlated_targets(inp, cfg.rho)
        R, g = _run(rnd, inp, h_target=ht)
        res, rep = compare_round(inp, g, h_target=ht)
        _report(f"{cfg.name}/{seed}", rep)


def test_tiny_sampled_target_only_f32(rnd):
    cfg = synth.CONFIGS["tiny_sampled_f32"].with_(verify="target_only")
    for seed in (303, 304, 305, 306):
        inp = synth.make_inputs(cfg.with_(seed=seed))
        ht = correlated_targets(inp, cfg.rho)
        R, g = _run(rnd, inp, h_target=ht)
        res, rep = compare_round(inp, g, h_target=ht)
        _report(f"{cfg.name}/target_only/{seed}", rep)


def test_ragged_mixed_target_only_bf16(rnd):
    cfg = synth.RoundConfig(name="ragged_mixed_target_only", B=6, H=512, V=3001, Hq=8, Hkv=2,
                            d=64, F=768, n_layers=2, K=7, ctx_min=0, ctx_max=700, dtype="bf16",
                            tau_mode="mixed", plant_frac=0.5, gain_std=0.1, verify="target_only",
                            seed=12)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g)
    _report(cfg.name, rep)
    # the device histogram of the round equals the oracle's statistics
    R.accept_stats()
    from oracle import dmtp as odm
    st = odm.acceptance_stats(res.accept_len, cfg.K)
    assert R.hist.cpu().numpy().tolist() == st["hist"]


def test_tiny_rounds_with_the_mtp_block(rnd):
    for name in ("tiny_greedy_f32", "tiny_sampled_f32"):
        cfg = synth.CONFIGS[name].with_(mtp_block=True, B=3, ctx_min=0, ctx_max=200, gain_std=0.1)
        inp = synth.make_inputs(cfg)
        R, g = _run(rnd, inp)
        res, rep = compare_round(inp, g)
        _report(f"{name}/mtp_block", rep)
        for l, (k, v) in enumerate(g["mtp_kv"]):
            assert max_rel(k[:, 0], res.mtp_kv[l][0][:, 0]) < 1e-4
            assert max_rel(v[:, 0], res.mtp_kv[l][1][:, 0]) < 1e-4


def test_ragged_mixed_bf16(rnd):
    """Several tiles, ragged contexts (including empty), mixed greedy/sampled, planted T1."""
    cfg = synth.RoundConfig(name="ragged_mixed", B=6, H=512, V=3001, Hq=8, Hkv=2, d=64, F=768,
                            n_layers=2, K=7, ctx_min=0, ctx_max=700, dtype="bf16",
                            tau_mode="mixed", plant_frac=0.5, gain_std=0.1, seed=11)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g)
    _report(cfg.name, rep)


@pytest.mark.parametrize("K", [2, 6])
def test_tiny_round_block_sizes(rnd, K):
    """K = 2 (a single MASK slot) and K = 6 (the literal five-MASK layout)."""
    cfg = synth.CONFIGS["tiny_greedy_f32"].with_(K=K, B=3, ctx_min=0, ctx_max=150, gain_std=0.1)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g)
    _report(f"tiny K={K}", rep)


def test_single_anchor_layout(rnd):
    cfg = synth.CONFIGS["tiny_greedy_f32"].with_(n_anchor=1, B=3, ctx_min=10, ctx_max=90)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g)
    _report("single_anchor", rep)


@pytest.mark.timeout(900)
def test_b32_greedy_bf16_full_size(rnd):
    cfg = synth.CONFIGS["b32_greedy_bf16"]
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g)
    _report(cfg.name, rep)
    # determinism: a second round on the same buffers is bit-identical
    R.run()
    g2 = R.results()
    for k in ("hd_mask", "out_tokens", "target_lse", "x_t1"):
        np.testing.assert_array_equal(g[k], g2[k])


@pytest.mark.timeout(900)
def test_b32_greedy_with_the_mtp_block_full_size(rnd):
    cfg = synth.CONFIGS["b32_greedy_bf16"].with_(mtp_block=True)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g, seqs=[0, 9, 31])
    _report(f"{cfg.name}/mtp_block", rep)


@pytest.mark.timeout(900)
def test_b32_zero_residual_is_bitwise_on_gpu(rnd):
    cfg = synth.CONFIGS["b32_greedy_bf16"].with_(w_zero=True)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    np.testing.assert_array_equal(g["x_t1"], inp.emb[g["t1"]].astype(np.float32))


@pytest.mark.timeout(900)
def test_chat_b128_mixed_full_size(rnd):
    cfg = synth.CONFIGS["chat_b128_mixed_bf16"]
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    seqs = list(range(0, cfg.B, 5))          # 26 sequences: greedy and sampled, planted or not
    res, rep = compare_round(inp, g, seqs=seqs)
    _report(cfg.name, rep)
    assert inp.tau[seqs].min() == 0 and inp.tau[seqs].max() > 0
    # the float32 logits rows the head stores for sampled sequences, element by
    # element against the oracle at the full vocabulary, for three sampled
    # sequences (candidate rows 0..K-1, then target rows 0..K)
    from oracle import dmtp as odm
    logits = R.logits.view(cfg.B, 2 * cfg.K + 1, cfg.V)
    sampled = [b for b in seqs if inp.tau[b] > 0][:3]
    assert sampled
    for b in sampled:
        ov = {k: v for k, v in rep["overrides"].items() if k[1] == b}
        ref = odm.run_round(inp, seqs=[b], overrides=ov, keep_logits=True)
        want = np.concatenate([ref.q_logits[0], ref.p_logits[0]])        # [2K + 1, V]
        got = logits[b].cpu().numpy().astype(np.float64)
        scale = np.max(np.abs(want), axis=1, keepdims=True)
        err = np.max(np.abs(got - want) / scale)
        print(f"chat logits seq {b}: max |gpu - oracle| / row max = {err:.2e}", flush=True)
        assert err < 2e-3, (b, err)


@pytest.mark.timeout(900)
def test_chat_b128_target_only_full_size(rnd):
    cfg = synth.CONFIGS["chat_b128_mixed_bf16"].with_(verify="target_only")
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    seqs = list(range(1, cfg.B, 5))
    res, rep = compare_round(inp, g, seqs=seqs)
    _report(f"{cfg.name}/target_only", rep)
    assert inp.tau[seqs].min() == 0 and inp.tau[seqs].max() > 0


@pytest.mark.timeout(900)
def test_long_block16_full_size(rnd):
    cfg = synth.CONFIGS["long_block16_bf16"]
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    # with the window test's sequences 3 and 6, every sequence of the batch is checked
    res, rep = compare_round(inp, g, seqs=[0, 1, 2, 4, 5, 7])
    _report(cfg.name, rep)


@pytest.mark.timeout(900)
def test_long_block16_anchor_window_full_size(rnd):
    """The pages' default visibility: the last 4096 context positions before the anchor."""
    cfg = synth.CONFIGS["long_block16_bf16"].with_(window=4096)
    inp = synth.make_inputs(cfg)
    R, g = _run(rnd, inp)
    res, rep = compare_round(inp, g, seqs=[3, 6])
    _report(f"{cfg.name}/window4096", rep)


@pytest.mark.timeout(900)
def test_whole_round_graph_replays_match_eager(rnd):
    """The round captured as one graph gives, on every replay, the eager round's
    results bit for bit; eager work and synchronisations sit between replays."""
    for name in ("tiny_sampled_f32", "chat_b128_mixed_bf16"):
        cfg = synth.CONFIGS[name]
        inp = synth.make_inputs(cfg)
        R = rnd(inp)
        R.run()
        want = R.results()
        R.capture()
        keys = ("t1", "x_t1", "hd_mask", "drafts", "target_argmax", "target_lse", "accept_len",
                "out_tokens", "n_out")
        for rep in range(4):
            # clobber the outputs eagerly, then replay into them
            R.out_tokens.fill_(-9)
            R.accept_len.fill_(-9)
            R.head_in[: R.n_draft_rows].zero_()
            torch.cuda.synchronize()
            R.replay()
            got = R.results()
            for k in keys:
                np.testing.assert_array_equal(got[k], want[k], err_msg=f"{name} replay {rep} {k}")
        if name == "tiny_sampled_f32":
            res, rep_ = compare_round(inp, want)
