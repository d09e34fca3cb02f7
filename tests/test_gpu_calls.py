"""Per-call parity of the HIP library with the oracle, at sizes the oracle
finishes in seconds that still cover several tiles and ragged tails."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dmtp as odm, numerics as onm, philox as oph  # noqa: E402

from tests._harness import NEAR_TIE, max_rel  # noqa: E402


@pytest.fixture(scope="module")
def dm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mtp_block_draft_amd as m
    return m


def _bf16_trunc(x):
    x = np.ascontiguousarray(x, dtype=np.float32).copy()
    x.view(np.uint32)[...] &= np.uint32(0xFFFF0000)
    return x


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def _store(a, dt):
    return _bf16_trunc(a) if dt == "bf16" else np.asarray(a, np.float32)


TD = {"bf16": torch.bfloat16, "f32": torch.float32}


# ---------------------------------------------------------------- fuse


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,H", [(1, 256), (37, 256), (32, 2048), (5, 1024), (32, 1536), (144, 320),
                                    (300, 2048)])
@pytest.mark.parametrize("residual", [False, True])
def test_fuse(dm, dt, rows, H, residual):
    print(f"fuse dt={dt} rows={rows} H={H} res={residual}", flush=True)
    r = np.random.default_rng(rows * 7 + H + residual)
    V = 300
    emb = _store(0.02 * r.standard_normal((V, H)), dt)
    x1 = _store(r.standard_normal((rows, H)), dt)
    ids = r.integers(0, V, size=rows).astype(np.int32)
    g1 = 1 + 0.1 * r.standard_normal(H).astype(np.float32)
    g2 = 1 + 0.1 * r.standard_normal(H).astype(np.float32)
    W = _store(0.02 * r.standard_normal((H, 2 * H)), dt)
    out = torch.empty(rows, H, dtype=torch.float32, device="cuda")
    E = _t(emb, TD[dt])
    I = _t(ids, torch.int32)
    dm.fuse(out, _t(W, TD[dt]), _t(g1, torch.float32), _t(g2, torch.float32), x1=_t(x1, TD[dt]),
            x2_ids=I, res_ids=I if residual else None, table=E, eps=1e-6)
    got = out.cpu().numpy()
    want = odm.fuse(x1, emb[ids], g1, g2, W, 1e-6, res=emb[ids] if residual else None)
    err = max_rel(got, want)
    print("  max rel", err)
    assert err < 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fuse_rows_wider_than_8192(dm, dt):
    # more than 32 rows take the prologue path; at H = 8256 each of its threads
    # holds 8 float4 of both streams and loads gains and residual as it stores
    test_fuse(dm, dt, 33, 8256, True)


@pytest.mark.parametrize("rows,H", [(32, 2048), (7, 512), (1, 4096), (8, 5120), (33, 1024)])
def test_fuse_residual_layout(dm, rows, H):
    """The DMTP residual's operand layout: x1 = ids of T1, x2 = float32 MTP rows,
    res = ids of T1, bf16 weights.  Rows <= 32 with H a multiple of 512 run the
    projection with the norms folded in; 33 rows take the prologue path.  Two
    ids fall outside the table and read zero rows."""
    print(f"fuse residual layout rows={rows} H={H}", flush=True)
    r = np.random.default_rng(rows * 13 + H)
    V = 257
    emb = _store(0.02 * r.standard_normal((V, H)), "bf16")
    ids = r.integers(0, V, size=rows).astype(np.int32)
    if rows > 2:
        ids[1], ids[rows - 1] = -3, V + 5
    x2 = r.standard_normal((rows, H)).astype(np.float32)
    g1 = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    g2 = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    W = _store(0.02 * r.standard_normal((H, 2 * H)), "bf16")
    out = torch.empty(rows, H, dtype=torch.float32, device="cuda")
    I = _t(ids, torch.int32)
    dm.fuse(out, _t(W, torch.bfloat16), _t(g1, torch.float32), _t(g2, torch.float32), x1_ids=I,
            x2=_t(x2, torch.float32), res_ids=I, table=_t(emb, torch.bfloat16), eps=1e-6)
    e_rows = np.where(((ids >= 0) & (ids < V))[:, None], emb[np.clip(ids, 0, V - 1)], 0.0)
    want = odm.fuse(e_rows, x2, g1, g2, W, 1e-6, res=e_rows)
    got = out.cpu().numpy()
    err = max_rel(got, want)
    print("  max rel", err)
    assert err < 1e-5
    # a row of the zero embedding normalises to zero: its x1 stream adds nothing
    if rows > 2:
        only_h = odm.fuse(np.zeros((1, H)), x2[1:2], g1, g2, W, 1e-6)
        assert max_rel(got[1:2], only_h) < 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fuse_zero_projection_is_bitwise_residual(dm, dt):
    r = np.random.default_rng(5)
    rows, H, V = 19, 512, 64
    emb = _store(0.02 * r.standard_normal((V, H)), dt)
    ids = r.integers(0, V, size=rows).astype(np.int32)
    x2 = r.standard_normal((rows, H)).astype(np.float32)
    out = torch.empty(rows, H, dtype=torch.float32, device="cuda")
    I = _t(ids, torch.int32)
    dm.fuse(out, torch.zeros(H, 2 * H, dtype=TD[dt], device="cuda"), _t(np.ones(H), torch.float32),
            _t(np.ones(H), torch.float32), x1_ids=I, x2=_t(x2, torch.float32), res_ids=I,
            table=_t(emb, TD[dt]))
    np.testing.assert_array_equal(out.cpu().numpy(), emb[ids].astype(np.float32))


# ---------------------------------------------------------------- LM head


def _head_case(seed, H, V, dt, M_norm=5, M_rows=20, M_strided=12):
    r = np.random.default_rng(seed)
    W = _store(0.02 * r.standard_normal((V, H)), dt)
    hid = r.standard_normal((M_norm, H)).astype(np.float32)
    g = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    rows = _store(r.standard_normal((M_rows, H)), dt)
    strided = _store(r.standard_normal((M_strided, 2 * H)), dt)
    rf = onm.round_to(dt)
    x = np.concatenate([rf(onm.rmsnorm(hid, g, 1e-6)), rows.astype(np.float64),
                        strided[:, :H].astype(np.float64)])
    return W, hid, g, rows, strided, x


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("H,V", [(256, 5003), (2048, 151936), (256, 2), (192, 130)])
def test_lm_head_greedy(dm, dt, H, V):
    print(f"lm_head greedy dt={dt} H={H} V={V}", flush=True)
    W, hid, g, rows, strided, x = _head_case(H + V, H, V, dt)
    M = x.shape[0]
    td = TD[dt]
    segs = [dm.head_segment(_t(hid, torch.float32), _t(g, torch.float32)),
            dm.head_segment(_t(rows, td)),
            dm.head_segment(_t(strided, td), n=strided.shape[0], ld=2 * H)]
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    rmax = torch.empty(M, dtype=torch.float32, device="cuda")
    gap = torch.empty(M, dtype=torch.float32, device="cuda")
    prep = torch.empty(M, H, dtype=td, device="cuda")
    dm.lm_head(_t(W, td), segs, tok, eps=1e-6, prepared=prep, lse=lse, row_max=rmax, gap=gap)
    # prepared rows: normalised rows rounded to the head dtype
    assert max_rel(prep.float().cpu().numpy(), x) < 2e-2
    ref = odm.lm_head(x, W.astype(np.float64), np.zeros(M))
    got = tok.cpu().numpy()
    for m in range(M):
        if got[m] != ref.token[m]:
            assert ref.margin[m] < NEAR_TIE, (m, got[m], ref.token[m], ref.margin[m])
    assert max_rel(lse.cpu().numpy(), ref.lse) < 1e-5
    assert max_rel(rmax.cpu().numpy(), ref.row_max) < 1e-4
    print("  exempt:", int((got != ref.token).sum()), "of", M)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_lm_head_sampled_planted_and_stored(dm, dt):
    H, V = 512, 7001
    W, hid, g, rows, strided, x = _head_case(11, H, V, dt, M_norm=6, M_rows=24, M_strided=9)
    M = x.shape[0]
    td = TD[dt]
    r = np.random.default_rng(12)
    tau = np.where(r.random(M) < 0.6, r.choice([1.0, 0.7, 1.3], size=M), 0.0).astype(np.float32)
    keys = (np.arange(M, dtype=np.uint64) * np.uint64(977) + np.uint64(5)).astype(np.uint64)
    keys[3] = np.uint64(0xFFFFFFFFFFFFFFFF)           # a no-draw row
    store = np.arange(M, dtype=np.int32)[::-1].copy()  # every row stored, reversed order
    plant = np.full(M, -1, np.int32)
    plant[[1, 7]] = [M - 1, 0]
    seed = 0x1234_5678_9ABC
    segs = [dm.head_segment(_t(hid, torch.float32), _t(g, torch.float32)),
            dm.head_segment(_t(rows, td)),
            dm.head_segment(_t(strided, td), n=strided.shape[0], ld=2 * H)]
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    logits = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
    dm.lm_head(_t(W, td), segs, tok, temperature=_t(tau, torch.float32),
               draw_key=_t(keys.view(np.int64), torch.int64), seed=seed,
               plant_row=_t(plant, torch.int32), store_row=_t(store, torch.int32), logits=logits,
               lse=lse)
    L = W.astype(np.float64)
    ref_logits = x @ L.T
    got_logits = logits.cpu().numpy()[store]
    assert max_rel(got_logits, ref_logits) < 2e-3
    t = np.where(tau > 0, tau, 1.0)
    assert max_rel(lse.cpu().numpy(), onm.logsumexp(ref_logits / t[:, None])) < 1e-4
    got = tok.cpu().numpy()
    n_ex = 0
    for m in range(M):
        if plant[m] >= 0:
            src = plant[m]
            want, margin = int(np.argmax(ref_logits[src])), float(onm.top2_gap(ref_logits[src]))
        elif tau[m] > 0 and keys[m] != np.uint64(0xFFFFFFFFFFFFFFFF):
            want, margin = oph.grouped_gumbel_argmax(ref_logits[m] / tau[m], seed, int(keys[m]))
        else:
            want, margin = int(np.argmax(ref_logits[m])), float(onm.top2_gap(ref_logits[m]))
        if got[m] != want:
            assert margin < NEAR_TIE, (m, got[m], want, margin)
            n_ex += 1
    print("exempt", n_ex)


@pytest.mark.parametrize("M", [32, 64, 200, 448, 901])
def test_lm_head_many_rows(dm, M):
    # 1 to 7 row tiles of 64 per workgroup, one and several row chunks, a
    # ragged vocabulary tile (7001 = 54 * 128 + 89)
    H, V = 512, 7001
    print(f"lm_head many rows M={M}", flush=True)
    W, hid, g, rows, strided, x = _head_case(31 + M, H, V, "bf16", M_norm=0, M_rows=M, M_strided=0)
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    rmax = torch.empty(M, dtype=torch.float32, device="cuda")
    gap = torch.empty(M, dtype=torch.float32, device="cuda")
    dm.lm_head(_t(W, torch.bfloat16), [dm.head_segment(_t(rows, torch.bfloat16))], tok, lse=lse,
               row_max=rmax, gap=gap)
    ref = odm.lm_head(x, W.astype(np.float64), np.zeros(M))
    got = tok.cpu().numpy()
    bad = np.nonzero(got != ref.token)[0]
    assert all(ref.margin[m] < NEAR_TIE for m in bad), [(m, got[m], ref.token[m]) for m in bad[:5]]
    assert max_rel(lse.cpu().numpy(), ref.lse) < 1e-5
    assert max_rel(rmax.cpu().numpy(), ref.row_max) < 1e-4
    print("  exempt:", len(bad), "of", M)


def test_lm_head_rows_do_not_depend_on_the_batch(dm):
    # Calls of 33 rows and more: 448 rows run 7 tiles per workgroup; 200 and
    # 385 rows take other tile counts and slice widths, which must not change
    # any row's result.  Calls of at most 32 rows take the weight-streaming
    # kernel, bit for bit the same among themselves; its k-split sums in
    # another order, so against the larger calls the rows agree to rounding.
    H, V = 2048, 20000
    W, hid, g, rows, strided, x = _head_case(21, H, V, "bf16", M_norm=0, M_rows=448, M_strided=0)
    Wt = _t(W, torch.bfloat16)
    X = _t(rows, torch.bfloat16)
    outs = {}
    for name, sl in (("all", slice(0, 448)), ("tail", slice(63, 448)), ("mid", slice(100, 300)),
                     ("one", slice(37, 38)), ("s20", slice(30, 50)), ("s32", slice(37, 69))):
        xs = X[sl].contiguous()
        n = xs.shape[0]
        tok = torch.empty(n, dtype=torch.int32, device="cuda")
        lse = torch.empty(n, dtype=torch.float32, device="cuda")
        gap = torch.empty(n, dtype=torch.float32, device="cuda")
        dm.lm_head(Wt, [dm.head_segment(xs)], tok, lse=lse, gap=gap)
        outs[name] = (tok.cpu().numpy(), lse.cpu().numpy(), gap.cpu().numpy())
    for j in (0, 1):
        np.testing.assert_array_equal(outs["tail"][j], outs["all"][j][63:])
        np.testing.assert_array_equal(outs["mid"][j], outs["all"][j][100:300])
        np.testing.assert_array_equal(outs["one"][j], outs["s32"][j][:1])
        np.testing.assert_array_equal(outs["s20"][j][7:], outs["s32"][j][:13])
    tok_s, lse_s, _ = outs["s32"]
    tok_a, lse_a, gap_a = (v[37:69] for v in outs["all"])
    assert max_rel(lse_s, lse_a) < 1e-6
    assert all(tok_s[i] == tok_a[i] or gap_a[i] < 1e-4 for i in range(32))


def test_head_pack_layout(dm):
    # the packed copy against its definition: block s of tile t holds, as
    # piece 8 r + j, columns 64 s + 8 (j ^ ((r >> 1) & 7)) .. + 7 of row
    # 128 t + r, with zero rows past V
    V, H = 300, 192
    print(f"head pack layout V={V} H={H}", flush=True)
    rng = np.random.default_rng(5)
    W = torch.from_numpy(rng.standard_normal((V, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    got = dm.pack_head_weight(W).view(torch.int16).cpu().numpy()
    T = (V + 127) // 128
    Wp = np.zeros((T * 128, H), np.int16)
    Wp[:V] = W.view(torch.int16).cpu().numpy()
    r = np.arange(128)[:, None]
    j = np.arange(8)[None, :]
    src = j ^ ((r >> 1) & 7)                                  # [128, 8] source chunk of piece (r, j)
    want = []
    for t in range(T):
        for sb in range(H // 64):
            blk = Wp[128 * t:128 * t + 128, 64 * sb:64 * sb + 64].reshape(128, 8, 8)
            want.append(blk[r, src, :].reshape(-1))
    np.testing.assert_array_equal(got, np.concatenate(want))


@pytest.mark.parametrize("V,H,M", [(7001, 512, 200), (7001, 512, 448), (20000, 2048, 448),
                                   (9000, 5120, 256), (3000, 1024, 901), (9000, 5120, 8),
                                   (7001, 512, 64), (20000, 2048, 100)])
def test_lm_head_packed_weights_bit_identical(dm, V, H, M):
    # The register-input GEMM (4, 5 and 7 row tiles per wave; one and three
    # row chunks; ragged last vocabulary tiles) and the 64-wide-slice kernel
    # of calls of 33 .. 128 rows, or of fewer rows when H is above 2048,
    # streaming the packed copy give every output bit for bit as they do from
    # W.  A packed copy of a zero matrix then shows the kernel reads the copy.
    print(f"lm_head packed V={V} H={H} M={M}", flush=True)
    W, hid, g, rows, strided, x = _head_case(41 + M, H, V, "bf16", M_norm=0, M_rows=M, M_strided=0)
    Wt, X = _t(W, torch.bfloat16), _t(rows, torch.bfloat16)
    n_st = min(M, 6)
    store = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    store[torch.arange(0, M, max(1, M // n_st), device="cuda")[:n_st]] = torch.arange(n_st, dtype=torch.int32,
                                                                                       device="cuda")
    outs = []
    for wp in (None, dm.pack_head_weight(Wt), dm.pack_head_weight(torch.zeros_like(Wt))):
        tok = torch.empty(M, dtype=torch.int32, device="cuda")
        lse = torch.empty(M, dtype=torch.float32, device="cuda")
        rmax = torch.empty(M, dtype=torch.float32, device="cuda")
        gap = torch.empty(M, dtype=torch.float32, device="cuda")
        logits = torch.full((n_st, V), float("nan"), dtype=torch.float32, device="cuda")
        dm.lm_head(Wt, [dm.head_segment(X)], tok, lse=lse, row_max=rmax, gap=gap, store_row=store,
                   logits=logits, w_packed=wp)
        outs.append([v.cpu().numpy() for v in (tok, lse, rmax, gap, logits)])
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
    assert np.all(outs[2][2] == 0) and np.all(outs[2][4] == 0)


@pytest.mark.parametrize("H", [512, 1024, 1536, 2048])
@pytest.mark.parametrize("M", [1, 9, 32])
def test_lm_head_at_most_32_rows(dm, H, M):
    # the weight-streaming kernel: normed, plain and strided segments, greedy,
    # sampled, planted and no-draw rows, stored logits, a ragged last
    # vocabulary tile (8191 = 255 * 32 + 31)
    V = 8191
    print(f"lm_head streaming H={H} M={M}", flush=True)
    n_norm, n_rows = (M + 2) // 3, M // 3
    W, hid, g, rows, strided, x = _head_case(7 * H + M, H, V, "bf16", M_norm=n_norm,
                                             M_rows=n_rows, M_strided=M - n_norm - n_rows)
    r = np.random.default_rng(H + M)
    tau = np.where(r.random(M) < 0.5, r.choice([1.0, 0.7], size=M), 0.0).astype(np.float32)
    keys = (np.arange(M, dtype=np.uint64) * np.uint64(131) + np.uint64(9)).astype(np.uint64)
    if M > 2:
        keys[2] = np.uint64(0xFFFFFFFFFFFFFFFF)
    plant = np.full(M, -1, np.int32)
    if M > 4:
        plant[4] = 0
    store = np.arange(M, dtype=np.int32)[::-1].copy()
    segs = [dm.head_segment(_t(hid, torch.float32), _t(g, torch.float32)),
            dm.head_segment(_t(rows, torch.bfloat16)),
            dm.head_segment(_t(strided, torch.bfloat16), n=strided.shape[0], ld=2 * H)]
    segs = [sg for sg, n in zip(segs, (n_norm, n_rows, M - n_norm - n_rows)) if n > 0]
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    rmax = torch.empty(M, dtype=torch.float32, device="cuda")
    logits = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
    seed = 0xDEC0DE
    dm.lm_head(_t(W, torch.bfloat16), segs, tok, eps=1e-6, temperature=_t(tau, torch.float32),
               draw_key=_t(keys.view(np.int64), torch.int64), seed=seed,
               plant_row=_t(plant, torch.int32), store_row=_t(store, torch.int32), logits=logits,
               lse=lse, row_max=rmax)
    ref_logits = x @ W.astype(np.float64).T
    assert max_rel(logits.cpu().numpy()[store], ref_logits) < 2e-3
    t = np.where(tau > 0, tau, 1.0)
    assert max_rel(lse.cpu().numpy(), onm.logsumexp(ref_logits / t[:, None])) < 1e-5
    assert max_rel(rmax.cpu().numpy(), ref_logits.max(axis=1)) < 1e-4
    got = tok.cpu().numpy()
    for m in range(M):
        if plant[m] >= 0:
            src = plant[m]
            want, margin = int(np.argmax(ref_logits[src])), float(onm.top2_gap(ref_logits[src]))
        elif tau[m] > 0 and keys[m] != np.uint64(0xFFFFFFFFFFFFFFFF):
            want, margin = oph.grouped_gumbel_argmax(ref_logits[m] / tau[m], seed, int(keys[m]))
        else:
            want, margin = int(np.argmax(ref_logits[m])), float(onm.top2_gap(ref_logits[m]))
        if got[m] != want:
            assert margin < NEAR_TIE, (m, got[m], want, margin)


# ---------------------------------------------------------------- block draft


def _spiked(k, ctx_lens, spike):
    """Keys of the context rows at position 50 mod 97 of each sequence times
    spike: their scores jump far above the rest in the middle of a chunk."""
    if spike:
        pos = np.concatenate([np.arange(n) for n in ctx_lens] + [np.zeros(0, np.int64)])
        k[:len(pos)][pos % 97 == 50] *= spike
    return k


def _draft_case(seed, dt, B, H, Hq, Hkv, d, F, NL, K, n_anchor, ctx_lens, V=500, window=0, spike=0.0):
    r = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(np.int32)
    tot = int(cu[-1])
    emb = _store(0.02 * r.standard_normal((V, H)), dt)
    layers = []
    for _ in range(NL):
        layers.append(dict(
            g_attn=(1 + 0.1 * r.standard_normal(H)).astype(np.float32),
            wqkv=_store(0.02 * r.standard_normal(((Hq + 2 * Hkv) * d, H)), dt),
            wo=_store(0.02 * r.standard_normal((H, Hq * d)), dt),
            g_ffn=(1 + 0.1 * r.standard_normal(H)).astype(np.float32),
            wg=_store(0.02 * r.standard_normal((F, H)), dt),
            wu=_store(0.02 * r.standard_normal((F, H)), dt),
            wd=_store(0.02 * r.standard_normal((H, F)), dt),
            ctx_k=_store(_spiked(r.standard_normal((max(tot, 1), Hkv, d)), ctx_lens, spike), dt),
            ctx_v=_store(r.standard_normal((max(tot, 1), Hkv, d)), dt)))
    anchor = r.integers(0, V - 1, size=B).astype(np.int32)
    x_t1 = (emb[r.integers(0, V - 1, size=B)] + 0.01 * r.standard_normal((B, H))).astype(np.float32)
    g_final = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    return dict(cu=cu, emb=emb, layers=layers, anchor=anchor, x_t1=x_t1, g_final=g_final,
                ctx_lens=np.asarray(ctx_lens))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    dict(B=3, H=256, Hq=4, Hkv=2, d=64, F=512, NL=2, K=7, n_anchor=2, ctx_lens=[0, 70, 200]),
    dict(B=2, H=512, Hq=8, Hkv=2, d=128, F=768, NL=1, K=7, n_anchor=1, ctx_lens=[130, 1]),
    dict(B=4, H=256, Hq=4, Hkv=4, d=64, F=256, NL=1, K=5, n_anchor=2, ctx_lens=[300, 64, 65, 5],
         window=100),
    dict(B=2, H=512, Hq=10, Hkv=2, d=128, F=512, NL=1, K=16, n_anchor=2, ctx_lens=[777, 2100]),
    # 48 query rows per kv head at d = 64, 32 slot rows
    dict(B=2, H=256, Hq=6, Hkv=2, d=64, F=512, NL=1, K=15, n_anchor=2, ctx_lens=[100, 300]),
    # 160 slot rows (one ragged 256-row GEMM tile), 16 query rows per kv head
    dict(B=20, H=256, Hq=4, Hkv=2, d=64, F=512, NL=1, K=7, n_anchor=2,
         ctx_lens=[0, 1, 31, 64, 100, 257, 513, 40, 9, 77, 5, 6, 7, 8, 300, 2, 3, 4, 65, 129]),
    # 144 slot rows, widths that end mid-tile, 48 query rows per kv head
    dict(B=9, H=320, Hq=6, Hkv=2, d=64, F=576, NL=1, K=15, n_anchor=2,
         ctx_lens=[0, 1, 31, 64, 100, 257, 513, 40, 9]),
    # 200 slot rows: a ragged second 128-row tile in every projection
    dict(B=25, H=1536, Hq=12, Hkv=4, d=128, F=1024, NL=1, K=7, n_anchor=2,
         ctx_lens=[(37 * i) % 300 for i in range(25)]),
    # the largest block (32 candidates, 33 slots): three query tiles share a chunk's K/V
    dict(B=2, H=256, Hq=2, Hkv=1, d=64, F=256, NL=1, K=32, n_anchor=2, ctx_lens=[50, 0]),
    # 170 query rows per kv head: six query tiles, two workgroups of four (two waves idle)
    dict(B=2, H=256, Hq=10, Hkv=1, d=64, F=256, NL=1, K=16, n_anchor=2, ctx_lens=[300, 40]),
    # the smallest block: one MASK slot
    dict(B=3, H=256, Hq=4, Hkv=2, d=64, F=256, NL=1, K=2, n_anchor=2, ctx_lens=[17, 0, 64]),
    # keys of scattered context rows times 40: a row's max jumps by far more
    # than 2^8 (log2 units) in the middle of a chunk, so the running reference
    # max moves and O and l are rescaled there; several query tiles per kv head
    dict(B=2, H=512, Hq=10, Hkv=2, d=128, F=512, NL=1, K=16, n_anchor=2, ctx_lens=[777, 2100],
         spike=40.0),
    # the same with one query tile per kv head
    dict(B=3, H=256, Hq=4, Hkv=2, d=64, F=512, NL=1, K=7, n_anchor=2, ctx_lens=[1500, 333, 64],
         spike=40.0),
])
def test_block_draft(dm, dt, shape):
    shape = dict(shape)
    window = shape.pop("window", 0)
    spike = shape.pop("spike", 0.0)
    print(f"block_draft dt={dt} {shape} window={window} spike={spike}", flush=True)
    c = _draft_case(sum(shape["ctx_lens"]) + shape["H"], dt, window=window, spike=spike, **shape)
    B, H, K, na = shape["B"], shape["H"], shape["K"], shape["n_anchor"]
    td = TD[dt]
    f32 = torch.float32
    lt = [{k: _t(v, f32 if k.startswith("g_") else td) for k, v in L.items()} for L in c["layers"]]
    Ls = [dm.layer_arg(**L) for L in lt]
    out = torch.empty(B * (K - 1), H, dtype=td, device="cuda")
    V = c["emb"].shape[0]
    S = K - 1 + na
    f32_rows = 128 if shape["d"] == 64 else 64
    if dt == "f32" and S * shape["Hq"] // shape["Hkv"] > f32_rows:
        # float32 context K/V doubles the LDS tiles: more than 128 (d = 64) or
        # 64 (d = 128) query rows per kv head do not fit one workgroup, and the
        # library refuses the shape
        with pytest.raises(dm.DmtpError):
            dm.block_draft(out, B=B, H=H, Hq=shape["Hq"], Hkv=shape["Hkv"], d=shape["d"],
                           F=shape["F"], K=K, n_anchor=na, layers=Ls,
                           anchor_ids=_t(c["anchor"], torch.int32), x_t1=_t(c["x_t1"], f32),
                           mask_id=V - 1, emb=_t(c["emb"], td), cu_ctx=_t(c["cu"], torch.int32),
                           max_ctx=int(max(c["ctx_lens"])), ctx_rows=int(c["cu"][-1]),
                           g_final=_t(c["g_final"], f32), window=window)
        return
    dm.block_draft(out, B=B, H=H, Hq=shape["Hq"], Hkv=shape["Hkv"], d=shape["d"], F=shape["F"], K=K,
                   n_anchor=na, layers=Ls, anchor_ids=_t(c["anchor"], torch.int32),
                   x_t1=_t(c["x_t1"], f32), mask_id=V - 1, emb=_t(c["emb"], td),
                   cu_ctx=_t(c["cu"], torch.int32), max_ctx=int(max(c["ctx_lens"])),
                   ctx_rows=int(c["cu"][-1]), g_final=_t(c["g_final"], f32), window=window)
    got = out.float().cpu().numpy().reshape(B, K - 1, H)
    slots = [odm.block_slots(c["emb"][c["anchor"][b]], c["x_t1"][b], c["emb"][V - 1], K, na)
             for b in range(B)]
    L64 = [odm.Layer64(*(np.asarray(L[k], np.float64) for k in
                         ("g_attn", "wqkv", "wo", "g_ffn", "wg", "wu", "wd"))) for L in c["layers"]]
    ref = odm.block_draft(slots, c["ctx_lens"], L64, [L["ctx_k"] for L in c["layers"]],
                          [L["ctx_v"] for L in c["layers"]], c["cu"], list(range(B)), c["g_final"],
                          onm.round_to(dt), Hq=shape["Hq"], Hkv=shape["Hkv"], d=shape["d"], eps=1e-6,
                          rope_base=1e6, window=window)
    ref = np.stack(ref)[:, na:, :]
    err = max_rel(got, ref)
    print("  max rel", err)
    assert err < (1e-4 if dt == "f32" else 2e-2)
    if dt == "bf16":
        # rounding flips only: almost every element is the same bf16 value
        assert np.mean(got != ref) < 0.02


def _hip_runtime():
    """The HIP runtime torch has loaded, for event handles (ctypes)."""
    import ctypes
    path = next(l.split()[-1] for l in open("/proc/self/maps").read().splitlines()
                if "libamdhip64" in l)
    hip = ctypes.CDLL(path)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def test_block_draft_attention_events(dm):
    # The profiling hook of the draft descriptor: the first layer's context
    # attention launched with a start/stop event pair of its own dispatch.
    # Outputs bit for bit as without it, and a positive duration.
    import ctypes
    shape = dict(B=3, H=256, Hq=4, Hkv=2, d=64, F=512, NL=2, K=7, n_anchor=2, ctx_lens=[1500, 333, 64])
    print("block_draft attention events", shape, flush=True)
    c = _draft_case(77, "bf16", **shape)
    B, H, K, na = shape["B"], shape["H"], shape["K"], shape["n_anchor"]
    td, f32 = TD["bf16"], torch.float32
    lt = [{k: _t(v, f32 if k.startswith("g_") else td) for k, v in L.items()} for L in c["layers"]]
    Ls = [dm.layer_arg(**L) for L in lt]
    V = c["emb"].shape[0]
    hip = _hip_runtime()
    ev = (ctypes.c_void_p(), ctypes.c_void_p())
    assert hip.hipEventCreate(ctypes.byref(ev[0])) == 0 and hip.hipEventCreate(ctypes.byref(ev[1])) == 0
    outs = []
    for events in (None, (ev[0].value, ev[1].value)):
        out = torch.empty(B * (K - 1), H, dtype=td, device="cuda")
        dm.block_draft(out, B=B, H=H, Hq=shape["Hq"], Hkv=shape["Hkv"], d=shape["d"], F=shape["F"], K=K,
                       n_anchor=na, layers=Ls, anchor_ids=_t(c["anchor"], torch.int32),
                       x_t1=_t(c["x_t1"], f32), mask_id=V - 1, emb=_t(c["emb"], td),
                       cu_ctx=_t(c["cu"], torch.int32), max_ctx=int(max(c["ctx_lens"])),
                       ctx_rows=int(c["cu"][-1]), g_final=_t(c["g_final"], f32), attn_events=events)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu().numpy())
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    hip.hipEventDestroy(ev[0])
    hip.hipEventDestroy(ev[1])
    print("  attention kernel", 1000.0 * ms.value, "us")
    assert ms.value > 0.0
    np.testing.assert_array_equal(outs[0], outs[1])


# ---------------------------------------------------------------- MTP block


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    dict(B=3, S=1, H=256, Hq=4, Hkv=2, d=64, F=512, NL=1, ctx_lens=[0, 5, 300]),
    dict(B=2, S=4, H=512, Hq=8, Hkv=2, d=128, F=768, NL=2, ctx_lens=[130, 1]),
    dict(B=5, S=3, H=256, Hq=4, Hkv=4, d=64, F=256, NL=1, ctx_lens=[64, 65, 0, 1000, 7]),
    dict(B=32, S=1, H=512, Hq=16, Hkv=4, d=128, F=512, NL=1,
         ctx_lens=list(range(40, 40 + 32 * 37, 37))),
    # 12 rows with K >= 1024: the weight-streaming projections (2 and 3 splits,
    # the gate/up pair as one call), two layers
    dict(B=6, S=2, H=1024, Hq=8, Hkv=2, d=128, F=1536, NL=2, ctx_lens=[0, 17, 300, 64, 1, 900]),
    # spiked context keys: a row's reference max moves in the middle of a chunk
    dict(B=4, S=3, H=256, Hq=8, Hkv=2, d=64, F=256, NL=1, ctx_lens=[600, 1, 250, 0], spike=40.0),
])
def test_mtp_block(dm, dt, shape):
    """The causal MTP block and the K/V rows it returns, against the oracle."""
    shape = dict(shape)
    print(f"mtp_block dt={dt} {shape}", flush=True)
    S = shape.pop("S")
    c = _draft_case(sum(shape["ctx_lens"]) + 7 * S, dt, K=2, n_anchor=1, **shape)
    B, H, Hq, Hkv, d, F = (shape[k] for k in ("B", "H", "Hq", "Hkv", "d", "F"))
    r = np.random.default_rng(B * 100 + S)
    x = r.standard_normal((B, S, H)).astype(np.float32)
    td = TD[dt]
    f32 = torch.float32
    lt = [{k: _t(v, f32 if k.startswith("g_") else td) for k, v in L.items()} for L in c["layers"]]
    Ls = [dm.layer_arg(**L) for L in lt]
    out = torch.empty(B, S, H, dtype=f32, device="cuda")
    k_new = [torch.empty(B, S, Hkv, d, dtype=td, device="cuda") for _ in Ls]
    v_new = [torch.empty(B, S, Hkv, d, dtype=td, device="cuda") for _ in Ls]
    dm.mtp_block(out, _t(x, f32), Hq=Hq, Hkv=Hkv, d=d, F=F, layers=Ls,
                 cu_ctx=_t(c["cu"], torch.int32), max_ctx=int(max(c["ctx_lens"])),
                 ctx_rows=int(c["cu"][-1]), dtype=1 if dt == "bf16" else 0, k_new=k_new,
                 v_new=v_new)
    L64 = [odm.Layer64(*(np.asarray(L[k], np.float64) for k in
                         ("g_attn", "wqkv", "wo", "g_ffn", "wg", "wu", "wd"))) for L in c["layers"]]
    cu = c["cu"]
    spans = [(int(cu[b]), int(cu[b + 1])) for b in range(B)]
    pos = np.asarray(c["ctx_lens"])[:, None] + np.arange(S)
    ref, kv = odm.mtp_block(x.astype(np.float64), pos, L64,
                            [[L["ctx_k"][lo:hi] for lo, hi in spans] for L in c["layers"]],
                            [[L["ctx_v"][lo:hi] for lo, hi in spans] for L in c["layers"]],
                            Hq=Hq, Hkv=Hkv, d=d, eps=1e-6, rope_base=1e6)
    err = max_rel(out.cpu().numpy(), ref)
    print("  max rel out", err)
    assert err < 1e-4
    rf = onm.round_to(dt)
    for l in range(len(Ls)):
        for got_t, want in ((k_new[l], kv[l][0]), (v_new[l], kv[l][1])):
            got = got_t.float().cpu().numpy()
            want_r = rf(want)
            e = max_rel(got, want_r)
            print("  max rel kv", e)
            # float32: accumulation error only; bf16: at most a rounding flip of one ulp
            assert e < (1e-4 if dt == "f32" else 1e-2)
            if dt == "bf16":
                assert np.mean(got != want_r) < 0.02


# ---------------------------------------------------------------- context K/V


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,NF,H,Hq,Hkv,d,NL", [(1, 5, 256, 4, 2, 64, 1), (37, 5, 512, 8, 2, 128, 2),
                                                (300, 3, 2048, 16, 4, 128, 1),
                                                # 150 rows: the two-plane layer GEMM on the 160-row
                                                # tile, the bf16 feature GEMM on 128-row tiles
                                                (150, 5, 512, 8, 2, 128, 2),
                                                # 200 rows of 1536: a ragged second 128-row tile
                                                (200, 2, 1536, 12, 4, 128, 1)])
def test_ctx_kv(dm, dt, N, NF, H, Hq, Hkv, d, NL):
    """Context K/V rows from target features, written into the named cache rows."""
    print(f"ctx_kv dt={dt} N={N} NF={NF} H={H} {Hq}/{Hkv}x{d} NL={NL}", flush=True)
    r = np.random.default_rng(N + H)
    rows = 2 * N + 5
    feats = _store(r.standard_normal((N, NF, H)), dt)
    w_fc = _store(0.02 * r.standard_normal((H, NF * H)), dt)
    pos = r.integers(0, 40000, size=N).astype(np.int32)
    dst = r.permutation(rows)[:N].astype(np.int32)
    if N > 2:
        dst[1], dst[2] = -1, rows + 3          # out of range: nothing written
    layers = [dict(g_attn=(1 + 0.1 * r.standard_normal(H)).astype(np.float32),
                   wqkv=_store(0.02 * r.standard_normal(((Hq + 2 * Hkv) * d, H)), dt))
              for _ in range(NL)]
    td, f32 = TD[dt], torch.float32
    z = lambda *sh: torch.zeros(*sh, dtype=td, device="cuda")   # noqa: E731
    Ls = [dm.layer_arg(g_attn=_t(L["g_attn"], f32), wqkv=_t(L["wqkv"], td), wo=z(64), g_ffn=z(64),
                       wg=z(64), wu=z(64), wd=z(64), ctx_k=z(64), ctx_v=z(64)) for L in layers]
    sentinel = 3.0
    kc = [torch.full((rows, Hkv, d), sentinel, dtype=td, device="cuda") for _ in range(NL)]
    vc = [torch.full((rows, Hkv, d), sentinel, dtype=td, device="cuda") for _ in range(NL)]
    c_out = torch.empty(N, H, dtype=f32, device="cuda")
    dm.ctx_kv(_t(feats, td), _t(pos, torch.int32), _t(dst, torch.int32), _t(w_fc, td), Hq=Hq,
              Hkv=Hkv, d=d, layers=Ls, k_cache=kc, v_cache=vc, ctx_out=c_out)
    L64 = [odm.Layer64(np.asarray(L["g_attn"], np.float64), np.asarray(L["wqkv"], np.float64),
                       None, None, None, None, None) for L in layers]
    c_ref, kv = odm.ctx_kv(feats.astype(np.float64), pos, w_fc.astype(np.float64), L64, Hq=Hq,
                           Hkv=Hkv, d=d, eps=1e-6, rope_base=1e6)
    assert max_rel(c_out.cpu().numpy(), c_ref) < 1e-5
    rf = onm.round_to(dt)
    ok = (dst >= 0) & (dst < rows)
    untouched = np.setdiff1d(np.arange(rows), dst[ok])
    for l in range(NL):
        for cache, want in ((kc[l], kv[l][0]), (vc[l], kv[l][1])):
            got = cache.float().cpu().numpy()
            e = max_rel(got[dst[ok]], rf(want[ok]))
            print("  max rel", e)
            assert e < (1e-4 if dt == "f32" else 1e-2)
            if dt == "bf16":
                assert np.mean(got[dst[ok]] != rf(want[ok])) < 0.02
            assert np.all(got[untouched] == sentinel)


# ---------------------------------------------------------------- verify


def _softmax_lse(l, tau):
    return onm.logsumexp(l / tau, axis=-1)


@pytest.mark.parametrize("V", [3001, 151936])
def test_verify_greedy_and_sampled(dm, V):
    B, K = 24, 7
    r = np.random.default_rng(V)
    tau = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
    tau[5] = 0.8
    logits = (1.5 * r.standard_normal((B, 2 * K + 1, V))).astype(np.float32)
    # candidates: from the q rows, with target rows made to agree on a planted prefix
    target = logits[:, K:, :].argmax(-1).astype(np.int32)
    drafts = r.integers(0, V, size=(B, K)).astype(np.int32)
    for b in range(B):
        k = (b // 2) % (K + 1)                # force acceptance up to row k (greedy rows)
        drafts[b, :k] = target[b, :k]
        if k < K and drafts[b, k] == target[b, k]:
            drafts[b, k] = (target[b, k] + 1) % V
    u = (r.integers(0, 1 << 24, size=(B, K)) * 2.0 ** -24).astype(np.float32)
    # sampled rows: force accept below row k (u = 0) and a sure rejection at row k
    for b in range(B):
        if tau[b] > 0:
            k = (b // 2) % (K + 1)
            u[b, :k] = 0.0
            if k < K:
                logits[b, K + k, drafts[b, k]] = -30.0
                u[b, k] = 0.999
    tt = np.where(tau > 0, tau, 1.0).astype(np.float64)
    lse = _softmax_lse(logits.astype(np.float64), tt[:, None, None]).astype(np.float32)
    seed = 77
    fkeys = np.arange(B, dtype=np.uint64) + np.uint64(1 << 33)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, K + 1, dtype=torch.int32, device="cuda")
    n_out = torch.empty(B, dtype=torch.int32, device="cuda")
    dm.verify(B=B, K=K, V=V, t1=_t(drafts[:, 0], torch.int32), drafts=_t(drafts[:, 1:], torch.int32),
              target=_t(target, torch.int32), accept_len=acc, out_tokens=out, n_out=n_out,
              temperature=_t(tau, torch.float32), logits=_t(logits.reshape(B * (2 * K + 1), V),
                                                            torch.float32),
              t1_lse=_t(lse[:, 0], torch.float32), draft_lse=_t(lse[:, 1:K], torch.float32),
              target_lse=_t(lse[:, K:], torch.float32), u_acc=_t(u, torch.float32), seed=seed,
              final_key=_t(fkeys.view(np.int64), torch.int64))
    acc, out, n_out = acc.cpu().numpy(), out.cpu().numpy(), n_out.cpu().numpy()
    L64 = logits.astype(np.float64)
    for b in range(B):
        if tau[b] == 0:
            L, toks = odm.verify_greedy(drafts[b], target[b])
            assert acc[b] == L and list(out[b, :L + 1]) == toks and n_out[b] == L + 1
            assert np.all(out[b, L + 1:] == -1)
            assert L == (b // 2) % (K + 1)
            continue
        q = np.exp(L64[b, :K] / tau[b] - onm.logsumexp(L64[b, :K] / tau[b])[:, None])
        p = np.exp(L64[b, K:] / tau[b] - onm.logsumexp(L64[b, K:] / tau[b])[:, None])
        margins = {}

        def accept(i, ratio):
            margins[("a", i)] = abs(np.log(u[b, i]) - np.log(ratio)) if u[b, i] > 0 else np.inf
            return bool(u[b, i] < ratio)

        def draw(i, w):
            with np.errstate(divide="ignore"):
                j, m = oph.grouped_gumbel_argmax(np.log(np.asarray(w)), seed, int(fkeys[b]))
            margins["final"] = m
            return j

        L, toks = odm.verify_rejection(drafts[b], p, q, accept, draw)
        if acc[b] != L:
            assert margins.get(("a", min(L, acc[b])), np.inf) < NEAR_TIE
            continue
        assert list(out[b, :L]) == toks[:L] and n_out[b] == L + 1
        if out[b, L] != toks[L]:
            assert margins["final"] < NEAR_TIE, (b, out[b, L], toks[L], margins["final"])
        k = (b // 2) % (K + 1)
        assert L == k


def test_verify_mass_pass_events(dm):
    # The profiling hook of the verify descriptor: the pass over the drawn
    # rows' logits launched with a start/stop event pair of its own dispatch.
    # Outputs bit for bit as without it, and a positive duration.
    import ctypes
    B, K, V = 8, 4, 3001
    print(f"verify mass events B={B} K={K} V={V}", flush=True)
    r = np.random.default_rng(11)
    tau = np.full(B, 1.0, np.float32)
    logits = (1.5 * r.standard_normal((B, 2 * K + 1, V))).astype(np.float32)
    drafts = r.integers(0, V, size=(B, K)).astype(np.int32)
    target = logits[:, K:, :].argmax(-1).astype(np.int32)
    u = (r.integers(0, 1 << 24, size=(B, K)) * 2.0 ** -24).astype(np.float32)
    u[::2] = 0.0                              # every second sequence accepts all: a bonus draw
    lse = _softmax_lse(logits.astype(np.float64), 1.0).astype(np.float32)
    fkeys = np.arange(B, dtype=np.uint64) + np.uint64(1 << 35)
    hip = _hip_runtime()
    ev = (ctypes.c_void_p(), ctypes.c_void_p())
    assert hip.hipEventCreate(ctypes.byref(ev[0])) == 0 and hip.hipEventCreate(ctypes.byref(ev[1])) == 0
    outs = []
    for events in (None, (ev[0].value, ev[1].value)):
        acc = torch.empty(B, dtype=torch.int32, device="cuda")
        out = torch.empty(B, K + 1, dtype=torch.int32, device="cuda")
        n_out = torch.empty(B, dtype=torch.int32, device="cuda")
        dm.verify(B=B, K=K, V=V, t1=_t(drafts[:, 0], torch.int32), drafts=_t(drafts[:, 1:], torch.int32),
                  target=_t(target, torch.int32), accept_len=acc, out_tokens=out, n_out=n_out,
                  temperature=_t(tau, torch.float32),
                  logits=_t(logits.reshape(B * (2 * K + 1), V), torch.float32),
                  t1_lse=_t(lse[:, 0], torch.float32), draft_lse=_t(lse[:, 1:K], torch.float32),
                  target_lse=_t(lse[:, K:], torch.float32), u_acc=_t(u, torch.float32), seed=5,
                  final_key=_t(fkeys.view(np.int64), torch.int64), mass_events=events)
        torch.cuda.synchronize()
        outs.append([acc.cpu().numpy(), out.cpu().numpy(), n_out.cpu().numpy()])
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    hip.hipEventDestroy(ev[0])
    hip.hipEventDestroy(ev[1])
    print("  mass pass", 1000.0 * ms.value, "us; accepted", outs[0][0].tolist())
    assert ms.value > 0.0
    assert np.all(outs[0][0][::2] == K)       # the planted bonus draws ran
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


def test_verify_target_only_compares_with_the_picks(dm):
    """Target-only: every sequence, sampled or not, commits the matching prefix of
    its candidates and the target's pick at the first mismatch (or the bonus);
    nothing but the picks is read."""
    B, K, V = 40, 7, 1000
    r = np.random.default_rng(9)
    picks = r.integers(0, V, size=(B, K + 1)).astype(np.int32)
    drafts = r.integers(0, V, size=(B, K)).astype(np.int32)
    for b in range(B):
        k = b % (K + 1)
        drafts[b, :k] = picks[b, :k]
        if k < K and drafts[b, k] == picks[b, k]:
            drafts[b, k] = (picks[b, k] + 1) % V
    tau = np.where(np.arange(B) % 3 == 0, 0.0, 1.0).astype(np.float32)
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    n_out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    dm.verify(B=B, K=K, V=V, t1=_t(drafts[:, 0], torch.int32), drafts=_t(drafts[:, 1:], torch.int32),
              target=_t(picks, torch.int32), accept_len=acc, out_tokens=out, n_out=n_out,
              temperature=_t(tau, torch.float32), target_only=True)
    acc, out, n_out = acc.cpu().numpy(), out.cpu().numpy(), n_out.cpu().numpy()
    for b in range(B):
        L, toks = odm.verify_target_only(drafts[b], lambda i: picks[b, i])
        assert acc[b] == L == b % (K + 1)
        assert list(out[b, :L + 1]) == toks and n_out[b] == L + 1
        assert np.all(out[b, L + 1:] == -1)


# ------------------------------------------------------------- acceptance stats


def _stats_summary(st, K):
    return np.array([st["per_verify"], st["first_candidate"]] + list(st["cumulative"]) +
                    list(st["conditional"]), dtype=np.float64)


@pytest.mark.parametrize("K", [1, 7, 16, 64])
def test_accept_stats_match_the_oracle(dm, K):
    r = np.random.default_rng(K)
    hist = torch.zeros(K + 1, dtype=torch.int64, device="cuda")
    summ = torch.zeros(2 + 2 * K, dtype=torch.float64, device="cuda")
    seen = []
    for B in (1, 300, 4097, 0):
        # skewed lengths, plus out-of-range values that are not counted
        L = np.minimum(r.geometric(0.35, size=B) - 1, K).astype(np.int32)
        if B > 10:
            L[:3] = [-1, K + 1, 1 << 20]
        dm.accept_stats(_t(L, torch.int32) if B else torch.empty(0, dtype=torch.int32, device="cuda"),
                        K, hist, summ)
        seen.extend(int(x) for x in L if 0 <= x <= K)
        st = odm.acceptance_stats(np.array(seen, dtype=np.int64), K)
        assert hist.cpu().numpy().tolist() == st["hist"]
        got = summ.cpu().numpy()
        np.testing.assert_allclose(got, _stats_summary(st, K), rtol=1e-14, equal_nan=True)


def test_accept_stats_of_an_empty_histogram_are_nan(dm):
    K = 5
    hist = torch.zeros(K + 1, dtype=torch.int64, device="cuda")
    summ = torch.zeros(2 + 2 * K, dtype=torch.float64, device="cuda")
    dm.accept_stats(torch.empty(0, dtype=torch.int32, device="cuda"), K, hist, summ)
    assert np.all(hist.cpu().numpy() == 0) and np.all(np.isnan(summ.cpu().numpy()))


def test_verify_one_candidate(dm):
    """K = 1: the MTP candidate alone, greedy, sampled and target-only."""
    B, K, V = 12, 1, 500
    r = np.random.default_rng(21)
    tau = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
    logits = (1.5 * r.standard_normal((B, 2 * K + 1, V))).astype(np.float32)
    target = logits[:, K:, :].argmax(-1).astype(np.int32)
    t1 = r.integers(0, V, size=B).astype(np.int32)
    t1[::3] = target[::3, 0]                 # some accepted, some rejected
    u = (r.integers(0, 1 << 24, size=(B, K)) * 2.0 ** -24).astype(np.float32)
    tt = np.where(tau > 0, tau, 1.0).astype(np.float64)
    lse = _softmax_lse(logits.astype(np.float64), tt[:, None, None]).astype(np.float32)
    fkeys = np.arange(B, dtype=np.uint64) + np.uint64(5 << 32)
    seed = 5
    L64 = logits.astype(np.float64)
    for target_only in (False, True):
        acc = torch.empty(B, dtype=torch.int32, device="cuda")
        out = torch.empty(B, K + 1, dtype=torch.int32, device="cuda")
        n_out = torch.empty(B, dtype=torch.int32, device="cuda")
        dm.verify(B=B, K=K, V=V, t1=_t(t1, torch.int32), drafts=None, target=_t(target, torch.int32),
                  accept_len=acc, out_tokens=out, n_out=n_out, temperature=_t(tau, torch.float32),
                  logits=_t(logits.reshape(B * 3, V), torch.float32),
                  t1_lse=_t(lse[:, 0], torch.float32), draft_lse=None,
                  target_lse=_t(lse[:, K:], torch.float32), u_acc=_t(u, torch.float32), seed=seed,
                  final_key=_t(fkeys.view(np.int64), torch.int64), target_only=target_only)
        acc, out, n_out = acc.cpu().numpy(), out.cpu().numpy(), n_out.cpu().numpy()
        for b in range(B):
            if target_only or tau[b] == 0:
                L, toks = odm.verify_greedy([t1[b]], target[b])
                assert acc[b] == L and list(out[b, :L + 1]) == toks and n_out[b] == L + 1
                assert np.all(out[b, L + 1:] == -1)
                continue
            q = np.exp(L64[b, :K] / tau[b] - onm.logsumexp(L64[b, :K] / tau[b])[:, None])
            p = np.exp(L64[b, K:] / tau[b] - onm.logsumexp(L64[b, K:] / tau[b])[:, None])
            m = {}

            def accept(i, ratio):
                m["a"] = abs(np.log(u[b, i]) - np.log(ratio)) if u[b, i] > 0 else np.inf
                return bool(u[b, i] < ratio)

            def draw(i, w):
                with np.errstate(divide="ignore"):
                    j, mg = oph.grouped_gumbel_argmax(np.log(np.asarray(w)), seed, int(fkeys[b]))
                m["final"] = mg
                return j

            L, toks = odm.verify_rejection([t1[b]], p, q, accept, draw)
            if acc[b] != L:
                assert m["a"] < NEAR_TIE
                continue
            assert list(out[b, :L]) == toks[:L] and n_out[b] == L + 1
            assert out[b, L] == toks[L] or m["final"] < NEAR_TIE
