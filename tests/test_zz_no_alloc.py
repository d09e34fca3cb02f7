"""dmtp_fuse_noalloc: the fusion call without a caller workspace.

Its scratch is a static device array inside the library, shared by every
call on one GPU.  Two calls in a row -- the second with fewer rows and a
smaller hidden size, so it reuses a scratch the first left dirty -- must each
give bit for bit what dmtp_fuse gives with its own workspace, and match the
oracle to the fusion call's bar.  A call whose need exceeds the static buffer
is refused on the host before anything runs.
"""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import dmtp as odm  # noqa: E402

from tests._harness import max_rel  # noqa: E402


def _bf16(a):
    x = np.ascontiguousarray(a, dtype=np.float32).copy()
    x.view(np.uint32)[...] &= np.uint32(0xFFFF0000)
    return x


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def _case(dm, rows, H, seed, layout):
    r = np.random.default_rng(seed)
    V = 300
    emb = _bf16(0.02 * r.standard_normal((V, H)))
    W = _bf16(0.02 * r.standard_normal((H, 2 * H)))
    g1 = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    g2 = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    ids = r.integers(0, V, size=rows).astype(np.int32)
    E, I = _t(emb, torch.bfloat16), _t(ids, torch.int32)
    keep = {}
    if layout == "mtp":          # x1 = hidden rows (bf16), x2 = ids, no residual
        x1 = _bf16(r.standard_normal((rows, H)))
        keep["x1"] = _t(x1, torch.bfloat16)
        kw = dict(x1=keep["x1"], x2_ids=I, table=E)
        want = odm.fuse(x1, emb[ids], g1, g2, W, 1e-6)
    else:                        # x1 = ids, x2 = float32 rows, residual = ids
        x2 = r.standard_normal((rows, H)).astype(np.float32)
        keep["x2"] = _t(x2, torch.float32)
        kw = dict(x1_ids=I, x2=keep["x2"], res_ids=I, table=E)
        want = odm.fuse(emb[ids], x2, g1, g2, W, 1e-6, res=emb[ids])
    Wt, G1, G2 = _t(W, torch.bfloat16), _t(g1, torch.float32), _t(g2, torch.float32)
    ref = torch.empty(rows, H, dtype=torch.float32, device="cuda")
    dm.fuse(ref, Wt, G1, G2, eps=1e-6, **kw)
    out = torch.full((rows, H), float("nan"), dtype=torch.float32, device="cuda")
    d = dm.fuse(out, Wt, G1, G2, eps=1e-6, run=False, **kw)
    keep.update(W=Wt, G1=G1, G2=G2, E=E, I=I)
    return d, out, ref, want, keep


@pytest.fixture(scope="module")
def dm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mtp_block_draft_amd as m
    return m


@pytest.mark.parametrize("first,second", [
    ((32, 2048, "mtp"), (7, 1024, "residual")),     # the folded-norm projection twice
    ((128, 2048, "residual"), (32, 2048, "mtp")),   # the prologue path, then the folded one
])
def test_noalloc_matches_fuse_on_two_calls(dm, first, second):
    for i, (rows, H, layout) in enumerate((first, second)):
        print(f"noalloc call {i}: rows={rows} H={H} layout={layout}", flush=True)
        d, out, ref, want, keep = _case(dm, rows, H, 11 + 7 * i + rows, layout)
        assert dm.lib.dmtp_fuse_ws(ctypes.byref(d)) <= (16 << 20)
        dm.fuse_noalloc(d)
        torch.cuda.synchronize()
        got, exp = out.cpu().numpy(), ref.cpu().numpy()
        np.testing.assert_array_equal(got, exp)
        err = max_rel(got, want)
        print("  max rel vs oracle", err)
        assert err < 1e-5


def test_noalloc_refuses_a_call_beyond_the_scratch(dm):
    rows, H = 32, 16384        # 2 MB x 32 splits of partials: far above 16 MiB
    out = torch.empty(rows, H, dtype=torch.float32, device="cuda")
    W = torch.zeros(H, 2 * H, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(H, dtype=torch.float32, device="cuda")
    x = torch.zeros(rows, H, dtype=torch.bfloat16, device="cuda")
    d = dm.fuse(out, W, g, g, x1=x, x2=x, run=False)
    assert dm.lib.dmtp_fuse_ws(ctypes.byref(d)) > (16 << 20)
    assert dm.lib.dmtp_fuse_noalloc(ctypes.byref(d), None) == -9
