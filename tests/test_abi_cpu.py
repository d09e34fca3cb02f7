"""The C-ABI library without a GPU: it loads, exports what include/dmtp.h
declares, its structs match the binding, and bad arguments are refused on
the host before anything is enqueued."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmtp.h")

abi = pytest.importorskip("mtp_block_draft_amd._abi")


@pytest.fixture(scope="module")
def lib():
    # DMTP_ABI_TEST_LIB: another build of the library to run these checks on
    # (the host-sanitized one; see test_abi_sanitized.py)
    path = os.environ.get("DMTP_ABI_TEST_LIB")
    return abi.load(path) if path else abi.load()


def test_exports_every_declared_function(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dmtp_[a-z_0-9]+)\s*\(", text, re.M))
    assert {"dmtp_fuse", "dmtp_block_draft", "dmtp_lm_head", "dmtp_verify"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(abi.SYMBOLS) == declared


def test_struct_sizes_and_version(lib):
    for i, st in enumerate(abi._STRUCTS):
        assert lib.dmtp_struct_size(i) == ctypes.sizeof(st)
    assert b"gfx950" in lib.dmtp_version()
    for code in abi.STATUS:
        assert lib.dmtp_status_str(code)


FAKE = 1 << 20   # aligned, never dereferenced: every call below fails validation first


def _fuse_desc(**over):
    d = abi.FuseDesc()
    d.rows, d.H, d.w_dtype, d.eps = 4, 256, abi.DMTP_BF16, 1e-6
    d.x1.rows, d.x1.dtype = FAKE, abi.DMTP_BF16
    d.x2.ids, d.x2.table, d.x2.table_rows = FAKE, FAKE, 100
    d.g1 = d.g2 = d.W = d.out = FAKE
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _call(lib, name, desc, ws_bytes=0):
    f = getattr(lib, name)
    return f(ctypes.byref(desc), ctypes.c_void_p(FAKE if ws_bytes else 0), ws_bytes, None)


def test_fuse_argument_errors(lib):
    assert lib.dmtp_fuse(None, None, 0, None) == -1
    assert _call(lib, "dmtp_fuse", _fuse_desc(H=100)) == -2          # not a multiple of 64
    assert _call(lib, "dmtp_fuse", _fuse_desc(rows=0)) == -2
    assert _call(lib, "dmtp_fuse", _fuse_desc(w_dtype=7)) == -3
    assert _call(lib, "dmtp_fuse", _fuse_desc(W=FAKE + 4)) == -5     # misaligned
    assert _call(lib, "dmtp_fuse", _fuse_desc(g1=None)) == -1
    d = _fuse_desc()
    d.x1.ids = FAKE                                                   # rows and ids both set
    assert _call(lib, "dmtp_fuse", d) == -8
    d = _fuse_desc()
    need = lib.dmtp_fuse_ws(ctypes.byref(d))
    assert need > 0
    assert _call(lib, "dmtp_fuse", d, ws_bytes=need - 1) == -4


def test_fuse_noalloc_refuses_a_call_beyond_its_static_scratch(lib):
    # 32 rows of H = 16384 need about 138 MB of partials; the static array is 16 MiB.
    d = _fuse_desc(rows=32, H=16384)
    assert lib.dmtp_fuse_ws(ctypes.byref(d)) > (16 << 20)
    assert lib.dmtp_fuse_noalloc(ctypes.byref(d), None) == -9
    assert b"scratch" in lib.dmtp_status_str(-9)
    # argument errors come first, as in dmtp_fuse
    assert lib.dmtp_fuse_noalloc(None, None) == -1
    assert lib.dmtp_fuse_noalloc(ctypes.byref(_fuse_desc(H=100)), None) == -2


def _draft_desc(layers, **over):
    d = abi.DraftDesc()
    d.B, d.H, d.Hq, d.Hkv, d.d, d.F, d.n_layers, d.K, d.n_anchor = 2, 256, 4, 4, 64, 512, 1, 7, 2
    d.dtype, d.eps, d.rope_base, d.window, d.max_ctx, d.ctx_rows, d.V = 0, 1e-6, 1e6, 0, 128, 256, 1024
    d.anchor_ids = d.x_t1 = d.emb = d.cu_ctx = d.g_final = d.out = FAKE
    d.mask_id = 1023
    d.layers = ctypes.cast(layers, ctypes.POINTER(abi.Layer))
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_block_draft_argument_errors(lib):
    L = abi.Layer(*([FAKE] * 9))
    arr = (abi.Layer * 1)(L)
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, d=96)) == -2       # head dim
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, Hq=6, Hkv=4)) == -2
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, K=1)) == -2
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, K=40)) == -2
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, n_anchor=3)) == -2
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, mask_id=1024)) == -2
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, anchor_ids=None)) == -1
    # too many query rows per kv head for one workgroup (S * G)
    assert _call(lib, "dmtp_block_draft", _draft_desc(arr, Hq=64, Hkv=1, d=128, K=16)) == -2
    bad = (abi.Layer * 1)(abi.Layer(*([FAKE] * 6 + [None] + [FAKE] * 2)))
    assert _call(lib, "dmtp_block_draft", _draft_desc(bad)) == -1
    d = _draft_desc(arr)
    need = lib.dmtp_block_draft_ws(ctypes.byref(d))
    assert need > 0 and _call(lib, "dmtp_block_draft", d, ws_bytes=need - 1) == -4


def _head_desc(**over):
    d = abi.HeadDesc()
    d.H, d.V, d.dtype, d.eps, d.n_seg = 256, 1000, abi.DMTP_BF16, 1e-6, 1
    d.seg[0].x, d.seg[0].n, d.seg[0].ld, d.seg[0].dtype = FAKE, 5, 256, abi.DMTP_BF16
    d.W = d.token = FAKE
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_lm_head_argument_errors(lib):
    assert _call(lib, "dmtp_lm_head", _head_desc(n_seg=0)) == -2
    assert _call(lib, "dmtp_lm_head", _head_desc(n_seg=5)) == -2
    assert _call(lib, "dmtp_lm_head", _head_desc(V=1)) == -2
    d = _head_desc()
    d.seg[0].g_norm = FAKE            # a normalised segment must be float32 hidden rows
    assert _call(lib, "dmtp_lm_head", d) == -3
    d = _head_desc()
    d.seg[0].ld = 100                 # row stride below H
    assert _call(lib, "dmtp_lm_head", d) == -2
    d = _head_desc(temperature=FAKE)  # sampling needs draw keys and stored logits
    assert _call(lib, "dmtp_lm_head", d) == -1
    d = _head_desc(store_row=FAKE)    # storing needs a logits buffer
    assert _call(lib, "dmtp_lm_head", d) == -1
    d = _head_desc()
    need = lib.dmtp_lm_head_ws(ctypes.byref(d))
    assert need > 0 and _call(lib, "dmtp_lm_head", d, ws_bytes=need - 1) == -4


def test_head_pack_argument_errors(lib):
    # size: ceil(V / 128) tiles of 128 rows x H bf16
    assert lib.dmtp_head_pack_bytes(151936, 2048) == 1187 * 128 * 2048 * 2
    assert lib.dmtp_head_pack_bytes(7001, 512) == 55 * 128 * 512 * 2
    assert lib.dmtp_head_pack_bytes(1, 512) == 0 and lib.dmtp_head_pack_bytes(300, 96) == 0
    n = lib.dmtp_head_pack_bytes(300, 128)
    ok = dict(W=FAKE, V=300, H=128, dtype=abi.DMTP_BF16, out=FAKE, nb=n)

    def pack(**kw):
        a = {**ok, **kw}
        return lib.dmtp_head_pack(a["W"], a["V"], a["H"], a["dtype"], a["out"], a["nb"], None)

    assert pack(W=0) == -1 and pack(out=0) == -1
    assert pack(H=96) == -2 and pack(V=1) == -2
    assert pack(dtype=abi.DMTP_F32) == -3
    assert pack(out=FAKE + 8) == -5 and pack(W=FAKE + 8) == -5
    assert pack(nb=n - 1) == -4
    assert pack() == -6               # valid, but no gfx950 here
    # the head call: a packed copy is bf16 only and 16-byte aligned
    assert _call(lib, "dmtp_lm_head", _head_desc(w_packed=FAKE + 8)) == -5
    d = _head_desc(w_packed=FAKE, dtype=abi.DMTP_F32)
    d.seg[0].dtype = abi.DMTP_F32
    assert _call(lib, "dmtp_lm_head", d) == -3


def test_verify_argument_errors(lib):
    d = abi.VerifyDesc()
    d.B, d.K, d.V = 3, 7, 1000
    d.t1 = d.drafts = d.target = d.accept_len = d.out_tokens = d.n_out = FAKE
    assert _call(lib, "dmtp_verify", abi.VerifyDesc()) == -2
    d.temperature = FAKE              # sampled verification needs its logits and uniforms
    assert _call(lib, "dmtp_verify", d) == -1
    d.temperature = None
    d.drafts = None
    assert _call(lib, "dmtp_verify", d) == -1
    d.drafts = FAKE
    need = lib.dmtp_verify_ws(ctypes.byref(d))
    assert need > 0 and _call(lib, "dmtp_verify", d, ws_bytes=need - 1) == -4
    d.target_only = 2                 # a flag: 0 or 1
    assert _call(lib, "dmtp_verify", d, ws_bytes=need) == -8


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_target_only_verify_needs_no_logits(lib):
    """Target-only verification reads only the picks: with temperatures but no
    logits, lse or uniforms it passes validation and reaches the device check."""
    d = abi.VerifyDesc()
    d.B, d.K, d.V = 3, 7, 1000
    d.t1 = d.drafts = d.target = d.accept_len = d.out_tokens = d.n_out = FAKE
    d.temperature = FAKE
    d.target_only = 1
    need = lib.dmtp_verify_ws(ctypes.byref(d))
    assert need > 0 and _call(lib, "dmtp_verify", d, ws_bytes=need) == -6


def test_accept_stats_argument_errors(lib):
    def st(**over):
        d = abi.StatsDesc()
        d.B, d.K, d.accept_len, d.hist, d.summary = 10, 7, FAKE, FAKE, FAKE
        for k, v in over.items():
            setattr(d, k, v)
        return lib.dmtp_accept_stats(ctypes.byref(d), None)

    assert lib.dmtp_accept_stats(None, None) == -1
    assert st(K=0) == -2
    assert st(K=65) == -2
    assert st(B=-1) == -2
    assert st(hist=None) == -1
    assert st(accept_len=None) == -1
    assert st(hist=FAKE + 4) == -5
    if torch.cuda.device_count() == 0:
        assert st(B=0, accept_len=None) == -6      # valid: only the device check is left
        assert st(summary=None) == -6


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_valid_call_without_gfx950_is_refused(lib):
    d = _fuse_desc()
    need = lib.dmtp_fuse_ws(ctypes.byref(d))
    assert _call(lib, "dmtp_fuse", d, ws_bytes=need) == -6


def test_binding_refuses_to_load_a_missing_library(tmp_path):
    with pytest.raises(ImportError):
        abi.load(str(tmp_path / "libdmtp.so"))


def test_mtp_block_argument_errors(lib):
    L = abi.Layer(*([FAKE] * 9))
    arr = (abi.Layer * 1)(L)

    def desc(**over):
        d = abi.MtpDesc()
        d.B, d.S, d.H, d.Hq, d.Hkv, d.d, d.F, d.n_layers, d.dtype = 4, 1, 256, 4, 2, 64, 512, 1, 1
        d.eps, d.rope_base, d.max_ctx, d.ctx_rows = 1e-6, 1e6, 100, 300
        d.x = d.cu_ctx = d.out = FAKE
        d.layers = ctypes.cast(arr, ctypes.POINTER(abi.Layer))
        for k, v in over.items():
            setattr(d, k, v)
        return d

    assert lib.dmtp_mtp_block(None, None, 0, None) == -1
    assert _call(lib, "dmtp_mtp_block", desc(S=0)) == -2
    assert _call(lib, "dmtp_mtp_block", desc(d=96)) == -2
    assert _call(lib, "dmtp_mtp_block", desc(Hq=6, Hkv=4)) == -2
    assert _call(lib, "dmtp_mtp_block", desc(dtype=5)) == -3
    assert _call(lib, "dmtp_mtp_block", desc(x=None)) == -1
    assert _call(lib, "dmtp_mtp_block", desc(out=FAKE + 8)) == -5
    bad = (abi.Layer * 1)(abi.Layer(*([FAKE] * 7 + [None, FAKE])))   # cache keys missing
    assert _call(lib, "dmtp_mtp_block", desc(layers=ctypes.cast(bad, ctypes.POINTER(abi.Layer)))) == -1
    mis = (ctypes.c_void_p * 1)(FAKE + 4)                              # misaligned K/V output
    assert _call(lib, "dmtp_mtp_block", desc(k_new=ctypes.cast(mis, ctypes.POINTER(ctypes.c_void_p)))) == -5
    d = desc()
    need = lib.dmtp_mtp_block_ws(ctypes.byref(d))
    assert need > 0 and _call(lib, "dmtp_mtp_block", d, ws_bytes=need - 1) == -4
    if torch.cuda.device_count() == 0:
        assert _call(lib, "dmtp_mtp_block", d, ws_bytes=need) == -6


def test_ctx_kv_argument_errors(lib):
    L = abi.Layer(*([FAKE] * 9))
    arr = (abi.Layer * 1)(L)
    caches = (ctypes.c_void_p * 1)(FAKE)

    def desc(**over):
        d = abi.CtxDesc()
        d.N, d.n_feat, d.H, d.Hq, d.Hkv, d.d, d.n_layers, d.dtype = 10, 5, 256, 4, 2, 64, 1, 1
        d.eps, d.rope_base, d.ctx_rows = 1e-6, 1e6, 100
        d.feats = d.positions = d.dst_rows = d.w_fc = FAKE
        d.layers = ctypes.cast(arr, ctypes.POINTER(abi.Layer))
        d.k_cache = ctypes.cast(caches, ctypes.POINTER(ctypes.c_void_p))
        d.v_cache = ctypes.cast(caches, ctypes.POINTER(ctypes.c_void_p))
        for k, v in over.items():
            setattr(d, k, v)
        return d

    assert lib.dmtp_ctx_kv(None, None, 0, None) == -1
    assert _call(lib, "dmtp_ctx_kv", desc(N=0)) == -2
    assert _call(lib, "dmtp_ctx_kv", desc(n_feat=9)) == -2
    assert _call(lib, "dmtp_ctx_kv", desc(H=100)) == -2
    assert _call(lib, "dmtp_ctx_kv", desc(dtype=3)) == -3
    assert _call(lib, "dmtp_ctx_kv", desc(dst_rows=None)) == -1
    assert _call(lib, "dmtp_ctx_kv", desc(k_cache=None)) == -1
    assert _call(lib, "dmtp_ctx_kv", desc(w_fc=FAKE + 2)) == -5
    d = desc()
    need = lib.dmtp_ctx_kv_ws(ctypes.byref(d))
    assert need > 0 and _call(lib, "dmtp_ctx_kv", d, ws_bytes=need - 1) == -4
    if torch.cuda.device_count() == 0:
        assert _call(lib, "dmtp_ctx_kv", d, ws_bytes=need) == -6
