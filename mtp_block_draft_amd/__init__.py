"""DMTP speculative-decoding round on MI355X: Python binding of libdmtp.so.

The four calls of include/dmtp.h with the same names, taking torch tensors
that live on the GPU.  This layer only marshals arguments (pointers, sizes,
the current HIP stream); every step of the round runs in the library's HIP
kernels.  Importing fails when the library is not built: there is no other
implementation to fall back on.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _abi
from ._abi import (DMTP_BF16, DMTP_F32, DMTP_NO_DRAW, DmtpError, DraftDesc, FuseDesc, HeadDesc,
                   CtxDesc, HeadSegment, Layer, MtpDesc, Rows, StatsDesc, VerifyDesc)

lib = _abi.load()

__all__ = ["lib", "fuse", "fuse_noalloc", "mtp_block", "ctx_kv", "block_draft", "lm_head", "pack_head_weight", "verify",
           "accept_stats", "call",
           "workspace_bytes",
           "DMTP_F32", "DMTP_BF16", "DMTP_NO_DRAW", "DmtpError", "version"]


def version() -> str:
    return lib.dmtp_version().decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("DMTP tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("DMTP tensors must be contiguous")
    return t.data_ptr()


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return DMTP_BF16
    if t == torch.float32:
        return DMTP_F32
    raise ValueError(f"unsupported dtype {t}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(name: str, desc) -> int:
    return int(getattr(lib, f"dmtp_{name}_ws")(ctypes.byref(desc)))


def call(name: str, desc, ws: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> None:
    """Run dmtp_<name> on a prepared descriptor; allocates the workspace if none is given."""
    need = workspace_bytes(name, desc)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    st = getattr(lib, f"dmtp_{name}")(ctypes.byref(desc), ctypes.c_void_p(ws.data_ptr()),
                                      ws.numel() * ws.element_size(),
                                      ctypes.c_void_p(_stream() if stream is None else stream))
    if st != 0:
        raise DmtpError(f"dmtp_{name}", st, lib.dmtp_status_str(st).decode())


def rows_arg(rows: Optional[torch.Tensor] = None, ids: Optional[torch.Tensor] = None,
             table: Optional[torch.Tensor] = None) -> Rows:
    r = Rows()
    if rows is not None:
        r.rows = _ptr(rows)
        r.dtype = dtype_code(rows.dtype)
    elif ids is not None:
        if ids.dtype != torch.int32:
            raise ValueError("ids must be int32")
        r.ids = _ptr(ids)
        r.table = _ptr(table)
        r.table_rows = table.shape[0]
    return r


def fuse(out: torch.Tensor, W: torch.Tensor, g1: torch.Tensor, g2: torch.Tensor, *,
         x1: Optional[torch.Tensor] = None, x1_ids: Optional[torch.Tensor] = None,
         x2: Optional[torch.Tensor] = None, x2_ids: Optional[torch.Tensor] = None,
         res: Optional[torch.Tensor] = None, res_ids: Optional[torch.Tensor] = None,
         table: Optional[torch.Tensor] = None, eps: float = 1e-6,
         ws: Optional[torch.Tensor] = None, run: bool = True) -> FuseDesc:
    """out = res + W [RMSNorm(x1; g1); RMSNorm(x2; g2)] (dmtp_fuse)."""
    d = FuseDesc()
    d.rows, d.H = out.shape
    d.w_dtype = dtype_code(W.dtype)
    d.eps = eps
    d.x1 = rows_arg(x1, x1_ids, table)
    d.x2 = rows_arg(x2, x2_ids, table)
    d.res = rows_arg(res, res_ids, table)
    d.g1, d.g2, d.W, d.out = _ptr(g1), _ptr(g2), _ptr(W), _ptr(out)
    if run:
        call("fuse", d, ws)
    return d


def fuse_noalloc(desc: FuseDesc, stream: Optional[int] = None) -> None:
    """dmtp_fuse_noalloc on a prepared fuse descriptor (no workspace: the
    library's static scratch)."""
    st = lib.dmtp_fuse_noalloc(ctypes.byref(desc),
                               ctypes.c_void_p(_stream() if stream is None else stream))
    if st != 0:
        raise DmtpError("dmtp_fuse_noalloc", st, lib.dmtp_status_str(st).decode())


def layer_arg(g_attn, wqkv, wo, g_ffn, wg, wu, wd, ctx_k, ctx_v) -> Layer:
    L = Layer()
    L._keep = (g_attn, wqkv, wo, g_ffn, wg, wu, wd, ctx_k, ctx_v)
    L.g_attn, L.wqkv, L.wo, L.g_ffn = _ptr(g_attn), _ptr(wqkv), _ptr(wo), _ptr(g_ffn)
    L.wg, L.wu, L.wd = _ptr(wg), _ptr(wu), _ptr(wd)
    L.ctx_k, L.ctx_v = _ptr(ctx_k), _ptr(ctx_v)
    return L


def block_draft(out: torch.Tensor, *, B: int, H: int, Hq: int, Hkv: int, d: int, F: int, K: int,
                n_anchor: int, layers: Sequence[Layer], anchor_ids: Optional[torch.Tensor],
                x_t1: torch.Tensor, mask_id: int, emb: torch.Tensor, cu_ctx: torch.Tensor,
                max_ctx: int, ctx_rows: int, g_final: torch.Tensor, eps: float = 1e-6,
                rope_base: float = 1e6, window: int = 0, ws: Optional[torch.Tensor] = None,
                run: bool = True, attn_events: Optional[Tuple[int, int]] = None) -> DraftDesc:
    """Block drafter layers + final norm of the MASK slots (dmtp_block_draft).

    attn_events: optional (start, stop) hipEvent_t handles that time the
    first layer's context-attention kernel from its own dispatch."""
    D = DraftDesc()
    D.B, D.H, D.Hq, D.Hkv, D.d, D.F = B, H, Hq, Hkv, d, F
    D.n_layers, D.K, D.n_anchor = len(layers), K, n_anchor
    D.dtype = dtype_code(emb.dtype)
    D.eps, D.rope_base, D.window, D.max_ctx, D.ctx_rows = eps, rope_base, window, max_ctx, ctx_rows
    D.V = emb.shape[0]
    arr = (Layer * len(layers))(*layers)
    D.layers = ctypes.cast(arr, ctypes.POINTER(Layer))
    D._layers_keepalive = arr
    D.anchor_ids = _ptr(anchor_ids)
    D.x_t1, D.mask_id, D.emb, D.cu_ctx = _ptr(x_t1), mask_id, _ptr(emb), _ptr(cu_ctx)
    D.g_final, D.out = _ptr(g_final), _ptr(out)
    if attn_events is not None:
        D.attn_start_event, D.attn_stop_event = attn_events
    if run:
        call("block_draft", D, ws)
    return D


def mtp_block(out: torch.Tensor, x: torch.Tensor, *, Hq: int, Hkv: int, d: int, F: int,
              layers: Sequence[Layer], cu_ctx: torch.Tensor, max_ctx: int, ctx_rows: int,
              dtype: int, k_new: Optional[Sequence[torch.Tensor]] = None,
              v_new: Optional[Sequence[torch.Tensor]] = None, eps: float = 1e-6,
              rope_base: float = 1e6, ws: Optional[torch.Tensor] = None,
              run: bool = True) -> MtpDesc:
    """The MTP decoder block over x [B, S, H] float32 (dmtp_mtp_block)."""
    D = MtpDesc()
    D.B, D.S, D.H = x.shape
    D.Hq, D.Hkv, D.d, D.F, D.n_layers, D.dtype = Hq, Hkv, d, F, len(layers), dtype
    D.eps, D.rope_base, D.max_ctx, D.ctx_rows = eps, rope_base, max_ctx, ctx_rows
    arr = (Layer * len(layers))(*layers)
    D.layers = ctypes.cast(arr, ctypes.POINTER(Layer))
    keep = [arr, x, out, cu_ctx]
    D.x, D.cu_ctx, D.out = _ptr(x), _ptr(cu_ctx), _ptr(out)
    for name, ts in (("k_new", k_new), ("v_new", v_new)):
        if ts is not None:
            ptrs = (ctypes.c_void_p * len(layers))(*[_ptr(t) for t in ts])
            setattr(D, name, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)))
            keep += [ptrs, list(ts)]
    D._keep = keep
    if run:
        call("mtp_block", D, ws)
    return D


def ctx_kv(feats: torch.Tensor, positions: torch.Tensor, dst_rows: torch.Tensor,
           w_fc: torch.Tensor, *, Hq: int, Hkv: int, d: int, layers: Sequence[Layer],
           k_cache: Sequence[torch.Tensor], v_cache: Sequence[torch.Tensor],
           ctx_out: Optional[torch.Tensor] = None, eps: float = 1e-6, rope_base: float = 1e6,
           ws: Optional[torch.Tensor] = None, run: bool = True) -> CtxDesc:
    """Drafter context K/V rows from target features [N, n_feat, H] (dmtp_ctx_kv)."""
    if positions.dtype != torch.int32 or dst_rows.dtype != torch.int32:
        raise ValueError("positions and dst_rows must be int32")
    D = CtxDesc()
    D.N, D.n_feat, D.H = feats.shape
    D.Hq, D.Hkv, D.d, D.n_layers = Hq, Hkv, d, len(layers)
    D.dtype = dtype_code(feats.dtype)
    D.eps, D.rope_base = eps, rope_base
    D.feats, D.positions, D.dst_rows, D.w_fc = _ptr(feats), _ptr(positions), _ptr(dst_rows), _ptr(w_fc)
    arr = (Layer * len(layers))(*layers)
    D.layers = ctypes.cast(arr, ctypes.POINTER(Layer))
    D.ctx_rows = k_cache[0].shape[0]
    kp = (ctypes.c_void_p * len(layers))(*[_ptr(t) for t in k_cache])
    vp = (ctypes.c_void_p * len(layers))(*[_ptr(t) for t in v_cache])
    D.k_cache = ctypes.cast(kp, ctypes.POINTER(ctypes.c_void_p))
    D.v_cache = ctypes.cast(vp, ctypes.POINTER(ctypes.c_void_p))
    D.ctx_out = _ptr(ctx_out)
    D._keep = (arr, kp, vp, feats, positions, dst_rows, w_fc, list(k_cache), list(v_cache), ctx_out)
    if run:
        call("ctx_kv", D, ws)
    return D


def head_segment(x: torch.Tensor, g_norm: Optional[torch.Tensor] = None, n: Optional[int] = None,
                 ld: Optional[int] = None) -> HeadSegment:
    s = HeadSegment()
    s._keep = (x, g_norm)   # the struct holds raw pointers: keep the tensors alive with it
    s.x = _ptr(x)
    s.n = x.shape[0] if n is None else n
    s.ld = x.shape[-1] if ld is None else ld
    s.dtype = dtype_code(x.dtype)
    s.g_norm = _ptr(g_norm)
    return s


def lm_head(W: torch.Tensor, segments: Sequence[HeadSegment], token: torch.Tensor, *,
            eps: float = 1e-6, temperature: Optional[torch.Tensor] = None,
            draw_key: Optional[torch.Tensor] = None, seed: int = 0,
            plant_row: Optional[torch.Tensor] = None, store_row: Optional[torch.Tensor] = None,
            logits: Optional[torch.Tensor] = None, prepared: Optional[torch.Tensor] = None,
            row_max: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            gap: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
            w_packed: Optional[torch.Tensor] = None, run: bool = True) -> HeadDesc:
    """Shared LM head with argmax / Gumbel-max draws (dmtp_lm_head).  w_packed:
    W's packed copy from pack_head_weight, streamed by the matrix-core GEMM."""
    D = HeadDesc()
    D.V, D.H = W.shape
    D.dtype = dtype_code(W.dtype)
    D.eps = eps
    D.n_seg = len(segments)
    D._keep = list(segments)
    for i, s in enumerate(segments):
        D.seg[i] = s
    D.W = _ptr(W)
    D.temperature, D.draw_key, D.seed = _ptr(temperature), _ptr(draw_key), seed
    D.plant_row, D.store_row, D.logits = _ptr(plant_row), _ptr(store_row), _ptr(logits)
    D.logits_rows = logits.shape[0] if logits is not None else 0
    D.prepared, D.token = _ptr(prepared), _ptr(token)
    D.row_max, D.lse, D.gap = _ptr(row_max), _ptr(lse), _ptr(gap)
    D.w_packed = _ptr(w_packed)
    if w_packed is not None:
        D._keep.append(w_packed)
    if run:
        call("lm_head", D, ws)
    return D


def pack_head_weight(W: torch.Tensor) -> torch.Tensor:
    """W [V, H] bf16 copied once into the layout the LM-head GEMM streams
    (dmtp_head_pack); pass the result to lm_head as w_packed."""
    if W.dtype != torch.bfloat16 or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("pack_head_weight takes a contiguous bf16 [V, H] matrix")
    V, H = W.shape
    n = lib.dmtp_head_pack_bytes(V, H)
    if n == 0:
        raise ValueError(f"unsupported head shape V={V}, H={H}")
    out = torch.empty(n // 2, dtype=torch.bfloat16, device=W.device)
    st = lib.dmtp_head_pack(ctypes.c_void_p(W.data_ptr()), V, H, DMTP_BF16,
                            ctypes.c_void_p(out.data_ptr()), n, ctypes.c_void_p(_stream()))
    if st != 0:
        raise DmtpError("dmtp_head_pack", st, lib.dmtp_status_str(st).decode())
    return out


def verify(*, B: int, K: int, V: int, t1: torch.Tensor, drafts: Optional[torch.Tensor],
           target: torch.Tensor, accept_len: torch.Tensor, out_tokens: torch.Tensor,
           n_out: torch.Tensor, temperature: Optional[torch.Tensor] = None,
           logits: Optional[torch.Tensor] = None, t1_lse: Optional[torch.Tensor] = None,
           draft_lse: Optional[torch.Tensor] = None, target_lse: Optional[torch.Tensor] = None,
           u_acc: Optional[torch.Tensor] = None, seed: int = 0,
           final_key: Optional[torch.Tensor] = None, target_only: bool = False,
           ws: Optional[torch.Tensor] = None, run: bool = True,
           mass_events: Optional[Tuple[int, int]] = None) -> VerifyDesc:
    """Greedy, rejection-sampling or target-only block verification (dmtp_verify).

    mass_events: optional (start, stop) hipEvent_t handles that time the pass
    over the drawn rows' logits from its own dispatch."""
    D = VerifyDesc()
    D.B, D.K, D.V = B, K, V
    D.t1, D.drafts, D.target = _ptr(t1), _ptr(drafts), _ptr(target)
    D.temperature, D.logits = _ptr(temperature), _ptr(logits)
    D.t1_lse, D.draft_lse, D.target_lse = _ptr(t1_lse), _ptr(draft_lse), _ptr(target_lse)
    D.u_acc, D.seed, D.final_key = _ptr(u_acc), seed, _ptr(final_key)
    D.accept_len, D.out_tokens, D.n_out = _ptr(accept_len), _ptr(out_tokens), _ptr(n_out)
    D.target_only = 1 if target_only else 0
    if mass_events is not None:
        D.mass_start_event, D.mass_stop_event = mass_events
    if run:
        call("verify", D, ws)
    return D


def accept_stats(accept_len: torch.Tensor, K: int, hist: torch.Tensor,
                 summary: Optional[torch.Tensor] = None, run: bool = True) -> StatsDesc:
    """Add accept_len's histogram to hist (int64 [K+1]); summary float64 [2+2K] (dmtp_accept_stats)."""
    if accept_len.dtype != torch.int32 or hist.dtype != torch.int64:
        raise ValueError("accept_len must be int32 and hist int64")
    if summary is not None and summary.dtype != torch.float64:
        raise ValueError("summary must be float64")
    D = StatsDesc()
    D.B, D.K = accept_len.numel(), K
    D.accept_len, D.hist, D.summary = _ptr(accept_len), _ptr(hist), _ptr(summary)
    D._keep = (accept_len, hist, summary)
    if run:
        st = lib.dmtp_accept_stats(ctypes.byref(D), ctypes.c_void_p(_stream()))
        if st != 0:
            raise DmtpError("dmtp_accept_stats", st, lib.dmtp_status_str(st).decode())
    return D
