"""One DMTP round on the GPU as a sequence of the four ABI calls.

Round(inputs) uploads the seeded inputs once, allocates every output and one
shared workspace, and prebuilds the call descriptors; run() then enqueues,
on the current stream:

  1. dmtp_fuse        h' = M [RMSNorm(h); RMSNorm(E(A))]             (MTP fusion)
     dmtp_mtp_block   h_MTP = the MTP decoder block over h' (workloads with
                      one; it also returns the K/V rows its cache appends),
                      else h_MTP = h'
  2. dmtp_lm_head     T1 from RMSNorm(h_MTP; g_f)                       (MTP candidate)
  3. dmtp_fuse        x_T1 = E(T1) + W [RMS_e(E(T1)); RMS_m(h_MTP)]     (DMTP residual)
  4. dmtp_block_draft MASK-slot rows of the drafter                    (block draft)
  5. dmtp_lm_head     candidates 1..K-1 and the K+1 target rows         (shared head)
  6. dmtp_verify      accepted prefix + correction/bonus                (verification)

Buffer layout (row-major, device): the LM-head input of step 5 is one
[B (K-1) + B (K+1), H] buffer in the head dtype -- the drafter writes its
MASK rows into the first B (K-1) rows and the target rows sit after them --
so step 5 reads one contiguous matrix.  Sampled sequences keep their float32
logits rows in a [B, 2K+1, V] buffer: candidate rows 0..K-1, target rows
K..2K.  The planted workload (T1 set to the target argmax) adds the B target
rows of position 0 to step 2 as a second, strided segment.

Verification follows the configuration: "rejection" (greedy at temperature 0,
rejection sampling above it) or "target_only", where step 5 draws the
target's own pick at each target row of a sampled sequence (its draw keys)
and step 6 compares the candidates with those picks.  accept_stats() adds
the round's accepted lengths to a running histogram on the device.

capture() records the six calls once into a HIP graph (through torch's graph
capture of the stream they are enqueued on); replay() then submits the whole
round -- T1 head, candidate write, embedding gather, residual, drafter, head
and verification -- as one launch.  The calls allocate nothing and record no
memset, so the captured round reads and writes the same buffers as run().
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np
import torch

from . import (DMTP_NO_DRAW, accept_stats, block_draft, call, fuse, head_segment, layer_arg, lib,
               lm_head, mtp_block, pack_head_weight, verify, workspace_bytes)


def _dev(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


class Round:
    def __init__(self, inp, h_target: Optional[np.ndarray] = None, device: str = "cuda",
                 pack_head: bool = True):
        cfg = inp.cfg
        self.cfg = cfg
        B, H, V, K = cfg.B, cfg.H, cfg.V, cfg.K
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        f32 = torch.float32
        i32 = torch.int32
        dv = torch.device(device)
        up = lambda a, dt=tdt: _dev(a, dt, dv)  # noqa: E731

        self.emb = up(inp.emb)
        self.w_head = up(inp.w_head)
        # the head matrix's packed copy (made once, with the weights), which the
        # matrix-core LM-head GEMM streams as contiguous 16 KB stages
        self.w_head_packed = (pack_head_weight(self.w_head)
                              if pack_head and tdt == torch.bfloat16 and H % 64 == 0 else None)
        self.fuse_M = up(inp.fuse_M)
        self.fuse_W = up(inp.fuse_W)
        g = {k: up(getattr(inp, k), f32) for k in ("g_h", "g_e", "g_e2", "g_m", "g_f", "g_final")}
        self.gains = g
        def layer_t(lw):
            return {k: up(getattr(lw, k), f32 if k.startswith("g_") else tdt)
                    for k in ("g_attn", "wqkv", "wo", "g_ffn", "wg", "wu", "wd", "ctx_k", "ctx_v")}
        self.layers_t = [layer_t(lw) for lw in inp.layers]
        self.has_mtp = bool(getattr(cfg, "mtp_block", False))
        self.mtp_layers_t = [layer_t(lw) for lw in inp.mtp_layers] if self.has_mtp else []
        self.cu_ctx = up(inp.cu_ctx, i32)
        self.anchor = up(inp.anchor, i32)
        self.h_prev = up(inp.h_prev)
        ht = inp.h_target if h_target is None else h_target
        nd = B * (K - 1)
        self.n_draft_rows = nd
        self.head_in = torch.empty(nd + B * (K + 1), H, dtype=tdt, device=dv)
        self.head_in[nd:] = up(np.asarray(ht, dtype=np.float32).reshape(B * (K + 1), H))

        tau = inp.tau.astype(np.float32)
        sampled = tau > 0
        self.any_sampled = bool(sampled.any())
        self.target_only = getattr(cfg, "verify", "rejection") == "target_only"
        plant = inp.plant.astype(bool)
        self.any_plant = bool(plant.any())
        self.seed = int(inp.philox_seed)

        # outputs
        self.h_mtp = torch.empty(B, H, dtype=f32, device=dv)
        self.h_fused = torch.empty(B, H, dtype=f32, device=dv) if self.has_mtp else self.h_mtp
        self.mtp_k_new = [torch.empty(B, 1, cfg.Hkv, cfg.d, dtype=tdt, device=dv)
                          for _ in self.mtp_layers_t]
        self.mtp_v_new = [torch.empty(B, 1, cfg.Hkv, cfg.d, dtype=tdt, device=dv)
                          for _ in self.mtp_layers_t]
        self.x_t1 = torch.empty(B, H, dtype=f32, device=dv)
        M1 = 2 * B if self.any_plant else B
        self.M1 = M1
        self.t1_token = torch.empty(M1, dtype=i32, device=dv)
        self.t1_lse = torch.empty(M1, dtype=f32, device=dv)
        self.t1_max = torch.empty(M1, dtype=f32, device=dv)
        self.t1_gap = torch.empty(M1, dtype=f32, device=dv)
        self.t1_prep = torch.empty(M1, H, dtype=tdt, device=dv)
        M2 = nd + B * (K + 1)
        self.M2 = M2
        self.tok = torch.empty(M2, dtype=i32, device=dv)
        self.lse = torch.empty(M2, dtype=f32, device=dv)
        self.rmax = torch.empty(M2, dtype=f32, device=dv)
        self.gap = torch.empty(M2, dtype=f32, device=dv)
        self.accept_len = torch.empty(B, dtype=i32, device=dv)
        self.out_tokens = torch.empty(B, K + 1, dtype=i32, device=dv)
        self.n_out = torch.empty(B, dtype=i32, device=dv)
        R2 = 2 * K + 1
        self.logits = (torch.empty(B * R2, V, dtype=f32, device=dv) if self.any_sampled else None)

        # per-launch row tables (sampling, storage, planting)
        if self.any_sampled:
            t1_temp = np.concatenate([tau, np.zeros(M1 - B, np.float32)])
            t1_key = np.full(M1, DMTP_NO_DRAW, dtype=np.uint64)
            t1_key[:B] = inp.draft_keys[:, 0]
            t1_store = np.full(M1, -1, np.int32)
            t1_store[:B] = np.where(sampled, np.arange(B) * R2, -1)
            tm = np.repeat(tau, K - 1)
            tt = np.repeat(tau, K + 1)
            c_temp = np.concatenate([tm, tt]).astype(np.float32)
            c_key = np.full(M2, DMTP_NO_DRAW, dtype=np.uint64)
            c_key[:nd] = inp.draft_keys[:, 1:].reshape(-1)
            if self.target_only:
                # the target's own picks at the rows of sampled sequences
                c_key[nd:] = np.where(np.repeat(sampled, K + 1), inp.target_keys.reshape(-1),
                                      DMTP_NO_DRAW).astype(np.uint64)
            bb = np.repeat(np.arange(B), K - 1)
            jj = np.tile(np.arange(K - 1), B)
            s_mask = np.where(sampled[bb], bb * R2 + 1 + jj, -1)
            bt = np.repeat(np.arange(B), K + 1)
            it = np.tile(np.arange(K + 1), B)
            s_tgt = np.where(sampled[bt], bt * R2 + K + it, -1)
            c_store = np.concatenate([s_mask, s_tgt]).astype(np.int32)
            self.t1_temp = up(t1_temp, f32)
            self.t1_key = up(t1_key.view(np.int64), torch.int64)
            self.t1_store = up(t1_store, i32)
            self.c_temp = up(c_temp, f32)
            self.c_key = up(c_key.view(np.int64), torch.int64)
            self.c_store = up(c_store, i32)
            self.v_temp = up(tau, f32)
            self.u_acc = up(inp.u_acc, f32)
            self.final_key = up(inp.final_keys.view(np.int64), torch.int64)
        else:
            self.t1_temp = self.t1_key = self.t1_store = None
            self.c_temp = self.c_key = self.c_store = None
            self.v_temp = self.u_acc = self.final_key = None
        if self.any_plant:
            pr = np.full(M1, -1, np.int32)
            pr[:B] = np.where(plant, B + np.arange(B), -1)
            self.plant_row = up(pr, i32)
        else:
            self.plant_row = None

        # descriptors
        eps = cfg.eps
        self.d_fuse_mtp = fuse(self.h_fused, self.fuse_M, g["g_h"], g["g_e"], x1=self.h_prev,
                               x2_ids=self.anchor, table=self.emb, eps=eps, run=False)
        if self.has_mtp:
            self._mtp_layers = [layer_arg(**lt) for lt in self.mtp_layers_t]
            self.d_mtp = mtp_block(self.h_mtp.view(B, 1, H), self.h_fused.view(B, 1, H), Hq=cfg.Hq,
                                   Hkv=cfg.Hkv, d=cfg.d, F=cfg.F, layers=self._mtp_layers,
                                   cu_ctx=self.cu_ctx, max_ctx=int(inp.ctx_len.max()),
                                   ctx_rows=int(inp.cu_ctx[-1]),
                                   dtype=1 if cfg.dtype == "bf16" else 0, k_new=self.mtp_k_new,
                                   v_new=self.mtp_v_new, eps=eps, rope_base=cfg.rope_base,
                                   run=False)
        segs = [head_segment(self.h_mtp, g["g_f"])]
        if self.any_plant:
            segs.append(head_segment(self.head_in[nd:], None, n=B, ld=(K + 1) * H))
        self.d_head_t1 = lm_head(self.w_head, segs, self.t1_token, eps=eps,
                                 temperature=self.t1_temp, draw_key=self.t1_key, seed=self.seed,
                                 plant_row=self.plant_row, store_row=self.t1_store,
                                 logits=self.logits, prepared=self.t1_prep, row_max=self.t1_max,
                                 lse=self.t1_lse, gap=self.t1_gap, w_packed=self.w_head_packed,
                                 run=False)
        t1_ids = self.t1_token[:B]
        self.d_fuse_delta = fuse(self.x_t1, self.fuse_W, g["g_e2"], g["g_m"], x1_ids=t1_ids,
                                 x2=self.h_mtp, res_ids=t1_ids, table=self.emb, eps=eps, run=False)
        L = [layer_arg(**lt) for lt in self.layers_t]
        self._layers = L
        self.d_draft = block_draft(self.head_in[:nd], B=B, H=H, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d,
                                   F=cfg.F, K=K, n_anchor=cfg.n_anchor, layers=L,
                                   anchor_ids=self.anchor, x_t1=self.x_t1, mask_id=cfg.mask_id,
                                   emb=self.emb, cu_ctx=self.cu_ctx, max_ctx=int(inp.ctx_len.max()),
                                   ctx_rows=int(inp.cu_ctx[-1]), g_final=g["g_final"], eps=eps,
                                   rope_base=cfg.rope_base, window=cfg.window, run=False)
        self.d_head_c = lm_head(self.w_head, [head_segment(self.head_in)], self.tok, eps=eps,
                                temperature=self.c_temp, draw_key=self.c_key, seed=self.seed,
                                store_row=self.c_store, logits=self.logits, row_max=self.rmax,
                                lse=self.lse, gap=self.gap, w_packed=self.w_head_packed, run=False)
        self.d_verify = verify(B=B, K=K, V=V, t1=t1_ids, drafts=self.tok[:nd],
                               target=self.tok[nd:], accept_len=self.accept_len,
                               out_tokens=self.out_tokens, n_out=self.n_out,
                               temperature=self.v_temp, logits=self.logits,
                               t1_lse=self.t1_lse[:B], draft_lse=self.lse[:nd],
                               target_lse=self.lse[nd:], u_acc=self.u_acc, seed=self.seed,
                               final_key=self.final_key, target_only=self.target_only,
                               run=False)
        self.hist = torch.zeros(K + 1, dtype=torch.int64, device=dv)
        self.summary = torch.zeros(2 + 2 * K, dtype=torch.float64, device=dv)
        self.steps = [("fuse", self.d_fuse_mtp)]
        self.step_names = ["fuse_mtp"]
        if self.has_mtp:
            self.steps.append(("mtp_block", self.d_mtp))
            self.step_names.append("mtp_block")
        self.step_names += ["lm_head_t1", "fuse_delta", "block_draft", "lm_head_draft_target",
                            "verify"]
        self.steps += [("lm_head", self.d_head_t1),
                      ("fuse", self.d_fuse_delta), ("block_draft", self.d_draft),
                      ("lm_head", self.d_head_c), ("verify", self.d_verify)]
        need = max(workspace_bytes(n, d) for n, d in self.steps)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dv)
        self._fns = [(getattr(lib, f"dmtp_{n}"), ctypes.byref(d)) for n, d in self.steps]
        self._ws_ptr = ctypes.c_void_p(self.ws.data_ptr())
        self._ws_bytes = self.ws.numel()

    def run_step(self, i: int, stream: Optional[int] = None) -> None:
        name, desc = self.steps[i]
        call(name, desc, self.ws, stream)

    def run(self, stream: Optional[int] = None) -> None:
        """Enqueue the whole round on `stream` (default: torch's current stream)."""
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream if stream is None else stream)
        for (fn, ref), (name, _) in zip(self._fns, self.steps):
            st = fn(ref, self._ws_ptr, self._ws_bytes, s)
            if st != 0:
                raise RuntimeError(f"dmtp_{name}: {lib.dmtp_status_str(st).decode()}")

    def capture(self) -> None:
        """Record one round into a HIP graph for replay()."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()           # first calls outside capture: kernel attributes, device checks
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g

    def replay(self) -> None:
        """Submit the captured round on the current stream."""
        self.graph.replay()

    def accept_stats(self) -> None:
        """Add this round's accepted lengths to self.hist and refresh self.summary."""
        accept_stats(self.accept_len, self.cfg.K, self.hist, self.summary)

    def results(self) -> Dict[str, np.ndarray]:
        torch.cuda.synchronize()
        cfg = self.cfg
        B, K, nd = cfg.B, cfg.K, self.n_draft_rows
        f = lambda t: t.detach().float().cpu().numpy()  # noqa: E731
        i = lambda t: t.detach().cpu().numpy().astype(np.int64)  # noqa: E731
        out = {
            "h_mtp": f(self.h_mtp), "h_fused": f(self.h_fused), "z1": f(self.t1_prep[:B]), "t1": i(self.t1_token[:B]),
            "t1_lse": f(self.t1_lse[:B]), "t1_max": f(self.t1_max[:B]), "t1_gap": f(self.t1_gap[:B]),
            "x_t1": f(self.x_t1), "hd_mask": f(self.head_in[:nd]).reshape(B, K - 1, cfg.H),
            "drafts_rest": i(self.tok[:nd]).reshape(B, K - 1),
            "target_argmax": i(self.tok[nd:]).reshape(B, K + 1),
            "draft_lse": f(self.lse[:nd]).reshape(B, K - 1),
            "target_lse": f(self.lse[nd:]).reshape(B, K + 1),
            "draft_max": f(self.rmax[:nd]).reshape(B, K - 1),
            "target_max": f(self.rmax[nd:]).reshape(B, K + 1),
            "gap": f(self.gap), "accept_len": i(self.accept_len),
            "out_tokens": i(self.out_tokens), "n_out": i(self.n_out),
        }
        out["drafts"] = np.concatenate([out["t1"][:, None], out["drafts_rest"]], axis=1)
        out["mtp_kv"] = [(f(k), f(v)) for k, v in zip(self.mtp_k_new, self.mtp_v_new)]
        return out
