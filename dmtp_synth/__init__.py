"""Seeded synthetic inputs for one DMTP speculative-decoding round.

This module only *draws* inputs: random weights, embeddings, context K/V,
hidden states, temperatures, uniforms and the integer keys that name each
random draw.  It holds none of the method's arithmetic (no norms, no
projections, no softmax, no rounding of results), so that the CPU oracle and
the HIP path can both consume it without sharing any step of the computation.

Shapes follow the workloads the pages describe (the DMTP blog: a 7-candidate
block, one MTP candidate plus six parallel MASK proposals, batch 32 in the
serving evaluation of section 7; contexts inside the 4096-position anchor
window of section 6.2).  Every tensor is drawn from its own NumPy stream,
``default_rng([seed, tensor_id])``, so one tensor can be regenerated without
the others and adding a tensor never shifts the values of another.

bf16 configurations store weights as float32 arrays whose values are exactly
representable in bfloat16: the float32 draw is truncated to its top 16 bits.
That is an input-generation choice (a bf16 random variable), not a rounding
step of the method.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, List, Optional

import numpy as np

# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class RoundConfig:
    """Shapes and knobs of one synthetic DMTP round.

    K         candidates per round (T1 from the MTP head + K-1 MASK proposals)
    n_anchor  2: slots [A, T1, MASK x (K-1)]  (two anchors, the main layout)
              1: slots [T1, MASK x (K-1)]     (single-anchor variant)
    S         draft slots = K - 1 + n_anchor; R = K + 1 target rows to verify
    """

    name: str
    B: int
    H: int
    V: int
    Hq: int
    Hkv: int
    d: int
    F: int
    n_layers: int
    K: int
    ctx_min: int
    ctx_max: int
    dtype: str = "bf16"          # "f32" or "bf16" storage of weights/activations
    tau_mode: str = "greedy"     # "greedy" | "sample" | "mixed"
    rho: Optional[float] = None  # target/draft hidden correlation (sampled tiny case)
    plant_frac: float = 0.0      # fraction of rows whose T1 is set to the target argmax
    w_zero: bool = False         # DMTP residual projection W zero-initialised
    n_anchor: int = 2
    verify: str = "rejection"    # "rejection" | "target_only" (rows with tau > 0)
    mtp_block: bool = False      # h_MTP from an MTP decoder block over h' (else h_MTP = h')
    window: int = 4096           # the drafter reads the last `window` context positions before
    #                              the anchor (0 = all of them)
    rope_base: float = 1.0e6
    eps: float = 1.0e-6
    weight_std: float = 0.02
    gain_std: float = 0.0        # gains are 1 + N(0, gain_std)
    seed: int = 0

    @property
    def S(self) -> int:
        return self.K - 1 + self.n_anchor

    @property
    def R(self) -> int:
        return self.K + 1

    @property
    def qkv_dim(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.d

    @property
    def mask_id(self) -> int:
        # The pages do not name the MASK token; the last vocabulary id is used.
        return self.V - 1

    def with_(self, **kw) -> "RoundConfig":
        return replace(self, **kw)


# The five workloads: tiny fp32 greedy, B32 greedy, tiny fp32 sampled,
# long-block stress, short-chat high-batch with a greedy/sampled mix.
CONFIGS: Dict[str, RoundConfig] = {
    "tiny_greedy_f32": RoundConfig(
        name="tiny_greedy_f32", B=1, H=256, V=1024, Hq=4, Hkv=4, d=64, F=512,
        n_layers=1, K=7, ctx_min=128, ctx_max=128, dtype="f32", seed=101),
    "b32_greedy_bf16": RoundConfig(
        name="b32_greedy_bf16", B=32, H=2048, V=151936, Hq=16, Hkv=4, d=128,
        F=6144, n_layers=1, K=7, ctx_min=1024, ctx_max=4096, dtype="bf16",
        seed=202),
    "tiny_sampled_f32": RoundConfig(
        name="tiny_sampled_f32", B=1, H=256, V=1024, Hq=4, Hkv=4, d=64, F=512,
        n_layers=1, K=7, ctx_min=128, ctx_max=128, dtype="f32",
        tau_mode="sample", rho=0.8, seed=303),
    "long_block16_bf16": RoundConfig(
        name="long_block16_bf16", B=8, H=5120, V=151936, Hq=40, Hkv=8, d=128,
        F=13824, n_layers=2, K=16, ctx_min=32768, ctx_max=32768, dtype="bf16",
        window=0, seed=404),
    "chat_b128_mixed_bf16": RoundConfig(
        name="chat_b128_mixed_bf16", B=128, H=2048, V=151936, Hq=16, Hkv=4,
        d=128, F=6144, n_layers=1, K=7, ctx_min=64, ctx_max=512, dtype="bf16",
        tau_mode="mixed", plant_frac=0.8, seed=505),
}

# Stable ids of the per-tensor random streams.
_TID = {
    "emb": 1, "w_head": 2, "fuse_M": 3, "fuse_W": 4, "g_h": 5, "g_e": 6,
    "g_e2": 7, "g_m": 8, "g_f": 9, "g_final": 10, "ctx_len": 11, "anchor": 12,
    "h_prev": 13, "h_target": 14, "tau": 15, "u_acc": 16, "plant": 17,
    "philox_seed": 18,
    # per-layer tensors: 100 + 16 * layer + j
    "g_attn": 0, "wqkv": 1, "wo": 2, "g_ffn": 3, "wg": 4, "wu": 5, "wd": 6,
    "ctx_k": 7, "ctx_v": 8,
}

# Purposes of the counter-based random draws (upper 32 bits of a draw key).
DRAW_DRAFT = 1   # sampling of candidate i of sequence b from the draft distribution
DRAW_FINAL = 2   # the correction/bonus draw of sequence b during verification
DRAW_TARGET = 3  # the target's own pick at verify row i of sequence b (target-only verify)


def draft_draw_key(b: int, i: int) -> int:
    """Key of the draw that samples candidate i (0 = T1) of sequence b."""
    return (DRAW_DRAFT << 32) | (int(b) << 8) | int(i)


def final_draw_key(b: int) -> int:
    """Key of the correction/bonus draw of sequence b."""
    return (DRAW_FINAL << 32) | int(b)


def target_pick_key(b: int, i: int) -> int:
    """Key of the draw that picks the target's token at verify row i of sequence b."""
    return (DRAW_TARGET << 32) | (int(b) << 8) | int(i)


def _rng(cfg: RoundConfig, tid: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, tid])


def _layer_tid(layer: int, name: str) -> int:
    return 100 + 16 * layer + _TID[name]


def _mtp_tid(name: str) -> int:
    return 2000 + _TID[name]


_CHUNK = 1 << 22  # elements per independent random stream of a large tensor
_POOL: Optional[ThreadPoolExecutor] = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = ThreadPoolExecutor(max_workers=n)
    return _POOL


def _normal_t(cfg: RoundConfig, tid: int, shape, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) tensor; element chunk c is drawn from stream [seed, tid, c].

    The chunking makes generation parallel and independent of the thread count.
    """
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n_chunks = (out.size + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        view = out[c * _CHUNK:(c + 1) * _CHUNK]
        np.random.default_rng([cfg.seed, tid, c]).standard_normal(out=view, dtype=np.float32)
        if std != 1.0:
            view *= np.float32(std)
        if dtype == "bf16":
            _truncate_to_bf16_inplace(view)

    if n_chunks <= 1:
        if n_chunks == 1:
            fill(0)
    else:
        list(_pool().map(fill, range(n_chunks)))
    return out.reshape(shape)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        _truncate_to_bf16_inplace(x)
    return x


def _truncate_to_bf16_inplace(x: np.ndarray) -> None:
    """Make every value bf16-representable by dropping the low 16 bits."""
    bits = x.view(np.uint32)
    np.bitwise_and(bits, np.uint32(0xFFFF0000), out=bits)


def _gain(cfg: RoundConfig, tid: int, n: int) -> np.ndarray:
    if cfg.gain_std == 0.0:
        return np.ones(n, dtype=np.float32)
    g = 1.0 + _normal(_rng(cfg, tid), (n,), cfg.gain_std, "f32")
    if cfg.dtype == "bf16":
        _truncate_to_bf16_inplace(g)
    return g


@dataclass
class LayerInputs:
    g_attn: np.ndarray   # [H]
    wqkv: np.ndarray     # [(Hq + 2 Hkv) d, H]  rows: q heads, then k heads, then v heads
    wo: np.ndarray       # [H, Hq d]
    g_ffn: np.ndarray    # [H]
    wg: np.ndarray       # [F, H]
    wu: np.ndarray       # [F, H]
    wd: np.ndarray       # [H, F]
    ctx_k: np.ndarray    # [sum L_b, Hkv, d]  context keys, already rotated
    ctx_v: np.ndarray    # [sum L_b, Hkv, d]


@dataclass
class RoundInputs:
    cfg: RoundConfig
    emb: np.ndarray        # [V, H]   token embedding, shared with the target
    w_head: np.ndarray     # [V, H]   shared LM head (out x in)
    fuse_M: np.ndarray     # [H, 2H]  MTP input projection, columns [h ; e]
    fuse_W: np.ndarray     # [H, 2H]  DMTP residual projection, columns [e ; h]
    g_h: np.ndarray        # [H] RMSNorm gain of the target hidden in the MTP fusion
    g_e: np.ndarray        # [H] RMSNorm gain of the anchor embedding in the MTP fusion
    g_e2: np.ndarray       # [H] RMS_e gain of the residual (T1 embedding stream)
    g_m: np.ndarray        # [H] RMS_m gain of the residual (MTP hidden stream)
    g_f: np.ndarray        # [H] final norm before the LM head, MTP rows
    g_final: np.ndarray    # [H] final norm of the block drafter
    layers: List[LayerInputs]
    mtp_layers: List[LayerInputs]  # the MTP decoder block (empty unless cfg.mtp_block); its
    #                                ctx_k / ctx_v are the block's own causal KV cache, one row
    #                                per context position (lengths ctx_len, offsets cu_ctx)
    ctx_len: np.ndarray    # [B] int32
    cu_ctx: np.ndarray     # [B + 1] int32 prefix sums of ctx_len
    anchor: np.ndarray     # [B] int32   A: emitted, not yet processed by the target
    h_prev: np.ndarray     # [B, H]      target hidden at x_{a-1}, after its final norm
    h_target: np.ndarray   # [B, K + 1, H] target-side hidden rows fed to the LM head
    tau: np.ndarray        # [B] float32, 0 = greedy
    u_acc: np.ndarray      # [B, K] float32 uniforms of the accept tests
    plant: np.ndarray      # [B] bool, T1 := target argmax of row 0
    philox_seed: int       # key of the counter-based generator
    draft_keys: np.ndarray  # [B, K] uint64 draw keys for candidate sampling
    final_keys: np.ndarray  # [B] uint64 draw keys for correction/bonus draws
    target_keys: np.ndarray  # [B, K + 1] uint64 draw keys of the target's picks


def make_inputs(cfg: RoundConfig, *, with_layers: bool = True) -> RoundInputs:
    """Draw every input of one round for ``cfg`` (deterministic in cfg.seed)."""
    B, H, V, K = cfg.B, cfg.H, cfg.V, cfg.K
    dt, std = cfg.dtype, cfg.weight_std
    emb = _normal_t(cfg, _TID["emb"], (V, H), std, dt)
    w_head = _normal_t(cfg, _TID["w_head"], (V, H), std, dt)
    fuse_M = _normal_t(cfg, _TID["fuse_M"], (H, 2 * H), std, dt)
    if cfg.w_zero:
        fuse_W = np.zeros((H, 2 * H), dtype=np.float32)
    else:
        fuse_W = _normal_t(cfg, _TID["fuse_W"], (H, 2 * H), std, dt)

    r = _rng(cfg, _TID["ctx_len"])
    ctx_len = r.integers(cfg.ctx_min, cfg.ctx_max + 1, size=B).astype(np.int32)
    cu_ctx = np.zeros(B + 1, dtype=np.int32)
    cu_ctx[1:] = np.cumsum(ctx_len)
    total = int(cu_ctx[-1])

    layers: List[LayerInputs] = []
    if with_layers:
        for l in range(cfg.n_layers):
            def t(name, shape, sd):
                return _normal_t(cfg, _layer_tid(l, name), shape, sd, dt)
            layers.append(LayerInputs(
                g_attn=_gain(cfg, _layer_tid(l, "g_attn"), H),
                wqkv=t("wqkv", (cfg.qkv_dim, H), std),
                wo=t("wo", (H, cfg.Hq * cfg.d), std),
                g_ffn=_gain(cfg, _layer_tid(l, "g_ffn"), H),
                wg=t("wg", (cfg.F, H), std),
                wu=t("wu", (cfg.F, H), std),
                wd=t("wd", (H, cfg.F), std),
                ctx_k=t("ctx_k", (total, cfg.Hkv, cfg.d), 1.0),
                ctx_v=t("ctx_v", (total, cfg.Hkv, cfg.d), 1.0),
            ))

    mtp_layers: List[LayerInputs] = []
    if with_layers and cfg.mtp_block:
        def tm(name, shape, sd):
            return _normal_t(cfg, _mtp_tid(name), shape, sd, dt)
        mtp_layers.append(LayerInputs(
            g_attn=_gain(cfg, _mtp_tid("g_attn"), H),
            wqkv=tm("wqkv", (cfg.qkv_dim, H), std),
            wo=tm("wo", (H, cfg.Hq * cfg.d), std),
            g_ffn=_gain(cfg, _mtp_tid("g_ffn"), H),
            wg=tm("wg", (cfg.F, H), std),
            wu=tm("wu", (cfg.F, H), std),
            wd=tm("wd", (H, cfg.F), std),
            ctx_k=tm("ctx_k", (total, cfg.Hkv, cfg.d), 1.0),
            ctx_v=tm("ctx_v", (total, cfg.Hkv, cfg.d), 1.0),
        ))

    anchor = _rng(cfg, _TID["anchor"]).integers(0, V - 1, size=B).astype(np.int32)
    h_prev = _normal_t(cfg, _TID["h_prev"], (B, H), 1.0, dt)
    h_target = _normal_t(cfg, _TID["h_target"], (B, K + 1, H), 1.0, dt)

    if cfg.tau_mode == "greedy":
        tau = np.zeros(B, dtype=np.float32)
    elif cfg.tau_mode == "sample":
        tau = np.ones(B, dtype=np.float32)
    elif cfg.tau_mode == "mixed":
        coin = _rng(cfg, _TID["tau"]).random(B) < 0.5
        tau = np.where(coin, 1.0, 0.0).astype(np.float32)
    else:
        raise ValueError(cfg.tau_mode)

    # uniforms on the 2^-24 grid of [0, 1): exactly representable in float32
    ui = _rng(cfg, _TID["u_acc"]).integers(0, 1 << 24, size=(B, K))
    u_acc = (ui.astype(np.float64) * 2.0 ** -24).astype(np.float32)

    if cfg.plant_frac > 0.0:
        plant = _rng(cfg, _TID["plant"]).random(B) < cfg.plant_frac
    else:
        plant = np.zeros(B, dtype=bool)

    philox_seed = int(_rng(cfg, _TID["philox_seed"]).integers(0, 2 ** 63))
    draft_keys = np.array([[draft_draw_key(b, i) for i in range(K)] for b in range(B)],
                          dtype=np.uint64)
    final_keys = np.array([final_draw_key(b) for b in range(B)], dtype=np.uint64)
    target_keys = np.array([[target_pick_key(b, i) for i in range(K + 1)] for b in range(B)],
                           dtype=np.uint64)

    return RoundInputs(
        cfg=cfg, emb=emb, w_head=w_head, fuse_M=fuse_M, fuse_W=fuse_W,
        g_h=_gain(cfg, _TID["g_h"], H), g_e=_gain(cfg, _TID["g_e"], H),
        g_e2=_gain(cfg, _TID["g_e2"], H), g_m=_gain(cfg, _TID["g_m"], H),
        g_f=_gain(cfg, _TID["g_f"], H), g_final=_gain(cfg, _TID["g_final"], H),
        layers=layers, mtp_layers=mtp_layers, ctx_len=ctx_len, cu_ctx=cu_ctx, anchor=anchor,
        h_prev=h_prev, h_target=h_target, tau=tau, u_acc=u_acc, plant=plant,
        philox_seed=philox_seed, draft_keys=draft_keys, final_keys=final_keys,
        target_keys=target_keys)


__all__ = [
    "RoundConfig", "CONFIGS", "RoundInputs", "LayerInputs", "make_inputs",
    "draft_draw_key", "final_draw_key", "target_pick_key", "DRAW_DRAFT", "DRAW_FINAL",
    "DRAW_TARGET",
]
