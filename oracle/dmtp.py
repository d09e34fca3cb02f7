"""The DMTP round, step by step, in float64 -- oracle side (test infrastructure).

Sources (cited by page title and section):
  [DMTP]   "DMTP: A Better First Token for Block Drafting via MTP"
  [DvM]    "DFlash vs MTP: Two Paths to Breaking the Autoregressive Decoding
           Bottleneck"
  [colibri] colibri's notes on speculative decoding (MTP and prompt lookup)

One round for a sequence whose last emitted-but-unprocessed token is A:
  1. MTP input fusion  h' = M [RMSNorm(h); RMSNorm(Emb(A))]      ([DvM] "MTP:
     Sequential Prediction Heads ...", module-input equation; [colibri]: the
     head input pairs the backbone's post-final-norm output with the next
     token's embedding).  h_MTP is the output of the MTP decoder block over h'
     (a pre-norm Transformer block with its own causal KV cache: [DvM] the
     same section; [DMTP] section 6.5; [colibri]) when the workload has one,
     else h' itself.
  2. T1 = the MTP candidate: LM head on RMSNorm(h_MTP), argmax or a draw
     ([DMTP] section 5, step 1; section 6.4 keeps highest-probability selection).
  3. DMTP residual  Delta = W [RMS_e(e_T1); RMS_m(h_MTP)],  e~ = e_T1 + Delta
     ([DMTP] section 3, the two displayed equations; W starts at zero so e~ = e_T1).
  4. Block draft over [E(A), e~_T1, E(MASK) x (K-1)] (two anchors, eight slots for
     K = 7: [DMTP] section 3 "Two Anchors and Training Boundaries" and the
     Nov-9 update), one parallel forward ([DMTP] section 5 step 2; [DvM] "DFlash:
     Block Diffusion ...": bidirectional attention inside the block, attention to
     the clean target context whose K/V the target features provide).
  5. Shared LM head on every MASK slot: slot j proposes the token at its own
     position ([DvM]: shared output head; block diffusion unmasks in place).
  6. Target verification of the K candidates: the longest accepted prefix plus
     one correction or bonus token ([DMTP] section 5 step 3; [colibri]: a pick
     that equals the next draft accepts it, the first differing pick ends the
     verify).  Greedy compares with the target argmax; at temperature tau > 0
     the accept test is u < p(d)/q(d) and a rejection draws from
     normalize(max(0, p - q)), all accepted draws the bonus from p ([DvM]
     reference 8, Leviathan et al.; [DvM] "DFlash's Lossless Guarantee Breaks at
     Non-Zero Temperature": the draft sampler uses the same tau as the target).
     Target-only verification, the verifier the pages' experiments use ([DMTP]
     section 5, the note after step 3; [colibri]: a sampled pick that equals the
     next draft accepts it), instead compares each candidate with the target's
     own pick y_i ~ softmax(lt_i / tau): the accepted prefix runs to the first
     mismatch and the pick there (or y_K) is committed.

Precision reading (the pages fix none beyond bf16 weights): weights, embeddings,
context K/V and target rows are inputs in the configuration's dtype; every
intermediate is exact (float64 here); the rows that enter the LM head are
rounded to the configuration's dtype ("rf": bf16 round-to-nearest-even, or
float32), because the LM head is a bf16 x bf16 product.  Every discrete decision
is recorded with its margin so that a comparison can exempt near-ties.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import numerics as nm
from .philox import grouped_gumbel_argmax

# ---------------------------------------------------------------------------
# step 1 and 3: fusion projections
# ---------------------------------------------------------------------------


def fuse(x1: np.ndarray, x2: np.ndarray, g1: np.ndarray, g2: np.ndarray,
         w_cat: np.ndarray, eps: float, res: Optional[np.ndarray] = None) -> np.ndarray:
    """res + Wcat [RMSNorm(x1; g1); RMSNorm(x2; g2)] for rows x1, x2 [n, H].

    Wcat is [H, 2H]: its first H columns multiply the normalised x1 stream,
    the last H the normalised x2 stream.  Covers the MTP input fusion
    (x1 = h, x2 = Emb(A), no residual: [DvM] "MTP: Sequential ...") and the
    DMTP residual (x1 = e_T1, x2 = h_MTP, res = e_T1: [DMTP] section 3).
    """
    cat = np.concatenate([nm.rmsnorm(x1, g1, eps), nm.rmsnorm(x2, g2, eps)], axis=-1)
    out = nm.matmul_nt(cat, w_cat)
    if res is not None:
        out = np.asarray(res, dtype=np.float64) + out
    return out


# ---------------------------------------------------------------------------
# step 2 and 5: shared LM head and token selection
# ---------------------------------------------------------------------------


@dataclass
class HeadRows:
    """LM-head results for a set of rows (one launch's worth)."""
    token: np.ndarray     # [M] chosen index
    margin: np.ndarray    # [M] decision margin (top-2 gap of the deciding score)
    row_max: np.ndarray   # [M] max logit
    lse: np.ndarray       # [M] logsumexp(l / tau) (tau = 1 for greedy rows)
    logits: np.ndarray    # [M, V] float64 logits


def lm_logits(rows: np.ndarray, w_head: np.ndarray) -> np.ndarray:
    """Logits l = W_head x for each row x (W_head [V, H], rows [M, H]), float64."""
    return nm.matmul_nt(rows, w_head)


def select_tokens(logits: np.ndarray, tau: np.ndarray, seed: int,
                  keys: Optional[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Per row: argmax when tau = 0, else a draw from softmax(l / tau).

    The draw is the two-level Gumbel-max form of sampling of
    philox.grouped_gumbel_argmax over l / tau with the row's draw key.  Lowest
    index on exact ties.
    """
    M = logits.shape[0]
    tok = np.empty(M, dtype=np.int64)
    mar = np.empty(M, dtype=np.float64)
    for m in range(M):
        if tau[m] > 0.0:
            tok[m], mar[m] = grouped_gumbel_argmax(logits[m] / tau[m], seed, int(keys[m]))
        else:
            tok[m] = nm.argmax_first(logits[m])
            mar[m] = nm.top2_gap(logits[m])
    return tok, mar


def lm_head(rows: np.ndarray, w_head: np.ndarray, tau: np.ndarray, seed: int = 0,
            keys: Optional[np.ndarray] = None) -> HeadRows:
    """Shared LM head on rows that are already the head's input (normed, rounded)."""
    logits = lm_logits(rows, w_head)
    tok, mar = select_tokens(logits, tau, seed, keys)
    t = np.where(np.asarray(tau) > 0.0, tau, 1.0).astype(np.float64)
    lse = nm.logsumexp(logits / t[:, None], axis=-1)
    return HeadRows(token=tok, margin=mar, row_max=logits.max(axis=-1), lse=lse,
                    logits=logits)


# ---------------------------------------------------------------------------
# step 4: the block drafter
# ---------------------------------------------------------------------------


def block_slots(anchor_emb: np.ndarray, x_t1: np.ndarray, mask_emb: np.ndarray,
                K: int, n_anchor: int) -> np.ndarray:
    """Draft input slots of one sequence.

    Two anchors: [E(A), E(T1) + Delta, E(MASK) x (K-1)];  one anchor:
    [E(T1) + Delta, E(MASK) x (K-1)].  Only the T1 slot carries the residual.
    """
    masks = [np.asarray(mask_emb, dtype=np.float64)] * (K - 1)
    head = [np.asarray(anchor_emb, dtype=np.float64)] if n_anchor == 2 else []
    return np.stack(head + [np.asarray(x_t1, dtype=np.float64)] + masks)


@dataclass
class Layer64:
    """Weights of one drafter layer (any float dtype; products are taken in float64)."""
    g_attn: np.ndarray
    wqkv: np.ndarray
    wo: np.ndarray
    g_ffn: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray


def layer64(lw) -> Layer64:
    return Layer64(lw.g_attn, lw.wqkv, lw.wo, lw.g_ffn, lw.wg, lw.wu, lw.wd)


def decoder_layer(X: np.ndarray, positions: np.ndarray, lw: Layer64,
                  ctx_k: Sequence[np.ndarray], ctx_v: Sequence[np.ndarray], *, Hq: int, Hkv: int,
                  d: int, eps: float, rope_base: float, window: int = 0, causal: bool = False):
    """One pre-norm decoder layer over n sequences of S new rows each.

    X is [n, S, H], positions [n, S]; ctx_k[i] / ctx_v[i] are the keys /
    values [L_i, Hkv, d] that row i's sequence already holds (already rotated).
    x^ = RMSNorm(X; g_attn); q, k, v = x^ Wqkv^T; q and k rotated at the row
    positions; each query reads the held keys (the last `window` when
    window > 0) and the new rows' keys -- all S of them, or, when causal, rows
    0..j for row j; GQA maps query head h to kv head h // (Hq / Hkv);
    X1 = X + o Wo^T; X2 = X1 + (silu(x^2 Wg^T) * (x^2 Wu^T)) Wd^T with
    x^2 = RMSNorm(X1; g_ffn).  Returns (X2, k, v), k rotated, both [n, S, Hkv, d]:
    the rows a cache appends.  The projections are row-wise, so they are
    taken for all sequences at once.
    """
    n, S, H = X.shape
    xh = nm.rmsnorm(X, lw.g_attn, eps)
    qkv = nm.matmul_nt(xh.reshape(n * S, H), lw.wqkv).reshape(n, S, -1)
    group = Hq // Hkv
    o = np.empty((n, S, Hq, d))
    k_all = np.empty((n, S, Hkv, d))
    v_all = np.empty((n, S, Hkv, d))
    for i in range(n):
        q = nm.rope(qkv[i, :, : Hq * d].reshape(S, Hq, d), positions[i], rope_base)
        k = nm.rope(qkv[i, :, Hq * d: (Hq + Hkv) * d].reshape(S, Hkv, d), positions[i], rope_base)
        v = qkv[i, :, (Hq + Hkv) * d:].reshape(S, Hkv, d)
        k_all[i], v_all[i] = k, v
        ck = np.asarray(ctx_k[i], dtype=np.float64)
        cv = np.asarray(ctx_v[i], dtype=np.float64)
        if window > 0 and ck.shape[0] > window:
            ck, cv = ck[-window:], cv[-window:]
        keys = np.concatenate([ck, k], axis=0)     # [n_ctx + S, Hkv, d]
        vals = np.concatenate([cv, v], axis=0)
        n_ctx = ck.shape[0]
        for kv in range(Hkv):
            kk = np.ascontiguousarray(keys[:, kv])
            vv = np.ascontiguousarray(vals[:, kv])
            for h in range(kv * group, (kv + 1) * group):
                if not causal:
                    o[i, :, h] = nm.attention(q[:, h], kk, vv)
                else:
                    for j in range(S):
                        o[i, j, h] = nm.attention(q[j: j + 1, h], kk[: n_ctx + j + 1],
                                                  vv[: n_ctx + j + 1])[0]
    X1 = X + nm.matmul_nt(o.reshape(n * S, Hq * d), lw.wo).reshape(n, S, H)
    xh2 = nm.rmsnorm(X1, lw.g_ffn, eps).reshape(n * S, H)
    a = nm.silu(nm.matmul_nt(xh2, lw.wg)) * nm.matmul_nt(xh2, lw.wu)
    return X1 + nm.matmul_nt(a, lw.wd).reshape(n, S, H), k_all, v_all


def draft_layer(X: np.ndarray, positions: np.ndarray, lw: Layer64,
                ctx_k: Sequence[np.ndarray], ctx_v: Sequence[np.ndarray], *, Hq: int, Hkv: int,
                d: int, eps: float, rope_base: float, window: int = 0) -> np.ndarray:
    """One layer of the block drafter: decoder_layer over the S draft slots with
    no mask -- every slot's query reads its sequence's context keys and all S
    block keys, the block-diagonal (bidirectional) part plus the offset
    block-causal part of the DFlash mask, which for one block is "see
    everything" ([DvM] "DFlash: Block Diffusion ...", three-component mask;
    [DMTP] section 6.2 window)."""
    return decoder_layer(X, positions, lw, ctx_k, ctx_v, Hq=Hq, Hkv=Hkv, d=d, eps=eps,
                         rope_base=rope_base, window=window)[0]


def mtp_block(X: np.ndarray, positions: np.ndarray, layers64: Sequence[Layer64],
              cache_k: Sequence[Sequence[np.ndarray]], cache_v: Sequence[Sequence[np.ndarray]], *,
              Hq: int, Hkv: int, d: int, eps: float, rope_base: float):
    """The MTP decoder block over S new rows per sequence ([DvM] "MTP: Sequential
    Prediction Heads ...": a dedicated Transformer block after the input
    projection; [DMTP] section 6.5: full-history causal attention, projections,
    normalisation and a feed-forward network; [colibri]: the head keeps its own
    causal KV cache, to which every completed pair contributes its K/V).

    X [n, S, H] holds the fused inputs h' of the new rows, at positions
    [n, S]; cache_k[l][i] / cache_v[l][i] are layer l's cached keys / values of
    sequence i (the whole history: no window).  Row j attends to the cache and
    to new rows 0..j.  Returns (h_MTP [n, S, H] -- the block output, with no
    final norm -- and per layer the (k, v) rows [n, S, Hkv, d] to append).
    """
    kv = []
    for l, lw in enumerate(layers64):
        X, k, v = decoder_layer(X, positions, lw, cache_k[l], cache_v[l], Hq=Hq, Hkv=Hkv, d=d,
                                eps=eps, rope_base=rope_base, window=0, causal=True)
        kv.append((k, v))
    return X, kv


def ctx_kv(feats: np.ndarray, positions: np.ndarray, w_fc: np.ndarray, layers64: Sequence[Layer64],
           *, Hq: int, Hkv: int, d: int, eps: float, rope_base: float):
    """The drafter's context K/V of new target rows ([DvM] "DFlash: Block
    Diffusion ...": KV injection -- hidden features from a few target layers go
    into the key/value cache of every draft layer; [DMTP] section 3, ablation
    notes: context fusion concatenates five target feature streams and projects
    them back to the hidden size).

    feats [N, n_feat, H] are the target features of N committed rows at
    `positions` [N]; c = W_fc [f_1; ...; f_n] (W_fc [H, n_feat H]).  Reading
    where the pages stop: c enters every drafter layer the way a block row does,
    so layer l's cache rows are k = RoPE(RMSNorm(c; g_attn) Wk^T, pos) and
    v = RMSNorm(c; g_attn) Wv^T with Wk, Wv the key and value rows of Wqkv.
    Returns c [N, H] and per layer (k, v) [N, Hkv, d].
    """
    N, nf, H = feats.shape
    c = nm.matmul_nt(np.asarray(feats, dtype=np.float64).reshape(N, nf * H), w_fc)
    out = []
    for lw in layers64:
        xh = nm.rmsnorm(c, lw.g_attn, eps)
        kvw = np.asarray(lw.wqkv, dtype=np.float64)[Hq * d:]
        kv = nm.matmul_nt(xh, kvw)
        k = nm.rope(kv[:, : Hkv * d].reshape(N, Hkv, d), np.asarray(positions), rope_base)
        v = kv[:, Hkv * d:].reshape(N, Hkv, d)
        out.append((k, v))
    return c, out


def block_draft(slots: Sequence[np.ndarray], ctx_len: np.ndarray, layers64: Sequence[Layer64],
                ctx_k: Sequence[np.ndarray], ctx_v: Sequence[np.ndarray], cu_ctx: np.ndarray,
                seqs: Sequence[int], g_final: np.ndarray, rf: Callable, *, Hq: int, Hkv: int,
                d: int, eps: float, rope_base: float, window: int = 0) -> List[np.ndarray]:
    """All layers of the drafter for each sequence, then rf(RMSNorm(X; g_final)).

    slots[i] is [S, H] for sequence seqs[i]; slot j sits at position
    ctx_len[b] + j (the anchor A is the first position after the context).
    """
    seqs = list(seqs)
    X = np.stack([np.asarray(x, dtype=np.float64) for x in slots])
    S = X.shape[1]
    pos = np.stack([int(ctx_len[b]) + np.arange(S) for b in seqs])
    spans = [(int(cu_ctx[b]), int(cu_ctx[b + 1])) for b in seqs]
    for li, lw in enumerate(layers64):
        X = draft_layer(X, pos, lw, [ctx_k[li][lo:hi] for lo, hi in spans],
                        [ctx_v[li][lo:hi] for lo, hi in spans], Hq=Hq, Hkv=Hkv, d=d, eps=eps,
                        rope_base=rope_base, window=window)
    return list(rf(nm.rmsnorm(X, g_final, eps)))


# ---------------------------------------------------------------------------
# step 6: verification
# ---------------------------------------------------------------------------


def verify_greedy(drafts: Sequence[int], target_argmax: Sequence[int]) -> Tuple[int, List[int]]:
    """Greedy block verification.

    Row i of the target (after the prefix and d_0..d_{i-1}) verifies d_i.  The
    accepted length L is the first i with d_i != y_i (K if none differ); the
    commit is d_0..d_{L-1} followed by y_L, the correction (L < K) or the bonus
    (L = K).
    """
    K = len(drafts)
    L = 0
    while L < K and int(drafts[L]) == int(target_argmax[L]):
        L += 1
    return L, [int(t) for t in drafts[:L]] + [int(target_argmax[L])]


def verify_target_only(drafts: Sequence[int], pick: Callable[[int], int]) -> Tuple[int, List[int]]:
    """Target-only block verification ([DMTP] section 5, the note after step 3).

    pick(i) is the target's own token at row i (row i follows the prefix and
    d_0..d_{i-1}): a draw from its distribution at temperature tau, or its
    argmax at tau = 0.  Candidate d_i is accepted while it equals that pick; the
    first pick that differs is committed in its place as the correction, and
    when all K match the pick of row K is the bonus.  Picks of rows past the
    first mismatch are never needed (pick is called in increasing i).
    """
    K = len(drafts)
    for i in range(K):
        y = int(pick(i))
        if y != int(drafts[i]):
            return i, [int(t) for t in drafts[:i]] + [y]
    return K, [int(t) for t in drafts] + [int(pick(K))]


class VerifyOps:
    """Arithmetic used by the rejection verifier, float64 NumPy version."""

    @staticmethod
    def ratio(p_row, q_row, tok):
        return float(p_row[tok]) / float(q_row[tok])

    @staticmethod
    def residual(p_row, q_row):
        return np.maximum(0.0, np.asarray(p_row) - np.asarray(q_row))

    @staticmethod
    def total(w):
        return float(np.sum(w))


def verify_rejection(drafts: Sequence[int], p_rows, q_rows, accept: Callable, draw: Callable,
                     ops=VerifyOps) -> Tuple[int, List[int]]:
    """Rejection-sampling block verification of one sequence.

    p_rows[i] (i = 0..K) is the target distribution at row i, q_rows[i]
    (i = 0..K-1) the draft distribution candidate d_i was proposed from.
    For i = 0, 1, ...: accept d_i with probability min(1, p_i(d_i)/q_i(d_i))
    (accept(i, ratio) decides); at the first rejection draw the correction
    from normalize(max(0, p_i - q_i)) (draw(i, weights) decides), falling back
    to p_i when that residual is zero (only reachable through rounding); when
    all K are accepted, draw the bonus from p_K.
    """
    K = len(drafts)
    for i in range(K):
        if accept(i, ops.ratio(p_rows[i], q_rows[i], int(drafts[i]))):
            continue
        r = ops.residual(p_rows[i], q_rows[i])
        y = draw(i, r) if ops.total(r) > 0 else draw(i, p_rows[i])
        return i, [int(t) for t in drafts[:i]] + [int(y)]
    return K, [int(t) for t in drafts] + [int(draw(K, p_rows[K]))]


# ---------------------------------------------------------------------------
# the round
# ---------------------------------------------------------------------------


@dataclass
class RoundResult:
    seqs: List[int]
    h_fused: np.ndarray      # [n, H] h' = M [RMSNorm(h); RMSNorm(E(A))]
    h_mtp: np.ndarray        # [n, H] h' or the MTP block's output
    z1: np.ndarray           # [n, H] rounded LM-head input of the T1 rows
    x_t1: np.ndarray         # [n, H] E(T1) + Delta
    hd: np.ndarray           # [n, S, H] rounded final-normed drafter output, all slots
    t1: np.ndarray           # [n]
    drafts: np.ndarray       # [n, K]  d_0 = T1, d_i from MASK slot i + n_anchor - 1
    target_argmax: np.ndarray  # [n, K + 1] the target's pick per row: argmax, or a draw (target-only, tau > 0)
    q_lse: np.ndarray        # [n, K]   lse(l / tau) of the candidate rows
    p_lse: np.ndarray        # [n, K + 1]
    q_max: np.ndarray
    p_max: np.ndarray
    accept_len: np.ndarray   # [n]
    out_tokens: np.ndarray   # [n, K + 1], -1 padded
    n_out: np.ndarray        # [n]
    decisions: List[Tuple[tuple, int, float]] = field(default_factory=list)
    mtp_kv: Optional[list] = None            # per MTP layer (k, v) [n, 1, Hkv, d] to append
    q_logits: Optional[np.ndarray] = None   # [n, K, V] when keep_logits
    p_logits: Optional[np.ndarray] = None   # [n, K + 1, V]


def head_rows_for_target(inp, seqs) -> np.ndarray:
    """Target-side LM-head input rows [n, K + 1, H] (inputs, used as given)."""
    return np.asarray(inp.h_target[list(seqs)], dtype=np.float64)


def run_round(inp, seqs: Optional[Sequence[int]] = None,
              overrides: Optional[Dict[tuple, int]] = None, keep_logits: bool = False,
              h_target: Optional[np.ndarray] = None) -> RoundResult:
    """One DMTP round over sequences `seqs` (default: all) of the inputs `inp`.

    overrides forces discrete decisions by name, for replaying a comparison
    whose other side took a near-tie the other way:
      ("T1", b), ("draft", b, i), ("y", b, i)  -> token
      ("accept", b, i) -> 0/1,  ("final", b) -> token
    h_target optionally replaces inp.h_target (all B sequences).
    """
    cfg = inp.cfg
    ov = dict(overrides or {})
    B, H, V, K = cfg.B, cfg.H, cfg.V, cfg.K
    seqs = list(range(B)) if seqs is None else [int(b) for b in seqs]
    n = len(seqs)
    rf = nm.round_to(cfg.dtype)
    eps = cfg.eps
    E = inp.emb
    w_head64 = inp.w_head
    tau = inp.tau[seqs].astype(np.float64)
    seed = int(inp.philox_seed)
    decisions: List[Tuple[tuple, int, float]] = []
    ht_all = inp.h_target if h_target is None else h_target
    ht = np.asarray(ht_all[seqs], dtype=np.float64)             # [n, K+1, H]

    def decide(key, value, margin):
        if key in ov:
            value = int(ov[key])
        decisions.append((key, int(value), float(margin)))
        return int(value)

    # -- target rows: the verifying logits (the target forward is an input) --
    p_logits = lm_logits(ht.reshape(n * (K + 1), H), w_head64).reshape(n, K + 1, V)
    tgt_argmax = nm.argmax_first(p_logits)
    tgt_gap = nm.top2_gap(p_logits)
    tt = np.where(tau > 0, tau, 1.0)

    # -- 1. MTP input fusion, then the MTP decoder block when the workload has one
    #       (otherwise h_MTP = h') --
    h_fused = fuse(inp.h_prev[seqs], E[inp.anchor[seqs]], inp.g_h, inp.g_e, inp.fuse_M, eps)
    mtp_kv = None
    if getattr(cfg, "mtp_block", False):
        spans = [(int(inp.cu_ctx[b]), int(inp.cu_ctx[b + 1])) for b in seqs]
        ml = inp.mtp_layers
        out, mtp_kv = mtp_block(h_fused[:, None, :], inp.ctx_len[seqs][:, None].astype(np.int64),
                                [layer64(lw) for lw in ml],
                                [[lw.ctx_k[lo:hi] for lo, hi in spans] for lw in ml],
                                [[lw.ctx_v[lo:hi] for lo, hi in spans] for lw in ml],
                                Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, eps=eps, rope_base=cfg.rope_base)
        h_mtp = out[:, 0]
    else:
        h_mtp = h_fused

    # -- 2. T1 from the shared head on RMSNorm(h_MTP; g_f), rounded to the head dtype --
    z1 = rf(nm.rmsnorm(h_mtp, inp.g_f, eps))
    l1 = lm_logits(z1, w_head64)
    t1 = np.empty(n, dtype=np.int64)
    for r, b in enumerate(seqs):
        if inp.plant[b]:
            # planted workload: T1 := the target's argmax at row 0 (a synthetic
            # stand-in for an MTP head that agrees with the target)
            v, m = tgt_argmax[r, 0], tgt_gap[r, 0]
        elif tau[r] > 0:
            v, m = grouped_gumbel_argmax(l1[r] / tau[r], seed, int(inp.draft_keys[b, 0]))
        else:
            v, m = nm.argmax_first(l1[r]), nm.top2_gap(l1[r])
        t1[r] = decide(("T1", b), v, m)

    # -- 3. DMTP residual on T1's embedding slot --
    e_t1 = E[t1]
    x_t1 = fuse(e_t1, h_mtp, inp.g_e2, inp.g_m, inp.fuse_W, eps, res=e_t1)

    # -- 4. block draft --
    slots = [block_slots(E[inp.anchor[b]], x_t1[r], E[cfg.mask_id], K, cfg.n_anchor)
             for r, b in enumerate(seqs)]
    L64 = [layer64(lw) for lw in inp.layers]
    hd = block_draft(slots, inp.ctx_len, L64, [lw.ctx_k for lw in inp.layers],
                     [lw.ctx_v for lw in inp.layers], inp.cu_ctx, seqs, inp.g_final, rf,
                     Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, eps=eps, rope_base=cfg.rope_base,
                     window=cfg.window)
    hd = np.stack(hd)                                     # [n, S, H]

    # -- 5. LM head on the MASK slots: candidate i >= 1 from slot i + n_anchor - 1 --
    first = cfg.n_anchor
    ld = lm_logits(hd[:, first:, :].reshape(n * (K - 1), H), w_head64).reshape(n, K - 1, V)
    q_logits = np.concatenate([l1[:, None, :], ld], axis=1)       # [n, K, V]
    drafts = np.empty((n, K), dtype=np.int64)
    drafts[:, 0] = t1
    for r, b in enumerate(seqs):
        for i in range(1, K):
            row = q_logits[r, i]
            if tau[r] > 0:
                v, m = grouped_gumbel_argmax(row / tau[r], seed, int(inp.draft_keys[b, i]))
            else:
                v, m = nm.argmax_first(row), nm.top2_gap(row)
            drafts[r, i] = decide(("draft", b, i), v, m)

    q_lse = nm.logsumexp(q_logits / tt[:, None, None], axis=-1)
    p_lse = nm.logsumexp(p_logits / tt[:, None, None], axis=-1)

    # -- 6. verification --
    accept_len = np.empty(n, dtype=np.int64)
    out_tokens = np.full((n, K + 1), -1, dtype=np.int64)
    y_final = np.empty((n, K + 1), dtype=np.int64)
    target_only = getattr(cfg, "verify", "rejection") == "target_only"
    for r, b in enumerate(seqs):
        for i in range(K + 1):
            if target_only and tau[r] > 0:
                # the target's own pick: a draw from softmax(lt_i / tau)
                v, m = grouped_gumbel_argmax(p_logits[r, i] / tau[r], seed, int(inp.target_keys[b, i]))
            else:
                v, m = tgt_argmax[r, i], tgt_gap[r, i]
            y_final[r, i] = decide(("y", b, i), v, m)
        if target_only:
            # at tau = 0 the picks are the argmax and this is greedy verification
            L, toks = verify_target_only(drafts[r], lambda i, r=r: y_final[r, i])
        elif tau[r] > 0:
            p_rows = np.exp(p_logits[r] / tau[r] - p_lse[r][:, None])
            q_rows = np.exp(q_logits[r] / tau[r] - q_lse[r][:, None])
            u = inp.u_acc[b].astype(np.float64)

            def accept(i, ratio, b=b, u=u):
                margin = abs(np.log(u[i]) - np.log(ratio)) if u[i] > 0 else np.inf
                return bool(decide(("accept", b, i), int(u[i] < ratio), margin))

            def draw(i, w, b=b):
                with np.errstate(divide="ignore"):
                    lw = np.log(np.asarray(w, dtype=np.float64))
                v, m = grouped_gumbel_argmax(lw, seed, int(inp.final_keys[b]))
                return decide(("final", b), v, m)

            L, toks = verify_rejection(drafts[r], p_rows, q_rows, accept, draw)
        else:
            L, toks = verify_greedy(drafts[r], y_final[r])
        accept_len[r] = L
        out_tokens[r, : len(toks)] = toks

    return RoundResult(
        seqs=seqs, h_fused=h_fused, h_mtp=h_mtp, z1=z1, x_t1=x_t1, hd=hd, t1=t1, drafts=drafts,
        target_argmax=y_final, q_lse=q_lse, p_lse=p_lse,
        q_max=q_logits.max(axis=-1), p_max=p_logits.max(axis=-1),
        accept_len=accept_len, out_tokens=out_tokens, n_out=accept_len + 1,
        decisions=decisions, mtp_kv=mtp_kv,
        q_logits=q_logits if keep_logits else None,
        p_logits=p_logits if keep_logits else None)


def acceptance_stats(accept_len: np.ndarray, K: int) -> Dict[str, object]:
    """Acceptance statistics of a set of verify rounds ([DMTP] sections 7 and 8).

    per_verify      1 + sum_k k * hist[k] / sum hist   (includes the correction/bonus)
    first_candidate 1 - hist[0] / sum hist
    cumulative[k]   P(L >= k) for k = 1..K
    conditional[k]  P(L >= k | L >= k - 1), acceptance of candidate k given the first k-1
    """
    a = np.asarray(accept_len, dtype=np.int64)
    hist = np.bincount(a, minlength=K + 1)[: K + 1]
    tot = int(hist.sum())
    per_verify = 1.0 + float(np.dot(np.arange(K + 1), hist)) / tot if tot else float("nan")
    first = 1.0 - hist[0] / tot if tot else float("nan")
    cum = [float((a >= k).mean()) if tot else float("nan") for k in range(1, K + 1)]
    prev = [1.0] + cum[:-1]
    cond = [c / p if p > 0 else float("nan") for c, p in zip(cum, prev)]
    return {"hist": hist.tolist(), "per_verify": per_verify, "first_candidate": float(first),
            "cumulative": cum, "conditional": cond}
