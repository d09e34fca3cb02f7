#!/usr/bin/env python3
"""Throughput of one DMTP draft+verify round on one MI355X.

A step is one whole round (MTP fusion, T1 head, DMTP residual, block draft,
shared LM head over draft and target rows, verification) over one batch of
synthetic, seeded inputs already resident in HBM.  Default workload: batch 32,
hidden 2048, vocabulary 151936, one block-draft layer (16 query / 4 kv heads
x 128, SwiGLU 6144), 7 candidates (8 draft slots, 8 verify rows), context
lengths uniform in [1024, 4096], greedy.

Prints one JSON line.  value = rounds/s; committed tokens/s, the roofline of
the dominant kernel (the LM-head call over the 448 draft+target rows) and the
CPU oracle timed on a bounded sample are extra fields.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

METRIC = "draft+verify rounds/s and accepted tokens/s at B32; % MFMA / HBM peak"


def _workload_desc(cfg) -> str:
    return (f"{cfg.name}: B={cfg.B}, H={cfg.H}, V={cfg.V}, {cfg.n_layers} draft layer(s) "
            f"{cfg.Hq}q/{cfg.Hkv}kv x{cfg.d}, F={cfg.F}, K={cfg.K} candidates "
            f"({cfg.S} slots, {cfg.R} verify rows), ctx U[{cfg.ctx_min},{cfg.ctx_max}], "
            f"tau={cfg.tau_mode}")


def cpu_baseline(inp, n_seq: int):
    from threadpoolctl import threadpool_info
    from oracle import dmtp as odm

    seqs = list(range(min(n_seq, inp.cfg.B)))
    t0 = time.perf_counter()
    odm.run_round(inp, seqs=seqs)
    dt = time.perf_counter() - t0
    scale = inp.cfg.B / len(seqs)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": 1.0 / (dt * scale), "unit": "rounds/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle on {len(seqs)} of {inp.cfg.B} sequences of one round "
                      f"({dt:.1f} s), scaled x{scale:g} to a whole round",
            "seconds": dt}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="b32_greedy_bf16")
    ap.add_argument("--cpu-seqs", type=int, default=8, help="sequences in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the round is "
              "data-parallel over sequences and is not sharded here", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import dmtp_synth as synth
    from mtp_block_draft_amd.round import Round

    cfg = synth.CONFIGS[args.config]
    inp = synth.make_inputs(cfg)
    R = Round(inp)
    stream = torch.cuda.current_stream()
    s_ptr = stream.cuda_stream
    import ctypes
    sp = ctypes.c_void_p(s_ptr)
    n_calls = len(R._fns)

    def one_round(evs=None):
        for i, (fn, ref) in enumerate(R._fns):
            if evs is not None:
                evs[i][0].record(stream)
            st = fn(ref, R._ws_ptr, R._ws_bytes, sp)
            if evs is not None:
                evs[i][1].record(stream)
            if st != 0:
                raise RuntimeError(f"call {i} failed with status {st}")

    for _ in range(args.warmup):
        one_round()
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(n_calls)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        one_round(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    per_call_us = [1000.0 * float(np.mean([evs[k][i][0].elapsed_time(evs[k][i][1])
                                           for k in range(args.steps)])) for i in range(n_calls)]
    res = R.results()
    committed = int(res["n_out"].sum())
    rounds_s = 1000.0 / ms_step

    # dominant kernel: the LM-head call over draft (B(K-1)) and target (B(K+1)) rows
    M = R.M2
    flops = 2.0 * M * cfg.V * cfg.H
    w_bytes = cfg.V * cfg.H * (2 if cfg.dtype == "bf16" else 4)
    head_us = per_call_us[4]
    achieved = flops / (head_us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": f"dmtp_lm_head over {M} rows (prep + GEMM with fused row statistics + merge)",
                "algorithmic_flops": flops, "algorithmic_bytes": w_bytes + M * cfg.H * 2,
                "avg_us": round(head_us, 2)}

    out = {
        "metric": METRIC, "value": round(rounds_s, 2), "unit": "rounds/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded random-init weights and inputs)",
        "config": {"workload": _workload_desc(cfg), "global_batch": cfg.B,
                   "candidates": cfg.K, "parallelism": "single GPU"},
        "accepted_tokens_per_s": round(rounds_s * committed, 1),
        "committed_tokens_per_round": committed,
        "phases_us": dict(zip(["fuse_mtp", "lm_head_t1", "fuse_delta", "block_draft",
                               "lm_head_draft_target", "verify"], [round(x, 2) for x in per_call_us])),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seqs)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
