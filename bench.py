#!/usr/bin/env python3
"""Throughput of one DMTP draft+verify round on one MI355X.

A step is one whole round (MTP fusion, T1 head, DMTP residual, block draft,
shared LM head over draft and target rows, verification) over one batch of
synthetic, seeded inputs already resident in HBM.  Default workload: batch 32,
hidden 2048, vocabulary 151936, one block-draft layer (16 query / 4 kv heads
x 128, SwiGLU 6144), 7 candidates (8 draft slots, 8 verify rows), context
lengths uniform in [1024, 4096], greedy.

Prints one JSON line.  value = rounds/s over the timed steps: W untimed
rounds, then K rounds back to back between two events, holding nothing but
the ABI calls of each round.  Extra fields, each from its own pass after the
timed loop:
  round_us_warm / round_us_cold  median, p10 and p90 of rounds timed one by one
      (cold: each after writes that evict the last-level cache);
  roofline  the dominant kernel (the LM-head GEMM over the 448 draft+target
      rows), timed by the events attached to its own dispatch on every round
      of a dedicated pass;
  phases    per-call medians with each call's algorithmic bytes and its
      fraction of the HBM (or matrix-core) peak;
  attention the drafter's context-attention kernel (first layer), timed by
      the events of its own dispatch in the same pass as the dominant kernel,
      against the context K/V bytes it reads;
  verify_scan  (sampled workloads verified by rejection sampling) the
      verifier's pass over the drawn rows' logits, timed the same way, against
      the float32 rows it reads;
  cpu_baseline  the CPU oracle on a bounded sample, with the host CPU model.
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
            f"({cfg.S} slots, {cfg.R} verify rows), ctx U[{cfg.ctx_min},{cfg.ctx_max}] "
            f"(drafter window {cfg.window or 'all'}), "
            f"tau={cfg.tau_mode}"
            + (f", verify={cfg.verify}" if cfg.tau_mode != "greedy" else ", greedy verify")
            + (", MTP decoder block" if cfg.mtp_block else ""))


# Sources the LM-head GEMM is compiled from; a counter summary taken on other
# sources is stale and its traffic figure is not reported.
HEAD_SOURCES = ("mtp_block_draft_amd/csrc/lm_head.hip", "mtp_block_draft_amd/csrc/dma.hpp",
                "mtp_block_draft_amd/csrc/common.hpp", "mtp_block_draft_amd/csrc/gemm_core.hpp")
TRAFFIC_SUMMARY = "profiles/lm_head_gemm_b32_448rows_counters.md"


def head_kernel_name(M: int, packed: bool = False) -> str:
    """The kernel dmtp_lm_head runs for its vocabulary GEMM over M bf16 rows (H a
    multiple of 128, more than 32 rows): row chunks of at most 448, 64-row tiles
    per workgroup; three or more tiles take the register-input kernel, which
    streams the packed copy of the weights when the call is given one."""
    nc = -(-M // 448)
    tb = -(-(-(-M // nc)) // 64)
    if tb >= 3:
        return f"head_gemm_xr_kernel<{tb}, 4, {'true' if packed else 'false'}>"
    return f"head_gemm_mf32_kernel<{tb}, 64>"


def head_fingerprint() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in HEAD_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the LM-head GEMM from the committed counter summary,
    or None when there is none or it was taken on different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_fingerprint") != head_fingerprint():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def rocprof_summary(args) -> int:
    """Print markdown summary lines from rocprofv3 CSV output (kernel stats, or
    FETCH_SIZE / WRITE_SIZE counter collections with the copy-probe calibration)."""
    import csv
    import re

    def short(name):
        n = re.sub(r"\(anonymous namespace\)::|dmtp::", "", name)
        return re.sub(r"\(.*", "", n)

    if args.stats:
        rows = list(csv.DictReader(open(args.stats)))
        print("| kernel | calls | avg us | min us | max us | share |")
        print("|---|---|---|---|---|---|")
        for r in rows[:args.top]:
            print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.1f}% |")
        return 0

    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault((short(r["Kernel_Name"]), int(r["Grid_Size"])), []).append(
                float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in out.items()}

    fetch = per_kernel(args.fetch, "FETCH_SIZE")
    write = per_kernel(args.write, "WRITE_SIZE")
    copy_bytes = args.copy_mib * 2 ** 20

    def pick(d, pat):
        cands = [(k, v) for k, v in d.items() if pat in k[0]]
        if not cands:
            raise SystemExit(f"no kernel matching {pat!r}")
        return max(cands, key=lambda kv: kv[1])

    (_, cf) = pick(fetch, args.copy_kernel)
    (_, cw) = pick(write, args.copy_kernel)
    f_scale = copy_bytes / (cf * 1024)
    w_scale = copy_bytes / (cw * 1024)
    (kk, kf) = pick(fetch, args.kernel)
    kw = write.get(kk, 0.0)
    traffic = kf * 1024 * f_scale + kw * 1024 * w_scale
    print(f"- kernel: `{kk[0]}` (grid {kk[1]})")
    print(f"- kernel_fingerprint: `{head_fingerprint()}`")
    print(f"- fetch_kib_per_launch: {kf:.1f}")
    print(f"- write_kib_per_launch: {kw:.1f}")
    print(f"- copy_probe_bytes: {copy_bytes}")
    print(f"- copy_probe_fetch_kib: {cf:.1f}")
    print(f"- copy_probe_write_kib: {cw:.1f}")
    print(f"- fetch_scale: {f_scale:.4f}")
    print(f"- write_scale: {w_scale:.4f}")
    print(f"- traffic_bytes_per_launch: {traffic:.0f}")
    return 0


def cpu_baseline(inp, n_seq: int, min_seconds: float = 10.0):
    """The oracle as it stands, on the host cores: whole rounds (or the first
    n_seq sequences of one, scaled) repeated until min_seconds have passed."""
    from threadpoolctl import threadpool_info
    from oracle import dmtp as odm

    seqs = list(range(min(n_seq, inp.cfg.B)))
    reps, t0 = 0, time.perf_counter()
    while True:
        odm.run_round(inp, seqs=seqs)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    scale = inp.cfg.B / len(seqs)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": reps / (dt * scale), "unit": "rounds/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle, {reps} repetitions of {len(seqs)} of {inp.cfg.B} "
                      f"sequences of one round ({dt:.1f} s)"
                      + (f", scaled x{scale:g} to a whole round" if scale != 1 else ""),
            "seconds": dt}


def ctx_kv_bench(R, cfg, stream, steps: int, warmup: int):
    """Time dmtp_ctx_kv on the rows one round can commit (B (K + 1)), five bf16
    feature streams per row, into fresh caches of the drafter layers' shapes."""
    import torch
    from mtp_block_draft_amd import call, ctx_kv, layer_arg, lib, workspace_bytes

    N, H, nf = cfg.B * (cfg.K + 1), cfg.H, 5
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed + 7)
    feats = torch.randn(N, nf, H, generator=gen, device="cuda").to(tdt)
    w_fc = (0.02 * torch.randn(H, nf * H, generator=gen, device="cuda")).to(tdt)
    pos = torch.arange(N, dtype=torch.int32, device="cuda") + 4096
    dst = torch.arange(N, dtype=torch.int32, device="cuda")
    layers = [layer_arg(**lt) for lt in R.layers_t]
    kc = [torch.empty(N, cfg.Hkv, cfg.d, dtype=tdt, device="cuda") for _ in layers]
    vc = [torch.empty(N, cfg.Hkv, cfg.d, dtype=tdt, device="cuda") for _ in layers]
    desc = ctx_kv(feats, pos, dst, w_fc, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, layers=layers, k_cache=kc,
                  v_cache=vc, eps=cfg.eps, rope_base=cfg.rope_base, run=False)
    ws = torch.empty(max(workspace_bytes("ctx_kv", desc), 256), dtype=torch.uint8, device="cuda")
    call("ctx_kv", desc, ws)
    # the entry point itself, as the round loop calls it (no per-call query)
    import ctypes
    fn, ref = lib.dmtp_ctx_kv, ctypes.byref(desc)
    wsp, wsn, sp = ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(stream.cuda_stream)
    for _ in range(warmup):
        fn(ref, wsp, wsn, sp)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        if fn(ref, wsp, wsn, sp) != 0:
            raise RuntimeError("dmtp_ctx_kv failed")
    b.record(stream)
    torch.cuda.synchronize()
    us = 1000.0 * a.elapsed_time(b) / steps
    esz = 2 if cfg.dtype == "bf16" else 4
    nbytes = (H * nf * H + len(layers) * 2 * cfg.Hkv * cfg.d * H + N * nf * H
              + len(layers) * 2 * N * cfg.Hkv * cfg.d) * esz
    return {"rows": N, "feature_streams": nf, "layers": len(layers), "us": round(us, 2),
            "algorithmic_bytes": nbytes, "gb_s": round(nbytes / us / 1e3, 1),
            "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}


def _pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs, dtype=np.float64), q)), 2)


def _dist(us):
    """Median and 10th / 90th percentiles of per-round microseconds."""
    return {"n": len(us), "median_us": _pct(us, 50), "p10_us": _pct(us, 10), "p90_us": _pct(us, 90)}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def phase_model(cfg, inp, n_sampled_rows: int):
    """Algorithmic bytes (and flops) of each call of one round, and its bound.

    Bytes count what the call must move at least once: weights and tables in
    the storage dtype, the context keys and values the drafter reads (the last
    `window` rows of each sequence), input and output rows.  The LM-head call
    over draft and target rows is a matrix-core bound when it has at least 312
    rows (the bf16 ridge of 2.5 PFLOP/s over 8 TB/s)."""
    import numpy as np
    esz = 2 if cfg.dtype == "bf16" else 4
    B, H, V, K, S = cfg.B, cfg.H, cfg.V, cfg.K, cfg.S
    fuse_b = 2 * H * H * esz + 2 * B * H * esz + B * H * 4
    head_w = V * H * esz
    L = np.asarray(inp.ctx_len, dtype=np.int64)
    if cfg.window:
        L = np.minimum(L, cfg.window)
    kv_rows = int(L.sum())
    layer_w = (cfg.qkv_dim * H + H * cfg.Hq * cfg.d + 3 * cfg.F * H) * esz
    draft_b = cfg.n_layers * (layer_w + 2 * kv_rows * cfg.Hkv * cfg.d * esz) + B * S * H * esz
    m2 = B * (K - 1) + B * (K + 1)
    logits_b = n_sampled_rows * V * 4
    out = {
        "fuse_mtp": {"bound": "hbm", "bytes": fuse_b},
        "lm_head_t1": {"bound": "hbm", "bytes": head_w + B * H * 4},
        "fuse_delta": {"bound": "hbm", "bytes": fuse_b},
        "block_draft": {"bound": "hbm", "bytes": draft_b},
        "lm_head_draft_target": {"bound": "mfma" if m2 >= 312 else "hbm",
                                 "bytes": head_w + m2 * H * esz + logits_b,
                                 "flops": 2.0 * m2 * V * H},
        "verify": {"bound": "latency", "bytes": None},
    }
    if cfg.mtp_block:
        # the block reads its whole cache (no window)
        cache_rows = int(np.asarray(inp.ctx_len, dtype=np.int64).sum())
        out["mtp_block"] = {"bound": "hbm",
                            "bytes": layer_w + 2 * cache_rows * cfg.Hkv * cfg.d * esz}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="b32_greedy_bf16")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the round captured as one HIP graph (the LM-head "
                         "GEMM is still timed by its dispatch events in an eager pass)")
    ap.add_argument("--verify", choices=["rejection", "target_only"], default=None,
                    help="verification of sampled rows (default: the workload's)")
    ap.add_argument("--ctx-kv", action="store_true",
                    help="also time dmtp_ctx_kv on the rows one round can commit")
    ap.add_argument("--mtp-block", action="store_true",
                    help="h_MTP from an MTP decoder block (drafter layer shapes, causal over its "
                         "own KV cache) instead of h_MTP = h'")
    ap.add_argument("--dist-rounds", type=int, default=200,
                    help="rounds timed one by one (warm, and after a cache flush) for the "
                         "median and p10 / p90")
    ap.add_argument("--kernel-rounds", type=int, default=100,
                    help="rounds of the pass that times the dominant kernel by its own "
                         "dispatch events")
    ap.add_argument("--cpu-seqs", type=int, default=32, help="sequences in the oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warm-up, copy this many MiB device-to-device once (a kernel "
                         "of known traffic, for calibrating FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--rocprof-summary", action="store_true",
                    help="summarise rocprofv3 CSV output instead of running (see --stats, "
                         "--fetch, --write)")
    ap.add_argument("--stats", help="rocprofv3 kernel_stats.csv")
    ap.add_argument("--top", type=int, default=20)
    ap.add_argument("--fetch", help="counter_collection.csv of a FETCH_SIZE pass")
    ap.add_argument("--write", help="counter_collection.csv of a WRITE_SIZE pass")
    ap.add_argument("--kernel", default="head_gemm_xr_kernel<7,")
    ap.add_argument("--copy-kernel", default="elementwise")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="repeat each LM-head call of the round alone for this many seconds "
                         "(for power and clock readings taken alongside), then exit")
    args = ap.parse_args()
    if args.rocprof_summary:
        return rocprof_summary(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the round is "
              "data-parallel over sequences and is not sharded here", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import dmtp_synth as synth
    from mtp_block_draft_amd.round import Round

    cfg = synth.CONFIGS[args.config]
    if args.verify:
        cfg = cfg.with_(verify=args.verify)
    if args.mtp_block:
        cfg = cfg.with_(mtp_block=True)
    inp = synth.make_inputs(cfg)
    R = Round(inp)
    stream = torch.cuda.current_stream()
    s_ptr = stream.cuda_stream
    import ctypes
    sp = ctypes.c_void_p(s_ptr)
    n_calls = len(R._fns)

    # The head GEMM of the draft + target call can be timed by its own
    # dispatch: the descriptor carries a start/stop hipEvent pair, which the
    # library hands to hipExtLaunchKernel, so no extra command enters the
    # stream.  Events come from the HIP runtime torch has loaded.
    hip_path = next(l.split()[-1] for l in open("/proc/self/maps").read().splitlines()
                    if "libamdhip64" in l)
    hip = ctypes.CDLL(hip_path)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    head_desc = R.d_head_c
    draft_desc = R.d_draft
    verify_desc = R.d_verify
    # the verifier's pass over the drawn rows' logits runs when sequences are
    # sampled and verified by rejection sampling
    has_scan = bool((inp.tau > 0).any()) and cfg.verify == "rejection"

    def one_round(gemm_ev=None, call_evs=None, attn_ev=None, mass_ev=None):
        head_desc.gemm_start_event = gemm_ev[0] if gemm_ev else None
        head_desc.gemm_stop_event = gemm_ev[1] if gemm_ev else None
        draft_desc.attn_start_event = attn_ev[0] if attn_ev else None
        draft_desc.attn_stop_event = attn_ev[1] if attn_ev else None
        verify_desc.mass_start_event = mass_ev[0] if mass_ev else None
        verify_desc.mass_stop_event = mass_ev[1] if mass_ev else None
        for i, (fn, ref) in enumerate(R._fns):
            if call_evs is not None:
                call_evs[i][0].record(stream)
            st = fn(ref, R._ws_ptr, R._ws_bytes, sp)
            if call_evs is not None:
                call_evs[i][1].record(stream)
            if st != 0:
                raise RuntimeError(f"call {i} failed with status {st}")

    def ev():
        return torch.cuda.Event(enable_timing=True)

    if args.sustain > 0:
        # each head call of the round on its own, back to back, for a few
        # seconds: a steady load for readings of power and clocks
        one_round()
        torch.cuda.synchronize()
        for name in ("lm_head_draft_target", "lm_head_t1"):
            fn, ref = R._fns[R.step_names.index(name)]
            t0 = time.time()
            n = 0
            while time.time() - t0 < args.sustain:
                for _ in range(20):
                    if fn(ref, R._ws_ptr, R._ws_bytes, sp) != 0:
                        raise RuntimeError(f"{name} failed")
                torch.cuda.synchronize()
                n += 20
            t1 = time.time()
            print(json.dumps({"sustain": name, "start": round(t0, 3), "end": round(t1, 3), "calls": n,
                              "us_per_call": round((t1 - t0) / n * 1e6, 2)}), flush=True)
        return 0

    if args.copy_probe_mib:
        # one elementwise kernel that reads and writes exactly N MiB
        src = torch.ones((args.copy_probe_mib << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- rounds timed one by one: an event pair around each round (warm), and
    # the same after 512 MB of writes that evict the 256 MB last-level cache
    # (cold: back-to-back rounds share part of that cache -- drafter weights,
    # context K/V -- which a target forward pass between rounds would evict)
    n_dist = max(args.dist_rounds, 1)
    wev = [(ev(), ev()) for _ in range(n_dist)]
    for a, b in wev:
        a.record(stream)
        one_round()
        b.record(stream)
    torch.cuda.synchronize()
    warm_us = [1000.0 * a.elapsed_time(b) for a, b in wev]
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
    fev = [(ev(), ev()) for _ in range(n_dist)]
    for k, (a, b) in enumerate(fev):
        flush.fill_(float(k))
        a.record(stream)
        one_round()
        b.record(stream)
    torch.cuda.synchronize()
    cold_us = [1000.0 * a.elapsed_time(b) for a, b in fev]
    del flush
    print(f"# {n_dist} single rounds: warm median {np.median(warm_us):.1f} us, cold median "
          f"{np.median(cold_us):.1f} us", file=sys.stderr, flush=True)

    # ---- the dominant kernel, timed by the events attached to its own
    # dispatch on every round of a dedicated pass, after untimed rounds that
    # let the caches and clocks settle from the flushes above
    n_settle = 16
    for _ in range(n_settle):
        one_round()
    n_k = max(args.kernel_rounds, 1)

    def hip_pairs():
        out = []
        for _ in range(n_k):
            pair = (ctypes.c_void_p(), ctypes.c_void_p())
            if hip.hipEventCreate(ctypes.byref(pair[0])) or hip.hipEventCreate(ctypes.byref(pair[1])):
                raise RuntimeError("hipEventCreate failed")
            out.append(pair)
        return out

    def hip_elapsed_us(pairs):
        out = []
        for a, b in pairs:
            ms = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(ms), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(1000.0 * ms.value)
            hip.hipEventDestroy(a)
            hip.hipEventDestroy(b)
        return out

    # the context attention of the drafter's first layer is timed the same
    # way, in the same rounds (a kernel inside the block_draft call)
    gev, aev = hip_pairs(), hip_pairs()
    mev = hip_pairs() if has_scan else [None] * n_k
    for k in range(n_k):
        one_round(gemm_ev=gev[k], attn_ev=aev[k], mass_ev=mev[k])
    torch.cuda.synchronize()
    gemm_us = hip_elapsed_us(gev)
    attn_us = hip_elapsed_us(aev)
    mass_us = hip_elapsed_us(mev) if has_scan else None
    one_round()   # leaves the descriptors without events
    torch.cuda.synchronize()

    # ---- per-call durations, from a separate pass (events between calls add
    # a few microseconds each, so they stay out of the passes above)
    n_diag = 50
    evs = [[[ev(), ev()] for _ in range(n_calls)] for _ in range(n_diag)]
    for k in range(n_diag):
        one_round(call_evs=evs[k])
    torch.cuda.synchronize()
    per_call_us = [1000.0 * float(np.median([evs[k][i][0].elapsed_time(evs[k][i][1])
                                             for k in range(n_diag)])) for i in range(n_calls)]
    pre_rounds = 2 * n_dist + n_settle + n_k + 1 + n_diag

    # ---- the headline: W untimed rounds, then exactly K rounds back to back,
    # with nothing but the round's calls between the two events.  It runs after
    # the diagnostic passes above, so it measures a GPU in its steady state: on
    # a GPU fresh from idle the LM-head GEMM runs up to 30 % slower for the
    # first 20 to 30 rounds while the power controller settles.
    for _ in range(args.warmup):
        one_round()
    torch.cuda.synchronize()
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        one_round()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    print(f"# headline: {args.steps} rounds, {1000.0 * ms_step:.2f} us per round", file=sys.stderr,
          flush=True)

    graph_ms_step = None
    if args.graph:
        R.capture()
        for _ in range(args.warmup):
            R.replay()
        torch.cuda.synchronize()
        g0, g1 = ev(), ev()
        g0.record(stream)
        for _ in range(args.steps):
            R.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms_step = g0.elapsed_time(g1) / args.steps

    res = R.results()
    committed = int(res["n_out"].sum())
    eager_ms_step = ms_step
    if graph_ms_step is not None:
        ms_step = graph_ms_step
    rounds_s = 1000.0 / ms_step

    # dominant kernel: the LM-head GEMM over draft (B(K-1)) and target (B(K+1)) rows
    M = R.M2
    flops = 2.0 * M * cfg.V * cfg.H
    w_bytes = cfg.V * cfg.H * (2 if cfg.dtype == "bf16" else 4)
    head_us = float(np.mean(gemm_us))
    achieved = flops / (head_us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = recorded_traffic() if args.config == "b32_greedy_bf16" else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": f"{head_kernel_name(M, R.w_head_packed is not None)} of dmtp_lm_head over {M} rows (bf16 GEMM "
                          f"with fused row statistics), timed by the events of its own "
                          f"dispatch on each of {n_k} rounds of a dedicated pass",
                "algorithmic_flops": flops, "algorithmic_bytes": w_bytes + M * cfg.H * 2,
                "avg_us": round(head_us, 2), "median_us": _pct(gemm_us, 50),
                "p10_us": _pct(gemm_us, 10), "p90_us": _pct(gemm_us, 90)}

    n_sampled = int((inp.tau > 0).sum()) * (2 * cfg.K + 1)
    model = phase_model(cfg, inp, n_sampled)
    phases = {}
    for name, us in zip(R.step_names, per_call_us):
        m = model.get(name, {"bound": "latency", "bytes": None})
        e = {"us": round(us, 2), "bound": m["bound"]}
        if m.get("bytes"):
            e["bytes"] = int(m["bytes"])
            e["hbm_frac"] = round(m["bytes"] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        if m.get("flops") and m["bound"] == "mfma":
            e["mfma_frac"] = round(m["flops"] / (us * 1e-6) / 1e12 / peak, 4)
        phases[name] = e

    # context K/V bytes the first layer's attention kernel reads (the last
    # `window` rows of each sequence, keys and values of every kv head)
    L = np.asarray(inp.ctx_len, dtype=np.int64)
    if cfg.window:
        L = np.minimum(L, cfg.window)
    attn_bytes = int(L.sum()) * 2 * cfg.Hkv * cfg.d * (2 if cfg.dtype == "bf16" else 4)
    attn_avg = float(np.mean(attn_us))
    attention = {"kernel": "context attention of draft layer 0 (attn_wave_kernel), timed by the "
                           f"events of its own dispatch on each of {n_k} rounds of the same pass",
                 "bound": "hbm", "bytes": attn_bytes, "avg_us": round(attn_avg, 2),
                 "median_us": _pct(attn_us, 50), "p10_us": _pct(attn_us, 10),
                 "p90_us": _pct(attn_us, 90),
                 "hbm_frac": round(attn_bytes / (attn_avg * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}

    scan = None
    if has_scan:
        # the rows the pass reads: p and q of each residual draw, p of each
        # bonus draw (sampled sequences; the round is seeded, so every round
        # draws the same)
        acc_len = R.accept_len.cpu().numpy()
        samp = np.asarray(inp.tau) > 0
        n_res = int(((acc_len < cfg.K) & samp).sum())
        n_bon = int(((acc_len >= cfg.K) & samp).sum())
        scan_bytes = (2 * n_res + n_bon) * cfg.V * 4
        m_avg = float(np.mean(mass_us))
        scan = {"kernel": "verify_mass_kernel (block masses of max(0, p - q) and of p over the drawn "
                          f"rows), timed by the events of its own dispatch on each of {n_k} rounds of "
                          "the same pass",
                "bound": "hbm", "residual_draws": n_res, "bonus_draws": n_bon, "bytes": scan_bytes,
                "avg_us": round(m_avg, 2), "median_us": _pct(mass_us, 50),
                "p10_us": _pct(mass_us, 10), "p90_us": _pct(mass_us, 90),
                "hbm_frac": round(scan_bytes / (m_avg * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}

    greedy = not bool((inp.tau > 0).any())
    out = {
        "metric": METRIC, "value": round(rounds_s, 2), "unit": "rounds/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded random-init weights and inputs)",
        "config": {"workload": _workload_desc(cfg), "global_batch": cfg.B,
                   "candidates": cfg.K, "verify": "greedy" if greedy else cfg.verify,
                   "parallelism": "single GPU",
                   "submission": "one HIP graph per round" if args.graph else
                   f"{n_calls} calls per round"},
        "pre_rounds": pre_rounds,
        "accepted_tokens_per_s": round(rounds_s * committed, 1),
        "committed_tokens_per_round": committed,
        "round_us_warm": _dist(warm_us),
        "round_us_cold": dict(_dist(cold_us), note="each round after 512 MB of writes that "
                              "evict the 256 MB last-level cache"),
        "phases": phases,
        "attention": attention,
        "roofline": roofline,
        "host_cpu": host_cpu_model(),
    }
    if scan is not None:
        out["verify_scan"] = scan
    if graph_ms_step is not None:
        out["eager_rounds_per_s"] = round(1000.0 / eager_ms_step, 2)
    if args.ctx_kv:
        out["ctx_kv"] = ctx_kv_bench(R, cfg, stream, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seqs, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
