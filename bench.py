#!/usr/bin/env python3
"""Benchmark: block-sparse video attention on one MI355X.

One step = one vsa_forward call (layout -> selection -> attention) over the
whole workload, inputs already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config hunyuan]

The headline workload is the HunyuanVideo 720p attention shape (B=1, H=24,
N=30x48x80=115200, d=128, tiles 6x8x8, sliding tile window 3x3x5).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("ms/attention call + effective TFLOP/s on retained blocks, "
          "HunyuanVideo-720p shape")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ATTN_SOURCES = ["block_sparse_attention_tile_amd/csrc/attend.hip",
                "block_sparse_attention_tile_amd/csrc/attn_core.h",
                "block_sparse_attention_tile_amd/csrc/attn_core_f8.h"]


def _src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data[kernel_key][workload]
    except (KeyError, ValueError):
        return None
    if ent.get("source_hash") != _src_hash(ATTN_SOURCES):
        return None
    return ent.get("bytes_per_launch")


def _oracle_rows(wl, qn, kn, mem):
    """Kept key tiles of every query tile of one head, by the oracle's own
    selection (static window / sink / dense, or scores with Top-K / Top-P)."""
    from oracle import geometry, select
    nt = geometry.tile_counts(wl.grid, wl.tile)
    nT = len(mem)
    K = min(wl.topk, nT) if wl.topk else (min(select.frac_count(wl.topk_frac, nT), nT) if wl.topk_frac else 0)
    if K or wl.topp:
        S = select.summarized_scores(qn, kn, mem, select.default_scale(wl.d), wl.summarizer)
        rows, _ = select.select_rows(S, nt, window=wl.window, win_mode=wl.win_mode, k=K, p=wl.topp,
                                     sink=wl.sink)
        return rows
    if wl.window is None and not wl.sink:
        return [list(range(nT))] * nT
    rows, _ = select.select_rows(None, nt, window=wl.window, win_mode=wl.win_mode, sink=wl.sink)
    return rows


def _cpu_baseline(wl, q, k, v, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload: its
    own mask, then masked-softmax attention of sampled query tiles (the
    timed part, like the GPU's attention stage)."""
    import numpy as np
    from oracle import attention, geometry
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    mem = geometry.tile_members(wl.grid, wl.tile)
    nT = len(mem)
    done, flops, dt = 0, 0.0, 0.0
    heads = 0
    head_flops = []  # retained FLOPs of each sampled head under the oracle's mask
    for h in range(wl.B * wl.H):
        b_, hh = divmod(h, wl.H)
        qn, kn, vn = (t[b_, hh].float().cpu().numpy() for t in (q, k, v))
        rows = _oracle_rows(wl, qn, kn, mem)
        head_flops.append(sum(4.0 * wl.d * len(mem[i]) * sum(len(mem[j]) for j in rows[i])
                              for i in range(nT)))
        t0 = time.perf_counter()
        for i in np.random.default_rng(h).permutation(nT):
            attention.block_sparse_attention(qn, kn, vn, mem, rows, query_tiles=[int(i)])
            done += 1
            flops += 4.0 * wl.d * len(mem[i]) * sum(len(mem[j]) for j in rows[i])
            if dt + time.perf_counter() - t0 > budget_s:
                break
        dt += time.perf_counter() - t0
        heads += 1
        if dt > budget_s:
            break
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} query tiles of {nT} per head over {heads} head(s) "
                      f"({done * len(mem[0])} query rows), fp64 numpy masked-softmax "
                      f"attention; {dt:.1f} s; {flops:.3e} retained FLOPs",
            "ms_per_call_extrapolated": dt / flops * (sum(head_flops) / len(head_flops)) * wl.B * wl.H * 1e3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="hunyuan")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--summarizer", choices=["mean", "max", "minmax"], default=None,
                    help="override the workload's block summarizer (dynamic masks)")
    ap.add_argument("--sink", type=int, default=None, help="override the workload's sink tiles")
    ap.add_argument("--compute", choices=["bf16", "fp8"], default=None,
                    help="override the attention arithmetic (fp8 = E4M3 Q, K, V and probabilities)")
    ap.add_argument("--no-fp8-leg", action="store_true",
                    help="skip the E4M3 (VSA_COMPUTE_FP8) measurement of the same workload")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: every stage is independent per (batch, head), so N GPUs would each take H/N heads with no exchange; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import block_sparse_attention_tile_amd as vsa
    from synth import CONFIGS, smooth_field_qkv
    from block_sparse_attention_tile_amd.workload import plan_structs as structs_of

    wl = CONFIGS[args.config]
    if args.summarizer is not None:
        wl = wl.with_(summarizer=args.summarizer)
    if args.sink is not None:
        wl = wl.with_(sink=args.sink)
    if args.compute is not None:
        wl = wl.with_(compute=args.compute)
    f8 = wl.compute == "fp8"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name} inputs", file=sys.stderr, flush=True)
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0,
                               device="cuda")
    o = torch.empty_like(q)
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    plan.workspace()
    stream = torch.cuda.current_stream()

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        plan.forward(q, k, v, o)
    torch.cuda.synchronize()
    pairs, flops = plan.retained_work()

    # ---- timed region: exactly `steps` whole calls
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        plan.forward(q, k, v, o)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} calls: {ms:.3f} ms/call", file=sys.stderr, flush=True)

    # ---- per-stage times (same stream, HIP events around each stage)
    def stage(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n_st = max(5, args.steps)
    ms_layout = stage(lambda: plan.layout(q, k, v), n_st)
    ms_select = stage(lambda: plan.select(q, k, v), n_st)
    ms_attend = stage(lambda: plan.attend(o, q, k, v), n_st)
    # a whole call that reuses the mask already in the workspace
    ms_cached = stage(lambda: plan.forward_cached(q, k, v, o), n_st)

    BH = wl.B * wl.H
    # read Q, K, V + write the tile-major copies (no layout stage for the
    # fine-grained mask, which reads the raster tensors directly)
    # (E4M3: one more read of Q, K, V for the per-head maxima, 1-byte writes)
    bytes_layout = 0.0 if wl.fine_group else BH * wl.N * wl.d * (15.0 if f8 else 12.0)
    attn_tflops = flops / (ms_attend * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if f8 else PEAK_BF16_TFLOPS
    traffic = _traffic("attend_fp8" if f8 else "attend", wl.name)
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                "traffic": traffic}

    fp8_leg = None
    if not f8 and not wl.fine_group and not args.no_fp8_leg:
        fp8_leg = _fp8_leg(wl, q, k, v, o, n_st, stage, flops)

    choice = None
    if wl.candidates:  # heads per chosen blocking (SICS or profiling selector)
        import numpy as np
        _, _, cand = plan.read_selection()
        counts = np.bincount(np.asarray(cand), minlength=len(wl.candidates))
        choice = {"x".join(map(str, c)): int(n) for c, n in zip(wl.candidates, counts)}

    cpu = None
    if args.cpu_budget > 0 and not wl.fine_group and not wl.candidates and not f8:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = _cpu_baseline(wl, q, k, v, args.cpu_budget)

    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if f8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} H={wl.H} N={wl.N} "
                               f"({wl.grid[0]}x{wl.grid[1]}x{wl.grid[2]}) d={wl.d} "
                               f"tile {wl.tile[0]}x{wl.tile[1]}x{wl.tile[2]}",
                   "mask": _mask_desc(wl), "retained_pairs": pairs,
                   "retained_flops": flops, "parallelism": "single GPU"},
        "stages_ms": {"layout": round(ms_layout, 4), "select": round(ms_select, 4),
                      "attend": round(ms_attend, 4)},
        "ms_per_call_cached_mask": round(ms_cached, 4),
        "heads_per_blocking": choice,
        "layout_gbs": round(bytes_layout / (ms_layout * 1e-3) / 1e9, 1) if bytes_layout else None,
        "layout_hbm_frac": (round(bytes_layout / (ms_layout * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                            if bytes_layout else None),
        "attend_tflops": round(attn_tflops, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "fp8": fp8_leg,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def _fp8_leg(wl, q, k, v, o, n, stage, flops):
    """The same workload and mask with E4M3 attention (VSA_COMPUTE_FP8):
    whole-call and per-stage times, and the attention kernel against the
    fp8 MFMA peak."""
    import block_sparse_attention_tile_amd as vsa
    from block_sparse_attention_tile_amd.workload import plan_structs
    print("[bench] E4M3 leg", file=sys.stderr, flush=True)
    plan8 = vsa.Plan(*plan_structs(wl.with_(compute="fp8")))
    ms_call = stage(lambda: plan8.forward(q, k, v, o), n)
    ms_layout = stage(lambda: plan8.layout(q, k, v), n)
    ms_attend = stage(lambda: plan8.attend(o, q, k, v), n)
    tf = flops / (ms_attend * 1e-3) / 1e12
    return {"dtype": "fp8-e4m3", "ms_per_call": round(ms_call, 4),
            "value": round(flops / (ms_call * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "stages_ms": {"layout": round(ms_layout, 4), "attend": round(ms_attend, 4)},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": _traffic("attend_fp8", wl.name)}}


def _mask_desc(wl):
    parts = []
    if wl.window:
        parts.append(f"window {wl.window[0]}x{wl.window[1]}x{wl.window[2]} tiles ({wl.win_mode})")
    if wl.topk:
        parts.append(f"top-{wl.topk}")
    if wl.topk_frac:
        parts.append(f"top-k {wl.topk_frac:.0%} of tiles")
    if wl.topp:
        parts.append(f"top-p {wl.topp}")
    if wl.candidates:
        if wl.selector == "profile":
            parts.append(f"profiling selector per head ({(wl.profile_frac or 0.01):.0%} of query rows, "
                         f"candidates {' / '.join('x'.join(map(str, c)) for c in wl.candidates)})")
        else:
            parts.append("SICS blocking choice per head")
    if wl.fine_group:
        parts.append(f"fine M={wl.fine_group} keep {wl.fine_keep:.0%}")
    if (wl.topk or wl.topk_frac or wl.topp) and wl.summarizer != "mean":
        parts.append(f"{wl.summarizer} summarizer")
    if wl.sink:
        parts.append(f"sink {wl.sink} tiles")
    return ", ".join(parts) or "dense"


if __name__ == "__main__":
    main()
