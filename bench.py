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


def _src_hash(paths):
    """Hash of the code in source files: comments and whitespace do not count
    (a kernel is unchanged when only its comments change)."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = "block_sparse_attention_tile_amd/csrc"


def _kernel_sources(name):
    """The source files a kernel is built from: the csrc file that defines
    its base name and every local header that file reaches."""
    import re
    base = re.match(r"(?:void\s+)?(?:\w+::)*(\w+)", name.strip()).group(1)
    files = []
    for f in sorted(os.listdir(os.path.join(ROOT, CSRC))):
        if f.endswith(".hip") and re.search(r"void\s+%s\s*\(" % re.escape(base),
                                             open(os.path.join(ROOT, CSRC, f)).read()):
            files.append(f"{CSRC}/{f}")
    if not files:
        return base, None
    todo, seen = list(files), []
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.append(f)
        for inc in re.findall(r'^#include "([^"]+)"', open(os.path.join(ROOT, f)).read(), re.M):
            todo.append(os.path.normpath(os.path.join(os.path.dirname(f), inc)))
    return base, seen


def _traffic(fragment, workload):
    """HBM bytes of one attention stage: the kernels whose names contain
    `fragment` (one launch per blocking), from the committed rocprofv3
    counter runs of `workload`; None when there are none or a kernel's
    sources changed since they were taken."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        kernels = json.load(open(TRAFFIC_JSON))["workloads"][workload]["kernels"]
    except (KeyError, ValueError):
        return None
    hits = [e for n, e in kernels.items() if fragment in n]
    if not hits or any(e.get("source_hash") != _src_hash(e["sources"]) for e in hits):
        return None
    return sum(e["bytes_per_launch"] for e in hits)


def _short_name(name):
    """A rocprofv3 kernel name without its parameter list, leading `void` or
    anonymous namespaces: `vsa::attend_kernel<vsa::Bf16Core<128>, 12, 4, 1, false>`."""
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(", 1)[0].strip()


def _counter_csv(path, counter):
    """Per-dispatch values of one counter from a rocprofv3 counter_collection
    csv: {kernel name: [value per dispatch]}."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            key = (_short_name(r["Kernel_Name"]), r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), val in per.items():
        out.setdefault(name, []).append(val)
    return out


def write_traffic(workload, fetch_csv, write_csv, command):
    """Record HBM bytes per dispatch (medians) of every kernel of one
    workload's counter runs in profiles/traffic.json.  The scale of each
    counter comes from the largest plain device copy (`--copy-calib`, 1 GiB)
    in the same run: bytes = counter KiB x 1024 / (counter KiB of the copy /
    bytes the copy reads or writes)."""
    import statistics
    fetch, write = _counter_csv(fetch_csv, "FETCH_SIZE"), _counter_csv(write_csv, "WRITE_SIZE")
    copy = "__amd_rocclr_copyBuffer"
    if copy not in fetch or copy not in write:
        raise SystemExit("no device copy in the counter runs: run bench.py with --copy-calib")
    nbytes = 1 << 30
    f_cal, w_cal = max(fetch[copy]), max(write[copy])
    ff, wf = f_cal * 1024.0 / nbytes, w_cal * 1024.0 / nbytes
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data.setdefault("workloads", {})
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        base, srcs = _kernel_sources(name)
        if srcs is None:
            continue  # not a kernel of this library (torch, the runtime's copies)
        fk, wk = statistics.median(fetch[name]), statistics.median(write[name])
        fb, wb = fk * 1024.0 / ff, wk * 1024.0 / wf
        kernels[name] = {"base": base, "sources": srcs, "source_hash": _src_hash(srcs),
                         "dispatches": len(fetch[name]), "fetch_kib_raw": fk, "write_kib_raw": wk,
                         "fetch_bytes": round(fb), "write_bytes": round(wb),
                         "bytes_per_launch": round(fb + wb)}
    data["workloads"][workload] = {
        "command": command,
        "calibration": {"kernel": f"{copy}, device copy of 1 GiB", "bytes": nbytes,
                        "FETCH_SIZE_kib": f_cal, "WRITE_SIZE_kib": w_cal,
                        "fetch_factor": ff, "write_factor": wf},
        "kernels": kernels}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    for name, e in kernels.items():
        print(f"{name[:90]:90s} x{e['dispatches']:3d}  read {e['fetch_bytes'] / 1e9:8.3f} GB"
              f"  written {e['write_bytes'] / 1e9:8.3f} GB")


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
            "kind": "oracle", "host_cores": os.cpu_count(), "cpu_model": _cpu_model(),
            "sample": f"{done} query tiles of {nT} per head over {heads} head(s) "
                      f"({done * len(mem[0])} query rows), fp64 numpy masked-softmax "
                      f"attention; {dt:.1f} s; {flops:.3e} retained FLOPs",
            "ms_per_call_extrapolated": dt / flops * (sum(head_flops) / len(head_flops)) * wl.B * wl.H * 1e3}


def _cpu_model():
    """The host CPU's model name (lscpu), for the CPU baseline's record."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    return None


def _copy_gbs(dev, stage):
    """Device-to-device copy of 1 GiB (torch copy_) in the same run: the
    practical ceiling of a read+write HBM stream on this part."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    ms = stage(lambda: b.copy_(a), 10)
    del a, b
    return 2.0 * (1 << 30) / (ms * 1e-3) / 1e9


def _gemm_tflops(dev, stage):
    """A dense bf16 GEMM (torch.matmul, 8192^3, random operands) in the same
    run: what a library contraction with data-dependent operand toggling
    reaches on this part, next to the datasheet peak."""
    import torch
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
    ms = stage(lambda: torch.matmul(a, b, out=c), 20)
    del a, b, c
    return 2.0 * 8192 ** 3 / (ms * 1e-3) / 1e12


def _ceilings(dev, stage):
    """Same-run practical ceilings (libvsa_probe.so): the attention's MFMA
    shape (32x32x16 bf16) issued back to back at 12 waves per CU on random
    operands that change at every product, and a plain 2 GiB HBM read
    (best over grid sizes, with and without non-temporal loads)."""
    import torch
    from block_sparse_attention_tile_amd import probe
    g = torch.Generator(device=dev).manual_seed(1)
    src = torch.randn(64 * probe.SLICE_BYTES // 2, device=dev, dtype=torch.bfloat16, generator=g)
    wgs, iters = 256 * 4, 3000
    out = torch.empty(wgs * probe.WAVES * 64, device=dev, dtype=torch.float32)
    flops = probe.mfma_rate(src, out, wgs, iters)
    ms = stage(lambda: probe.mfma_rate(src, out, wgs, iters), 5)
    mfma = flops / (ms * 1e-3) / 1e12
    del src, out
    buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev).fill_(0x5A)
    rd = []
    for wg in (1024, 4096, 16384):
        o = torch.empty(wg * 256, dtype=torch.int32, device=dev)
        for nt in (False, True):
            ms = stage(lambda: probe.read_rate(buf, o, wg, nt), 5)
            rd.append(buf.numel() / (ms * 1e-3) / 1e9)
    del buf
    return {"mfma_bf16_random_tflops": round(mfma, 1), "hbm_read_gbs": round(max(rd), 1),
            "mfma_probe": f"{wgs} workgroups x 12 waves x {iters} x 64 products, random operands"}


def _clamp_leg(wl, q, k, v, o, n, stage):
    """The same static workload with the window clamped at the grid edge
    (every window keeps its full 3x3x5 size: 13,500 tile pairs per head at
    HunyuanVideo instead of 9,152)."""
    import block_sparse_attention_tile_amd as vsa
    from block_sparse_attention_tile_amd.workload import plan_structs
    print("[bench] clamped-window leg", file=sys.stderr, flush=True)
    plan_c = vsa.Plan(*plan_structs(wl.with_(win_mode="clamp")))
    ms_call = stage(lambda: plan_c.forward(q, k, v, o), n)
    ms_attend = stage(lambda: plan_c.attend(o, q, k, v), n)
    pairs, flops = plan_c.retained_work()
    return {"mask": _mask_desc(wl.with_(win_mode="clamp")), "retained_pairs": pairs,
            "retained_flops": flops, "ms_per_call": round(ms_call, 4),
            "attend_ms": round(ms_attend, 4),
            "value": round(flops / (ms_call * 1e-3) / 1e12, 2),
            "attend_tflops": round(flops / (ms_attend * 1e-3) / 1e12, 2),
            "attend_frac": round(flops / (ms_attend * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


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
    ap.add_argument("--no-clamp-leg", action="store_true",
                    help="skip the clamped-window measurement of a static-window workload")
    ap.add_argument("--no-fp8-leg", action="store_true",
                    help="skip the E4M3 (VSA_COMPUTE_FP8) measurement of the same workload")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: record the HBM bytes per dispatch of the config's kernels "
                         "from two rocprofv3 counter_collection csv files (FETCH_SIZE, then "
                         "WRITE_SIZE, each a run of bench.py --copy-calib) in profiles/traffic.json")
    ap.add_argument("--command", default="",
                    help="with --write-traffic: the profiling command to record beside the numbers")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.config, args.write_traffic[0], args.write_traffic[1], args.command)
        return
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
    # an event between consecutive calls gives each call's own time as well
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        plan.forward(q, k, v, o)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_call = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
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
    # bf16: read K, V (and Q for dynamic masks' summaries) + write tile-major K
    # and V^T (the attention reads Q in raster order); E4M3: read Q, K, V for
    # the per-head maxima, again for the 1-byte tile-major copies of all three.
    # No layout stage for the fine-grained mask (it reads the raster tensors).
    pool = bool(wl.topk or wl.topk_frac or wl.topp)
    per_tok = 15.0 if f8 else (10.0 if pool else 8.0)
    bytes_layout = 0.0 if wl.fine_group else BH * wl.N * wl.d * per_tok
    attn_tflops = flops / (ms_attend * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if f8 else PEAK_BF16_TFLOPS
    traffic = _traffic(("fine_attend_kernel" if wl.fine_group else
                        "attend_kernel<vsa::F8Core" if f8 else "attend_kernel<vsa::Bf16Core"), wl.name)
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                "traffic": traffic}

    fp8_leg = None
    if not f8 and not wl.fine_group and not args.no_fp8_leg:
        fp8_leg = _fp8_leg(wl, q, k, v, o, n_st, stage, flops)
    clamp_leg = None
    if wl.window and wl.win_mode == "truncate" and not (wl.topk or wl.topk_frac or wl.topp) \
            and not wl.candidates and not f8 and not args.no_clamp_leg:
        clamp_leg = _clamp_leg(wl, q, k, v, o, n_st, stage)
    copy_gbs = None if wl.fine_group else _copy_gbs(dev, stage)
    gemm_tflops = None if wl.fine_group or f8 else _gemm_tflops(dev, stage)
    ceilings = None if wl.fine_group else _ceilings(dev, stage)

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
        "ms_per_step_median": round(per_call[len(per_call) // 2], 4),
        "ms_per_step_min": round(per_call[0], 4),
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
        "hbm_copy_gbs": round(copy_gbs, 1) if copy_gbs else None,
        "layout_copy_frac": (round(bytes_layout / (ms_layout * 1e-3) / 1e9 / copy_gbs, 4)
                             if bytes_layout and copy_gbs else None),
        "attend_tflops": round(attn_tflops, 2),
        "gemm_bf16_tflops": round(gemm_tflops, 1) if gemm_tflops else None,
        "attend_gemm_frac": round(attn_tflops / gemm_tflops, 4) if gemm_tflops else None,
        "ceilings": ceilings,
        "attend_mfma_ceiling_frac": (round(attn_tflops / ceilings["mfma_bf16_random_tflops"], 4)
                                     if ceilings and not f8 else None),
        "layout_read_ceiling_frac": (round(bytes_layout / (ms_layout * 1e-3) / 1e9 / ceilings["hbm_read_gbs"], 4)
                                     if ceilings and bytes_layout else None),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "fp8": fp8_leg,
        "clamp_window": clamp_leg,
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
                         "traffic": _traffic("attend_kernel<vsa::F8Core", wl.name)}}


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
