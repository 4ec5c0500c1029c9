"""Turn a workload description (any object with the attributes below) into
the C structs of the library.

Attributes read: B, H, d, grid, tile, candidates, window, win_mode, topk,
topk_frac, topp, fine_group, fine_keep, summarizer ("mean", "max" or
"minmax"; optional, default mean), sink (optional, default 0), compute
("bf16" or "fp8"; optional, default bf16), selector ("sics" or "profile":
how a head picks among the candidates; optional, default sics) and
profile_frac (optional, default 0 = 1%).
"""
from __future__ import annotations

from . import _lib


def flags_of(wl):
    if wl.fine_group:
        return _lib.VSA_FINE
    f = 0
    if wl.window is not None:
        f |= _lib.VSA_WINDOW
    if wl.topk:
        f |= _lib.VSA_TOPK
    if wl.topk_frac:
        f |= _lib.VSA_TOPK_FRAC
    if wl.topp:
        f |= _lib.VSA_TOPP
    if wl.candidates:
        f |= _lib.VSA_PROFILE_SELECT if getattr(wl, "selector", "sics") == "profile" else _lib.VSA_SICS_SELECT
    return f or _lib.VSA_DENSE


def plan_structs(wl):
    prob = _lib.make_problem(wl.B, wl.H, wl.d, wl.grid, wl.tile, wl.candidates)
    mode = _lib.VSA_WIN_CLAMP if wl.win_mode == "clamp" else _lib.VSA_WIN_TRUNCATE
    summ = {"mean": _lib.VSA_SUMM_MEAN, "max": _lib.VSA_SUMM_MAX,
            "minmax": _lib.VSA_SUMM_MINMAX}[getattr(wl, "summarizer", "mean")]
    pol = _lib.make_policy(flags_of(wl), win=wl.window or (1, 1, 1), win_mode=mode,
                           topk=wl.topk, topk_frac=wl.topk_frac, topp=wl.topp,
                           fine_group=wl.fine_group, fine_keep=wl.fine_keep,
                           summarizer=summ, sink=getattr(wl, "sink", 0),
                           compute={"bf16": _lib.VSA_COMPUTE_BF16,
                                    "fp8": _lib.VSA_COMPUTE_FP8}[getattr(wl, "compute", "bf16")],
                           profile_frac=getattr(wl, "profile_frac", 0.0))
    return prob, pol
