"""Shared test helpers: workload -> C structs, and oracle pipelines."""
from __future__ import annotations

import numpy as np

import block_sparse_attention_tile_amd as vsa
from oracle import attention, fine, geometry, select, sics


from block_sparse_attention_tile_amd.workload import flags_of, plan_structs as structs_of  # noqa: E402,F401

# Summation error of one E4M3 matrix product (v_mfma_f32_32x32x64_f8f6f4) per
# output element, as a fraction of its largest |term|: the bound the E4M3
# attention's parity tolerance is derived from, measured on the hardware by
# tests/test_gpu_probe.py.
C_MFMA = 2.0 ** -10


def oracle_tile_rows(wl, q_h, k_h, tile):
    """Oracle selection for one head: (rows, margins, members)."""
    mem = geometry.tile_members(wl.grid, tile)
    nt = geometry.tile_counts(wl.grid, tile)
    nT = len(mem)
    K = 0
    if wl.topk:
        K = min(wl.topk, nT)
    elif wl.topk_frac:
        K = min(select.frac_count(wl.topk_frac, nT), nT)
    S = None
    if K or wl.topp:
        S = select.summarized_scores(q_h, k_h, mem, select.default_scale(wl.d), wl.summarizer)
    if wl.window is None and not K and not wl.topp:
        return [list(range(nT))] * nT, [np.inf] * nT, mem
    rows, margins = select.select_rows(S, nt, window=wl.window, win_mode=wl.win_mode,
                                       k=K, p=wl.topp, sink=wl.sink)
    return rows, margins, mem


def unambiguous(tiles, margins):
    """The query tiles whose oracle selection is unique (no Top-P cut within
    1e-9 of the mass the oracle's rounding could move): only these are
    compared bit-exactly, and their O against the oracle's own kept tiles."""
    return [int(i) for i in tiles if margins[i] > 1e-9]


def csr_rows(row_ptr, col, bh, max_tiles, n_tiles):
    base = bh * max_tiles
    return [col[row_ptr[base + i]:row_ptr[base + i + 1]].tolist() for i in range(n_tiles)]


def oracle_candidate(wl, q_h, k_h):
    sc = sics.candidate_scores(q_h, k_h, wl.grid, wl.candidates)
    return sics.choose(sc), sc
