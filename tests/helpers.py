"""Shared test helpers: workload -> C structs, and oracle pipelines."""
from __future__ import annotations

import numpy as np

import block_sparse_attention_tile_amd as vsa
from oracle import attention, fine, geometry, select, sics


def flags_of(wl):
    f = 0
    if wl.fine_group:
        return vsa.VSA_FINE
    if wl.window is not None:
        f |= vsa.VSA_WINDOW
    if wl.topk:
        f |= vsa.VSA_TOPK
    if wl.topk_frac:
        f |= vsa.VSA_TOPK_FRAC
    if wl.topp:
        f |= vsa.VSA_TOPP
    if wl.candidates:
        f |= vsa.VSA_SICS_SELECT
    if f == 0:
        f = vsa.VSA_DENSE
    return f


def structs_of(wl):
    prob = vsa.make_problem(wl.B, wl.H, wl.d, wl.grid, wl.tile, wl.candidates)
    pol = vsa.make_policy(flags_of(wl), win=wl.window or (1, 1, 1),
                          win_mode=vsa.VSA_WIN_CLAMP if wl.win_mode == "clamp" else vsa.VSA_WIN_TRUNCATE,
                          topk=wl.topk, topk_frac=wl.topk_frac, topp=wl.topp,
                          fine_group=wl.fine_group, fine_keep=wl.fine_keep)
    return prob, pol


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
        pq = select.pooled_means(q_h, mem)
        pk = select.pooled_means(k_h, mem)
        S = select.tile_scores(pq, pk, select.default_scale(wl.d))
    if wl.window is None and not K and not wl.topp:
        return [list(range(nT))] * nT, [np.inf] * nT, mem
    rows, margins = select.select_rows(S, nt, window=wl.window, win_mode=wl.win_mode,
                                       k=K, p=wl.topp)
    return rows, margins, mem


def csr_rows(row_ptr, col, bh, max_tiles, n_tiles):
    base = bh * max_tiles
    return [col[row_ptr[base + i]:row_ptr[base + i + 1]].tolist() for i in range(n_tiles)]


def oracle_candidate(wl, q_h, k_h):
    sc = sics.candidate_scores(q_h, k_h, wl.grid, wl.candidates)
    return sics.choose(sc), sc
