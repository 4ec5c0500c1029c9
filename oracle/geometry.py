"""Tiling of a T x H x W token grid into 3D tiles (oracle; test infrastructure).

A tile is a contiguous cube of tokens and one tile is one attention block;
token order inside a tile is kept consecutive (Sliding Tile Attention
verdict page, pith_extraction.key_machinery; SPADE review page, Figure 3:
blockings given as (T, H, W) extents).

Readings where the pages are silent:
  * tokens are numbered in raster order (t, h, w), w fastest;
  * tiles are numbered in raster order of tile coordinates;
  * inside a tile the valid tokens keep their raster order;
  * edge tiles that overhang the grid hold only the tokens inside it.
"""
from __future__ import annotations

import math

import numpy as np


def tile_counts(grid, tile):
    """Tiles per axis: ceil(grid_a / tile_a)."""
    return tuple(int(math.ceil(g / t)) for g, t in zip(grid, tile))


def token_coords(grid):
    """(t, h, w) coordinates of every token, in raster order."""
    T, Hh, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W),
                          indexing="ij")
    return t.ravel(), h.ravel(), w.ravel()


def token_tile_id(grid, tile):
    """Tile id of every raster token."""
    nt = tile_counts(grid, tile)
    t, h, w = token_coords(grid)
    return (t // tile[0] * nt[1] + h // tile[1]) * nt[2] + w // tile[2]


def tile_members(grid, tile):
    """List over tiles of the raster token ids inside each tile.

    Each list is in raster order (the in-tile order of the tiled layout).
    """
    tid = token_tile_id(grid, tile)
    order = np.argsort(tid, kind="stable")   # stable: keeps raster order
    nT = int(np.prod(tile_counts(grid, tile)))
    counts = np.bincount(tid, minlength=nT)
    bounds = np.concatenate([[0], np.cumsum(counts)])
    return [order[bounds[i]:bounds[i + 1]] for i in range(nT)]


def tile_coord(i, ntiles):
    """Tile coordinates (it, ih, iw) of tile id i."""
    return (i // (ntiles[1] * ntiles[2]), (i // ntiles[2]) % ntiles[1],
            i % ntiles[2])


def _axis_range(c, r, n, mode):
    if mode == "clamp" and n >= 2 * r + 1:
        lo = min(max(c - r, 0), n - (2 * r + 1))
        return lo, lo + 2 * r
    return max(c - r, 0), min(c + r, n - 1)


def window(i, ntiles, win, mode="truncate"):
    """Key tiles inside the 3D tile window of query tile i, ascending.

    win gives the full window extent per axis in tiles (odd), so the radius
    is (win - 1) / 2.  A query tile attends to every key tile whose tile
    coordinates are within the radius on all three axes (Sliding Tile
    Attention verdict page, pith_extraction.pith_summary and key_machinery:
    the window slides over tiles, not tokens).  "truncate" cuts the window
    at the grid edge; "clamp" shifts it inward so it keeps its full size.
    """
    c = tile_coord(i, ntiles)
    rng = [_axis_range(c[a], (win[a] - 1) // 2, ntiles[a], mode)
           for a in range(3)]
    out = []
    for t in range(rng[0][0], rng[0][1] + 1):
        for h in range(rng[1][0], rng[1][1] + 1):
            for w in range(rng[2][0], rng[2][1] + 1):
                out.append((t * ntiles[1] + h) * ntiles[2] + w)
    return sorted(out)
