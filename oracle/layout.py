"""Tile-major layout and its inverse (oracle; test infrastructure).

The layout transform puts the tokens of each tile next to each other so a
block-sparse kernel reads contiguous blocks (SPADE review page, "What
carries the argument": fused layout transform in the executor; Sparse
VideoGen verdict page, pith_extraction.key_machinery: the transposed layout
is what lets the block-sparse kernel reach its speedup).

tile-major x_t[b, h, i, s, :] = x[b, h, members[i][s], :] for s < n_i, and
zero for the padded slots n_i <= s < slots.
"""
from __future__ import annotations

import numpy as np


def to_tile_major(x, members, slots):
    """x: [B, H, N, d] -> [B, H, nT, slots, d] (zero pads)."""
    B, H, N, d = x.shape
    out = np.zeros((B, H, len(members), slots, d), dtype=x.dtype)
    for i, m in enumerate(members):
        out[:, :, i, :len(m), :] = x[:, :, m, :]
    return out


def from_tile_major(xt, members, N):
    """Inverse: [B, H, nT, slots, d] -> [B, H, N, d], dropping pads."""
    B, H, nT, slots, d = xt.shape
    out = np.zeros((B, H, N, d), dtype=xt.dtype)
    for i, m in enumerate(members):
        out[:, :, m, :] = xt[:, :, i, :len(m), :]
    return out
