"""SICS tile-coherence score and per-head blocking choice (oracle).

SPADE review page, "Core claim" and "What carries the argument": each
candidate 3D blocking of the Q/K token grid is scored by the Sum of
Intra-block Cosine Similarities (SICS), the sum over all token pairs inside
a block of their cosine similarity, computed in O(BS * d) with cumulative
partial sums; the blocking with the highest score is selected per head.
Figure 3 of that page lists spatial, temporal and mixed candidates.

Readings where the page is silent (the equations are named but not printed):
  * a zero vector has unit vector 0 (contributes nothing);
  * blockings with different block sizes are compared by the MEAN pairwise
    cosine, SICS_i / (n_i (n_i - 1) / 2), averaged over tiles with n_i >= 2
    (equal block sizes, the only case the page shows, rank identically to
    the raw sum);
  * Q and K are both scored and their two means averaged;
  * ties between candidates go to the lower candidate index.
"""
from __future__ import annotations

import numpy as np

from . import geometry


def unit_rows(x):
    x64 = np.asarray(x, dtype=np.float64)
    n = np.sqrt((x64 * x64).sum(axis=1, keepdims=True))
    return np.where(n > 0, x64 / np.where(n > 0, n, 1.0), 0.0)


def sics_pairwise(x):
    """Brute force: sum_{a<b} cos(x_a, x_b) over the rows of x."""
    u = unit_rows(x)
    n = u.shape[0]
    s = 0.0
    for a in range(n):
        for b in range(a + 1, n):
            s += float(u[a] @ u[b])
    return s


def sics_cumulative(x):
    """Same sum with running partial sums: sum_b u_b . (u_0 + .. + u_{b-1})."""
    u = unit_rows(x)
    prefix = np.cumsum(u, axis=0)
    before = np.vstack([np.zeros((1, u.shape[1])), prefix[:-1]])
    return float((u * before).sum())


def tile_sics(x, members):
    """SICS of every tile of one head: x [N, d] -> fp64 [nT]."""
    return np.array([sics_cumulative(x[m]) for m in members])


def mean_pair_cosine(x, members):
    """Average over tiles (n_i >= 2) of SICS_i / pairs_i."""
    vals = []
    for m in members:
        n = len(m)
        if n >= 2:
            vals.append(sics_cumulative(x[m]) / (n * (n - 1) / 2.0))
    return float(np.mean(vals))


def candidate_scores(q, k, grid, candidates):
    """Score per candidate blocking for one head (q, k: [N, d])."""
    out = []
    for tile in candidates:
        mem = geometry.tile_members(grid, tile)
        out.append(0.5 * (mean_pair_cosine(q, mem) + mean_pair_cosine(k, mem)))
    return np.array(out)


def choose(scores):
    """Index of the highest score; ties to the lower index."""
    return int(np.argmax(scores))        # argmax returns the first maximum
