"""Online profiling selector (oracle; test infrastructure).

Sparse VideoGen verdict page (pith_extraction.key_machinery and
core_discovery; skeptic_critique): every head is either spatial or temporal
at a given step; per head, a small sample of the query rows (1%) is run
through full attention and through each candidate sparse pattern, and the
pattern whose output on those rows is closest to the full one (lowest mean
squared error) is kept for the whole head.

Readings taken here (the page gives neither the mask generators nor the
sampling procedure, referee_report.minor_comments):
  * the candidates are the plan's candidate blockings, each under the
    policy's static tile mask (sliding window, sink, or dense).  One-frame
    tiles (1, th, tw) give a spatial pattern and tiles spanning all frames
    (T, th, tw) a temporal one;
  * the sample is n = clamp(round(frac * N / 32), 1, floor(N / 32)) runs of
    32 consecutive raster tokens, run r starting at floor(r * N / n): an
    evenly spread, deterministic sample in place of a random one.  With
    N < 32 it is the single run of all N tokens;
  * MSE = mean over the sampled rows and the d channels of (O_c - O_full)^2,
    with O_full the unmasked softmax attention; the argmin wins, ties to the
    lower candidate index.
"""
from __future__ import annotations

import numpy as np

from . import attention, geometry, select

RUN = 32


def n_runs(N, frac):
    if N < RUN:
        return 1
    return int(min(max(int(np.floor(frac * N / RUN + 0.5)), 1), N // RUN))


def sample_rows(N, frac):
    """Raster token ids of the sampled query rows (ascending)."""
    if N < RUN:
        return np.arange(N)
    n = n_runs(N, frac)
    starts = [(r * N) // n for r in range(n)]
    return np.concatenate([np.arange(s, s + RUN) for s in starts])


def candidate_rows(grid, tile, window=None, win_mode="truncate", sink=0):
    """Kept key tiles of every query tile of one blocking under a static
    mask (window and / or sink; dense when window is None and sink = 0)."""
    nt = geometry.tile_counts(grid, tile)
    nT = int(np.prod(nt))
    if window is None and sink == 0:
        return [list(range(nT))] * nT
    rows, _ = select.select_rows(None, nt, window=window, win_mode=win_mode, sink=sink)
    return rows


def masked_outputs(q, k, v, grid, tile, rows, qids, scale=None):
    """Output of the sampled query rows qids under one blocking's mask: each
    row attends to the keys of the kept tiles of its own tile."""
    members = geometry.tile_members(grid, tile)
    tid = geometry.token_tile_id(grid, tile)
    out = np.zeros((len(qids), v.shape[1]))
    for n, qi in enumerate(qids):
        keys = np.concatenate([members[j] for j in rows[tid[qi]]])
        out[n] = attention.attention_dense(q[qi:qi + 1], k[keys], v[keys], None, scale)[0]
    return out


def profile_mse(q, k, v, grid, candidates, window=None, win_mode="truncate", sink=0,
                frac=0.01, scale=None):
    """One head: MSE of every candidate's masked output against full
    attention on the sampled rows (fp64)."""
    qids = sample_rows(q.shape[0], frac)
    full = attention.attention_dense(q[qids], k, v, None, scale)
    mse = []
    for tile in candidates:
        rows = candidate_rows(grid, tile, window, win_mode, sink)
        o = masked_outputs(q, k, v, grid, tile, rows, qids, scale)
        mse.append(float(np.mean((o - full) ** 2)))
    return np.array(mse)


def choose(mse):
    """Argmin, ties to the lower index."""
    return int(np.argmin(mse))
