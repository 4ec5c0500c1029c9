"""Pins of the profiling selector oracle (oracle/profile.py).

Checked against things other than itself: the sample's counts and bounds
(closed form), a dense candidate's MSE (exactly 0), a token-level brute
force of the masked outputs (explicit distance tests over every key, not
the tile lists), and planted spatial / temporal heads, which must pick the
one-frame / all-frames blocking (the dichotomy of the Sparse VideoGen
verdict page).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, profile


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * scale).to(torch.bfloat16).double().numpy()


def test_sample_rows_counts_and_bounds():
    rows = profile.sample_rows(115200, 0.01)
    assert rows.size == 36 * 32 and profile.n_runs(115200, 0.01) == 36
    runs = rows.reshape(-1, 32)
    assert np.all(np.diff(runs, axis=1) == 1)                # 32 consecutive tokens
    assert np.all(runs[1:, 0] - runs[:-1, 31] >= 1)          # disjoint, ascending
    assert runs[0, 0] == 0 and runs[-1, 31] < 115200
    assert profile.sample_rows(20, 0.01).tolist() == list(range(20))
    assert profile.n_runs(1000, 1e-6) == 1 and profile.n_runs(1000, 1.0) == 31
    full = profile.sample_rows(1000, 1.0)
    assert len(set(full.tolist())) == 31 * 32 and full.max() < 1000


def test_dense_candidate_has_zero_mse():
    grid, d = (3, 4, 8), 16
    N = 96
    q, k, v = (_bf16((N, d), s) for s in (1, 2, 3))
    mse = profile.profile_mse(q, k, v, grid, [(1, 4, 8), (3, 2, 2)], window=None, frac=1.0)
    assert np.all(mse < 1e-28)


def _brute_masked(q, k, v, grid, tile, win, qids):
    """Each sampled row attends to the keys whose tile coordinates lie within
    the window radius of its own tile's, by an explicit loop over all keys
    (truncate mode)."""
    T, H, W = grid
    coords = [(t, h, w) for t in range(T) for h in range(H) for w in range(W)]
    rad = [(x - 1) // 2 for x in win]
    out = np.zeros((len(qids), v.shape[1]))
    for n, qi in enumerate(qids):
        qc = [coords[qi][a] // tile[a] for a in range(3)]
        keys = [j for j, c in enumerate(coords)
                if all(abs(c[a] // tile[a] - qc[a]) <= rad[a] for a in range(3))]
        out[n] = attention.attention_dense(q[qi:qi + 1], k[keys], v[keys])[0]
    return out


def test_masked_outputs_match_token_level_brute_force():
    grid, d = (4, 6, 10), 16
    N = 240
    q, k, v = (_bf16((N, d), s) for s in (4, 5, 6))
    cands = [(1, 3, 5), (4, 2, 2), (2, 3, 4)]
    win = (1, 3, 3)
    qids = profile.sample_rows(N, 0.2)
    full = attention.attention_dense(q[qids], k, v)
    want = [float(np.mean((_brute_masked(q, k, v, grid, t, win, qids) - full) ** 2)) for t in cands]
    got = profile.profile_mse(q, k, v, grid, cands, window=win, frac=0.2)
    np.testing.assert_allclose(got, want, rtol=1e-12)


def _planted(grid, d, kind, seed):
    """q = k = a one-hot code of the frame (spatial head) or of the (h, w)
    position (temporal head), times 4, plus small noise; v random."""
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    code = (t if kind == "spatial" else h * W + w).ravel() % d
    emb = np.eye(d)[code] * 4.0
    noise = _bf16(emb.shape, seed, 0.05)
    q = torch.tensor(emb + noise).to(torch.bfloat16).double().numpy()
    v = _bf16(emb.shape, seed + 1)
    return q, q.copy(), v


@pytest.mark.parametrize("kind,want", [("spatial", 0), ("temporal", 1)])
def test_planted_heads_pick_their_pattern(kind, want):
    grid = (6, 4, 4)
    cands = [(1, 4, 4), (6, 1, 1)]   # one frame per tile / one position across all frames
    q, k, v = _planted(grid, 16, kind, 7)
    mse = profile.profile_mse(q, k, v, grid, cands, window=(1, 1, 1), frac=1.0)
    assert profile.choose(mse) == want, mse
    assert mse[want] < 0.1 * mse[1 - want]


def test_choose_ties_to_lower_index():
    assert profile.choose(np.array([0.5, 0.2, 0.2])) == 1
    assert profile.choose(np.array([0.0, 0.0])) == 0
