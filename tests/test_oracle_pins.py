"""Pins of the CPU oracle against things other than itself.

Each check compares the oracle with a library routine, a closed form, a
brute-force enumeration, or a value printed on the pages, so that a
dropped term, a wrong sign or a transposed operand in the oracle fails.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention, fine, geometry, layout, select, sics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).float().numpy()


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- geometry

def test_tile_major_equals_torch_view_permute():
    grid, tile = (4, 8, 12), (2, 4, 4)
    x = _bf16((1, 3, 4 * 8 * 12, 16), 1)
    mem = geometry.tile_members(grid, tile)
    xt = layout.to_tile_major(x, mem, 32)
    T, Hh, W = grid
    tt, th, tw = tile
    ref = torch.from_numpy(x).view(1, 3, T // tt, tt, Hh // th, th, W // tw, tw, 16)
    ref = ref.permute(0, 1, 2, 4, 6, 3, 5, 7, 8).reshape(1, 3, -1, tt * th * tw, 16)
    assert np.array_equal(xt, ref.numpy())


def test_members_bruteforce_tiny():
    grid, tile = (4, 8, 8), (2, 4, 4)
    nt = (2, 2, 2)
    expect = [[] for _ in range(8)]
    for t in range(4):
        for h in range(8):
            for w in range(8):
                i = ((t // 2) * nt[1] + h // 4) * nt[2] + w // 4
                expect[i].append((t * 8 + h) * 8 + w)
    got = geometry.tile_members(grid, tile)
    assert [list(m) for m in got] == expect


@pytest.mark.parametrize("grid,tile", [((21, 30, 52), (3, 6, 8)),
                                       ((21, 45, 80), (1, 16, 16)),
                                       ((21, 45, 80), (3, 8, 8)),
                                       ((5, 7, 9), (2, 3, 4))])
def test_partition_and_counts(grid, tile):
    mem = geometry.tile_members(grid, tile)
    allt = np.concatenate(mem)
    N = grid[0] * grid[1] * grid[2]
    assert sorted(allt.tolist()) == list(range(N))
    nt = geometry.tile_counts(grid, tile)
    for i, m in enumerate(mem):
        c = geometry.tile_coord(i, nt)
        ext = [min(tile[a], grid[a] - c[a] * tile[a]) for a in range(3)]
        assert len(m) == ext[0] * ext[1] * ext[2]
        assert list(m) == sorted(m)


def test_roundtrip_ragged():
    grid, tile = (5, 7, 9), (2, 3, 4)
    x = _bf16((2, 2, 5 * 7 * 9, 8), 2)
    mem = geometry.tile_members(grid, tile)
    xt = layout.to_tile_major(x, mem, 32)
    assert np.array_equal(layout.from_tile_major(xt, mem, x.shape[2]), x)
    # pads are zero
    for i, m in enumerate(mem):
        assert not xt[:, :, i, len(m):, :].any()


def test_spade_figure3_blockings_hold_64_tokens():
    grid = (16, 8, 8)
    for name, T, H, W, n in _golden("spade_fig3_blockings.txt"):
        mem = geometry.tile_members(grid, (int(T), int(H), int(W)))
        assert all(len(m) == int(n) for m in mem), name


def test_sta_block_pair_count():
    (video, tile, per_axis, pairs), = _golden("sta_theorem31_blocks.txt")
    nt = geometry.tile_counts((int(video),) * 3, (int(tile),) * 3)
    assert nt == (int(per_axis),) * 3
    assert (nt[0] * nt[1] * nt[2]) ** 2 == int(pairs)


# ------------------------------------------------------------------ window

def _closed_form_pairs(ntiles, win, mode):
    tot = 1
    for n, w in zip(ntiles, win):
        r = (w - 1) // 2
        if mode == "clamp" and n >= w:
            tot *= n * w
        else:
            tot *= sum(min(i + r, n - 1) - max(i - r, 0) + 1 for i in range(n))
    return tot


@pytest.mark.parametrize("ntiles,win,mode,expect", [
    ((5, 6, 10), (3, 3, 5), "truncate", 9152),     # HunyuanVideo 720p
    ((5, 6, 10), (3, 3, 5), "clamp", 13500),
    ((7, 5, 7), (3, 3, 3), "truncate", 4693),      # Wan-2.1 480p
    ((2, 2, 2), (3, 3, 3), "truncate", 64),        # tiny: all-ones
])
def test_window_pair_counts(ntiles, win, mode, expect):
    assert _closed_form_pairs(ntiles, win, mode) == expect
    nT = ntiles[0] * ntiles[1] * ntiles[2]
    got = sum(len(geometry.window(i, ntiles, win, mode)) for i in range(nT))
    assert got == expect


def test_window_matches_token_level_definition():
    # A query token attends a key token iff their TILE coordinates differ by
    # at most the radius on every axis; the result has only full blocks.
    grid, tile, win = (6, 6, 8), (2, 3, 2), (3, 3, 5)
    nt = geometry.tile_counts(grid, tile)
    mem = geometry.tile_members(grid, tile)
    rows = [geometry.window(i, nt, win) for i in range(len(mem))]
    tm = attention.token_mask(mem, rows, 6 * 6 * 8)
    t, h, w = geometry.token_coords(grid)
    ct, ch, cw = t // tile[0], h // tile[1], w // tile[2]
    ref = ((np.abs(ct[:, None] - ct[None]) <= 1) & (np.abs(ch[:, None] - ch[None]) <= 1)
           & (np.abs(cw[:, None] - cw[None]) <= 2))
    assert np.array_equal(tm, ref)


def test_clamp_window_keeps_full_size():
    nt = (5, 6, 10)
    for i in range(300):
        assert len(geometry.window(i, nt, (3, 3, 5), "clamp")) == 45


# ------------------------------------------------------------ pooled means

def test_pooled_means_match_torch_mean():
    grid, tile = (4, 8, 8), (2, 4, 4)
    x = _bf16((256, 64), 3)
    mem = geometry.tile_members(grid, tile)
    got = select.pooled_means(x, mem)
    ref = torch.from_numpy(x).double().view(2, 2, 2, 4, 2, 4, 64)
    ref = ref.permute(0, 2, 4, 1, 3, 5, 6).reshape(8, 32, 64).mean(dim=1).float()
    assert np.array_equal(got, ref.numpy())


def test_pooled_ragged_tile_uses_valid_count():
    grid, tile = (1, 1, 52), (1, 1, 8)          # last tile has 4 tokens
    x = _bf16((52, 16), 4)
    got = select.pooled_means(x, geometry.tile_members(grid, tile))
    assert np.array_equal(got[-1], x[48:52].astype(np.float64).mean(0).astype(np.float32))


def test_pooled_constant_tile():
    x = np.full((32, 8), 0.375, dtype=np.float32)
    assert np.all(select.pooled_means(x, [np.arange(32)]) == np.float32(0.375))


def test_pooled_exactness_guard_fires():
    x = np.zeros((4, 1))
    x[0, 0] = 2.0 ** 40
    x[1, 0] = 2.0 ** -40
    with pytest.raises(AssertionError):
        select.pooled_means(x, [np.arange(4)])


# ------------------------------------------------- max / min summarizers

def test_pooled_extrema_match_torch_amax_amin():
    grid, tile = (4, 8, 8), (2, 4, 4)
    x = _bf16((256, 64), 13)
    mx, mn = select.pooled_extrema(x, geometry.tile_members(grid, tile))
    ref = torch.from_numpy(x).view(2, 2, 2, 4, 2, 4, 64).permute(0, 2, 4, 1, 3, 5, 6).reshape(8, 32, 64)
    assert np.array_equal(mx, ref.amax(dim=1).numpy())
    assert np.array_equal(mn, ref.amin(dim=1).numpy())


def test_pooled_extrema_ragged_tile_uses_valid_tokens():
    grid, tile = (1, 1, 52), (1, 1, 8)          # last tile has 4 tokens
    x = _bf16((52, 16), 14)
    mx, mn = select.pooled_extrema(x, geometry.tile_members(grid, tile))
    assert np.array_equal(mx[-1], x[48:52].max(0)) and np.array_equal(mn[-1], x[48:52].min(0))


def test_minmax_score_bounds_every_key_of_the_tile():
    grid, tile = (2, 6, 6), (1, 3, 3)
    q, k = _bf16((72, 32), 15), _bf16((72, 32), 16)
    mem = geometry.tile_members(grid, tile)
    S = select.summarized_scores(q, k, mem, 0.25, "minmax")
    pq = select.pooled_means(q, mem).astype(np.float64)
    for j, m in enumerate(mem):
        exact = (pq @ k[m].astype(np.float64).T).max(axis=1) * 0.25   # best key of tile j
        assert np.all(S[:, j] >= exact - 1e-12)


def test_summarizers_coincide_on_one_token_tiles():
    grid, tile = (1, 3, 4), (1, 1, 1)
    q, k = _bf16((12, 16), 17), _bf16((12, 16), 18)
    mem = geometry.tile_members(grid, tile)
    ref = (q.astype(np.float64) @ k.astype(np.float64).T) * 0.5         # closed form
    for summ in ("mean", "max", "minmax"):
        assert np.allclose(select.summarized_scores(q, k, mem, 0.5, summ), ref, rtol=1e-12, atol=1e-12)


def test_max_summarizer_scores_against_the_key_maxima():
    grid, tile = (4, 8, 8), (2, 4, 4)
    q, k = _bf16((256, 64), 19), _bf16((256, 64), 20)
    mem = geometry.tile_members(grid, tile)
    kmax = torch.from_numpy(k).view(2, 2, 2, 4, 2, 4, 64).permute(0, 2, 4, 1, 3, 5, 6).reshape(8, 32, 64).amax(1)
    ref = torch.from_numpy(select.pooled_means(q, mem)).double() @ kmax.double().T * 0.125
    assert np.allclose(select.summarized_scores(q, k, mem, 0.125, "max"), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_sink_is_kept_in_every_row():
    S = np.arange(64, dtype=np.float64).reshape(8, 8)          # col 7 best
    rows, _ = select.select_rows(S, (2, 2, 2), window=(1, 1, 1), k=1, sink=2)
    for i, r in enumerate(rows):
        assert r == sorted({0, 1, i, 7})
    assert select.select_rows(S, (2, 2, 2), window=(1, 1, 1), sink=0)[0] == [[i] for i in range(8)]
    assert all(r == list(range(8)) for r in select.select_rows(S, (2, 2, 2), window=(1, 1, 1), sink=99)[0])


# ------------------------------------------------------------- tile scores

def test_scores_match_fp64_matmul():
    pq = np.random.default_rng(0).standard_normal((20, 64)).astype(np.float32)
    pk = np.random.default_rng(1).standard_normal((20, 64)).astype(np.float32)
    s = select.tile_scores(pq, pk, 0.125)
    ref = (torch.from_numpy(pq).double() @ torch.from_numpy(pk).double().T * 0.125).numpy()
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(s, select.tile_scores(pq, pk, 0.125))


def test_scores_order_is_left_to_right():
    # 1 + 2^-53 + 2^-53 loses both small terms left to right but not exactly.
    pq = np.array([[1.0, 2.0 ** -26, 2.0 ** -26]], dtype=np.float32)
    pk = np.array([[1.0, 2.0 ** -27, 2.0 ** -27]], dtype=np.float32)
    assert select.tile_scores(pq, pk, 1.0)[0, 0] == 1.0
    pq2 = pq[:, ::-1].copy()
    pk2 = pk[:, ::-1].copy()
    assert select.tile_scores(pq2, pk2, 1.0)[0, 0] == 1.0 + 2.0 ** -52


# ------------------------------------------------------------ Top-K / Top-P

def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(5)
    for _ in range(50):
        row = rng.integers(0, 6, size=17).astype(np.float64)   # many ties
        k = int(rng.integers(1, 17))
        ref = sorted(sorted(range(17), key=lambda j: (-row[j], j))[:k])
        assert select.topk(row, k) == ref
    assert select.topk(row, 17) == list(range(17))


def test_topp_bruteforce():
    rng = np.random.default_rng(6)
    for _ in range(50):
        row = rng.standard_normal(23) * 2
        p = float(rng.uniform(0.05, 0.99))
        mx = max(row)
        e = [math.exp(v - mx) for v in row]
        z = math.fsum(e)
        order = sorted(range(23), key=lambda j: (-row[j], j))
        acc = 0.0
        for m, j in enumerate(order):
            acc += e[j] / z
            if acc >= p:
                break
        got, margin = select.topp(row, p)
        if margin > 1e-9:
            assert got == sorted(order[:m + 1])


def test_topp_special_cases():
    row = np.array([0.3, -1.0, 2.0, 2.0, 0.1])
    assert select.topp(row, 1.0)[0] == [0, 1, 2, 3, 4]
    assert select.topp(row, 1e-12)[0] == [2]                 # tie -> lower index
    assert select.topp(row + 7.25, 0.6)[0] == select.topp(row, 0.6)[0]
    assert np.allclose(scipy.special.softmax(row).sum(), 1.0)


def test_frac_count():
    assert select.frac_count(0.2, 315) == 63
    assert select.frac_count(0.2, 720) == 144
    assert select.frac_count(0.2, 420) == 84
    assert select.frac_count(0.2, 3) == 1
    assert fine.keep_count(0.15, 512, 32760) == 2515968


def test_select_rows_union():
    S = np.arange(64, dtype=np.float64).reshape(8, 8)[:, ::-1].copy()  # col 0 best
    rows, _ = select.select_rows(S, (2, 2, 2), window=(1, 1, 1), k=2)
    for i, r in enumerate(rows):
        assert r == sorted({i, 0, 1})


# -------------------------------------------------------------------- SICS

@pytest.mark.parametrize("n", [2, 3, 5, 16, 32])
def test_sics_cumulative_equals_pairwise(n):
    x = _bf16((n, 24), 10 + n)
    assert math.isclose(sics.sics_cumulative(x), sics.sics_pairwise(x),
                        rel_tol=1e-12, abs_tol=1e-12)
    u = sics.unit_rows(x)
    closed = (np.sum(u.sum(0) ** 2) - n) / 2.0
    assert math.isclose(sics.sics_cumulative(x), closed, rel_tol=1e-10, abs_tol=1e-10)


def test_sics_special_cases():
    v = np.random.default_rng(0).standard_normal(16)
    par = np.stack([v * c for c in (1.0, 2.0, 0.5, 3.0, 7.0)])
    assert math.isclose(sics.sics_cumulative(par), 10.0, rel_tol=1e-12)
    assert abs(sics.sics_cumulative(np.eye(6))) < 1e-15
    assert math.isclose(sics.sics_cumulative(np.stack([v, -v])), -1.0, rel_tol=1e-12)
    withzero = np.vstack([par, np.zeros((1, 16))])
    assert math.isclose(sics.sics_cumulative(withzero), 10.0, rel_tol=1e-12)


def test_sics_prefers_blocking_along_long_correlation():
    from synth import smooth_field
    grid = (14, 16, 16)
    cands = ((1, 16, 16), (7, 4, 4), (3, 8, 8))
    for ell, want in (((8.0, 1.0, 1.0), 1), ((1.0, 8.0, 8.0), 0)):
        q = smooth_field((1, 1, 32), grid, [ell], seed=3)[0, 0].float().numpy()
        k = smooth_field((1, 1, 32), grid, [ell], seed=4)[0, 0].float().numpy()
        sc = sics.candidate_scores(q, k, grid, cands)
        assert sics.choose(sc) == want, sc


def test_choose_tie_goes_low():
    assert sics.choose(np.array([0.5, 0.7, 0.7])) == 1


# -------------------------------------------------------------------- fine

def test_fine_threshold_and_lists():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((9, 50))
    kc = fine.keep_count(0.15, 9, 50)
    tau = fine.threshold(s, kc)
    assert tau == np.sort(s.ravel())[::-1][kc - 1]
    lists = fine.kept_lists(s, tau)
    assert sum(len(l) for l in lists) == kc          # no ties in random data
    dense = fine.kept_lists(s, fine.threshold(s, s.size))
    assert all(len(l) == 50 for l in dense)


def test_fine_group_means_and_scores():
    q = _bf16((130, 16), 8)
    k = _bf16((40, 16), 9)
    qb = fine.group_means(q, 64)
    assert qb.shape == (3, 16)
    assert np.array_equal(qb[2], q[128:130].astype(np.float64).mean(0).astype(np.float32))
    s = fine.group_scores(qb, k)
    ref = qb.astype(np.float64) @ k.astype(np.float64).T
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- attention

def test_dense_attention_matches_torch_sdpa():
    q, k, v = (_bf16((1, 2, 96, 32), s) for s in (20, 21, 22))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double(),
        torch.from_numpy(v).double()).numpy()
    for h in range(2):
        got = attention.attention_dense(q[0, h], k[0, h], v[0, h])
        assert np.allclose(got, ref[0, h], rtol=1e-12, atol=1e-12)


def test_probabilities_rows_sum_to_one():
    q, k = _bf16((40, 16), 30), _bf16((70, 16), 31)
    allowed = np.random.default_rng(1).random((40, 70)) < 0.4
    allowed[:, 0] = True
    P = attention.attention_dense(q, k, np.eye(70), allowed)
    ref = scipy.special.softmax(np.where(allowed, q.astype(np.float64) @ k.T / 4.0,
                                         -np.inf), axis=1)
    assert np.allclose(P, ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(P.sum(1), 1.0, atol=1e-12)
    assert not P[~allowed].any()


def test_constant_v_and_empty_rows():
    q, k = _bf16((10, 8), 40), _bf16((12, 8), 41)
    v = np.full((12, 5), -1.5)
    assert np.allclose(attention.attention_dense(q, k, v), -1.5, atol=1e-14)
    allowed = np.ones((10, 12), dtype=bool)
    allowed[3] = False
    out = attention.attention_dense(q, k, v, allowed)
    assert not out[3].any()


def test_block_sparse_equals_dense_with_token_mask():
    grid, tile = (4, 6, 8), (2, 3, 4)
    N = 4 * 6 * 8
    q, k, v = (_bf16((N, 16), s) for s in (50, 51, 52))
    mem = geometry.tile_members(grid, tile)
    rng = np.random.default_rng(2)
    rows = [sorted(set(rng.choice(8, size=3, replace=False).tolist()) | {i}) for i in range(8)]
    got = attention.block_sparse_attention(q, k, v, mem, rows)
    ref = attention.attention_dense(q, k, v, attention.token_mask(mem, rows, N))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_tiny_workload_is_dense_attention():
    from synth import get, smooth_field_qkv
    wl = get("tiny")
    q, k, v = (t.float().numpy() for t in smooth_field_qkv(1, 2, 64, wl.grid, wl.ell_per_head()))
    mem = geometry.tile_members(wl.grid, wl.tile)
    nt = geometry.tile_counts(wl.grid, wl.tile)
    S = select.tile_scores(select.pooled_means(q[0, 0], mem), select.pooled_means(k[0, 0], mem), 0.125)
    rows, _ = select.select_rows(S, nt, window=wl.window, k=wl.topk)
    assert all(r == list(range(8)) for r in rows)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double(), torch.from_numpy(v).double())
    got = attention.block_sparse_attention(q[0, 0], k[0, 0], v[0, 0], mem, rows)
    assert np.allclose(got, ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_fine_attention_dense_when_all_kept():
    q, k, v = (_bf16((70, 8), s) for s in (60, 61, 62))
    g = fine.groups(70, 32)
    got = attention.fine_attention(q, k, v, g, [np.arange(70)] * len(g))
    assert np.allclose(got, attention.attention_dense(q, k, v), rtol=1e-12, atol=1e-13)


def test_tile_sics_equals_bruteforce_per_tile():
    """Per-tile SICS against explicit pairwise cosines over every token pair
    of each (ragged) tile."""
    grid, tile = (3, 5, 7), (2, 3, 4)
    x = _bf16((3 * 5 * 7, 16), 31).astype(np.float64)
    mem = geometry.tile_members(grid, tile)
    got = sics.tile_sics(x, mem)
    for i, m in enumerate(mem):
        want = 0.0
        for a, b in itertools.combinations(m, 2):
            want += float(x[a] @ x[b]) / (np.linalg.norm(x[a]) * np.linalg.norm(x[b]))
        assert math.isclose(got[i], want, rel_tol=1e-10, abs_tol=1e-10), (i, got[i], want)


def test_mean_pair_cosine_special_cases():
    """Parallel tokens give 1 per pair, orthonormal tokens 0; one-token tiles
    are left out of the mean."""
    grid, tile = (1, 4, 6), (1, 2, 3)
    mem = geometry.tile_members(grid, tile)
    par = np.tile(np.arange(1.0, 9.0), (24, 1))
    assert math.isclose(sics.mean_pair_cosine(par, mem), 1.0, rel_tol=1e-12)
    orth = np.zeros((24, 24))
    orth[np.arange(24), np.arange(24)] = 1.0
    assert abs(sics.mean_pair_cosine(orth, mem)) < 1e-15
    mem1 = [[0], [1, 2]]                      # a one-token tile and a pair of opposite tokens
    x = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, -1.0]])
    assert math.isclose(sics.mean_pair_cosine(x, mem1), -1.0, rel_tol=1e-12)


def test_token_tile_id_bruteforce():
    """Tile id of every token of a ragged grid by explicit coordinate loops."""
    grid, tile = (5, 7, 9), (2, 3, 4)
    nt = [-(-g // t) for g, t in zip(grid, tile)]
    want = [((t // tile[0]) * nt[1] + h // tile[1]) * nt[2] + w // tile[2]
            for t in range(grid[0]) for h in range(grid[1]) for w in range(grid[2])]
    assert geometry.token_tile_id(grid, tile).tolist() == want


def test_default_scale():
    assert select.default_scale(64) == 0.125
    assert select.default_scale(128) == 1.0 / math.sqrt(128.0)
    assert math.isclose(select.default_scale(128) ** 2 * 128, 1.0, rel_tol=1e-15)


def test_candidate_scores_worked_example():
    """Two blockings of different block sizes on a 1 x 1 x 4 grid (d = 2),
    worked out by hand.  Tokens 0, 1 are e1; tokens 2, 3 are at 60 degrees to
    e1.  Blocking 0 (1x1x2) has tiles {0,1}, {2,3}: pair cosines 1 and 1, mean
    pair cosine 1, SICS sum 2.  Blocking 1 (1x1x4) has one tile: pair cosines
    1, 1 and four times 0.5, SICS 4, mean pair cosine 4/6.

    With K = Q the score is the mean pair cosine, [1, 2/3]: blocking 0 wins,
    while a raw SICS sum (2 vs 4, or its mean over tiles, 1 vs 4) would pick
    blocking 1.  With K = (e1, -e1, e1, -e1) the K mean pair cosines are -1
    (tiles {0,1}, {2,3}) and -2/6 (one tile: four pairs at -1, two at +1), so
    the averaged scores are [0, 1/6] and blocking 1 wins, while Q alone would
    still pick blocking 0."""
    grid = (1, 1, 4)
    cands = ((1, 1, 2), (1, 1, 4))
    c60 = (0.5, math.sqrt(3.0) / 2.0)
    q = np.array([[1.0, 0.0], [1.0, 0.0], c60, c60])
    sc = sics.candidate_scores(q, q, grid, cands)
    assert np.allclose(sc, [1.0, 2.0 / 3.0], rtol=0, atol=1e-12), sc
    assert sics.choose(sc) == 0
    k = np.array([[1.0, 0.0], [-1.0, 0.0], [1.0, 0.0], [-1.0, 0.0]])
    sc = sics.candidate_scores(q, k, grid, cands)
    assert np.allclose(sc, [0.0, 1.0 / 6.0], rtol=0, atol=1e-12), sc
    assert sics.choose(sc) == 1
