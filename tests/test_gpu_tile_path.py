"""GPU parity of the tile path (layout, selection, attention) against the oracle.

Every case prints its name before touching the GPU so a failing run names it.
Tolerances: tile indices bit-exact; pooled means bit-exact (exact sums,
one rounding); attention output max-abs <= 2e-2 (bf16 I/O, fp32 accumulate).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import attention, geometry, layout, select
from synth import CONFIGS, Workload, smooth_field_qkv
from tests.helpers import csr_rows, oracle_tile_rows, structs_of, unambiguous

pytestmark = pytest.mark.gpu
ATOL = 2e-2

SMALL = {
    # dense 8-tile problem, 32-token tiles, d=64
    "tiny": CONFIGS["tiny"],
    # ragged edge tiles (grid not divisible), 24-token tiles -> 32 slots
    "ragged_d64": Workload("ragged_d64", 1, 3, 64, (5, 7, 9), (2, 3, 4), window=(3, 3, 3), topk=3),
    # Wan-480p tile shape (144 tokens -> 160 slots, a 32-key tail chunk),
    # partial last W tile, Top-P + window
    "w480_mini": Workload("w480_mini", 1, 2, 128, (6, 12, 20), (3, 6, 8), window=(3, 3, 3), topp=0.9),
    # HunyuanVideo tile shape (384 tokens), static window 3x3x5, d=128
    "hy_mini": Workload("hy_mini", 1, 2, 128, (12, 16, 24), (6, 8, 8), window=(3, 3, 5)),
    # clamp-mode window
    "hy_mini_clamp": Workload("hy_mini_clamp", 1, 1, 128, (12, 16, 40), (6, 8, 8), window=(1, 1, 3),
                              win_mode="clamp"),
    # dense, two batches
    "dense_b2": Workload("dense_b2", 2, 2, 64, (3, 5, 6), (1, 5, 6)),
    # Top-K only (scores decide everything), d=128, 112-token tiles
    "topk_only": Workload("topk_only", 1, 2, 128, (7, 8, 8), (7, 4, 4), topk=3),
    # max summarizer of K (scores against per-channel key maxima)
    "topk_max": Workload("topk_max", 1, 2, 128, (7, 8, 8), (7, 4, 4), topk=3, summarizer="max"),
    # max/min bound estimator + attention sink + window, ragged tiles, d=64
    "topp_minmax_sink": Workload("topp_minmax_sink", 1, 3, 64, (5, 7, 9), (2, 3, 4), window=(3, 3, 3),
                                 topp=0.9, summarizer="minmax", sink=2),
    # static window + sink (the plan's static counts include the sink)
    "window_sink": Workload("window_sink", 1, 2, 128, (12, 16, 24), (6, 8, 8), window=(1, 1, 3), sink=4),
    # eight 32-row slabs per tile (eight-wave workgroups, 4-stage ring), window + Top-K
    "eight_slab": Workload("eight_slab", 1, 2, 128, (4, 16, 32), (1, 16, 16), window=(3, 1, 1), topk=2),
    # seven slabs (224-token tiles), ragged on every axis, Top-P, d=64
    "seven_slab_ragged": Workload("seven_slab_ragged", 1, 2, 64, (5, 9, 30), (2, 8, 14), topp=0.9),
    # static window over 144-token tiles: query tiles run in pairs (union of their kept
    # lists); 9 tiles, so the last pair has one tile, and the last W tile is half full
    "pair_window_odd": Workload("pair_window_odd", 1, 2, 128, (3, 18, 20), (3, 6, 8), window=(3, 3, 3)),
    # paired 105-token tiles (4 slabs): 16-key units with 9 valid keys end every full
    # tile, 45-token edge tiles end with 13; Top-P + window
    "pair_units_105": Workload("pair_units_105", 1, 2, 128, (6, 10, 17), (3, 5, 7), window=(3, 3, 3),
                               topp=0.9),
    # paired 168-token tiles (6 slabs, 16-key units), d=64, 144-token edge tiles, Top-P only
    "pair_units_d64": Workload("pair_units_d64", 1, 2, 64, (4, 12, 40), (2, 6, 14), topp=0.8),
    # 96-token tiles (a 32-key tail chunk per tile), Top-K + window, two batches, d=64
    "topk_96": Workload("topk_96", 2, 2, 64, (6, 8, 24), (2, 4, 12), window=(3, 1, 1), topk=2),
    # 336-token tiles (eleven-wave workgroups, 4-stage ring, a 16-key tail chunk per tile),
    # static window, ragged H
    # Top-K over 192-token tiles: query tiles paired, interleaved schedule
    "topk_pair_192": Workload("topk_pair_192", 1, 2, 128, (6, 16, 24), (3, 8, 8), topk=3),
    # the same with ragged edge tiles, an odd tile count (the last pair has one tile) and d=64
    "topk_pair_ragged": Workload("topk_pair_ragged", 1, 3, 64, (7, 8, 20), (3, 8, 8), topk=4),
    "eleven_slab_units": Workload("eleven_slab_units", 1, 2, 128, (12, 13, 24), (6, 7, 8), window=(3, 3, 3)),
    # Top-K over 112-token tiles (four-wave workgroups, two per CU), three t tiles
    "topk_112": Workload("topk_112", 1, 2, 128, (21, 8, 12), (7, 4, 4), topk=5),
    # the same with ragged tiles on every axis (a 2-frame last t tile), two batches, d=64
    "topk_112_ragged": Workload("topk_112_ragged", 2, 2, 64, (16, 9, 10), (7, 4, 4), topk_frac=0.3),
}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _inputs(wl, device="cuda", seed=0):
    return smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=seed, device=device)


def _run_all(wl, q, k, v):
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    return plan, o


@pytest.mark.parametrize("name", list(SMALL))
def test_layout_roundtrip_and_tile_major(name):
    wl = SMALL[name]
    _say(f"layout {name}")
    q, k, v = _inputs(wl)
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    plan.layout(q, k, v)
    slots = plan.info.slots[0]
    mem = geometry.tile_members(wl.grid, wl.tile)
    nT = len(mem)
    # the bf16 attention reads Q in raster order: no tile-major Q exists
    with pytest.raises(vsa.VsaError):
        plan.untile(0, torch.zeros_like(q))
    back_k = plan.untile(1, torch.zeros_like(k))
    torch.cuda.synchronize()
    assert torch.equal(back_k, k)
    want_k = layout.to_tile_major(k.view(torch.int16).cpu().numpy(), mem, slots)
    got_k = plan.region(_lib.VSA_WS_KT, torch.int16).view(wl.B, wl.H, nT, slots, wl.d).cpu().numpy()
    assert np.array_equal(got_k, want_k)
    want_v = layout.to_tile_major(v.view(torch.int16).cpu().numpy(), mem, slots)
    got_vt = plan.region(_lib.VSA_WS_VT, torch.int16).view(wl.B, wl.H, nT, wl.d, slots).cpu().numpy()
    assert np.array_equal(got_vt.transpose(0, 1, 2, 4, 3), want_v)


@pytest.mark.parametrize("name", [n for n, w in SMALL.items() if w.topk or w.topp])
def test_pooled_means_bit_exact(name):
    wl = SMALL[name]
    _say(f"pooled {name}")
    q, k, v = _inputs(wl)
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    plan.layout(q, k, v)
    torch.cuda.synchronize()
    mem = geometry.tile_members(wl.grid, wl.tile)
    nT = len(mem)
    pq = plan.region(_lib.VSA_WS_POOLED_Q, torch.float32).view(wl.B * wl.H, nT, wl.d).cpu().numpy()
    # K summaries are channel-major [head][d][tile]
    pk = plan.region(_lib.VSA_WS_POOLED_K, torch.float32).view(wl.B * wl.H, wl.d, nT).transpose(1, 2).cpu().numpy()
    if wl.summarizer == "minmax":
        pkn = plan.region(_lib.VSA_WS_POOLED_KMIN, torch.float32).view(wl.B * wl.H, wl.d, nT).transpose(1, 2).cpu().numpy()
    qn, kn = q.float().cpu().numpy(), k.float().cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            assert np.array_equal(pq[b * wl.H + h], select.pooled_means(qn[b, h], mem))
            if wl.summarizer == "mean":
                assert np.array_equal(pk[b * wl.H + h], select.pooled_means(kn[b, h], mem))
            else:
                kmax, kmin = select.pooled_extrema(kn[b, h], mem)
                assert np.array_equal(pk[b * wl.H + h], kmax)
                if wl.summarizer == "minmax":
                    assert np.array_equal(pkn[b * wl.H + h], kmin)


# (pair, units) the plan must choose for the cases that exist to run the
# paired / unit kernels (and for two that must not)
KERNELS = {"w480_mini": (1, 1), "pair_window_odd": (1, 1), "pair_units_105": (1, 1),
           "pair_units_d64": (1, 1), "eleven_slab_units": (0, 0), "hy_mini": (0, 0),
           "topk_only": (0, 0), "topk_max": (0, 0), "topk_pair_192": (1, 0), "topk_pair_ragged": (1, 0)}
# Top-K pairs (six-slab tiles) stream the interleaved schedule
INTERLEAVED = {"topk_pair_192", "topk_pair_ragged"}


@pytest.mark.parametrize("name", list(SMALL))
def test_selection_and_attention_small(name):
    wl = SMALL[name]
    _say(f"forward {name}")
    q, k, v = _inputs(wl)
    plan, o = _run_all(wl, q, k, v)
    if name in KERNELS:  # (pair, units)
        assert (plan.info.pair[0], plan.info.units[0]) == KERNELS[name]
    assert plan.info.interleave[0] == int(name in INTERLEAVED), list(plan.info.interleave)
    # score-only masks (no window) order the attention head by head
    assert plan.info.head_sync == int(wl.window is None and bool(wl.topk or wl.topk_frac or wl.topp))
    row_ptr, col, _ = plan.read_selection()
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    on = o.float().cpu().numpy()
    nT = plan.info.n_tiles[0]
    for b in range(wl.B):
        for h in range(wl.H):
            bh = b * wl.H + h
            rows, margins, mem = oracle_tile_rows(wl, qn[b, h], kn[b, h], wl.tile)
            got = csr_rows(row_ptr, col, bh, plan.info.max_tiles, nT)
            ok = unambiguous(range(nT), margins)
            for i in ok:
                assert got[i] == rows[i], (b, h, i)
            ref = attention.block_sparse_attention(qn[b, h], kn[b, h], vn[b, h], mem, rows, query_tiles=ok)
            for i in ok:
                err = np.abs(on[b, h][mem[i]] - ref[mem[i]]).max()
                assert err <= ATOL, (b, h, i, err)


def test_forward_is_deterministic_and_stage_split_matches():
    wl = SMALL["w480_mini"]
    _say("determinism w480_mini")
    q, k, v = _inputs(wl, seed=5)
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    o1 = plan.forward(q, k, v)
    ws = plan.workspace()
    ws.fill_(0xFF)                      # poison: NaN patterns everywhere
    o2 = plan.forward(q, k, v)
    o3 = torch.empty_like(q)
    plan.layout(q, k, v)
    plan.select()
    plan.attend(o3, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_hunyuan_full_size_sampled():
    """HunyuanVideo 720p shape: all heads' selection, sampled query tiles of O."""
    wl = CONFIGS["hunyuan"]
    _say("hunyuan full size")
    q, k, v = _inputs(wl)
    plan, o = _run_all(wl, q, k, v)
    row_ptr, col, _ = plan.read_selection()
    nT = plan.info.n_tiles[0]
    mem = geometry.tile_members(wl.grid, wl.tile)
    nt = geometry.tile_counts(wl.grid, wl.tile)
    want = [geometry.window(i, nt, wl.window) for i in range(nT)]
    for bh in range(wl.B * wl.H):
        assert csr_rows(row_ptr, col, bh, plan.info.max_tiles, nT) == want
    rng = np.random.default_rng(0)
    for h in (0, 13, 23):
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        on = o[0, h].float().cpu().numpy()
        tiles = sorted(set(rng.choice(nT, 6, replace=False).tolist()) | {0, nT - 1, 155})
        ref = attention.block_sparse_attention(qn, kn, vn, mem, want, query_tiles=tiles)
        for i in tiles:
            err = np.abs(on[mem[i]] - ref[mem[i]]).max()
            assert err <= ATOL, (h, i, err)


def test_wan480_full_size_sampled():
    """Wan-2.1 480p shape (window 3x3x3 united with Top-P 0.9; 144-token tiles,
    the last W tile of every row half full): pooled means and the kept tiles
    of every head against the oracle (bit-exact; a row whose Top-P cut sits
    within the margin of the oracle's rounding is counted, not compared),
    and O on sampled query tiles of three heads, partial tiles included."""
    wl = CONFIGS["wan480"]
    _say("wan480 full size")
    q, k, v = _inputs(wl)
    plan, o = _run_all(wl, q, k, v)
    row_ptr, col, _ = plan.read_selection()
    nT = plan.info.n_tiles[0]
    mem = geometry.tile_members(wl.grid, wl.tile)
    assert nT == len(mem) == 245
    pq = plan.region(_lib.VSA_WS_POOLED_Q, torch.float32).view(wl.H, nT, wl.d).cpu().numpy()
    pk = plan.region(_lib.VSA_WS_POOLED_K, torch.float32).view(wl.H, wl.d, nT).transpose(1, 2).cpu().numpy()
    rng = np.random.default_rng(1)
    near_cut = 0
    for h in range(wl.H):
        qn, kn = (t[0, h].float().cpu().numpy() for t in (q, k))
        assert np.array_equal(pq[h], select.pooled_means(qn, mem)), h
        assert np.array_equal(pk[h], select.pooled_means(kn, mem)), h
        rows, margins, _ = oracle_tile_rows(wl, qn, kn, wl.tile)
        got = csr_rows(row_ptr, col, h, plan.info.max_tiles, nT)
        ok = unambiguous(range(nT), margins)
        near_cut += nT - len(ok)
        for i in ok:
            assert got[i] == rows[i], (h, i)
        if h in (0, 5, 11):
            vn = v[0, h].float().cpu().numpy()
            on = o[0, h].float().cpu().numpy()
            # tile 6 and 244 are partial (4 of 8 W columns); 122 is interior
            tiles = unambiguous(sorted(set(rng.choice(nT, 4, replace=False).tolist()) | {0, 6, 122, nT - 1}),
                                margins)
            ref = attention.block_sparse_attention(qn, kn, vn, mem, rows, query_tiles=tiles)
            for i in tiles:
                err = np.abs(on[mem[i]] - ref[mem[i]]).max()
                assert err <= ATOL, (h, i, err)
    assert near_cut <= nT * wl.H // 100, near_cut


MAXIMA = {
    # 4096 tiles (the plan's limit) of one token each: the selection sorts
    # 4096 scores per row; every key tile is a 32-slot chunk with one key
    "max_tiles_topk": Workload("max_tiles_topk", 1, 1, 64, (16, 16, 16), (1, 1, 1), window=(3, 3, 3),
                               topk=8),
    "max_tiles_topp": Workload("max_tiles_topp", 1, 1, 64, (16, 16, 16), (1, 1, 1), topp=0.3),
    # two tiles of 4096 tokens (the tile-size limit): 128 slabs per tile, so
    # eleven workgroups of twelve waves per tile, the last with four idle waves
    "max_tile": Workload("max_tile", 1, 1, 128, (16, 16, 32), (16, 16, 16), window=(1, 1, 3)),
}


@pytest.mark.parametrize("name", list(MAXIMA))
def test_maximum_sizes(name):
    """The limits the plan accepts: the kept tiles of every row bit-exact and
    O within 2e-2 on every query row (sampled query tiles for the 4096-tile
    cases)."""
    wl = MAXIMA[name]
    _say(f"maximum {name}")
    q, k, v = _inputs(wl)
    plan, o = _run_all(wl, q, k, v)
    row_ptr, col, _ = plan.read_selection()
    qn, kn, vn = (t[0, 0].float().cpu().numpy() for t in (q, k, v))
    rows, margins, mem = oracle_tile_rows(wl, qn, kn, wl.tile)
    nT = len(mem)
    assert plan.info.n_tiles[0] == nT
    got = csr_rows(row_ptr, col, 0, plan.info.max_tiles, nT)
    for i in unambiguous(range(nT), margins):
        assert got[i] == rows[i], i
    tiles = unambiguous(list(range(nT)) if nT <= 2 else sorted(set(range(0, nT, 37)) | {nT - 1}), margins)
    ref = attention.block_sparse_attention(qn, kn, vn, mem, rows, query_tiles=tiles)
    on = o[0, 0].float().cpu().numpy()
    for i in tiles:
        err = np.abs(on[mem[i]] - ref[mem[i]]).max()
        assert err <= ATOL, (i, err)
