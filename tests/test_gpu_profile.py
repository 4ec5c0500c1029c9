"""GPU parity of the online profiling selector (VSA_PROFILE_SELECT) against
the oracle (oracle/profile.py).

Per head: the MSE of every candidate on the sampled rows, the chosen
blocking, and the attention output under it.

Tolerance of an MSE: the kernel's outputs carry bf16-rounded probabilities
and fp32 sums, each off from the fp64 ones by less than delta = 2^-7 max|v|
(four times the 2^-9 rounding of one probability, relative to the spread of
V); then |(a + e1)^2 - a^2| summed as a mean gives
|MSE_gpu - MSE| <= 2 sqrt(MSE) delta + delta^2.  The choice must match the
oracle's whenever the two best MSEs are further apart than twice that.
Attention output: max-abs <= 2e-2, as for every bf16 path.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import attention, geometry, profile
from synth import Workload, smooth_field_qkv
from tests.helpers import csr_rows, structs_of

pytestmark = pytest.mark.gpu
ATOL = 2e-2

CASES = {
    # anisotropic heads (temporal-like ell = (8,1,1) and spatial-like (1,8,8)), three candidates
    "aniso_d128": Workload("aniso_d128", 1, 4, 128, (14, 16, 16), (1, 16, 16),
                           candidates=((1, 16, 16), (7, 4, 4), (7, 8, 8)), window=(1, 1, 1),
                           ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0), selector="profile",
                           profile_frac=0.05),
    # clamp-mode window plus a sink, W < 64 (one chunk per line), ragged tiles
    "clamp_sink": Workload("clamp_sink", 1, 2, 128, (6, 12, 20), (1, 6, 8),
                           candidates=((1, 6, 8), (3, 3, 4)), window=(1, 3, 3), win_mode="clamp",
                           sink=2, selector="profile", profile_frac=0.1),
    # long lines (W = 96: two chunks per line, a 32-key tail), d = 64, two batches
    "wide_d64": Workload("wide_d64", 2, 2, 64, (4, 4, 96), (1, 4, 32),
                         candidates=((1, 4, 32), (4, 1, 8)), window=(1, 1, 3), selector="profile",
                         profile_frac=0.25),
    # fewer than 32 tokens: one run of all rows
    "tiny_n": Workload("tiny_n", 1, 2, 64, (1, 4, 6), (1, 2, 3), candidates=((1, 2, 3), (1, 4, 6)),
                       window=(1, 1, 1), selector="profile"),
}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _check_plan(wl, q, k, v):
    plan = vsa.Plan(*structs_of(wl))
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    BH = wl.B * wl.H
    nb = len(wl.candidates)
    mse = plan.region(_lib.VSA_WS_CAND_SCORE, torch.float32).view(BH, nb).cpu().numpy()
    row_ptr, col, cand = plan.read_selection()
    on = o.float().cpu().numpy()
    frac = wl.profile_frac or 0.01
    chosen = []
    for b in range(wl.B):
        for h in range(wl.H):
            bh = b * wl.H + h
            qn, kn, vn = (t[b, h].float().cpu().numpy() for t in (q, k, v))
            want = profile.profile_mse(qn, kn, vn, wl.grid, wl.candidates, wl.window, wl.win_mode,
                                       wl.sink, frac)
            delta = 2.0 ** -7 * np.abs(vn).max()
            tol = 2.0 * np.sqrt(want) * delta + delta ** 2
            assert np.all(np.abs(mse[bh] - want) <= tol), (bh, mse[bh], want, tol)
            order = np.sort(want)
            best = profile.choose(want)
            if len(order) < 2 or order[1] - order[0] > 2.0 * tol.max():
                assert int(cand[bh]) == best, (bh, int(cand[bh]), best, want)
            c = int(cand[bh])
            chosen.append(c)
            tile = wl.candidates[c]
            mem = geometry.tile_members(wl.grid, tile)
            rows = profile.candidate_rows(wl.grid, tile, wl.window, wl.win_mode, wl.sink)
            got = csr_rows(row_ptr, col, bh, plan.info.max_tiles, len(mem))
            assert got == rows, bh
            ref = attention.block_sparse_attention(qn, kn, vn, mem, rows)
            err = float(np.abs(on[b, h] - ref).max())
            assert err <= ATOL, (bh, err)
    return chosen


@pytest.mark.parametrize("name", list(CASES))
def test_profile_choice_and_attention(name):
    wl = CASES[name]
    _say(f"profile {name}")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0, device="cuda")
    _check_plan(wl, q, k, v)


def _planted(grid, d, kind, seed):
    """q = k = 8 x a one-hot code of the frame (spatial head) or of the (h, w)
    position (temporal head), plus small noise; v random.  With d = 64 the
    matching keys then score 64 / 8 = 8 above the rest (weight e^8 each), so
    each head's attention sits on its pattern's keys."""
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    code = (t if kind == "spatial" else h * W + w).ravel() % d
    rng = np.random.default_rng(seed)
    qk = np.eye(d)[code] * 8.0 + rng.standard_normal((code.size, d)) * 0.05
    return qk, qk.copy(), rng.standard_normal((code.size, d))


def test_planted_spatial_and_temporal_heads():
    # one-frame tiles vs one position across all frames: the Sparse VideoGen dichotomy
    wl = Workload("planted", 1, 2, 64, (6, 8, 8), (1, 8, 8), candidates=((1, 8, 8), (6, 1, 1)),
                  window=(1, 1, 1), selector="profile", profile_frac=1.0)
    _say("profile planted")
    heads = [_planted(wl.grid, wl.d, kind, 3 + i) for i, kind in enumerate(("spatial", "temporal"))]
    q, k, v = (torch.tensor(np.stack([hd[x] for hd in heads])[None]).to(torch.bfloat16).cuda()
               for x in range(3))
    assert _check_plan(wl, q, k, v) == [0, 1]



def test_profile_hunyuan_full_size_sampled():
    """HunyuanVideo 720p shape with the spatial / temporal candidates: the
    MSEs and choice of two heads (one of each field kind) against the
    oracle over the same 1% sample, and sampled query tiles of O."""
    from synth import CONFIGS
    wl = CONFIGS["hunyuan_svg"]
    _say("profile hunyuan_svg full size")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0, device="cuda")
    plan = vsa.Plan(*structs_of(wl))
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    nb = len(wl.candidates)
    mse = plan.region(_lib.VSA_WS_CAND_SCORE, torch.float32).view(wl.H, nb).cpu().numpy()
    row_ptr, col, cand = plan.read_selection()
    for h in (0, 1):
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        want = profile.profile_mse(qn, kn, vn, wl.grid, wl.candidates, wl.window, wl.win_mode, wl.sink, 0.01)
        delta = 2.0 ** -7 * np.abs(vn).max()
        tol = 2.0 * np.sqrt(want) * delta + delta ** 2
        assert np.all(np.abs(mse[h] - want) <= tol), (h, mse[h], want, tol)
        c = int(cand[h])
        if abs(want[0] - want[1]) > 2.0 * tol.max():
            assert c == profile.choose(want), (h, c, want)
        tile = wl.candidates[c]
        mem = geometry.tile_members(wl.grid, tile)
        rows = profile.candidate_rows(wl.grid, tile, wl.window, wl.win_mode, wl.sink)
        assert csr_rows(row_ptr, col, h, plan.info.max_tiles, len(mem)) == rows
        tiles = [0, len(mem) // 2, len(mem) - 1]
        ref = attention.block_sparse_attention(qn, kn, vn, mem, rows, query_tiles=tiles)
        on = o[0, h].float().cpu().numpy()
        for i in tiles:
            assert np.abs(on[mem[i]] - ref[mem[i]]).max() <= ATOL, (h, i)
