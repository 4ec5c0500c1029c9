"""GPU parity of the cached-mask forward (vsa_forward_cached).

A mask computed on one input (A) is reused on another (B): the selection in
the workspace must stay bit-identical, and the output on B must equal the
oracle's masked attention on B under A's selection (and, for SICS, under A's
blocking choice).  A workspace whose selection was never written must give
zeros, not out-of-bounds accesses.  Tolerance: attention max-abs <= 2e-2.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import attention, fine, geometry
from synth import Workload, smooth_field_qkv
from tests.helpers import csr_rows, oracle_candidate, oracle_tile_rows, structs_of, unambiguous

pytestmark = pytest.mark.gpu
ATOL = 2e-2

CASES = {
    # Top-P + window, Wan-480p tile shape (partial chunks)
    "w480_mini": Workload("w480_mini", 1, 2, 128, (6, 12, 20), (3, 6, 8), window=(3, 3, 3), topp=0.9),
    # Top-K only, ragged tiles, d=64, two batches
    "topk_ragged": Workload("topk_ragged", 2, 2, 64, (5, 7, 9), (2, 3, 4), topk=3),
    # SICS blocking choice + Top-K fraction (the blocking is part of the cached mask)
    "sics": Workload("sics", 1, 4, 128, (14, 16, 16), (1, 16, 16),
                     candidates=((1, 16, 16), (7, 4, 4), (7, 8, 8)), topk_frac=0.2,
                     ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
    # static window (the cached call skips nothing but the no-op selection)
    "hy_mini": Workload("hy_mini", 1, 2, 128, (12, 16, 24), (6, 8, 8), window=(3, 3, 5)),
}
FINE = Workload("fine_cached", 1, 2, 128, (5, 8, 16), (1, 1, 1), fine_group=64, fine_keep=0.15)


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _inputs(wl, seed):
    return smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=seed, device="cuda")


@pytest.mark.parametrize("name", list(CASES))
def test_cached_mask_reused_on_new_input(name):
    wl = CASES[name]
    _say(f"cached {name}")
    plan = vsa.Plan(*structs_of(wl))
    qa, ka, va = _inputs(wl, 0)
    qb, kb, vb = _inputs(wl, 7)
    plan.forward(qa, ka, va)
    torch.cuda.synchronize()
    rp_a, col_a, cand_a = plan.read_selection()
    ob = plan.forward_cached(qb, kb, vb)
    torch.cuda.synchronize()
    rp_b, col_b, cand_b = plan.read_selection()
    assert np.array_equal(rp_a, rp_b) and np.array_equal(col_a, col_b) and np.array_equal(cand_a, cand_b)
    tiles = wl.candidates or (wl.tile,)
    mt = plan.info.max_tiles
    worst = 0.0
    for b in range(wl.B):
        for h in range(wl.H):
            bh = b * wl.H + h
            # A's selection is the oracle's on A (Top-P rows at the rounding margin excepted)
            qa_h, ka_h = (t[b, h].float().cpu().numpy() for t in (qa, ka))
            if wl.candidates:
                c_ref, _ = oracle_candidate(wl, qa_h, ka_h)
                assert int(cand_a[bh]) == c_ref, (bh, int(cand_a[bh]), c_ref)
            tile = tiles[int(cand_a[bh])] if wl.candidates else wl.tile
            mem = geometry.tile_members(wl.grid, tile)
            rows = csr_rows(rp_a, col_a, bh, mt, len(mem))
            rows_ref, margins, _ = oracle_tile_rows(wl, qa_h, ka_h, tile)
            for i in unambiguous(range(len(mem)), margins):
                assert rows[i] == list(rows_ref[i]), (bh, i)
            qn, kn, vn = (t[b, h].float().cpu().numpy() for t in (qb, kb, vb))
            ref = attention.block_sparse_attention(qn, kn, vn, mem, rows)
            worst = max(worst, float(np.abs(ob[b, h].float().cpu().numpy() - ref).max()))
    assert worst <= ATOL, worst


def test_cached_fine_mask_reused_on_new_input():
    wl = FINE
    _say("cached fine")
    plan = vsa.Plan(*structs_of(wl))
    qa, ka, va = _inputs(wl, 0)
    qb, kb, vb = _inputs(wl, 7)
    plan.forward(qa, ka, va)
    torch.cuda.synchronize()
    BH, G, N = wl.B * wl.H, plan.info.fine_groups, wl.N
    count = plan.region(_lib.VSA_WS_FINE_COUNT, torch.int32).view(BH, G).cpu().numpy().copy()
    idx = plan.region(_lib.VSA_WS_FINE_IDX, torch.int32).view(BH, G, N).cpu().numpy().copy()
    ob = plan.forward_cached(qb, kb, vb)
    torch.cuda.synchronize()
    assert np.array_equal(count, plan.region(_lib.VSA_WS_FINE_COUNT, torch.int32).view(BH, G).cpu().numpy())
    grp = fine.groups(N, wl.fine_group)
    for bh in range(BH):
        lists = [idx[bh, g, :count[bh, g]] for g in range(G)]
        # A's mask is the oracle's on A
        s_a = fine.group_scores(fine.group_means(qa[0, bh].float().cpu().numpy(), wl.fine_group),
                                ka[0, bh].float().cpu().numpy())
        ref_lists = fine.kept_lists(s_a, fine.threshold(s_a, fine.keep_count(wl.fine_keep, G, N)))
        assert all(np.array_equal(a, r) for a, r in zip(lists, ref_lists)), bh
        qn, kn, vn = (t[0, bh].float().cpu().numpy() for t in (qb, kb, vb))
        ref = attention.fine_attention(qn, kn, vn, grp, lists)
        err = float(np.abs(ob[0, bh].float().cpu().numpy() - ref).max())
        assert err <= ATOL, (bh, err)


@pytest.mark.parametrize("name", ["topk_ragged", "sics", "fine"])
def test_cached_on_unwritten_selection_gives_zeros(name):
    wl = FINE if name == "fine" else CASES[name]
    _say(f"cached unwritten {name}")
    plan = vsa.Plan(*structs_of(wl))
    plan.workspace().fill_(0xFF)  # every selection field reads -1
    q, k, v = _inputs(wl, 3)
    o = torch.full_like(q, 7.0)
    plan.forward_cached(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    # the host-side getters refuse the poisoned fields instead of indexing with them
    # (blocking index -1 under SICS, row length -1 otherwise)
    if name != "fine":
        with pytest.raises(vsa.VsaError, match="corrupt blocking index" if name == "sics" else "corrupt row length"):
            plan.read_selection()
    with pytest.raises(vsa.VsaError, match="corrupt"):
        plan.retained_work()

