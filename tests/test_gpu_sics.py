"""GPU parity of the SICS blocking choice (Wan-14B path) against the oracle.

Tolerances: per-tile SICS and candidate scores 1e-3 relative (absolute floor
1e-3 x pairs for tiles whose sum cancels); the chosen blocking exact (the
score margin between the two best candidates is printed); kept tiles
bit-exact under the chosen blocking; O max-abs <= 2e-2.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import attention, geometry, sics
from synth import CONFIGS, Workload, smooth_field_qkv
from tests.helpers import csr_rows, oracle_tile_rows, structs_of

pytestmark = pytest.mark.gpu
ATOL = 2e-2
CANDS = ((1, 16, 16), (7, 4, 4), (3, 8, 8))

SMALL = {
    "sics_d128": Workload("sics_d128", 1, 4, 128, (14, 16, 16), (1, 16, 16), candidates=CANDS,
                          topk_frac=0.2, ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
    # ragged: H=20 is not a multiple of 16 or 8; two batches; d=64; window too
    "sics_ragged_d64": Workload("sics_ragged_d64", 2, 2, 64, (7, 20, 16), (1, 16, 16),
                                candidates=((1, 16, 16), (7, 4, 4)), topk_frac=0.25,
                                window=(1, 1, 3), ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
    # 72 heads: the head-synchronous attention order finds the r-th head of a
    # blocking across two 64-head ballot windows
    "sics_72_heads": Workload("sics_72_heads", 2, 36, 64, (7, 16, 16), (1, 16, 16),
                              candidates=((1, 16, 16), (7, 4, 4)), topk_frac=0.25,
                              ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _check_head(wl, plan, qn, kn, bh, sics_t, scores, cand, row_ptr, col, tol_log):
    for c, tile in enumerate(wl.candidates):
        mem = geometry.tile_members(wl.grid, tile)
        for x, arr in ((0, qn), (1, kn)):
            ref = sics.tile_sics(arr, mem)
            got = sics_t[bh, c, x, :len(mem)]
            pairs = np.array([len(m) * (len(m) - 1) / 2.0 for m in mem])
            err = np.abs(got - ref)
            assert np.all(err <= 1e-3 * np.maximum(np.abs(ref), pairs * 1.0)), (bh, c, x, err.max())
    want_c, sc = sics.candidate_scores(qn, kn, wl.grid, wl.candidates), None
    ref_scores = want_c
    assert np.allclose(scores[bh], ref_scores, rtol=1e-3, atol=1e-4), (bh, scores[bh], ref_scores)
    order = np.sort(ref_scores)[::-1]
    margin = order[0] - order[1] if len(order) > 1 else np.inf
    tol_log.append(margin)
    best = sics.choose(ref_scores)
    if margin > 1e-4:
        assert cand[bh] == best, (bh, cand[bh], best, ref_scores)
    return int(cand[bh])


@pytest.mark.parametrize("name", list(SMALL))
def test_sics_choice_selection_attention(name):
    wl = SMALL[name]
    _say(f"sics {name}")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=1, device="cuda")
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    # Top-K without a window: attention workgroups ordered head by head
    assert plan.info.head_sync == (wl.window is None)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    nb = len(wl.candidates)
    BH = wl.B * wl.H
    mt = plan.info.max_tiles
    sics_t = plan.region(_lib.VSA_WS_TILE_SICS, torch.float32).view(BH, nb, 2, mt).cpu().numpy()
    scores = plan.region(_lib.VSA_WS_CAND_SCORE, torch.float32).view(BH, nb).cpu().numpy()
    row_ptr, col, cand = plan.read_selection()
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    on = o.float().cpu().numpy()
    margins = []
    chosen = []
    for b in range(wl.B):
        for h in range(wl.H):
            bh = b * wl.H + h
            c = _check_head(wl, plan, qn[b, h], kn[b, h], bh, sics_t, scores, cand, row_ptr, col,
                            margins)
            chosen.append(c)
            tile = wl.candidates[c]
            rows, tmarg, mem = oracle_tile_rows(wl, qn[b, h], kn[b, h], tile)
            got = csr_rows(row_ptr, col, bh, mt, len(mem))
            assert got == rows, (b, h)
            ref = attention.block_sparse_attention(qn[b, h], kn[b, h], vn[b, h], mem, rows)
            err = np.abs(on[b, h] - ref).max()
            assert err <= ATOL, (b, h, err)
    print(f"chosen blockings {chosen}, min score margin {min(margins):.3e}", flush=True)
    # heads alternate between temporal and spatial correlation; the choice follows
    assert chosen[0] != chosen[1]


def test_wan14b_full_size():
    """Wan-14B 720p shape: SICS scores, blocking choice and Top-K selection of
    all 40 heads against the oracle; per-tile SICS and O on sampled heads."""
    wl = CONFIGS["wan14b"]
    _say("wan14b full size")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0, device="cuda")
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    nb = len(wl.candidates)
    mt = plan.info.max_tiles
    scores = plan.region(_lib.VSA_WS_CAND_SCORE, torch.float32).view(wl.H, nb).cpu().numpy()
    sics_t = plan.region(_lib.VSA_WS_TILE_SICS, torch.float32).view(wl.H, nb, 2, mt).cpu().numpy()
    row_ptr, col, cand = plan.read_selection()
    margins = []
    rng = np.random.default_rng(0)
    sample = sorted(set(rng.choice(wl.H, 6, replace=False).tolist()) | {0, 1})
    for h in range(wl.H):
        # every head: candidate scores, the chosen blocking and its kept tiles;
        # the sampled heads also per-tile SICS and O on sampled query tiles
        qn, kn = (t[0, h].float().cpu().numpy() for t in (q, k))
        if h in sample:
            c = _check_head(wl, plan, qn, kn, h, sics_t, scores, cand, row_ptr, col, margins)
        else:
            ref_scores = sics.candidate_scores(qn, kn, wl.grid, wl.candidates)
            assert np.allclose(scores[h], ref_scores, rtol=1e-3, atol=1e-4), (h, scores[h], ref_scores)
            order = np.sort(ref_scores)[::-1]
            margins.append(order[0] - order[1])
            assert margins[-1] > 1e-4 and int(cand[h]) == sics.choose(ref_scores), (h, ref_scores)
            c = int(cand[h])
        tile = wl.candidates[c]
        rows, _, mem = oracle_tile_rows(wl, qn, kn, tile)
        got = csr_rows(row_ptr, col, h, mt, len(mem))
        assert got == rows, h
        assert all(len(r) == plan.info.topk[c] for r in got)
        if h in sample:
            vn = v[0, h].float().cpu().numpy()
            on = o[0, h].float().cpu().numpy()
            tiles = sorted(set(rng.choice(len(mem), 4, replace=False).tolist()) | {len(mem) - 1})
            ref = attention.block_sparse_attention(qn, kn, vn, mem, rows, query_tiles=tiles)
            for i in tiles:
                err = np.abs(on[mem[i]] - ref[mem[i]]).max()
                assert err <= ATOL, (h, i, err)
    print(f"cand per head {cand.tolist()}, min margin {min(margins):.3e}", flush=True)
    assert set(cand[0::2].tolist()) == {1} and set(cand[1::2].tolist()) == {0}


def test_side_streams_join_the_callers_stream():
    """Per-head blockings launch on side streams forked from and joined into the caller's
    stream: on a non-default stream the output equals the default stream's bit for bit, and
    work enqueued on that stream right after the call (a copy of the output) sees all of it."""
    wl = SMALL["sics_d128"]
    _say("side streams on a user stream")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=2, device="cuda")
    plan = vsa.Plan(*structs_of(wl))
    assert plan.info.n_blockings == 3
    ref = plan.forward(q, k, v)
    torch.cuda.synchronize()
    _, _, cand = plan.read_selection()
    assert len(set(cand.tolist())) >= 2  # at least two blockings' launches in flight together
    s = torch.cuda.Stream()
    snaps = []
    with torch.cuda.stream(s):
        for _ in range(3):
            o = torch.full_like(q, 7.0)
            plan.forward(q, k, v, o)
            snaps.append(o.clone())
    torch.cuda.synchronize()
    for snap in snaps:
        assert torch.equal(snap, ref)


def test_concurrent_callers_share_the_side_streams():
    """Two host threads, each with its own plan, workspace and stream, call the library at the
    same time (the binding releases the interpreter lock during each call): both plans launch
    per-blocking work on the device's one set of side streams, and every output still equals
    that plan's single-threaded result bit for bit."""
    import threading

    wl_a, wl_b = SMALL["sics_d128"], SMALL["sics_ragged_d64"]
    _say("two threads, two plans, shared side streams")
    qa, ka, va = smooth_field_qkv(wl_a.B, wl_a.H, wl_a.d, wl_a.grid, wl_a.ell_per_head(), seed=4,
                                  device="cuda")
    qb, kb, vb = smooth_field_qkv(wl_b.B, wl_b.H, wl_b.d, wl_b.grid, wl_b.ell_per_head(), seed=5,
                                  device="cuda")
    plan_a, plan_b = vsa.Plan(*structs_of(wl_a)), vsa.Plan(*structs_of(wl_b))
    assert plan_a.info.n_blockings == 3 and plan_b.info.n_blockings == 2
    ref_a, ref_b = plan_a.forward(qa, ka, va), plan_b.forward(qb, kb, vb)
    torch.cuda.synchronize()
    outs = {"a": [], "b": []}
    errors = []
    barrier = threading.Barrier(2)

    def worker(name, plan, q, k, v):
        try:
            s = torch.cuda.Stream()
            barrier.wait()
            with torch.cuda.stream(s):
                for _ in range(6):
                    o = torch.full_like(q, 3.0)
                    plan.forward(q, k, v, o)
                    outs[name].append(o.clone())
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=("a", plan_a, qa, ka, va)),
               threading.Thread(target=worker, args=("b", plan_b, qb, kb, vb))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    assert len(outs["a"]) == 6 and len(outs["b"]) == 6
    for o in outs["a"]:
        assert torch.equal(o, ref_a)
    for o in outs["b"]:
        assert torch.equal(o, ref_b)
