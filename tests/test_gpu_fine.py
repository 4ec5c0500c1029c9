"""GPU parity of the fine-grained M x 1 path against the oracle.

Bit-exact: group means, the per-head threshold tau, every group's kept-key
list (each group's row of the FINE_IDX region holds its FINE_COUNT kept keys,
ascending).  O max-abs <= 2e-2.  Planted inputs drive every way the library
can reach tau: the thin rescored band around it (smooth fields, a key of huge
norm), the exact path over every pair (all scores equal, so the band exceeds
the rescoring buffer; approximations beyond fp32 range), and ties at tau that
cover many whole groups.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import attention, fine
from synth import CONFIGS, Workload, smooth_field_qkv
from tests.helpers import structs_of

pytestmark = pytest.mark.gpu
ATOL = 2e-2

SMALL = {
    "fine_d128": Workload("fine_d128", 1, 2, 128, (5, 8, 16), (1, 1, 1), fine_group=64, fine_keep=0.15),
    # N = 189 is not a multiple of M = 32 (last group 29 rows); d = 64; 2 batches
    "fine_ragged_d64": Workload("fine_ragged_d64", 2, 2, 64, (3, 7, 9), (1, 1, 1), fine_group=32,
                                fine_keep=0.3),
    # keep everything: dense attention
    "fine_dense": Workload("fine_dense", 1, 1, 128, (2, 8, 12), (1, 1, 1), fine_group=64, fine_keep=1.0),
    # M = 128 (four waves per group)
    "fine_m128": Workload("fine_m128", 1, 2, 128, (4, 8, 16), (1, 1, 1), fine_group=128, fine_keep=0.2),
    # 32-row groups at d = 128 (a second, gather-only wave per workgroup), ragged last group
    "fine_m32_d128": Workload("fine_m32_d128", 1, 2, 128, (3, 6, 11), (1, 1, 1), fine_group=32,
                              fine_keep=0.2),
}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _device_mask(plan, wl):
    BH, G, d, N = wl.B * wl.H, plan.info.fine_groups, wl.d, wl.N
    qbar = plan.region(_lib.VSA_WS_FINE_QBAR, torch.float32).view(BH, G, d).cpu().numpy()
    tau = plan.region(_lib.VSA_WS_FINE_TAU, torch.float64)[:BH].cpu().numpy()
    count = plan.region(_lib.VSA_WS_FINE_COUNT, torch.int32).view(BH, G).cpu().numpy()
    idx = plan.region(_lib.VSA_WS_FINE_IDX, torch.int32).view(BH, G, N).cpu().numpy()
    return qbar, tau, count, idx


def _check_mask(wl, qn, kn, bh, qbar, tau, count, idx):
    """Group means, tau and every kept list bit-exact; returns the lists."""
    M = wl.fine_group
    qb_ref = fine.group_means(qn, M)
    assert np.array_equal(qbar[bh], qb_ref), bh
    s = fine.group_scores(qb_ref, kn)
    G, N = s.shape
    kc = fine.keep_count(wl.fine_keep, G, N)
    t_ref = fine.threshold(s, kc)
    assert tau[bh] == t_ref, (bh, tau[bh], t_ref)
    lists = fine.kept_lists(s, t_ref)
    for gi in range(G):
        got = idx[bh, gi, :count[bh, gi]]
        assert np.array_equal(got, lists[gi]), (bh, gi)
    return lists


def _check_head(wl, plan, qn, kn, vn, on, bh, qbar, tau, count, idx, groups=None):
    lists = _check_mask(wl, qn, kn, bh, qbar, tau, count, idx)
    N = kn.shape[0]
    G = len(lists)
    grp = fine.groups(N, wl.fine_group)
    sel = range(G) if groups is None else groups
    ref = attention.fine_attention(qn, kn, vn, grp, lists, query_groups=sel)
    for gi in sel:
        err = np.abs(on[grp[gi]] - ref[grp[gi]]).max()
        assert err <= ATOL, (bh, gi, err)


@pytest.mark.parametrize("name", list(SMALL))
def test_fine_small(name):
    wl = SMALL[name]
    _say(f"fine {name}")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=2, device="cuda")
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    qbar, tau, count, idx = _device_mask(plan, wl)
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    on = o.float().cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            _check_head(wl, plan, qn[b, h], kn[b, h], vn[b, h], on[b, h], b * wl.H + h, qbar, tau,
                        count, idx)
    pairs, flops = plan.retained_work()
    assert pairs == int(count.sum())


def test_fine_full_size_sampled():
    wl = CONFIGS["fine"]
    _say("fine full size")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0, device="cuda")
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    qbar, tau, count, idx = _device_mask(plan, wl)
    G = plan.info.fine_groups
    kept = count.sum(axis=1)
    print(f"kept pairs per head {kept.tolist()} (target {plan.info.fine_keep_count})", flush=True)
    assert np.all(kept >= plan.info.fine_keep_count)
    # a second call gives the identical mask
    plan.forward(q, k, v)
    torch.cuda.synchronize()
    _, tau2, count2, idx2 = _device_mask(plan, wl)
    assert np.array_equal(tau, tau2) and np.array_equal(count, count2)
    for h in range(wl.H):
        for gi in range(G):
            assert np.array_equal(idx[h, gi, :count[h, gi]], idx2[h, gi, :count[h, gi]])
    rng = np.random.default_rng(0)
    for h in range(wl.H):  # every head's mask; O on sampled groups of two heads
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        if h in (0, 7):
            on = o[0, h].float().cpu().numpy()
            groups = sorted(set(rng.choice(G, 5, replace=False).tolist()) | {G - 1})
            _check_head(wl, plan, qn, kn, vn, on, h, qbar, tau, count, idx, groups=groups)
        else:
            _check_mask(wl, qn, kn, h, qbar, tau, count, idx)


def _planted(kind):
    """Planted inputs (CPU, bf16) and the workload they belong to."""
    g = torch.Generator().manual_seed(11)
    if kind == "huge_key":
        # one key of norm ~1000x the others: its scores dwarf the rest
        wl = Workload("fine_huge_key", 1, 2, 128, (4, 8, 32), (1, 1, 1), fine_group=64, fine_keep=0.15)
        q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=5)
        k[0, 0, 37] = (k[0, 0, 37].float() * 1000).to(torch.bfloat16)
        k[0, 1, 5] = (k[0, 1, 5].float() * -1000).to(torch.bfloat16)
    elif kind == "all_equal":
        # every query row equal and every key equal: all G*N scores tie, so tau
        # is that score, every pair is kept, and the band (everything) exceeds
        # the rescoring buffer
        wl = Workload("fine_all_equal", 1, 1, 128, (4, 16, 64), (1, 1, 1), fine_group=16, fine_keep=0.15)
        row_q = torch.randn(128, generator=g)
        row_k = torch.randn(128, generator=g)
        q = row_q.expand(1, 1, wl.N, 128).to(torch.bfloat16).contiguous()
        k = row_k.expand(1, 1, wl.N, 128).to(torch.bfloat16).contiguous()
        v = torch.randn(1, 1, wl.N, 128, generator=g).to(torch.bfloat16)
    elif kind == "group_ties":
        # all keys equal and runs of 8 groups with identical rows: every score
        # of a run ties, so the ties at tau span 8 whole groups (8 N pairs)
        wl = Workload("fine_group_ties", 1, 2, 64, (3, 8, 40), (1, 1, 1), fine_group=32, fine_keep=0.3)
        G = -(-wl.N // 32)
        runs = torch.randn(wl.H, -(-G // 8), 64, generator=g)
        rows = runs.repeat_interleave(8 * 32, dim=1)[:, :wl.N]
        q = rows.unsqueeze(0).to(torch.bfloat16).contiguous()
        k = torch.randn(wl.H, 1, 64, generator=g).expand(wl.H, wl.N, 64).unsqueeze(0).to(torch.bfloat16).contiguous()
        v = torch.randn(1, wl.H, wl.N, 64, generator=g).to(torch.bfloat16)
    elif kind == "wide_range":
        # per-channel scales 2^-12 .. 2^12 on q and k: products of very different
        # magnitudes in every score, the hardest case for the approximate scores'
        # error bound (a violated bound shows up as a list that differs)
        # (integers up to 127 times a power of two: bf16-exact, and every group
        # sum stays exact, as the group-mean definition needs)
        wl = Workload("fine_wide_range", 1, 2, 128, (4, 8, 32), (1, 1, 1), fine_group=32, fine_keep=0.15)
        sq = torch.pow(2.0, torch.randint(-12, 13, (128,), generator=g).float())
        sk = torch.pow(2.0, torch.randint(-12, 13, (128,), generator=g).float())
        q = (torch.randint(-127, 128, (1, 2, wl.N, 128), generator=g).float() * sq).to(torch.bfloat16)
        k = (torch.randint(-127, 128, (1, 2, wl.N, 128), generator=g).float() * sk).to(torch.bfloat16)
        v = torch.randn(1, 2, wl.N, 128, generator=g).to(torch.bfloat16)
    elif kind == "zero_q":
        # one head with all-zero queries: every score is 0, every pair kept
        wl = Workload("fine_zero_q", 1, 2, 64, (2, 8, 16), (1, 1, 1), fine_group=32, fine_keep=0.2)
        q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=6)
        q[0, 1] = 0
    else:  # "beyond_fp32"
        # scores ~1e40 overflow the fp32 approximations (exact in fp64)
        wl = Workload("fine_beyond_fp32", 1, 1, 64, (2, 8, 16), (1, 1, 1), fine_group=32, fine_keep=0.2)
        q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=7)
        q = (q.float() * 1e20).to(torch.bfloat16)
        k = (k.float() * 1e20).to(torch.bfloat16)
    return wl, q, k, v


@pytest.mark.parametrize("kind", ["huge_key", "wide_range", "all_equal", "group_ties", "zero_q", "beyond_fp32"])
def test_fine_planted_exact(kind):
    wl, q, k, v = _planted(kind)
    _say(f"fine planted {kind}")
    q, k, v = (t.to("cuda") for t in (q, k, v))
    plan = vsa.Plan(*structs_of(wl))
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    qbar, tau, count, idx = _device_mask(plan, wl)
    plan.forward(q, k, v)  # identical on a second call
    torch.cuda.synchronize()
    _, tau2, count2, idx2 = _device_mask(plan, wl)
    assert np.array_equal(tau, tau2) and np.array_equal(count, count2)
    assert np.array_equal(np.where(np.arange(wl.N)[None, None, :] < count[..., None], idx, 0),
                          np.where(np.arange(wl.N)[None, None, :] < count2[..., None], idx2, 0))
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    on = o.float().cpu().numpy()
    for h in range(wl.H):
        if kind in ("beyond_fp32", "wide_range"):  # scores beyond the attention's fp32 range: mask only
            _check_mask(wl, qn[0, h], kn[0, h], h, qbar, tau, count, idx)
        else:
            _check_head(wl, plan, qn[0, h], kn[0, h], vn[0, h], on[0, h], h, qbar, tau, count, idx)
    if kind == "all_equal":
        assert int(count.sum()) == wl.N * plan.info.fine_groups
    if kind == "group_ties":
        kc = plan.info.fine_keep_count
        assert np.all(count.sum(axis=1) >= kc + wl.N)  # ties beyond K + N are all kept
