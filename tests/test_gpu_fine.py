"""GPU parity of the fine-grained M x 1 path against the oracle.

Bit-exact: group means, the per-head threshold tau, every group's kept-key
list.  O max-abs <= 2e-2.
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
    BH, G, d = wl.B * wl.H, plan.info.fine_groups, wl.d
    qbar = plan.region(_lib.VSA_WS_FINE_QBAR, torch.float32).view(BH, G, d).cpu().numpy()
    tau = plan.region(_lib.VSA_WS_FINE_TAU, torch.float64)[:BH].cpu().numpy()
    ptr = plan.region(_lib.VSA_WS_FINE_PTR, torch.int32).view(BH, G + 1).cpu().numpy()
    idx = plan.region(_lib.VSA_WS_FINE_IDX, torch.int32).view(BH, -1).cpu().numpy()
    return qbar, tau, ptr, idx


def _check_head(wl, plan, qn, kn, vn, on, bh, qbar, tau, ptr, idx, groups=None):
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
        got = idx[bh, ptr[bh, gi]:ptr[bh, gi + 1]]
        assert np.array_equal(got, lists[gi]), (bh, gi)
    grp = fine.groups(N, M)
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
    qbar, tau, ptr, idx = _device_mask(plan, wl)
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    on = o.float().cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            _check_head(wl, plan, qn[b, h], kn[b, h], vn[b, h], on[b, h], b * wl.H + h, qbar, tau,
                        ptr, idx)
    pairs, flops = plan.retained_work()
    assert pairs == int(ptr[:, -1].sum())


def test_fine_full_size_sampled():
    wl = CONFIGS["fine"]
    _say("fine full size")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0, device="cuda")
    prob, pol = structs_of(wl)
    plan = vsa.Plan(prob, pol)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    qbar, tau, ptr, idx = _device_mask(plan, wl)
    G = plan.info.fine_groups
    kept = ptr[:, -1]
    print(f"kept pairs per head {kept.tolist()} (target {plan.info.fine_keep_count})", flush=True)
    assert np.all(kept >= plan.info.fine_keep_count)
    rng = np.random.default_rng(0)
    for h in (0, 7):
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        on = o[0, h].float().cpu().numpy()
        groups = sorted(set(rng.choice(G, 5, replace=False).tolist()) | {G - 1})
        _check_head(wl, plan, qn, kn, vn, on, h, qbar, tau, ptr, idx, groups=groups)
