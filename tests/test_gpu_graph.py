"""HIP graph capture of vsa_forward and vsa_forward_cached.

The execution calls enqueue kernel launches only (no memset, copy or
allocation), so a stream capture records a graph that replays them.  Each
case makes one uncaptured call (which also sets the kernels' dynamic-LDS
limits), captures one call into a graph, and replays it several times with
eager work and synchronizations between the replays.  Every replay must
equal the eager output bit for bit: the kernels are deterministic.  The
captured input buffers are then refilled with new inputs, and the replay
must equal an eager call on those inputs.
"""
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from synth import Workload, smooth_field_qkv
from tests.helpers import structs_of

pytestmark = pytest.mark.gpu

CASES = {
    # static window (mask built in the plan)
    "window": Workload("hy_mini", 1, 2, 128, (12, 16, 24), (6, 8, 8), window=(3, 3, 5)),
    # window united with Top-P (pooled means, scores, selection on the GPU)
    "topp": Workload("w480_mini", 1, 2, 128, (6, 12, 20), (3, 6, 8), window=(3, 3, 3), topp=0.9),
    # SICS choice of a blocking per head, then Top-K
    "sics": Workload("sics", 1, 4, 128, (14, 16, 16), (1, 16, 16),
                     candidates=((1, 16, 16), (7, 4, 4), (7, 8, 8)), topk_frac=0.2,
                     ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
    # profiling selector (sampled-row MSE per candidate)
    "profile": Workload("profile", 1, 2, 128, (14, 16, 16), (1, 16, 16),
                        candidates=((1, 16, 16), (7, 4, 4)), window=(1, 1, 1), selector="profile",
                        ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0), profile_frac=0.05),
    # E4M3 attention (max-|x| pass, quantising layout)
    "fp8": Workload("hy_mini_fp8", 1, 2, 128, (12, 16, 24), (6, 8, 8), window=(3, 3, 5), compute="fp8"),
    # fine-grained mask (scores, histogram, radix select, lists) and gathered attention
    "fine": Workload("fine_d128", 1, 2, 128, (5, 8, 16), (1, 1, 1), fine_group=64, fine_keep=0.15),
}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _replays_match(plan, call, q, k, v, o, want, reps=4):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(q, k, v, o)
    for r in range(reps):
        o.fill_(1.0)                       # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want), r
        del junk
    return g


@pytest.mark.parametrize("cached", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name, cached):
    wl = CASES[name]
    _say(f"graph {name} cached={cached}")
    q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=0, device="cuda")
    plan = vsa.Plan(*structs_of(wl))
    o = torch.empty_like(q)
    plan.forward(q, k, v, o)               # uncaptured call: mask in the workspace, attributes set
    torch.cuda.synchronize()
    want = o.clone()
    call = plan.forward_cached if cached else plan.forward
    g = _replays_match(plan, call, q, k, v, o, want)
    # new inputs in the captured buffers
    q2, k2, v2 = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=7, device="cuda")
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = o.clone()
    ref = torch.empty_like(q)
    if cached:
        plan.forward_cached(q, k, v, ref)  # the mask the graph reused: the one in the workspace
    else:
        plan.forward(q, k, v, ref)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
