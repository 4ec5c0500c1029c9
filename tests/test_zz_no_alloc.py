"""vsa_forward_noalloc against vsa_forward, through the C ABI.

The allocation-free forward runs the same kernels on the library's own
per-device scratch array instead of a caller workspace, so its output must
be bit-identical to vsa_forward's.  Several calls in a row share that array
(each one rewrites everything it reads): a large call is followed by smaller
ones, and the fine-grained path and the E4M3 path take their turn.
"""
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from synth import Workload, smooth_field_qkv
from tests.helpers import structs_of

pytestmark = pytest.mark.gpu

SEQUENCE = [
    # Top-P + window on Wan-480p tiles (largest scratch of the sequence)
    Workload("na_topp", 1, 4, 128, (9, 24, 40), (3, 6, 8), window=(3, 3, 3), topp=0.9),
    # smaller: Top-K only, ragged tiles, d = 64, two batches
    Workload("na_topk", 2, 2, 64, (5, 7, 9), (2, 3, 4), topk=3),
    # fine-grained mask (its own scratch regions), then a small window case
    Workload("na_fine", 1, 2, 128, (5, 8, 16), (1, 1, 1), fine_group=64, fine_keep=0.15),
    Workload("na_window", 1, 1, 128, (4, 8, 8), (2, 4, 4), window=(3, 3, 3)),
    # E4M3 attention with SICS choice
    Workload("na_sics_fp8", 1, 2, 128, (7, 16, 16), (1, 16, 16),
             candidates=((1, 16, 16), (7, 4, 4)), topk_frac=0.3, compute="fp8",
             ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
]


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def test_noalloc_matches_forward_over_a_sequence_of_calls():
    sizes = []
    for n, wl in enumerate(SEQUENCE):
        _say(f"noalloc {wl.name}")
        plan = vsa.Plan(*structs_of(wl))
        assert plan.ws_bytes <= _lib.VSA_NOALLOC_BYTES
        sizes.append(plan.ws_bytes)
        q, k, v = smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=n,
                                   device="cuda")
        ref = plan.forward(q, k, v)
        got = torch.full_like(q, float("nan"))
        plan.forward_noalloc(q, k, v, got)
        # and once more on the same array (it keeps the previous call's contents)
        got2 = torch.full_like(q, float("nan"))
        plan.forward_noalloc(q, k, v, got2)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), wl.name
        assert torch.equal(got2.view(torch.int16), ref.view(torch.int16)), wl.name
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_plans_beyond_its_scratch():
    wl = Workload("na_big", 1, 24, 128, (30, 48, 80), (6, 8, 8), window=(3, 3, 5))
    plan = vsa.Plan(*structs_of(wl))
    assert plan.ws_bytes > _lib.VSA_NOALLOC_BYTES
    q = torch.zeros(1, 1, 8, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_forward_noalloc(plan.handle, q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                q.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert e.value.status == _lib.VSA_ERR_UNSUPPORTED
