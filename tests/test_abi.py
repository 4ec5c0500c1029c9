"""C-ABI checks that need no GPU: exports, plan validation, geometry facts."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import geometry
from synth import CONFIGS
from tests.helpers import structs_of

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "vsa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = ctypes.CDLL(_lib.LIB_PATH)
    declared = _declared_functions()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(_lib.EXPORTED) == declared


def test_library_has_no_unresolved_symbols():
    # RTLD_NOW resolves every symbol at load time (a missing kernel stub
    # would otherwise surface only when its launcher runs)
    ctypes.CDLL(_lib.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_status_strings():
    L = vsa.lib()
    assert L.vsa_status_string(0) == b"VSA_OK"
    assert L.vsa_status_string(3) == b"VSA_ERR_WORKSPACE_TOO_SMALL"


@pytest.mark.parametrize("name", ["tiny", "wan480", "hunyuan", "wan14b", "fine"])
def test_plan_for_every_workload(name):
    wl = CONFIGS[name]
    prob, pol = structs_of(wl)
    h = vsa.vsa_plan(prob, pol)
    info = vsa.vsa_plan_get_info(h)
    assert vsa.vsa_workspace_bytes(h) > 0
    if wl.fine_group:
        assert info.fine_groups == 512
        assert info.fine_keep_count == 2515968
    else:
        tiles = wl.candidates or (wl.tile,)
        for c, t in enumerate(tiles):
            nt = geometry.tile_counts(wl.grid, t)
            assert tuple(info.ntiles[c]) == nt
            bs = t[0] * t[1] * t[2]
            assert info.slots[c] == -(-bs // 32) * 32
    vsa.vsa_plan_destroy(h)


def _static_flops(wl, mode):
    mem = geometry.tile_members(wl.grid, wl.tile)
    nt = geometry.tile_counts(wl.grid, wl.tile)
    tot = 0.0
    pairs = 0
    for i in range(len(mem)):
        for j in geometry.window(i, nt, wl.window, mode):
            tot += len(mem[i]) * len(mem[j])
            pairs += 1
    return pairs, tot * 4 * wl.d * wl.B * wl.H


@pytest.mark.parametrize("mode,code", [("truncate", vsa.VSA_WIN_TRUNCATE), ("clamp", vsa.VSA_WIN_CLAMP)])
def test_static_window_work_matches_oracle(mode, code):
    wl = CONFIGS["hunyuan"]
    prob, _ = structs_of(wl)
    pol = vsa.make_policy(vsa.VSA_WINDOW, win=wl.window, win_mode=code)
    info = vsa.vsa_plan_get_info(vsa.vsa_plan(prob, pol))
    pairs, fl = _static_flops(wl, mode)
    assert info.static_pairs == pairs
    assert info.static_flops == pytest.approx(fl, rel=1e-12)
    assert info.row_cap == 45


def test_ragged_static_flops():
    wl = CONFIGS["wan480"].with_(topp=0.0)
    prob, pol = structs_of(wl)
    info = vsa.vsa_plan_get_info(vsa.vsa_plan(prob, pol))
    pairs, fl = _static_flops(wl, "truncate")
    assert info.static_pairs == pairs == 4693
    assert info.static_flops == pytest.approx(fl, rel=1e-12)


def test_static_window_with_sink_counts_the_union():
    wl = CONFIGS["hunyuan"]
    prob, _ = structs_of(wl)
    pol = vsa.make_policy(vsa.VSA_WINDOW, win=wl.window, sink=3)
    info = vsa.vsa_plan_get_info(vsa.vsa_plan(prob, pol))
    mem = geometry.tile_members(wl.grid, wl.tile)
    nt = geometry.tile_counts(wl.grid, wl.tile)
    pairs, fl = 0, 0.0
    for i in range(len(mem)):
        row = set(geometry.window(i, nt, wl.window, "truncate")) | {0, 1, 2}
        pairs += len(row)
        fl += sum(len(mem[i]) * len(mem[j]) for j in row)
    assert info.static_pairs == pairs
    assert info.static_flops == pytest.approx(fl * 4 * wl.d * wl.B * wl.H, rel=1e-12)
    assert info.row_cap == 48


def _err(prob, pol):
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_plan(prob, pol)
    return e.value.status


def test_plan_errors():
    ok = vsa.make_problem(1, 2, 64, (4, 8, 8), (2, 4, 4))
    win = vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3))
    assert _err(vsa.make_problem(1, 2, 96, (4, 8, 8), (2, 4, 4)), win) == vsa._lib.VSA_ERR_UNSUPPORTED
    assert _err(vsa.make_problem(0, 2, 64, (4, 8, 8), (2, 4, 4)), win) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(vsa.make_problem(1, 2, 64, (4, 8, 8), (8, 4, 4)), win) == vsa._lib.VSA_ERR_UNSUPPORTED
    assert _err(ok, vsa.make_policy(vsa.VSA_WINDOW, win=(2, 3, 3))) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(0)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_TOPP, topp=1.5)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_TOPK)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_TOPK | vsa.VSA_TOPK_FRAC, topk=2, topk_frac=0.5)) \
        == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_FINE | vsa.VSA_WINDOW, win=(3, 3, 3), fine_group=64,
                                    fine_keep=0.1)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_FINE, fine_group=40, fine_keep=0.1)) \
        == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_SICS_SELECT | vsa.VSA_TOPK, topk=2)) \
        == vsa._lib.VSA_ERR_INVALID_ARG          # n_cand = 0
    assert _err(ok, vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3), scale=-1.0)) \
        == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_TOPK, topk=2, summarizer=3)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3), sink=-1)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_FINE, fine_group=64, fine_keep=0.1, sink=1)) \
        == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3), compute=2)) == vsa._lib.VSA_ERR_INVALID_ARG
    assert _err(ok, vsa.make_policy(vsa.VSA_FINE, fine_group=64, fine_keep=0.1,
                                    compute=vsa.VSA_COMPUTE_FP8)) == vsa._lib.VSA_ERR_UNSUPPORTED
    # launch-size limits: B*H in the second grid dimension; one attention workgroup per
    # (head, tile, slab group) in a 1-D launch; (head, group) pairs of the fine path in 32 bits
    assert _err(vsa.make_problem(256, 256, 64, (4, 8, 8), (2, 4, 4)), win) == vsa._lib.VSA_ERR_UNSUPPORTED
    assert _err(vsa.make_problem(60, 1000, 64, (16, 16, 16), (1, 1, 1)), win) == vsa._lib.VSA_ERR_UNSUPPORTED
    assert _err(vsa.make_problem(1, 1024, 64, (1024, 1024, 1024), (1, 1, 1)),
                vsa.make_policy(vsa.VSA_FINE, fine_group=16, fine_keep=0.1)) == vsa._lib.VSA_ERR_UNSUPPORTED
    with pytest.raises(vsa.VsaError):
        vsa.vsa_plan(None, win) if False else _lib._check(vsa.lib().vsa_plan(None, None, None))


def test_fp8_workspace_regions():
    # E4M3 exponents [B*H][3] and partial maxima [B*H][3][128]; the bf16 plan has neither
    prob = vsa.make_problem(2, 3, 128, (4, 8, 8), (2, 4, 4))
    for compute, want_exp, want_amax in ((vsa.VSA_COMPUTE_BF16, 0, 0),
                                         (vsa.VSA_COMPUTE_FP8, 6 * 3 * 4, 6 * 3 * 128 * 4)):
        h = vsa.vsa_plan(prob, vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3), compute=compute))
        assert vsa.vsa_workspace_region(h, _lib.VSA_WS_F8_EXP)[1] == want_exp
        assert vsa.vsa_workspace_region(h, _lib.VSA_WS_F8_AMAX)[1] == want_amax
        # tile-major K keeps its bf16 size (E4M3 uses the first half); tile-major Q
        # exists only for E4M3 (the bf16 attention reads Q in raster order)
        want_q = 6 * 8 * 32 * 128 * 2 if compute == vsa.VSA_COMPUTE_FP8 else 0
        assert vsa.vsa_workspace_region(h, _lib.VSA_WS_QT)[1] == want_q
        assert vsa.vsa_workspace_region(h, _lib.VSA_WS_KT)[1] == 6 * 8 * 32 * 128 * 2
        assert vsa.vsa_workspace_region(h, _lib.VSA_WS_VT)[1] == 6 * 8 * 32 * 128 * 2


def test_exec_argument_errors_before_any_device_call():
    prob = vsa.make_problem(1, 2, 64, (4, 8, 8), (2, 4, 4))
    h = vsa.vsa_plan(prob, vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3)))
    n = vsa.vsa_workspace_bytes(h)
    L = vsa.lib()
    buf = ctypes.create_string_buffer(n + 512)
    base = (ctypes.addressof(buf) + 255) & ~255
    assert L.vsa_forward(h, None, 16, 16, 16, base, n, None) == vsa._lib.VSA_ERR_INVALID_ARG
    assert L.vsa_forward(h, 16, 16, 16, 16, base, n - 1, None) == vsa._lib.VSA_ERR_WORKSPACE_TOO_SMALL
    assert L.vsa_forward(h, 16, 16, 16, 16, base + 16, n, None) == vsa._lib.VSA_ERR_INVALID_ARG
    assert L.vsa_forward(h, 17, 16, 16, 16, base, n, None) == vsa._lib.VSA_ERR_INVALID_ARG
    assert b"workspace" in L.vsa_last_error() or b"aligned" in L.vsa_last_error()


def test_forward_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    prob = vsa.make_problem(1, 2, 64, (4, 8, 8), (2, 4, 4))
    h = vsa.vsa_plan(prob, vsa.make_policy(vsa.VSA_WINDOW, win=(3, 3, 3)))
    n = vsa.vsa_workspace_bytes(h)
    buf = ctypes.create_string_buffer(n + 512)
    base = (ctypes.addressof(buf) + 255) & ~255
    st = vsa.lib().vsa_forward(h, 16, 16, 16, 16, base, n, None)
    assert st == vsa._lib.VSA_ERR_HIP


def test_workspace_regions_disjoint_and_aligned():
    wl = CONFIGS["wan14b"]
    prob, pol = structs_of(wl)
    h = vsa.vsa_plan(prob, pol)
    total = vsa.vsa_workspace_bytes(h)
    spans = []
    for r in range(_lib.VSA_WS_NREGIONS):
        off, n = vsa.vsa_workspace_region(h, r)
        if n:
            assert off % 256 == 0
            assert off + n <= total
            spans.append((off, off + n))
    spans.sort()
    for a, b in zip(spans, spans[1:]):
        assert a[1] <= b[0]


def test_profile_errors_and_sizes():
    prob = vsa.make_problem(1, 2, 64, (4, 8, 8), (2, 4, 4), candidates=((2, 4, 4), (4, 2, 2)))
    bad = vsa.make_policy(vsa.VSA_PROFILE_SELECT | vsa.VSA_TOPK, topk=2)
    with pytest.raises(vsa.VsaError):
        vsa.vsa_plan(prob, bad)
    h = vsa.vsa_plan(prob, vsa.make_policy(vsa.VSA_PROFILE_SELECT | vsa.VSA_WINDOW, win=(1, 1, 1),
                                           profile_frac=0.5))
    runs = 4  # round(0.5 * 256 / 32)
    assert vsa.vsa_workspace_region(h, _lib.VSA_WS_PROF_SSE)[1] == 2 * runs * 2 * 4
    segs = min(-(-1024 // (2 * 1)), 4 * 8, 16)  # groups = B*H*ceil(runs/4) = 2; lines = 32
    assert vsa.vsa_workspace_region(h, _lib.VSA_WS_PROF_PART)[1] == 2 * runs * segs * 32 * (64 + 2) * 4


def test_attention_pairs_query_tiles_where_lists_overlap():
    """Plan-time choice of two query tiles per attention workgroup: tiles of 4 to 6 slabs
    under Top-P, or under a static mask whose neighbours' lists mostly coincide; under Top-K
    only tiles of 6 slabs, with the interleaved schedule; never for a 1x1x1 window or larger
    tiles."""
    from synth import CONFIGS, Workload
    from block_sparse_attention_tile_amd.workload import plan_structs

    def pair(wl):
        p = vsa.Plan(*plan_structs(wl))
        return list(p.info.pair)[:p.info.n_blockings]
    assert pair(CONFIGS["wan480"]) == [1]
    assert pair(Workload("w", 1, 2, 128, (3, 18, 20), (3, 6, 8), window=(3, 3, 3))) == [1]
    assert pair(Workload("w", 1, 2, 128, (6, 12, 40), (3, 6, 8), window=(1, 1, 1))) == [0]
    assert pair(Workload("k", 1, 2, 128, (7, 8, 8), (7, 4, 4), topk=3)) == [0]
    assert pair(CONFIGS["hunyuan"]) == [0]
    assert pair(CONFIGS["wan14b"]) == [0, 0, 1]  # 256-, 112- and 192-token tiles
    p = vsa.Plan(*plan_structs(CONFIGS["wan14b"]))
    assert list(p.info.interleave)[:3] == [0, 0, 1] and list(p.info.units)[:3] == [0, 0, 0]
    assert list(vsa.Plan(*plan_structs(CONFIGS["wan480"])).info.interleave)[:1] == [0]  # Top-P: union


def test_attention_units_where_tails_are_short():
    """Plan-time choice of units for pairs (16 keys for bf16, 32 for E4M3): when they cut the
    chunk count over all tiles by 5% or more, as for 144-token tiles (9 units vs 3 chunks; E4M3
    5 units of 32 vs 3 chunks) or 168-token ones (11 vs 12); not for 180-token tiles (12 units
    = 3 chunks), not for unpaired blockings."""
    from synth import CONFIGS, Workload
    from block_sparse_attention_tile_amd.workload import plan_structs

    def units(wl):
        p = vsa.Plan(*plan_structs(wl))
        return list(p.info.units)[:p.info.n_blockings]
    assert units(CONFIGS["wan480"]) == [1]
    assert units(CONFIGS["wan480"].with_(compute="fp8")) == [1]
    assert units(CONFIGS["hunyuan"]) == [0]
    assert units(CONFIGS["wan14b"]) == [0, 0, 0]
    assert units(CONFIGS["hunyuan_svg"]) == [0, 0]
    assert units(CONFIGS["tiny"]) == [0]
    assert units(Workload("u", 1, 2, 64, (4, 12, 40), (2, 6, 15), topp=0.8)) == [0]   # 180 = 12 units = 3 chunks
    assert units(Workload("u", 1, 2, 64, (4, 12, 40), (2, 6, 14), topp=0.8)) == [1]   # 168: 11 units < 3 chunks


def test_noalloc_refuses_a_plan_beyond_its_scratch_without_touching_the_gpu():
    # the size check comes before any device access, so this runs without a GPU
    wl = CONFIGS["hunyuan"]
    h = vsa.vsa_plan(*structs_of(wl))
    assert vsa.vsa_workspace_bytes(h) > _lib.VSA_NOALLOC_BYTES
    buf = (ctypes.c_char * 4096)()
    p = (ctypes.addressof(buf) + 255) & ~255
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_forward_noalloc(h, p, p, p, p, None)
    assert e.value.status == _lib.VSA_ERR_UNSUPPORTED
    assert b"vsa_forward_noalloc" in vsa.lib().vsa_last_error()
    vsa.vsa_plan_destroy(h)
