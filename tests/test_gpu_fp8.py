"""GPU parity of the E4M3 (FP8) tile path against the oracle (oracle/fp8.py).

Bit-exact: the per-head exponents, the E4M3 codes of tile-major Q and K and
of the (slot-permuted) V^T rows, and the selection.

Attention output, per query row, within a tolerance derived from the
arithmetic (all terms computed from the oracle's values):
  * the E4M3 MFMA sums each 64-term product with an error of at most
    C_MFMA = 2^-10 of its largest |term| (tests/test_gpu_probe.py measures
    the bare product against exact sums on uniform-code, normal,
    probability-like and cancelling operands and holds it to this bound; the
    accumulator input itself is kept in fp32), so a score may be off by dS = C_MFMA * sum over
    64-channel groups of max|q8| max|k8| (raw units), dt = dS * c2 in exp2
    units, plus 2^-20 (|t| + 16) for the fp32 rounding of c2, of the fma and
    of exp2;
  * a probability whose value 2^(t - r + 8) can cross an E4M3 rounding
    midpoint within +-dt may round to either neighbour: its code is not
    unique, and the kernel's pick moves O by at most
    dp (|v_j| + |o|) / (l - sum dp);
  * below 2^-5 (E4M3's subnormal range, with one power of two of slack for
    a reference the kernel rounds one step higher) the kernel may round
    against another power of two: dp <= 2^-9;
  * the PV and row-sum products add C_MFMA * max p8 (max|v| + |o|) per
    64-key chunk, over l;
  * bf16 output rounding adds 2^-8 |o|.
The tolerance is twice the sum, plus 1e-3, and never more than max|v| +
|o| (O is a convex combination of the kept rows of V); that bound alone is
used where the others stop being informative (sum dp > l / 2, e.g. one
huge key whose score error bound spans several powers of two).  Such rows
are counted: the smooth-field cases must have none (only the planted
degenerate heads may), and every case prints the median and largest
tolerance next to the largest observed error.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as vsa
from block_sparse_attention_tile_amd import _lib
from oracle import fp8, geometry, layout
from synth import CONFIGS, Workload, smooth_field_qkv
from tests.helpers import C_MFMA, csr_rows, oracle_candidate, oracle_tile_rows, structs_of, unambiguous

pytestmark = pytest.mark.gpu

CASES = {
    # HunyuanVideo tile shape (384 tokens, full 64-key chunks), static window
    "hy_mini": Workload("hy_mini", 1, 2, 128, (12, 16, 24), (6, 8, 8), window=(3, 3, 5), compute="fp8"),
    # Wan-480p tile shape (144 tokens -> 160 slots: a 32-key tail chunk), Top-P + window
    "w480_mini": Workload("w480_mini", 1, 2, 128, (6, 12, 20), (3, 6, 8), window=(3, 3, 3), topp=0.9,
                          compute="fp8"),
    # ragged edge tiles, every chunk a 32-key chunk, Top-K, d=64
    "ragged_d64": Workload("ragged_d64", 1, 3, 64, (5, 7, 9), (2, 3, 4), window=(3, 3, 3), topk=3,
                           compute="fp8"),
    # dense, two batches, d=64
    "dense_b2": Workload("dense_b2", 2, 2, 64, (3, 5, 6), (1, 5, 6), compute="fp8"),
    # SICS blocking choice per head + Top-K fraction
    "sics": Workload("sics", 1, 4, 128, (14, 16, 16), (1, 16, 16),
                     candidates=((1, 16, 16), (7, 4, 4), (7, 8, 8)), topk_frac=0.2,
                     ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0), compute="fp8"),
    # eight-wave and seven-wave workgroups (4-stage ring); the second ragged on every axis
    "eight_slab": Workload("eight_slab", 1, 2, 128, (4, 16, 32), (1, 16, 16), window=(3, 1, 1), topk=2,
                           compute="fp8"),
    "seven_slab_ragged": Workload("seven_slab_ragged", 1, 2, 64, (5, 9, 30), (2, 8, 14), topp=0.9,
                                  compute="fp8"),
    # paired 156-token tiles at d = 64: 32-key units (five per tile, the last with 28 keys),
    # 12-token edge tiles
    "pair_units_d64": Workload("pair_units_d64", 1, 2, 64, (4, 12, 40), (2, 6, 13), topp=0.8, compute="fp8"),
    # Top-K pairs of 192-token tiles (interleaved schedule), ragged, odd tile count
    "topk_pair_ragged": Workload("topk_pair_ragged", 1, 3, 64, (7, 8, 20), (3, 8, 8), topk=4, compute="fp8"),
    # window clamped at the grid edge (every row keeps its full window)
    "hy_mini_clamp": Workload("hy_mini_clamp", 1, 1, 128, (12, 16, 40), (6, 8, 8), window=(1, 1, 3),
                              win_mode="clamp", compute="fp8"),
    # max/min bound estimator + attention sink + window + Top-P, ragged tiles, d=64
    "topp_minmax_sink": Workload("topp_minmax_sink", 1, 3, 64, (5, 7, 9), (2, 3, 4), window=(3, 3, 3),
                                 topp=0.9, summarizer="minmax", sink=2, compute="fp8"),
}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)


def _inputs(wl, seed=0, device="cuda"):
    return smooth_field_qkv(wl.B, wl.H, wl.d, wl.grid, wl.ell_per_head(), seed=seed, device=device)


def _vslot(pp):
    """Slot stored at position pp of an E4M3 V^T row (bits b2 b4 b3 b1 b0)."""
    pp = np.asarray(pp)
    return (pp & ~31) | (((pp >> 2) & 3) << 3) | (((pp >> 4) & 1) << 2) | (pp & 3)


def fp8_reference(q_h, k_h, v_h, mem, rows, tiles, scale):
    """Oracle FP8 output of one head on the given query tiles, and the
    per-row tolerance of the module docstring."""
    N, d = q_h.shape
    (q8, k8, v8), _, (eq, ek, ev) = fp8.quantize_qkv(q_h, k_h, v_h)
    c2 = scale / math.log(2.0) * 2.0 ** -(eq + ek)
    vs = np.ldexp(v8, -ev)
    out = np.zeros((N, d))
    tol = np.zeros(N)
    hull_only = np.zeros(N, dtype=bool)
    groups = d // 64
    for i in tiles:
        if not rows[i]:
            continue
        qi = mem[i]
        keys = np.concatenate([mem[j] for j in rows[i]])
        t = fp8.prob_exponents(q8[qi], k8[keys], eq, ek, scale)
        p, p8, r = fp8.quantized_probs(t)
        l = p8.sum(axis=1)
        o = (p8 @ vs[keys]) / l[:, None]
        out[qi] = o
        omax = np.abs(o).max(axis=1)
        vmax = np.abs(vs[keys]).max(axis=1)
        mq = np.abs(q8[qi]).reshape(len(qi), groups, 64).max(axis=2)
        mk = np.abs(k8[keys]).reshape(len(keys), groups, 64).max(axis=2)
        dt = C_MFMA * (mq @ mk.T) * c2 + 2.0 ** -20 * (np.abs(t) + 16.0)
        lo = fp8.e4m3_round(np.exp2(t - dt - r + 8.0))
        hi = fp8.e4m3_round(np.minimum(np.exp2(t + dt - r + 8.0), 448.0))
        dp = hi - lo
        dp = np.where(p < 2.0 ** -5, np.maximum(dp, 2.0 ** -9), dp)
        den = l - dp.sum(axis=1)
        flip = (dp * (vmax[None, :] + omax[:, None])).sum(axis=1) / np.where(den > 0.5 * l, den, 1.0)
        starts = np.cumsum([0] + [len(mem[j]) for j in rows[i]])[:-1]
        cs = np.concatenate([np.arange(s0, s0 + len(mem[j]), 64) for s0, j in zip(starts, rows[i])])
        pmax = np.maximum.reduceat(p8, cs, axis=1)
        vmc = np.maximum.reduceat(vmax, cs)
        pv = C_MFMA * (pmax * (vmc[None, :] + omax[:, None])).sum(axis=1) / l
        # O is a convex combination of the kept rows of V whatever the
        # weights: where the score bounds allow every weight to move
        # (sum dp > l / 2), only that bound remains
        hull = vmax.max() + omax
        tol[qi] = np.where(den > 0.5 * l, np.minimum(2.0 * (2.0 ** -8 * omax + flip + pv) + 1e-3, hull), hull)
        hull_only[qi] = den <= 0.5 * l
    return out, tol, hull_only


def _check_head(on_h, q_h, k_h, v_h, mem, rows, tiles, scale, tag, allow_hull=False):
    """Per-row tolerance check; rows that fall back to the convex-hull bound
    must not occur unless allow_hull (planted degenerate heads)."""
    ref, tol, hull_only = fp8_reference(q_h, k_h, v_h, mem, rows, tiles, scale)
    errs, tols, n_hull = [], [], 0
    for i in tiles:
        if not rows[i]:
            continue
        err = np.abs(on_h[mem[i]] - ref[mem[i]]).max(axis=1)
        bad = np.nonzero(err > tol[mem[i]])[0]
        assert bad.size == 0, (tag, i, float(err[bad[0]]), float(tol[mem[i]][bad[0]]))
        errs.append(err)
        tols.append(tol[mem[i]])
        n_hull += int(hull_only[mem[i]].sum())
    errs, tols = np.concatenate(errs), np.concatenate(tols)
    print(f"[fp8 {tag}] rows {errs.size}, max err {errs.max():.4f}, tolerance median "
          f"{np.median(tols):.4f} max {tols.max():.4f}, hull-bound rows {n_hull}", flush=True)
    if not allow_hull:
        assert n_hull == 0, (tag, n_hull)
    return float(errs.max())


@pytest.mark.parametrize("name", ["hy_mini", "w480_mini", "ragged_d64", "sics"])
def test_fp8_layout_codes_bit_exact(name):
    wl = CASES[name]
    _say(f"fp8 layout {name}")
    q, k, v = _inputs(wl)
    plan = vsa.Plan(*structs_of(wl))
    plan.forward(q, k, v)
    torch.cuda.synchronize()
    BH = wl.B * wl.H
    exps = plan.region(_lib.VSA_WS_F8_EXP, torch.int32).view(BH, 3).cpu().numpy()
    _, _, cand = plan.read_selection()
    qt = plan.region(_lib.VSA_WS_QT, torch.uint8).cpu().numpy()
    kt = plan.region(_lib.VSA_WS_KT, torch.uint8).cpu().numpy()
    vt = plan.region(_lib.VSA_WS_VT, torch.uint8).cpu().numpy()
    head_bytes = qt.size // 2 // BH  # E4M3 uses the first half of the bf16-sized region
    for b in range(wl.B):
        for h in range(wl.H):
            bh = b * wl.H + h
            xs = [t[b, h].float().cpu().numpy() for t in (q, k, v)]
            codes, es = zip(*(fp8.quantize_head(x) for x in xs))
            assert list(exps[bh]) == list(es), (bh, exps[bh], es)
            c = int(cand[bh]) if wl.candidates else 0
            tile = wl.candidates[c] if wl.candidates else wl.tile
            mem = geometry.tile_members(wl.grid, tile)
            slots = plan.info.slots[c]
            nT, d = len(mem), wl.d
            want_q = layout.to_tile_major(codes[0][None, None], mem, slots)[0, 0]
            want_k = layout.to_tile_major(codes[1][None, None], mem, slots)[0, 0]
            want_v = layout.to_tile_major(codes[2][None, None], mem, slots)[0, 0]   # [nT, slots, d]
            base = bh * head_bytes
            n = nT * slots * d
            assert np.array_equal(qt[base:base + n].reshape(nT, slots, d), want_q)
            assert np.array_equal(kt[base:base + n].reshape(nT, slots, d), want_k)
            got_v = vt[base:base + n].reshape(nT, d, slots)
            perm = _vslot(np.arange(slots))
            assert np.array_equal(got_v, want_v.transpose(0, 2, 1)[:, :, perm])


# cases that exist to run the paired / unit kernels: the plan must choose them
PAIRED_UNITS = {"w480_mini": (1, 1), "pair_units_d64": (1, 1), "topk_pair_ragged": (1, 0)}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_attention_small(name):
    wl = CASES[name]
    _say(f"fp8 forward {name}")
    q, k, v = _inputs(wl)
    plan = vsa.Plan(*structs_of(wl))
    if name in PAIRED_UNITS:
        assert (plan.info.pair[0], plan.info.units[0]) == PAIRED_UNITS[name]
    assert plan.info.interleave[0] == int(name == "topk_pair_ragged")
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    row_ptr, col, cand = plan.read_selection()
    on = o.float().cpu().numpy()
    assert np.isfinite(on).all()
    scale = 1.0 / math.sqrt(wl.d)
    for b in range(wl.B):
        for h in range(wl.H):
            bh = b * wl.H + h
            qn, kn, vn = (t[b, h].float().cpu().numpy() for t in (q, k, v))
            if wl.candidates:
                c, _ = oracle_candidate(wl, qn, kn)
                assert int(cand[bh]) == c
                tile = wl.candidates[c]
            else:
                tile = wl.tile
            rows, margins, mem = oracle_tile_rows(wl, qn, kn, tile)
            got = csr_rows(row_ptr, col, bh, plan.info.max_tiles, len(mem))
            ok = unambiguous(range(len(mem)), margins)
            for i in ok:
                assert got[i] == rows[i], (b, h, i)
            _check_head(on[b, h], qn, kn, vn, mem, rows, ok, scale, (name, b, h))


def test_fp8_degenerate_heads():
    # head 0: all-zero V (e_v = 0, O = 0); head 1: constant K (equal scores
    # per row, every probability 256, O = mean of the kept V); head 2: one
    # huge value in K (a small exponent, most K codes round to zero)
    wl = Workload("degenerate", 1, 3, 128, (6, 8, 8), (3, 4, 8), window=(3, 3, 1), compute="fp8")
    _say("fp8 degenerate heads")
    q, k, v = _inputs(wl, seed=3)
    v[0, 0].zero_()
    k[0, 1] = 0.25
    k[0, 2, 5, 7] = 3000.0
    big = float(k[0, 2, 5, 7])
    plan = vsa.Plan(*structs_of(wl))
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    exps = plan.region(_lib.VSA_WS_F8_EXP, torch.int32).view(3, 3).cpu().numpy()
    assert exps[0, 2] == 0 and exps[2, 1] == fp8.scale_exponent(big)
    assert torch.count_nonzero(o[0, 0]).item() == 0
    row_ptr, col, _ = plan.read_selection()
    on = o.float().cpu().numpy()
    mem = geometry.tile_members(wl.grid, wl.tile)
    for h in range(3):
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        got = csr_rows(row_ptr, col, h, plan.info.max_tiles, len(mem))
        rows, _, _ = oracle_tile_rows(wl, qn, kn, wl.tile)
        assert got == rows, h
        _check_head(on[0, h], qn, kn, vn, mem, rows, range(len(mem)), 1.0 / math.sqrt(wl.d), ("deg", h),
                    allow_hull=True)


def test_fp8_cached_mask_reused_on_new_input():
    wl = CASES["w480_mini"]
    _say("fp8 cached w480_mini")
    plan = vsa.Plan(*structs_of(wl))
    qa, ka, va = _inputs(wl, seed=0)
    qb, kb, vb = _inputs(wl, seed=7)
    plan.forward(qa, ka, va)
    torch.cuda.synchronize()
    rp_a, col_a, _ = plan.read_selection()
    ob = plan.forward_cached(qb, kb, vb)
    torch.cuda.synchronize()
    rp_b, col_b, _ = plan.read_selection()
    assert np.array_equal(rp_a, rp_b) and np.array_equal(col_a, col_b)
    mem = geometry.tile_members(wl.grid, wl.tile)
    on = ob.float().cpu().numpy()
    for h in range(wl.H):
        rows = csr_rows(rp_a, col_a, h, plan.info.max_tiles, len(mem))
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (qb, kb, vb))
        _check_head(on[0, h], qn, kn, vn, mem, rows, range(len(mem)), 1.0 / math.sqrt(wl.d), ("cached", h))


def test_fp8_cached_on_unwritten_selection_gives_zeros():
    wl = CASES["ragged_d64"]
    _say("fp8 cached unwritten")
    plan = vsa.Plan(*structs_of(wl))
    plan.workspace().fill_(0xFF)
    q, k, v = _inputs(wl, seed=3)
    o = torch.full_like(q, 7.0)
    plan.forward_cached(q, k, v, o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0


def test_fp8_hunyuan_full_size_sampled():
    """HunyuanVideo 720p shape in E4M3: exponents and codes of one head,
    sampled query tiles of O for two heads."""
    wl = CONFIGS["hunyuan"].with_(compute="fp8")
    _say("fp8 hunyuan full size")
    q, k, v = _inputs(wl)
    plan = vsa.Plan(*structs_of(wl))
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    row_ptr, col, _ = plan.read_selection()
    nT = plan.info.n_tiles[0]
    mem = geometry.tile_members(wl.grid, wl.tile)
    nt = geometry.tile_counts(wl.grid, wl.tile)
    want = [geometry.window(i, nt, wl.window) for i in range(nT)]
    exps = plan.region(_lib.VSA_WS_F8_EXP, torch.int32).view(wl.H, 3).cpu().numpy()
    rng = np.random.default_rng(0)
    for h in (0, 23):
        assert csr_rows(row_ptr, col, h, plan.info.max_tiles, nT) == want
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        assert list(exps[h]) == [fp8.scale_exponent(np.abs(x).max()) for x in (qn, kn, vn)]
        tiles = sorted(set(rng.choice(nT, 3, replace=False).tolist()) | {0, nT - 1, 155})
        _check_head(o[0, h].float().cpu().numpy(), qn, kn, vn, mem, want, tiles,
                    1.0 / math.sqrt(wl.d), ("hunyuan", h))


def test_fp8_wan14b_full_size_sampled():
    """Wan-14B 720p shape in E4M3: per-head SICS blocking and Top-K 20%
    selection (bit-exact, as for bf16), sampled query tiles of O for one head
    of each blocking."""
    wl = CONFIGS["wan14b"].with_(compute="fp8")
    _say("fp8 wan14b full size")
    q, k, v = _inputs(wl)
    plan = vsa.Plan(*structs_of(wl))
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    row_ptr, col, cand = plan.read_selection()
    rng = np.random.default_rng(1)
    for h in (0, 1):  # the two anisotropic head kinds
        qn, kn, vn = (t[0, h].float().cpu().numpy() for t in (q, k, v))
        c, _ = oracle_candidate(wl, qn, kn)
        assert int(cand[h]) == c
        tile = wl.candidates[c]
        rows, margins, mem = oracle_tile_rows(wl, qn, kn, tile)
        got = csr_rows(row_ptr, col, h, plan.info.max_tiles, len(mem))
        tiles = unambiguous(sorted(set(rng.choice(len(mem), 3, replace=False).tolist()) | {0, len(mem) - 1}),
                            margins)
        for i in tiles:
            assert got[i] == rows[i], (h, i)
        _check_head(o[0, h].float().cpu().numpy(), qn, kn, vn, mem, rows, tiles, 1.0 / math.sqrt(wl.d),
                    ("wan14b", h))
