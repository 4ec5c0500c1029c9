"""GPU checks of the hardware probes (include/vsa_probe.h).

  * The MFMA rate probe does the work it is timed for: a wave's output sum
    equals the sum of every output element of its products, recomputed on
    the host from the fragments' row and column sums (the sum over all
    (m, n) of A.B is the sum over k of colsum_A[k] * rowsum_B[k]; lane l of
    a 32x32x16 fragment holds k = 8 * (l // 32) + t, t = 0..7).
  * The read probe's XOR fold equals the XOR of every 32-bit word read.
  * The bare E4M3 product (the E4M3 attention's score MFMA) stays within
    C_MFMA of its largest |term| of the exact sum, element by element, on
    operands drawn four ways: uniform over every finite code, normal values,
    probability-like powers of two against normal values, and pairs that
    cancel.  Products of E4M3 values and their 64-term sums are exact in
    fp64, so the reference has no rounding of its own.  This is the bound
    the E4M3 attention's parity tolerance (test_gpu_fp8.py) is built on.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_tile_amd import probe
from tests.helpers import C_MFMA

pytestmark = pytest.mark.gpu


def test_mfma_rate_probe_computes_its_products():
    print("[gpu case] probe mfma rate", flush=True)
    g = torch.Generator().manual_seed(5)
    n_slices, wgs, iters = 5, 3, 4
    src_h = torch.randn(n_slices * probe.SLICE_BYTES // 2, generator=g).to(torch.bfloat16)
    src = src_h.cuda()
    out = torch.full((wgs * probe.WAVES * 64,), float("nan"), device="cuda")
    flops = probe.mfma_rate(src, out, wgs, iters)
    torch.cuda.synchronize()
    assert flops == wgs * 12 * iters * 64 * 32768
    fr = src_h.double().numpy().reshape(n_slices, 16, 2, 32, 8)  # slice, frag, half, lane%32, t
    s = fr.sum(axis=3).reshape(n_slices, 16, 16)  # per k = 8 * half + t: sum over the 32 lanes
    got = out.cpu().double().numpy().reshape(wgs * 12, 64).sum(axis=1)
    for w in range(wgs * 12):
        sa, sb = s[w % n_slices, :8], s[w % n_slices, 8:]
        want = iters * sum(float(sa[ia] @ sb[(ia + ib) % 8]) for ia in range(8) for ib in range(8))
        scale = iters * sum(float(np.abs(sa[ia]) @ np.abs(sb[(ia + ib) % 8])) for ia in range(8) for ib in range(8))
        assert abs(got[w] - want) <= 1e-4 * scale + 1e-3, (w, got[w], want)


def test_read_rate_probe_reads_every_word():
    print("[gpu case] probe read rate", flush=True)
    rng = np.random.default_rng(3)
    words = rng.integers(0, 2 ** 32, size=4 * 12345, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    for wgs in (1, 3, 7):
        for nt in (False, True):
            out = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
            assert probe.read_rate(src, out, wgs, nt) == words.nbytes
            torch.cuda.synchronize()
            folded = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
            assert folded == np.bitwise_xor.reduce(words), (wgs, nt)


def _codes(x):
    """E4M3 codes of float values (round to nearest even, saturating in range)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)


def _values(c):
    return c.view(torch.float8_e4m3fn).double().numpy()


def _operands(kind, n, rng):
    if kind == "uniform_codes":
        finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
        a = torch.from_numpy(rng.choice(finite, size=(n, 32, 64)))
        b = torch.from_numpy(rng.choice(finite, size=(n, 32, 64)))
    elif kind == "normal":
        a, b = _codes(rng.standard_normal((n, 32, 64))), _codes(rng.standard_normal((n, 32, 64)))
    elif kind == "probability":  # p = 2^-u, u in [0, 12), against value-like rows
        a = _codes(np.exp2(-rng.uniform(0.0, 12.0, (n, 32, 64))))
        b = _codes(rng.standard_normal((n, 32, 64)) * 3.0)
    else:  # cancelling: each A row is x, -x over the two k halves against equal B halves
        x = rng.standard_normal((n, 32, 32)) * 8.0
        a = _codes(np.concatenate([x, -x], axis=2))
        y = rng.standard_normal((n, 32, 32))
        b = _codes(np.concatenate([y, y + rng.standard_normal((n, 32, 32)) * 2.0 ** -4], axis=2))
    return a.contiguous(), b.contiguous()


@pytest.mark.parametrize("kind", ["uniform_codes", "normal", "probability", "cancelling"])
def test_e4m3_product_error_within_the_parity_bound(kind):
    print(f"[gpu case] probe e4m3 product {kind}", flush=True)
    rng = np.random.default_rng(17)
    n = 64
    a, b = _operands(kind, n, rng)
    d = torch.full((n, 32, 32), float("nan"), device="cuda")
    probe.mfma_f8(a.cuda(), b.cuda(), d)
    torch.cuda.synchronize()
    av, bv = _values(a), _values(b)
    exact = np.einsum("pmk,pnk->pmn", av, bv)
    maxterm = np.abs(av)[:, :, None, :] * np.abs(bv)[:, None, :, :]
    maxterm = maxterm.max(axis=3)
    err = np.abs(d.cpu().double().numpy() - exact)
    assert np.all(np.isfinite(err))
    assert np.all(err <= C_MFMA * maxterm), float((err / np.maximum(maxterm, 1e-300)).max())
    ratio = float((err / np.where(maxterm > 0, maxterm, np.inf)).max())
    print(f"  largest error / largest term: 2^{math.log2(ratio) if ratio > 0 else -math.inf:.2f}"
          f" (bound 2^{math.log2(C_MFMA):.0f})", flush=True)
