"""GPU checks that the ceiling probes do the work they are timed for: the
MFMA probe's per-wave output sum equals the sum of every output element of
its products, recomputed on the host from the fragments' row and column
sums (sum over all (m, n) of A.B = sum over k of colsum_A[k] * rowsum_B[k];
lane l of a 32x32x16 fragment holds k = 8 * (l // 32) + t, t = 0..7), and
the read probe's XOR fold equals the XOR of every 32-bit word read."""
import numpy as np
import pytest
import torch

from block_sparse_attention_tile_amd import ceiling

pytestmark = pytest.mark.gpu


def test_mfma_probe_computes_its_products():
    print("[gpu case] ceiling mfma probe", flush=True)
    g = torch.Generator().manual_seed(5)
    n_slices, wgs, iters = 5, 3, 4
    src_h = torch.randn(n_slices * ceiling.SLICE_BYTES // 2, generator=g).to(torch.bfloat16)
    src = src_h.cuda()
    out = torch.full((wgs * ceiling.WAVES * 64,), float("nan"), device="cuda")
    flops = ceiling.mfma_bf16(src, out, wgs, iters)
    torch.cuda.synchronize()
    assert flops == wgs * 12 * iters * 64 * 32768
    fr = src_h.float().double().numpy().reshape(n_slices, 16, 2, 32, 8)  # slice, frag, half, lane%32, t
    s = fr.sum(axis=3).reshape(n_slices, 16, 16)  # per k = 8 * half + t: sum over the 32 lanes
    got = out.cpu().double().numpy().reshape(wgs * 12, 64).sum(axis=1)
    for w in range(wgs * 12):
        sa, sb = s[w % n_slices, :8], s[w % n_slices, 8:]
        want = iters * sum(float(sa[ia] @ sb[(ia + ib) % 8]) for ia in range(8) for ib in range(8))
        scale = iters * sum(float(np.abs(sa[ia]) @ np.abs(sb[(ia + ib) % 8])) for ia in range(8) for ib in range(8))
        assert abs(got[w] - want) <= 1e-4 * scale + 1e-3, (w, got[w], want)


def test_read_probe_reads_every_word():
    print("[gpu case] ceiling read probe", flush=True)
    rng = np.random.default_rng(3)
    words = rng.integers(0, 2 ** 32, size=4 * 12345, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    for wgs in (1, 3, 7):
        for nt in (False, True):
            out = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
            assert ceiling.read(src, out, wgs, nt) == words.nbytes
            torch.cuda.synchronize()
            folded = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
            assert folded == np.bitwise_xor.reduce(words), (wgs, nt)
