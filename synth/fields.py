"""Smooth 3D Gaussian random fields plus white noise, cast to bf16.

Recipe (stated once, used everywhere):
  * For every (head, channel) pair an independent field on the T x H x W
    token grid is drawn: white N(0,1) noise is filtered in Fourier space by
    exp(-pi^2 * sum_a (f_a * l_a)^2) (f_a in cycles per token, periodic
    boundary).  The filtered field has covariance exp(-|r|^2 / (2 l^2))
    per axis, i.e. length-scale l_a tokens along axis a.
  * Each channel is rescaled to unit empirical variance (zero mean).
  * Independent N(0, sigma^2) noise with sigma = 0.3 is added.
  * The result is rounded to bfloat16 (round-to-nearest-even) and laid out
    as [B, H, N, d] with N in raster (t, h, w) order, w fastest.
  * Q, K, V use seeds s, s+1, s+2.  Within one tensor the random stream is
    consumed in (batch, head, channel) order.
"""
from __future__ import annotations

import math
from typing import Sequence

import torch


def _filter(grid, ell, device):
    T, Hh, W = grid
    ft = torch.fft.fftfreq(T, device=device, dtype=torch.float64)
    fh = torch.fft.fftfreq(Hh, device=device, dtype=torch.float64)
    fw = torch.fft.rfftfreq(W, device=device, dtype=torch.float64)
    e = (ft[:, None, None] * ell[0]) ** 2 + (fh[None, :, None] * ell[1]) ** 2 \
        + (fw[None, None, :] * ell[2]) ** 2
    return torch.exp(-(math.pi ** 2) * e).to(torch.float32)


def smooth_field(shape_bhd: Sequence[int], grid: Sequence[int],
                 ell_per_head: Sequence[Sequence[float]], seed: int,
                 noise_sigma: float = 0.3, device="cpu",
                 head_chunk: int = 4) -> torch.Tensor:
    """One bf16 tensor [B, H, N, d] of smooth fields plus noise."""
    B, H, d = shape_bhd
    T, Hh, W = grid
    N = T * Hh * W
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=device)
    filters = {}
    for b in range(B):
        for h0 in range(0, H, head_chunk):
            h1 = min(H, h0 + head_chunk)
            nh = h1 - h0
            white = torch.randn((nh, d, T, Hh, W), generator=gen,
                                device=device, dtype=torch.float32)
            noise = torch.randn((nh, d, T, Hh, W), generator=gen,
                                device=device, dtype=torch.float32)
            spec = torch.fft.rfftn(white, dim=(2, 3, 4))
            for j in range(nh):
                ell = tuple(float(x) for x in ell_per_head[h0 + j])
                if ell not in filters:
                    filters[ell] = _filter(grid, ell, device)
                spec[j] *= filters[ell]
            fld = torch.fft.irfftn(spec, s=(T, Hh, W), dim=(2, 3, 4))
            fld = fld.reshape(nh, d, N)
            fld = fld - fld.mean(dim=2, keepdim=True)
            fld = fld / fld.std(dim=2, unbiased=False, keepdim=True).clamp_min(1e-12)
            fld = fld + noise_sigma * noise.reshape(nh, d, N)
            out[b, h0:h1] = fld.transpose(1, 2).to(torch.bfloat16)
    return out


def smooth_field_qkv(B, H, d, grid, ell_per_head, seed=0, device="cpu",
                     noise_sigma=0.3):
    """Q, K, V with seeds seed, seed+1, seed+2."""
    return tuple(smooth_field((B, H, d), grid, ell_per_head, seed + i,
                              noise_sigma=noise_sigma, device=device)
                 for i in range(3))
