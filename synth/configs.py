"""Named workloads: attention shapes of video DiTs and their mask policies.

Shapes are the latent token grids of the models' attention layers.  The
policy entries are plain parameters; how a mask is built from them lives
in the library (HIP path) and, independently, in the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    grid: Tuple[int, int, int]            # (T, H, W) tokens
    tile: Tuple[int, int, int]            # (tt, th, tw) tokens per tile
    candidates: Tuple[Tuple[int, int, int], ...] = ()   # SICS blockings
    window: Optional[Tuple[int, int, int]] = None       # full extents, odd
    win_mode: str = "truncate"            # or "clamp"
    topk: int = 0
    topk_frac: float = 0.0
    topp: float = 0.0
    fine_group: int = 0
    fine_keep: float = 0.0
    summarizer: str = "mean"              # block summary of K: "mean", "max", "minmax"
    sink: int = 0                         # leading key tiles always kept
    compute: str = "bf16"                 # attention arithmetic: "bf16" or "fp8" (E4M3)
    selector: str = "sics"                # per-head choice among candidates: "sics" or "profile"
    profile_frac: float = 0.0             # sampled query rows of the profiling selector (0 = 1%)
    ell: Tuple[float, float, float] = (2.0, 2.0, 2.0)
    ell_alt: Optional[Tuple[float, float, float]] = None  # odd heads
    note: str = ""

    @property
    def N(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    def ell_per_head(self) -> Sequence[Tuple[float, float, float]]:
        if self.ell_alt is None:
            return [self.ell] * self.H
        return [self.ell if h % 2 == 0 else self.ell_alt for h in range(self.H)]

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


CONFIGS = {
    # 8 tiles; the +-1 window covers every tile, so the mask is all-ones.
    "tiny": Workload("tiny", 1, 2, 64, (4, 8, 8), (2, 4, 4),
                     window=(3, 3, 3), topk=4),
    # Wan-2.1-1.3B 480p: +-1 tile window plus per-head Top-P 0.9.
    "wan480": Workload("wan480", 1, 12, 128, (21, 30, 52), (3, 6, 8),
                       window=(3, 3, 3), topp=0.9),
    # HunyuanVideo 720p: fixed sliding-tile window of 3x3x5 tiles.
    "hunyuan": Workload("hunyuan", 1, 24, 128, (30, 48, 80), (6, 8, 8),
                        window=(3, 3, 5)),
    # Wan-14B 720p: per-head SICS choice among three blockings, Top-K 20%.
    "wan14b": Workload("wan14b", 1, 40, 128, (21, 45, 80), (1, 16, 16),
                       candidates=((1, 16, 16), (7, 4, 4), (3, 8, 8)),
                       topk_frac=0.2, ell=(8.0, 1.0, 1.0),
                       ell_alt=(1.0, 8.0, 8.0)),
    # HunyuanVideo 720p shape, per-head spatial / temporal choice by the
    # profiling selector: whole-frame tiles (1, 48, 80) vs 4x4-position tiles
    # across all 30 frames (30, 4, 4), each attending within its own tile;
    # anisotropic heads as for Wan-14B.
    "hunyuan_svg": Workload("hunyuan_svg", 1, 24, 128, (30, 48, 80), (1, 48, 80),
                            candidates=((1, 48, 80), (30, 4, 4)), window=(1, 1, 1),
                            selector="profile", ell=(8.0, 1.0, 1.0), ell_alt=(1.0, 8.0, 8.0)),
    # Fine-grained M x 1 slices at the Wan-2.1-1.3B 480p shape.
    "fine": Workload("fine", 1, 12, 128, (21, 30, 52), (1, 1, 1),
                     fine_group=64, fine_keep=0.15),
}


def get(name: str) -> Workload:
    return CONFIGS[name]
