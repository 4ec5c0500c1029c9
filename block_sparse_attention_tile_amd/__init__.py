"""Block-sparse self-attention over 3D video token grids for MI355X (gfx950).

The compute lives in libvsa.so (hand-written HIP kernels behind the C ABI in
include/vsa.h); this package only binds it.  `Plan` bundles a plan handle
with its workspace; the module-level vsa_* functions mirror the C calls.
"""
from __future__ import annotations

from . import _lib
from ._lib import (  # noqa: F401
    VSA_DENSE, VSA_FINE, VSA_SICS_SELECT, VSA_TOPK, VSA_TOPK_FRAC, VSA_TOPP, VSA_WINDOW,
    VSA_SUMM_MAX, VSA_SUMM_MEAN, VSA_SUMM_MINMAX, VSA_WIN_CLAMP, VSA_WIN_TRUNCATE, VsaError, lib,
    VSA_COMPUTE_BF16, VSA_COMPUTE_FP8, VSA_PROFILE_SELECT,
    make_policy, make_problem, vsa_attend,
    vsa_forward, vsa_forward_cached, vsa_forward_noalloc, vsa_layout, vsa_plan, vsa_plan_destroy, vsa_plan_get_info,
    vsa_read_selection, vsa_retained_work, vsa_select, vsa_untile, vsa_workspace_bytes,
    vsa_workspace_region,
)


from .workload import flags_of, plan_structs  # noqa: E402,F401


def _ptr(t):
    return t.data_ptr() if t is not None else None


class Plan:
    """A plan plus a workspace tensor on one device (torch used for memory only)."""

    def __init__(self, problem, policy, device="cuda"):
        self.problem = problem
        self.policy = policy
        self.handle = vsa_plan(problem, policy)
        self.info = vsa_plan_get_info(self.handle)
        self.ws_bytes = vsa_workspace_bytes(self.handle)
        self.device = device
        self._ws = None

    @property
    def n_heads(self):
        return self.problem.B * self.problem.H

    def workspace(self):
        import torch
        if self._ws is None:
            self._ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def region(self, which, dtype):
        """View of one workspace region as a flat tensor of `dtype`."""
        import torch
        off, n = vsa_workspace_region(self.handle, which)
        ws = self.workspace()
        return ws[off:off + n].view(dtype)

    @staticmethod
    def _stream():
        import torch
        return torch.cuda.current_stream().cuda_stream

    def _check(self, *ts):
        import torch
        for t in ts:
            if t is None:
                continue
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
                raise ValueError("tensors must be contiguous bf16 on the GPU")
            p = self.problem
            n = p.grid[0] * p.grid[1] * p.grid[2]
            if tuple(t.shape) != (p.B, p.H, n, p.d):
                raise ValueError(f"expected shape {(p.B, p.H, n, p.d)}, got {tuple(t.shape)}")

    def forward(self, q, k, v, o=None):
        import torch
        if o is None:
            o = torch.empty_like(q)
        self._check(q, k, v, o)
        vsa_forward(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(self.workspace()),
                    self.ws_bytes, self._stream())
        return o

    def forward_cached(self, q, k, v, o=None):
        """Forward against the selection already in this plan's workspace
        (from the last forward/select): see vsa_forward_cached."""
        import torch
        if o is None:
            o = torch.empty_like(q)
        self._check(q, k, v, o)
        vsa_forward_cached(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(self.workspace()),
                           self.ws_bytes, self._stream())
        return o

    def forward_noalloc(self, q, k, v, o=None):
        """Forward on the library's own per-device scratch array instead of
        this plan's workspace: see vsa_forward_noalloc."""
        import torch
        if o is None:
            o = torch.empty_like(q)
        self._check(q, k, v, o)
        vsa_forward_noalloc(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), self._stream())
        return o

    def layout(self, q, k, v):
        self._check(q, k, v)
        vsa_layout(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(self.workspace()), self.ws_bytes,
                   self._stream())

    def select(self, q=None, k=None, v=None):
        self._check(q, k, v)
        vsa_select(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(self.workspace()), self.ws_bytes,
                   self._stream())

    def attend(self, o, q=None, k=None, v=None):
        self._check(q, k, v, o)
        vsa_attend(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(self.workspace()),
                   self.ws_bytes, self._stream())
        return o

    def untile(self, which, out):
        self._check(out)
        vsa_untile(self.handle, which, _ptr(self.workspace()), self.ws_bytes, _ptr(out),
                   self._stream())
        return out

    def read_selection(self):
        return vsa_read_selection(self.handle, _ptr(self.workspace()), self.ws_bytes,
                                  self._stream(), self.n_heads)

    def retained_work(self):
        return vsa_retained_work(self.handle, _ptr(self.workspace()), self.ws_bytes,
                                 self._stream())

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                vsa_plan_destroy(h)
            except Exception:
                pass
            self.handle = None
