"""ctypes binding of libvsa.so (the C ABI in include/vsa.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Functions keep the C names; the torch helpers at the bottom only
turn tensors into device pointers and the current HIP stream.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa.so")

VSA_OK = 0
VSA_ERR_INVALID_ARG = 1
VSA_ERR_UNSUPPORTED = 2
VSA_ERR_WORKSPACE_TOO_SMALL = 3
VSA_ERR_HIP = 4
VSA_BF16 = 1

VSA_DENSE = 0x01
VSA_WINDOW = 0x02
VSA_TOPK = 0x04
VSA_TOPK_FRAC = 0x08
VSA_TOPP = 0x10
VSA_SICS_SELECT = 0x20
VSA_FINE = 0x40
VSA_PROFILE_SELECT = 0x80
VSA_WIN_TRUNCATE = 0
VSA_WIN_CLAMP = 1
VSA_MAX_CAND = 4
VSA_SUMM_MEAN = 0
VSA_SUMM_MAX = 1
VSA_SUMM_MINMAX = 2
VSA_COMPUTE_BF16 = 0
VSA_COMPUTE_FP8 = 1
VSA_NOALLOC_BYTES = 256 << 20

(VSA_WS_QT, VSA_WS_KT, VSA_WS_VT, VSA_WS_POOLED_Q, VSA_WS_POOLED_K, VSA_WS_ROW_LEN,
 VSA_WS_COL_IDX, VSA_WS_CAND, VSA_WS_CAND_SCORE, VSA_WS_TILE_SICS, VSA_WS_ATOMS,
 VSA_WS_FINE_QBAR, VSA_WS_FINE_TAU, VSA_WS_FINE_COUNT, VSA_WS_FINE_IDX, VSA_WS_FINE_PTR,
 VSA_WS_FINE_MASK, VSA_WS_SCRATCH, VSA_WS_POOLED_KMIN, VSA_WS_F8_EXP, VSA_WS_F8_AMAX,
 VSA_WS_PROF_SSE, VSA_WS_PROF_PART, VSA_WS_NREGIONS) = range(24)

EXPORTED = [
    "vsa_plan", "vsa_plan_destroy", "vsa_plan_get_info", "vsa_workspace_bytes",
    "vsa_workspace_region", "vsa_forward", "vsa_forward_cached", "vsa_forward_noalloc", "vsa_layout",
    "vsa_select", "vsa_attend",
    "vsa_untile", "vsa_read_selection", "vsa_retained_work", "vsa_status_string",
    "vsa_last_error",
]


class vsa_problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("d", C.c_int32),
                ("grid", C.c_int32 * 3), ("tile", C.c_int32 * 3),
                ("n_cand", C.c_int32), ("cand_tile", (C.c_int32 * 3) * VSA_MAX_CAND),
                ("dtype", C.c_int32)]


class vsa_mask_policy(C.Structure):
    _fields_ = [("flags", C.c_uint32), ("win", C.c_int32 * 3), ("win_mode", C.c_int32),
                ("topk", C.c_int32), ("topk_frac", C.c_double), ("topp", C.c_double),
                ("fine_group", C.c_int32), ("fine_keep", C.c_double), ("scale", C.c_double),
                ("summarizer", C.c_int32), ("sink", C.c_int32), ("compute", C.c_int32),
                ("profile_frac", C.c_double)]


class vsa_plan_info(C.Structure):
    _fields_ = [("n_blockings", C.c_int32), ("ntiles", (C.c_int32 * 3) * VSA_MAX_CAND),
                ("n_tiles", C.c_int32 * VSA_MAX_CAND), ("slots", C.c_int32 * VSA_MAX_CAND),
                ("topk", C.c_int32 * VSA_MAX_CAND), ("max_tiles", C.c_int32),
                ("row_cap", C.c_int32), ("static_pairs", C.c_int64),
                ("static_flops", C.c_double), ("fine_groups", C.c_int32),
                ("fine_keep_count", C.c_int64), ("fine_cap", C.c_int64), ("scale", C.c_double),
                ("pair", C.c_int32 * VSA_MAX_CAND),
                ("units", C.c_int32 * VSA_MAX_CAND),
                ("interleave", C.c_int32 * VSA_MAX_CAND), ("head_sync", C.c_int32)]


class VsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libvsa.so; fail loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_tile_amd.build`")
    L = C.CDLL(LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)  # unresolved symbols fail here
    P = C.c_void_p
    sz = C.c_size_t
    L.vsa_plan.argtypes = [C.POINTER(vsa_problem), C.POINTER(vsa_mask_policy), C.POINTER(P)]
    L.vsa_plan_destroy.argtypes = [P]
    L.vsa_plan_destroy.restype = None
    L.vsa_plan_get_info.argtypes = [P, C.POINTER(vsa_plan_info)]
    L.vsa_workspace_bytes.argtypes = [P, C.POINTER(sz)]
    L.vsa_workspace_region.argtypes = [P, C.c_int, C.POINTER(sz), C.POINTER(sz)]
    for name in ("vsa_layout", "vsa_select"):
        getattr(L, name).argtypes = [P, P, P, P, P, sz, P]
    for name in ("vsa_forward", "vsa_forward_cached", "vsa_attend"):
        getattr(L, name).argtypes = [P, P, P, P, P, P, sz, P]
    L.vsa_forward_noalloc.argtypes = [P, P, P, P, P, P]
    L.vsa_untile.argtypes = [P, C.c_int, P, sz, P, P]
    L.vsa_read_selection.argtypes = [P, P, sz, C.POINTER(C.c_int32), C.POINTER(C.c_int32), sz,
                                     C.POINTER(C.c_int64), C.POINTER(C.c_int32), P]
    L.vsa_retained_work.argtypes = [P, P, sz, C.POINTER(C.c_int64), C.POINTER(C.c_double), P]
    L.vsa_status_string.argtypes = [C.c_int]
    L.vsa_status_string.restype = C.c_char_p
    L.vsa_last_error.argtypes = []
    L.vsa_last_error.restype = C.c_char_p
    for name in EXPORTED:
        if name not in ("vsa_plan_destroy", "vsa_status_string", "vsa_last_error"):
            getattr(L, name).restype = C.c_int
    _lib = L
    return L


def _status_name(status):
    try:
        return lib().vsa_status_string(status).decode()
    except Exception:  # pragma: no cover - only while the library is absent
        return str(status)


def _check(status):
    if status != VSA_OK:
        raise VsaError(status, lib().vsa_last_error().decode())


# ---------------------------------------------------------------- structs

def make_problem(B, H, d, grid, tile, candidates=()):
    p = vsa_problem()
    p.B, p.H, p.d = B, H, d
    p.grid[:] = list(grid)
    p.tile[:] = list(tile)
    p.n_cand = len(candidates)
    for c, t in enumerate(candidates):
        p.cand_tile[c][:] = list(t)
    p.dtype = VSA_BF16
    return p


def make_policy(flags, win=(1, 1, 1), win_mode=VSA_WIN_TRUNCATE, topk=0, topk_frac=0.0,
                topp=0.0, fine_group=0, fine_keep=0.0, scale=0.0, summarizer=VSA_SUMM_MEAN, sink=0,
                compute=VSA_COMPUTE_BF16, profile_frac=0.0):
    p = vsa_mask_policy()
    p.flags = flags
    p.win[:] = list(win)
    p.win_mode = win_mode
    p.topk = topk
    p.topk_frac = topk_frac
    p.topp = topp
    p.fine_group = fine_group
    p.fine_keep = fine_keep
    p.scale = scale
    p.summarizer = summarizer
    p.sink = sink
    p.compute = compute
    p.profile_frac = profile_frac
    return p


# ------------------------------------------------------------- C functions

def vsa_plan(problem, policy):
    h = C.c_void_p()
    _check(lib().vsa_plan(C.byref(problem), C.byref(policy), C.byref(h)))
    return h


def vsa_plan_destroy(plan):
    lib().vsa_plan_destroy(plan)


def vsa_plan_get_info(plan):
    info = vsa_plan_info()
    _check(lib().vsa_plan_get_info(plan, C.byref(info)))
    return info


def vsa_workspace_bytes(plan):
    n = C.c_size_t()
    _check(lib().vsa_workspace_bytes(plan, C.byref(n)))
    return n.value


def vsa_workspace_region(plan, region):
    off, n = C.c_size_t(), C.c_size_t()
    _check(lib().vsa_workspace_region(plan, region, C.byref(off), C.byref(n)))
    return off.value, n.value


def vsa_forward(plan, q, k, v, o, ws, ws_bytes, stream):
    _check(lib().vsa_forward(plan, q, k, v, o, ws, ws_bytes, stream))


def vsa_forward_cached(plan, q, k, v, o, ws, ws_bytes, stream):
    _check(lib().vsa_forward_cached(plan, q, k, v, o, ws, ws_bytes, stream))


def vsa_forward_noalloc(plan, q, k, v, o, stream):
    _check(lib().vsa_forward_noalloc(plan, q, k, v, o, stream))


def vsa_layout(plan, q, k, v, ws, ws_bytes, stream):
    _check(lib().vsa_layout(plan, q, k, v, ws, ws_bytes, stream))


def vsa_select(plan, q, k, v, ws, ws_bytes, stream):
    _check(lib().vsa_select(plan, q, k, v, ws, ws_bytes, stream))


def vsa_attend(plan, q, k, v, o, ws, ws_bytes, stream):
    _check(lib().vsa_attend(plan, q, k, v, o, ws, ws_bytes, stream))


def vsa_untile(plan, which, ws, ws_bytes, out, stream):
    _check(lib().vsa_untile(plan, which, ws, ws_bytes, out, stream))


def vsa_read_selection(plan, ws, ws_bytes, stream, n_heads):
    """(row_ptr, col_idx, cand) as numpy arrays; n_heads = B * H."""
    import numpy as np
    info = vsa_plan_get_info(plan)
    rows = n_heads * info.max_tiles
    row_ptr = np.zeros(rows + 1, dtype=np.int32)
    cap = rows * max(1, info.row_cap)
    col = np.zeros(cap, dtype=np.int32)
    cand = np.zeros(n_heads, dtype=np.int32)
    n = C.c_int64()
    i32p = C.POINTER(C.c_int32)
    _check(lib().vsa_read_selection(plan, ws, ws_bytes, row_ptr.ctypes.data_as(i32p),
                                    col.ctypes.data_as(i32p), cap, C.byref(n),
                                    cand.ctypes.data_as(i32p), stream))
    return row_ptr, col[:n.value].copy(), cand


def vsa_retained_work(plan, ws, ws_bytes, stream):
    pairs, flops = C.c_int64(), C.c_double()
    _check(lib().vsa_retained_work(plan, ws, ws_bytes, C.byref(pairs), C.byref(flops), stream))
    return pairs.value, flops.value
