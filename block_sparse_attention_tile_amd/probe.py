"""ctypes binding of libvsa_probe.so (include/vsa_probe.h): hardware probes
beside the attention library.  bench.py reports the two same-run ceilings;
the E4M3 parity tests measure the bare E4M3 product's summation error.

Argument marshalling only; the probes run in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa_probe.so")
EXPORTED = ["vsa_probe_mfma_rate", "vsa_probe_read_rate", "vsa_probe_mfma_f8"]
WAVES = 12            # VSA_PROBE_WAVES
SLICE_BYTES = 16384   # one wave's sixteen 1 KB fragments
FLOP_PER_ITER_WAVE = 64 * 32768

_lib = None


def lib():
    """Load libvsa_probe.so; fail loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_tile_amd.build`")
    L = C.CDLL(LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    P = C.c_void_p
    L.vsa_probe_mfma_rate.argtypes = [P, C.c_size_t, P, C.c_int, C.c_int, P]
    L.vsa_probe_read_rate.argtypes = [P, C.c_size_t, P, C.c_int, C.c_int, P]
    L.vsa_probe_mfma_f8.argtypes = [P, P, P, C.c_int, P]
    for n in EXPORTED:
        getattr(L, n).restype = C.c_int
    _lib = L
    return L


def _stream(t):
    import torch
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(name, st):
    if st != 0:
        raise RuntimeError(f"{name} failed with status {st}")


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def mfma_rate(src, out, workgroups: int, iters: int) -> float:
    """Launch the MFMA rate probe; returns the FLOPs it performs.  src: a
    device tensor of bf16 bits (a multiple of 16 KB); out: float32 device
    tensor of workgroups * 12 * 64 elements."""
    import torch
    _require(src.is_cuda and src.is_contiguous() and (src.numel() * src.element_size()) % SLICE_BYTES == 0,
             "src: contiguous device tensor of whole 16 KB slices")
    _require(out.is_cuda and out.dtype == torch.float32 and out.numel() >= workgroups * WAVES * 64,
             "out: float32 device tensor of workgroups * 12 * 64 elements")
    _check("vsa_probe_mfma_rate",
           lib().vsa_probe_mfma_rate(C.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                     C.c_void_p(out.data_ptr()), workgroups, iters, _stream(src)))
    return float(workgroups) * WAVES * iters * FLOP_PER_ITER_WAVE


def read_rate(src, out, workgroups: int, nontemporal: bool = False) -> int:
    """Launch the read probe over all of src; returns the bytes it reads.
    out: int32 device tensor of workgroups * 256 elements."""
    nbytes = src.numel() * src.element_size()
    _require(src.is_cuda and src.is_contiguous() and nbytes % 16 == 0,
             "src: contiguous device tensor of whole 16-byte units")
    _require(out.is_cuda and out.element_size() == 4 and out.numel() >= workgroups * 256,
             "out: 4-byte device tensor of workgroups * 256 elements")
    _check("vsa_probe_read_rate",
           lib().vsa_probe_read_rate(C.c_void_p(src.data_ptr()), nbytes, C.c_void_p(out.data_ptr()),
                                     workgroups, int(nontemporal), _stream(src)))
    return nbytes


def mfma_f8(a, b, d) -> None:
    """D[p] = A[p] B[p] by one E4M3 MFMA per problem.  a: uint8 [n, 32, 64]
    (rows, k); b: uint8 [n, 32, 64] (columns, k); d: float32 [n, 32, 32]."""
    import torch
    n = a.shape[0]
    for t, dt, shape, name in ((a, torch.uint8, (n, 32, 64), "a"), (b, torch.uint8, (n, 32, 64), "b"),
                               (d, torch.float32, (n, 32, 32), "d")):
        _require(t.is_cuda and t.dtype == dt and t.is_contiguous() and tuple(t.shape) == shape,
                 f"{name}: contiguous device tensor {dt} {shape}")
    _check("vsa_probe_mfma_f8",
           lib().vsa_probe_mfma_f8(C.c_void_p(a.data_ptr()), C.c_void_p(b.data_ptr()),
                                   C.c_void_p(d.data_ptr()), n, _stream(a)))
