"""ctypes binding of libvsa_ceiling.so (include/vsa_ceiling.h): the same-run
ceilings of this part that bench.py reports beside the attention.

Argument marshalling only; the probes run in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa_ceiling.so")
EXPORTED = ["vsa_ceiling_mfma_bf16", "vsa_ceiling_read"]
WAVES = 12            # VSA_CEILING_WAVES
SLICE_BYTES = 16384   # one wave's sixteen 1 KB fragments
FLOP_PER_ITER_WAVE = 64 * 32768

_lib = None


def lib():
    """Load libvsa_ceiling.so; fail loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_tile_amd.build`")
    L = C.CDLL(LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    P = C.c_void_p
    L.vsa_ceiling_mfma_bf16.argtypes = [P, C.c_size_t, P, C.c_int, C.c_int, P]
    L.vsa_ceiling_read.argtypes = [P, C.c_size_t, P, C.c_int, C.c_int, P]
    for n in EXPORTED:
        getattr(L, n).restype = C.c_int
    _lib = L
    return L


def _stream(t):
    import torch
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def mfma_bf16(src, out, workgroups: int, iters: int) -> float:
    """Launch the MFMA probe; returns the FLOPs it performs.  src: a device
    tensor of bf16 bits (a multiple of 16 KB); out: float32 device tensor of
    workgroups * 12 * 64 elements."""
    import torch
    assert src.is_cuda and src.is_contiguous() and (src.numel() * src.element_size()) % SLICE_BYTES == 0
    assert out.is_cuda and out.dtype == torch.float32 and out.numel() >= workgroups * WAVES * 64
    st = lib().vsa_ceiling_mfma_bf16(C.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                     C.c_void_p(out.data_ptr()), workgroups, iters, _stream(src))
    if st != 0:
        raise RuntimeError(f"vsa_ceiling_mfma_bf16 failed with status {st}")
    return float(workgroups) * WAVES * iters * FLOP_PER_ITER_WAVE


def read(src, out, workgroups: int, nontemporal: bool = False) -> int:
    """Launch the read probe over all of src; returns the bytes it reads.
    out: int32 device tensor of workgroups * 256 elements."""
    import torch
    nbytes = src.numel() * src.element_size()
    assert src.is_cuda and src.is_contiguous() and nbytes % 16 == 0
    assert out.is_cuda and out.element_size() == 4 and out.numel() >= workgroups * 256
    st = lib().vsa_ceiling_read(C.c_void_p(src.data_ptr()), nbytes, C.c_void_p(out.data_ptr()),
                                workgroups, int(nontemporal), _stream(src))
    if st != 0:
        raise RuntimeError(f"vsa_ceiling_read failed with status {st}")
    return nbytes
