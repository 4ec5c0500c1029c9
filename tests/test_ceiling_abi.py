"""CPU checks of the ceiling library (include/vsa_ceiling.h): it loads,
exports every declared call, and refuses bad arguments before any launch."""
import ctypes
import os
import re

from block_sparse_attention_tile_amd import ceiling

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "vsa_ceiling.h")


def test_ceiling_library_exports_every_declared_function():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(vsa_\w+)\s*\(", src)))
    L = ctypes.CDLL(ceiling.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    assert declared == sorted(ceiling.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_ceiling_calls_refuse_bad_arguments():
    L = ceiling.lib()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails its checks
    assert L.vsa_ceiling_mfma_bf16(None, 16384, fake, 1, 1, None) == 1
    assert L.vsa_ceiling_mfma_bf16(fake, 16384 + 16, fake, 1, 1, None) == 1  # not whole slices
    assert L.vsa_ceiling_mfma_bf16(fake, 16384, fake, 0, 1, None) == 1
    assert L.vsa_ceiling_mfma_bf16(fake, 16384, fake, 1, 0, None) == 1
    assert L.vsa_ceiling_mfma_bf16(ctypes.c_void_p((1 << 20) + 4), 16384, fake, 1, 1, None) == 1
    assert L.vsa_ceiling_read(fake, 24, fake, 1, 0, None) == 1  # not whole 16-byte units
    assert L.vsa_ceiling_read(fake, 0, fake, 1, 0, None) == 1
    assert L.vsa_ceiling_read(fake, 32, None, 1, 1, None) == 1
    assert L.vsa_ceiling_read(fake, 32, fake, 0, 1, None) == 1
