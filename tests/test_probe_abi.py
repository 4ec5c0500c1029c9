"""CPU checks of the probe library (include/vsa_probe.h): it loads, exports
every declared call, and refuses bad arguments before any launch."""
import ctypes
import os
import re

from block_sparse_attention_tile_amd import probe

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "vsa_probe.h")


def test_probe_library_exports_every_declared_function():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(vsa_\w+)\s*\(", src)))
    L = ctypes.CDLL(probe.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    assert declared == sorted(probe.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_probe_calls_refuse_bad_arguments():
    L = probe.lib()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails its checks
    odd = ctypes.c_void_p((1 << 20) + 4)
    assert L.vsa_probe_mfma_rate(None, 16384, fake, 1, 1, None) == 1
    assert L.vsa_probe_mfma_rate(fake, 16384 + 16, fake, 1, 1, None) == 1  # not whole slices
    assert L.vsa_probe_mfma_rate(fake, 16384, fake, 0, 1, None) == 1
    assert L.vsa_probe_mfma_rate(fake, 16384, fake, 1, 0, None) == 1
    assert L.vsa_probe_mfma_rate(odd, 16384, fake, 1, 1, None) == 1
    assert L.vsa_probe_read_rate(fake, 24, fake, 1, 0, None) == 1  # not whole 16-byte units
    assert L.vsa_probe_read_rate(fake, 0, fake, 1, 0, None) == 1
    assert L.vsa_probe_read_rate(fake, 32, None, 1, 1, None) == 1
    assert L.vsa_probe_read_rate(fake, 32, fake, 0, 1, None) == 1
    assert L.vsa_probe_mfma_f8(fake, fake, fake, 0, None) == 1
    assert L.vsa_probe_mfma_f8(odd, fake, fake, 1, None) == 1
    assert L.vsa_probe_mfma_f8(fake, None, fake, 1, None) == 1


def test_probe_binding_refuses_host_tensors():
    import pytest
    import torch
    with pytest.raises(ValueError):
        probe.mfma_rate(torch.zeros(8192, dtype=torch.bfloat16), torch.zeros(768), 1, 1)
    with pytest.raises(ValueError):
        probe.read_rate(torch.zeros(16, dtype=torch.uint8), torch.zeros(256, dtype=torch.int32), 1)
    with pytest.raises(ValueError):
        z8 = torch.zeros(1, 32, 64, dtype=torch.uint8)
        probe.mfma_f8(z8, z8, torch.zeros(1, 32, 32))
