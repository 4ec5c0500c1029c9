"""CPU checks of the entry points' contracts: bench.py refuses more than one
GPU with a message, the product path fails loudly without the HIP library,
and the build entry point exposes build() and smoke()."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from block_sparse_attention_tile_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libvsa.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()


def test_graft_entry_exposes_build_and_smoke():
    sys.path.insert(0, ROOT)
    import __graft_entry__ as g
    assert callable(g.build) and callable(g.smoke)
