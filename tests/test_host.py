"""Host-side behaviour that needs no GPU: the benchmark refuses more than one GPU before it
touches a device, and the binding raises instead of falling back when the library is missing."""
import os
import subprocess
import sys

import pytest

from mla_latent_kv_21_amd import binding as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "libmla.so"))
    with pytest.raises(RuntimeError, match="not built"):
        M.lib()
    w_dims = M.make_dims(512, 8, 64, 64, 128, 32, 8, 64, "f32")
    with pytest.raises(RuntimeError, match="not built"):
        M.mla_decode_workspace_bytes(w_dims, 1, 1, 1, 8)
