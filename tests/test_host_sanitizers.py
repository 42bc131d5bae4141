"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The library's host side (argument validation, workspace sizing, the block-table checker with
its stack bitmap and 64-bit index arithmetic, the path selector, the no-workspace decode's
size checks) is rebuilt with the sanitizers on its host code only (device code is untouched)
and the C-ABI tests run against that build in a child process with the sanitizer runtime
preloaded. Any invalid access or undefined operation aborts the child and fails this test.
"""
import glob
import os
import shutil
import subprocess
import sys
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_21_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-only instrumentation: each sanitizer flag applies to the host compilation alone
SAN = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=undefined".split()
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    extra = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] if src.endswith("decode_mfma.hip") else []
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    r = subprocess.run([HIPCC, *FLAGS, *SAN, *extra, *lang, "-c", src, "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC) or _runtime() is None,
                    reason="needs hipcc and clang's sanitizer runtime")
def test_abi_under_host_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    lib = os.path.join(OUT, "libmla_sanitized.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, MLA_LIB=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_select.py"),
                        os.path.join(ROOT, "tests", "test_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
