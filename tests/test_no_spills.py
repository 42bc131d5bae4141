"""Every kernel of the library compiles for gfx950 without private (scratch) memory.

A register spill inside the split-K core's main loop reloads through scratch, and the compiler
then waits for every outstanding global load before the reload, which drains the tile copies in
flight and slows the kernel by a third or more. The check compiles each HIP source for the device
with the library's own flags and reads the kernel descriptors: every kernel must declare a zero
private segment, and no scratch instruction may appear.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from mla_latent_kv_21_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                reason="needs hipcc")

HIP_SOURCES = [s for s in B.sources() if s.endswith(".hip")]


def device_asm(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in B.FLAGS if f not in ("-fPIC",)]
    cmd = [B.HIPCC, *flags, *B.EXTRA.get(os.path.basename(src), []), "-x", "hip",
           "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-2000:]}"
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            texts = list(ex.map(lambda s: device_asm(s, d), HIP_SOURCES))
    return dict(zip((os.path.basename(s) for s in HIP_SOURCES), texts))


def kernels(text):
    """(name, private segment bytes) for every kernel descriptor in an assembly listing."""
    names = re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", text, re.M)
    sizes = [int(v) for v in
             re.findall(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", text, re.M)]
    assert len(names) == len(sizes)
    return list(zip(names, sizes))


@pytest.mark.parametrize("src", [os.path.basename(s) for s in HIP_SOURCES])
def test_no_private_segment(asm, src):
    text = asm[src]
    spilled = [(n, s) for n, s in kernels(text) if s != 0]
    assert not spilled, f"{src}: kernels with scratch: {spilled}"
    assert not re.search(r"^\s*scratch_(load|store)", text, re.M), f"{src}: scratch access"


def test_the_core_variants_are_all_there(asm):
    """The split-K core's ten instantiations (one and two head blocks; four head blocks over
    bf16 and e4m3 rows, plain and forming a decode step's new rows, each with streaming and with
    default-policy tile copies) are all compiled and so all checked above."""
    names = [n for n, _ in kernels(asm["decode_mfma.hip"])]
    assert len([n for n in names if "decode_mfma_kernel" in n]) == 10
