"""The C ABI without a GPU: every declared symbol is exported, host-side validation returns the
documented status before anything is launched, workspace sizes follow their formula, and the
host block-table checker catches bad and shared block ids."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from mla_latent_kv_21_amd import binding as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        from mla_latent_kv_21_amd.build import build
        build()
    return M.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s+(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("mla_cache_append", "mla_absorb_q", "mla_decode", "gqla_expand", "gqla_decode"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    for name in M.EXPORTS:
        assert name in declared_functions()


def dims(**kw):
    base = dict(d_model=7168, n_heads=128, d_nope=128, d_v=128, d_c=512, d_r=64, n_groups=128,
                block_size=64, dtype="bf16")
    base.update(kw)
    return M.make_dims(**base)


P = ctypes.c_void_p
FAKE = 0x10000  # an aligned address that is never dereferenced: validation fails first


def decode_call(L, d, batch=2, s_q=1, q=FAKE, cache=FAKE, nb=8, table=FAKE, mb=4, lens=FAKE,
                wuv=FAKE, n_split=0, ws=None, ws_bytes=0, out=FAKE):
    dp = ctypes.byref(d) if d is not None else None
    return L.mla_decode(dp, batch, s_q, P(q), P(cache), nb, P(table), mb, P(lens), P(wuv),
                        n_split, P(ws), ws_bytes, P(out), None, None)


def test_decode_validation(L):
    d = dims()
    assert decode_call(L, None) == -1
    assert decode_call(L, dims(dtype=7)) == -3
    assert decode_call(L, dims(n_groups=3)) == -2          # 3 does not divide 128
    assert decode_call(L, dims(d_r=63)) == -2              # odd rotary width
    assert decode_call(L, dims(d_v=124)) == -2             # value rows are merged 16 bytes at a time
    assert decode_call(L, dims(d_c=500)) == -2             # latent width not a multiple of 8
    assert decode_call(L, d, batch=0) == 0                 # empty batch: nothing to do
    assert decode_call(L, d, s_q=0) == -4
    assert decode_call(L, d, n_split=M.MLA_MAX_SPLIT + 1) == -4
    assert decode_call(L, d, q=0) == -1
    assert decode_call(L, d, q=FAKE + 4) == -6             # misaligned
    assert decode_call(L, d, ws=None) == -5                # missing workspace
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 2, 1, 0, 4)
    assert decode_call(L, d, ws=FAKE, ws_bytes=need - 1) == -5


def test_workspace_sizes(L):
    d = dims()
    ns = L.mla_auto_split(ctypes.byref(d), 4, 1, 2048)
    assert ns == 64                                      # 4 sequences x 64 chunks = 256 CUs
    n = L.mla_decode_workspace_bytes(ctypes.byref(d), 4, 1, 64, 2048)
    rows = 4 * 128 * 64
    al = lambda x: (x + 255) // 256 * 256
    assert n == al(rows * 512 * 2) + al(rows * 4) + al(4 * 64 * 4)  # bf16 partial rows
    g = L.gqla_decode_workspace_bytes(ctypes.byref(d), 4, 2, 8, 2048)
    rows = 4 * 2 * 128 * 8
    assert g == al(rows * 128 * 2) + al(rows * 4) + al(4 * 2 * 8 * 4)
    assert L.mla_decode_workspace_bytes(ctypes.byref(d), 4, 1, M.MLA_MAX_SPLIT + 1, 2048) == 0
    # auto split: never more splits than 64-position chunks of the longest sequence
    assert L.mla_auto_split(ctypes.byref(d), 1, 1, 1) == 1
    assert L.mla_auto_split(ctypes.byref(d), 64, 1, 128) == 4


def test_append_absorb_expand_validation(L):
    d = dims()
    bd = ctypes.byref(d)
    # n_tok == 0 is a no-op
    assert L.mla_cache_append(bd, 0, None, None, None, None, None, None, None, 1, 1, 1, None,
                              None, 0, None) == 0
    assert L.mla_cache_append(bd, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None,
                              P(FAKE), 1, 4, 8, P(FAKE), P(FAKE), 1 << 30, None) == -1  # no W_KR
    assert L.mla_cache_append(bd, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE + 2), P(FAKE), P(FAKE),
                              P(FAKE), 1, 4, 8, P(FAKE), P(FAKE), 1 << 30, None) == -6
    need = L.mla_cache_append_workspace_bytes(bd, 4)
    assert need > 0
    assert L.mla_cache_append(bd, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                              P(FAKE), 1, 4, 8, P(FAKE), P(FAKE), need - 1, None) == -5
    assert L.mla_absorb_q(bd, 2, 0, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == -4
    assert L.mla_absorb_q(bd, 0, 1, None, None, None, None, None, None) == 0
    assert L.mla_absorb_q(bd, 2, 1, None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == -1
    assert L.gqla_expand(bd, 2, P(FAKE), 0, P(FAKE), 4, P(FAKE), None, P(FAKE), P(FAKE),
                         P(FAKE), None) == -4       # no blocks
    assert L.gqla_expand(bd, 2, P(FAKE), 8, P(FAKE), 4, P(FAKE), None, P(FAKE), None,
                         P(FAKE), None) == -1
    assert L.gqla_decode(bd, 2, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), 8, P(FAKE), 4, P(FAKE),
                         0, None, 0, P(FAKE), None, None) == -5


def test_status_strings(L):
    for st in M.STATUS:
        assert len(M.status_string(st)) >= 2
    assert M.status_string(12345) == "unknown status"


def test_validate_block_table(L):
    d = dims(block_size=4)
    table = torch.tensor([[3, 0, -1], [1, 2, 5]], dtype=torch.int32)
    lens = torch.tensor([6, 12], dtype=torch.int32)
    assert M.mla_validate_block_table(d, table, lens, 6) == 0
    assert M.mla_validate_block_table(d, table, lens, 5) == -8     # id 5 out of range
    bad = table.clone(); bad[1, 0] = 3
    assert M.mla_validate_block_table(d, bad, lens, 6) == -8       # block 3 used twice
    assert M.mla_validate_block_table(d, table, torch.tensor([6, 13], dtype=torch.int32), 6) == -4
    # unused entries (past ceil(L/bs)) are never looked at
    ok = table.clone(); ok[0, 2] = 99
    assert M.mla_validate_block_table(d, ok, lens, 6) == 0
    # a large random permutation table is accepted, a single collision is caught
    r = np.random.default_rng(0)
    ids = r.permutation(200_000).astype(np.int32)
    big = torch.from_numpy(ids[:131072].reshape(64, 2048).copy())
    blens = torch.full((64,), 2048 * 4, dtype=torch.int32)
    assert M.mla_validate_block_table(d, big, blens, 200_000) == 0
    big[63, 2047] = big[0, 0]
    assert M.mla_validate_block_table(d, big, blens, 200_000) == -8


def prefill_call(L, d, batch=2, s_q=300, q=FAKE, qpe=FAKE, qpos=FAKE, cache=FAKE, nb=16,
                 table=FAKE, mb=8, lens=FAKE, wuk=FAKE, wuv=FAKE, ws=None, ws_bytes=0, out=FAKE):
    dp = ctypes.byref(d) if d is not None else None
    return L.mla_prefill(dp, batch, s_q, P(q), P(qpe), P(qpos), P(cache), nb, P(table), mb,
                         P(lens), P(wuk), P(wuv), P(ws), ws_bytes, P(out), None, None)


def test_prefill_validation_and_workspace(L):
    """mla_prefill checks everything before the expansion is enqueued: a failing check leaves
    nothing launched (a half-done call would expand and then stop)."""
    d = dims()
    bd = ctypes.byref(d)
    need = L.mla_prefill_workspace_bytes(bd, 2, 300, 16, 8)
    al = lambda x: (x + 255) // 256 * 256
    kv = al(16 * 64 * (128 * (128 + 128) + 64) * 2)       # the expanded rows of 16 blocks
    assert need == kv + L.gqla_decode_workspace_bytes(bd, 2, 300, 0, 8)
    ok = dict(ws=FAKE, ws_bytes=need)
    assert prefill_call(L, None) == -1
    assert prefill_call(L, d, batch=0) == 0
    assert prefill_call(L, d, s_q=0, **ok) == -4
    assert prefill_call(L, d, ws=None) == -5
    assert prefill_call(L, d, ws=FAKE, ws_bytes=need - 1) == -5
    assert prefill_call(L, d, batch=300, s_q=300, **ok) == -5        # workspace sized for 2
    assert prefill_call(L, d, q=0, **ok) == -1
    assert prefill_call(L, d, wuv=0, **ok) == -1
    assert prefill_call(L, d, q=FAKE + 2, **ok) == -6
    assert prefill_call(L, d, out=FAKE + 8, **ok) == -6
    big = L.mla_prefill_workspace_bytes(bd, 300, 300, 16, 8)
    assert prefill_call(L, d, batch=300, s_q=300, ws=FAKE, ws_bytes=big) == -4  # B s_q > 65535


def test_layer_projection_validation(L):
    d = dims()
    bd = ctypes.byref(d)
    nq = L.mla_query_project_workspace_bytes(bd, 4, 1536)
    no = L.mla_output_project_workspace_bytes(bd, 4)
    assert nq > 0 and no > 0
    assert L.mla_query_project(bd, 0, 1536, None, None, None, None, None, None, None, None, 0,
                               None) == 0
    assert L.mla_query_project(bd, 4, 1536, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                               P(FAKE), P(FAKE), P(FAKE), nq - 1, None) == -5
    assert L.mla_query_project(bd, 4, 1536, None, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                               P(FAKE), P(FAKE), P(FAKE), nq, None) == -1
    assert L.mla_output_project(bd, 4, P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), no - 1,
                                None) == -5
    assert L.mla_output_project(bd, 4, P(FAKE + 2), P(FAKE), None, P(FAKE), P(FAKE), no,
                                None) == -6


def noalloc_call(L, d, batch=2, s_q=1, mb=4, n_split=0):
    dp = ctypes.byref(d) if d is not None else None
    return L.mla_decode_noalloc(dp, batch, s_q, P(FAKE), P(FAKE), 8, P(FAKE), mb, P(FAKE),
                                P(FAKE), n_split, P(FAKE), None, None)


def test_decode_noalloc_host_checks(L):
    """The no-workspace decode rejects what mla_decode rejects, and any batch whose partials
    would not fit its fixed device array, before it touches a device."""
    L.mla_decode_noalloc.restype = ctypes.c_int32
    d = dims()
    assert noalloc_call(L, None) == -1
    assert noalloc_call(L, d, batch=0) == 0
    assert noalloc_call(L, d, s_q=0) == -4
    assert noalloc_call(L, dims(n_groups=3)) == -2
    # 16 sequences x 128 heads x 64 uniform splits of bf16 partials: 134 MB > 36 MiB
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 16, 1, 64, 4096)
    assert need > M.MLA_NOALLOC_SCRATCH_BYTES
    assert noalloc_call(L, d, batch=16, mb=4096, n_split=64) == -5
    # the largest workload shapes fit: long context (4 x 64 splits) and the balanced plan
    assert L.mla_decode_workspace_bytes(ctypes.byref(d), 4, 1, 64, 2048) <= M.MLA_NOALLOC_SCRATCH_BYTES
    assert L.mla_decode_workspace_bytes(ctypes.byref(d), 32, 4, 0, 512) <= M.MLA_NOALLOC_SCRATCH_BYTES


def fp8_decode_call(L, d, scales=FAKE, ws=FAKE, ws_bytes=1 << 30, batch=2):
    return L.mla_decode_fp8(ctypes.byref(d), batch, 1, P(FAKE), P(FAKE), P(scales), 8, P(FAKE),
                            4, P(FAKE), P(FAKE), 0, P(ws), ws_bytes, P(FAKE), None, None)


def test_fp8_host_checks(L):
    """The e4m3 calls refuse, before launch, shapes their kernels do not cover (H != 128, the
    portable-kernel flag, fp32 dims, rows not a multiple of 16 bytes) and missing or misaligned
    scales; empty calls do nothing."""
    d = dims()
    assert fp8_decode_call(L, d, batch=0) == 0
    assert fp8_decode_call(L, dims(n_heads=64, n_groups=64)) == -2
    assert fp8_decode_call(L, dims(dtype="f32")) == -2
    assert fp8_decode_call(L, M.make_dims(7168, 128, 128, 128, 512, 64, 128, 64, "bf16",
                                          generic=True)) == -2
    assert fp8_decode_call(L, d, scales=0) == -1
    assert fp8_decode_call(L, d, scales=FAKE + 4) == -6
    assert fp8_decode_call(L, d, ws=None, ws_bytes=0) == -5
    assert L.mla_decode_fp8_splitk(ctypes.byref(d), 2, 1, P(FAKE), P(FAKE), None, 8, P(FAKE), 4,
                                   P(FAKE), 0, P(FAKE), 1 << 30, None) == -1
    assert L.mla_decode_fp8_merge(ctypes.byref(dims(block_size=48)), 2, 1, P(FAKE), P(FAKE),
                                  P(FAKE), 8, P(FAKE), 4, P(FAKE), P(FAKE), 0, P(FAKE), 1 << 30,
                                  P(FAKE), None, None) == -2
    # quantisation: rows of d_c + d_r values, 16-byte multiples of at most 1024
    qd = ctypes.byref(d)
    assert L.mla_cache_quantize_fp8(qd, 0, None, None, None, None) == 0
    assert L.mla_cache_quantize_fp8(qd, -1, P(FAKE), P(FAKE), P(FAKE), None) == -4
    assert L.mla_cache_quantize_fp8(qd, 4, P(FAKE), None, P(FAKE), None) == -1
    assert L.mla_cache_quantize_fp8(qd, 4, P(FAKE), P(FAKE), P(FAKE + 4), None) == -6
    assert L.mla_cache_quantize_fp8(ctypes.byref(dims(d_c=504)), 4, P(FAKE), P(FAKE), P(FAKE),
                                    None) == -2
    assert L.mla_cache_quantize_fp8(ctypes.byref(dims(dtype="f32")), 4, P(FAKE), P(FAKE),
                                    P(FAKE), None) == -2
    # append: the scales are required once there is a token to write
    need = L.mla_cache_append_workspace_bytes(qd, 4)
    assert L.mla_cache_append_fp8(qd, 0, None, None, None, None, None, None, None, 1, 1, 1, None,
                                  None, None, 0, None) == 0
    assert L.mla_cache_append_fp8(qd, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                  P(FAKE), 1, 4, 8, P(FAKE), None, P(FAKE), need, None) == -1
    assert L.mla_cache_append_fp8(qd, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                  P(FAKE), 1, 4, 8, P(FAKE), P(FAKE), P(FAKE), need - 1,
                                  None) == -5
    assert L.mla_cache_append_absorb_q_fp8(
        ctypes.byref(dims(d_r=40)), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
        P(FAKE), 1, 4, 8, P(FAKE), P(FAKE), P(FAKE), need, 1, P(FAKE), P(FAKE), P(FAKE),
        P(FAKE), P(FAKE), None) == -2                       # 552 values: not 16-byte rows


def test_decode_step_host_checks(L):
    """mla_decode_step refuses what its component calls refuse, and a short workspace, before
    anything is launched; an empty batch does nothing."""
    d = dims()
    dp = ctypes.byref(d)
    need = L.mla_decode_step_workspace_bytes(dp, 4, 1, 64, 2048)
    dec = L.mla_decode_workspace_bytes(dp, 4, 1, 64, 2048)
    assert need > dec > 0

    def call(dd=d, batch=4, s_q=1, x=FAKE, gamma=FAKE, w_uv=FAKE, ws=FAKE, ws_bytes=need,
             out=FAKE, n_split=64):
        return L.mla_decode_step(ctypes.byref(dd), batch, s_q, P(x), P(FAKE), P(gamma), P(FAKE),
                                 P(FAKE), P(FAKE), P(FAKE), P(w_uv), P(FAKE), 8192, P(FAKE),
                                 2048, P(FAKE), n_split, P(ws), ws_bytes, P(out), None, None)
    assert call(batch=0) == 0
    assert call(s_q=0) == -4
    assert call(n_split=M.MLA_MAX_SPLIT + 1) == -4
    assert call(ws_bytes=need - 1) == -5
    assert call(ws=None) == -1
    assert call(x=None) == -1                       # the append's input
    assert call(gamma=None) == -1
    assert call(w_uv=None) == -1
    assert call(out=FAKE + 4) == -6
    assert call(dd=dims(n_groups=3)) == -2


def test_decode_step_fp8_host_checks(L):
    """mla_decode_step_fp8 refuses what mla_decode_step and the e4m3 decode refuse (shapes
    without an e4m3 core, a missing or misaligned scale array), before anything is launched."""
    d = dims()
    dp = ctypes.byref(d)
    need = L.mla_decode_step_workspace_bytes(dp, 4, 1, 64, 2048)

    def call(dd=d, batch=4, x=FAKE, scale=FAKE, ws=FAKE, ws_bytes=need, n_split=64):
        return L.mla_decode_step_fp8(ctypes.byref(dd), batch, 1, P(x), P(FAKE), P(FAKE), P(FAKE),
                                     P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(scale), 8192,
                                     P(FAKE), 2048, P(FAKE), n_split, P(ws), ws_bytes, P(FAKE),
                                     None, None)
    assert call(batch=0) == 0
    assert call(scale=None) == -1
    assert call(scale=FAKE + 4) == -6
    assert call(ws_bytes=need - 1) == -5
    assert call(x=None) == -1
    assert call(n_split=M.MLA_MAX_SPLIT + 1) == -4
    assert call(dd=dims(n_heads=32, n_groups=32)) == -2            # no e4m3 core for H = 32
    assert call(dd=dims(generic=True)) == -2
