"""ctypes binding of libmla.so: the C ABI of include/mla.h under the same names.

Argument marshalling only: tensors become device pointers, the current torch stream becomes
the hipStream_t, and a non-OK status becomes an MlaError. Every step of the decode path runs
in the library's HIP kernels; if the library is missing this module raises instead of
computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB overrides the library path (the host-sanitizer test loads an instrumented build).
LIB_PATH = os.environ.get("MLA_LIB") or os.path.join(_HERE, "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
MLA_FLAG_GENERIC_KERNELS = 1
MLA_MAX_SPLIT = 256
MLA_NOALLOC_SCRATCH_BYTES = 36 << 20
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_RANGE", -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_ALIGN", -7: "MLA_ERR_HIP",
          -8: "MLA_ERR_BLOCK_TABLE"}
EXPORTS = ["mla_cache_append_workspace_bytes", "mla_cache_append", "mla_absorb_q",
           "mla_cache_append_absorb_q",
           "mla_query_project_workspace_bytes", "mla_query_project",
           "mla_output_project_workspace_bytes", "mla_output_project",
           "mla_decode_workspace_bytes", "mla_decode", "mla_decode_splitk", "mla_decode_merge",
           "mla_decode_noalloc", "mla_decode_step_workspace_bytes", "mla_decode_step",
           "mla_cache_quantize_fp8", "mla_cache_append_fp8", "mla_cache_append_absorb_q_fp8",
           "mla_decode_fp8", "mla_decode_fp8_splitk", "mla_decode_fp8_merge",
           "mla_decode_step_fp8", "gqla_expand",
           "gqla_decode_workspace_bytes", "gqla_decode",
           "mla_prefill_workspace_bytes", "mla_prefill", "mla_auto_split", "mla_select_path",
           "mla_status_string",
           "mla_validate_block_table"]


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class MlaDims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("d_r", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float)]


def make_dims(d_model, n_heads, d_nope, d_v, d_c, d_r, n_groups, block_size, dtype,
              rope_base=10000.0, rms_eps=1e-6, softmax_scale=0.0, generic=False) -> MlaDims:
    dt = {"f32": MLA_F32, "bf16": MLA_BF16, torch.float32: MLA_F32,
          torch.bfloat16: MLA_BF16}.get(dtype, dtype)
    return MlaDims(d_model, n_heads, d_nope, d_v, d_c, d_r, n_groups, block_size, dt,
                   MLA_FLAG_GENERIC_KERNELS if generic else 0, rope_base, rms_eps,
                   softmax_scale)


def dims_of(w, generic: bool = False, **kw) -> MlaDims:
    """mla_dims of a workloads.Workload."""
    return make_dims(w.d_model, w.n_heads, w.d_nope, w.d_v, w.d_c, w.d_r, w.n_groups,
                     w.block_size, w.dtype, generic=generic, **kw)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(or python mla_latent_kv_21_amd/build.py) first")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.POINTER(MlaDims)
        sig = {
            "mla_cache_append_workspace_bytes": (S, [D, I]),
            "mla_cache_append": (I, [D, I, P, P, P, P, P, P, P, I, I, I, P, P, S, P]),
            "mla_absorb_q": (I, [D, I, I, P, P, P, P, P, P]),
            "mla_cache_append_absorb_q": (I, [D, I, P, P, P, P, P, P, P, I, I, I, P, P, S, I, P,
                                              P, P, P, P, P]),
            "mla_query_project_workspace_bytes": (S, [D, I, I]),
            "mla_query_project": (I, [D, I, I, P, P, P, P, P, P, P, P, S, P]),
            "mla_output_project_workspace_bytes": (S, [D, I]),
            "mla_output_project": (I, [D, I, P, P, P, P, P, S, P]),
            "mla_decode_workspace_bytes": (S, [D, I, I, I, I]),
            "mla_decode": (I, [D, I, I, P, P, I, P, I, P, P, I, P, S, P, P, P]),
            "mla_decode_splitk": (I, [D, I, I, P, P, I, P, I, P, I, P, S, P]),
            "mla_decode_merge": (I, [D, I, I, P, P, I, P, I, P, P, I, P, S, P, P, P]),
            "mla_decode_noalloc": (I, [D, I, I, P, P, I, P, I, P, P, I, P, P, P]),
            "mla_decode_step_workspace_bytes": (S, [D, I, I, I, I]),
            "mla_decode_step": (I, [D, I, I, P, P, P, P, P, P, P, P, P, I, P, I, P, I, P, S, P,
                                    P, P]),
            "mla_decode_step_fp8": (I, [D, I, I, P, P, P, P, P, P, P, P, P, P, I, P, I, P, I, P,
                                        S, P, P, P]),
            "mla_cache_quantize_fp8": (I, [D, ctypes.c_int64, P, P, P, P]),
            "mla_cache_append_fp8": (I, [D, I, P, P, P, P, P, P, P, I, I, I, P, P, P, S, P]),
            "mla_cache_append_absorb_q_fp8": (I, [D, I, P, P, P, P, P, P, P, I, I, I, P, P, P, S,
                                                  I, P, P, P, P, P, P]),
            "mla_decode_fp8": (I, [D, I, I, P, P, P, I, P, I, P, P, I, P, S, P, P, P]),
            "mla_decode_fp8_splitk": (I, [D, I, I, P, P, P, I, P, I, P, I, P, S, P]),
            "mla_decode_fp8_merge": (I, [D, I, I, P, P, P, I, P, I, P, P, I, P, S, P, P, P]),
            "gqla_expand": (I, [D, I, P, I, P, I, P, P, P, P, P, P]),
            "gqla_decode_workspace_bytes": (S, [D, I, I, I, I]),
            "gqla_decode": (I, [D, I, I, P, P, P, P, I, P, I, P, I, P, S, P, P, P]),
            "mla_prefill_workspace_bytes": (S, [D, I, I, I, I]),
            "mla_prefill": (I, [D, I, I, P, P, P, P, I, P, I, P, P, P, P, S, P, P, P]),
            "mla_auto_split": (I, [D, I, I, I]),
            "mla_select_path": (I, [D, I, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                    ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]),
            "mla_status_string": (ctypes.c_char_p, [I]),
            "mla_validate_block_table": (I, [D, P, I, I, P, I]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmla must be contiguous")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(st: int, what: str):
    if st != 0:
        raise MlaError(st, what)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- entry points
def mla_cache_append_workspace_bytes(dims: MlaDims, n_tok: int) -> int:
    return lib().mla_cache_append_workspace_bytes(ctypes.byref(dims), n_tok)


def mla_cache_append(dims, x, seq_idx, pos, w_dkv, gamma, w_kr, block_table, num_blocks,
                     latent_cache, workspace=None):
    n_tok = x.shape[0]
    if workspace is None:
        workspace = _workspace(mla_cache_append_workspace_bytes(dims, n_tok), x.device)
    st = lib().mla_cache_append(ctypes.byref(dims), n_tok, _ptr(x), _ptr(seq_idx), _ptr(pos),
                                _ptr(w_dkv), _ptr(gamma), _ptr(w_kr), _ptr(block_table),
                                block_table.shape[0], block_table.shape[1], num_blocks,
                                _ptr(latent_cache), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "mla_cache_append")


def mla_cache_append_absorb_q(dims, x, seq_idx, pos, w_dkv, gamma, w_kr, block_table,
                              num_blocks, latent_cache, q_nope, q_pe, q_pos, w_uk, q_abs,
                              workspace=None):
    """mla_cache_append then mla_absorb_q (the absorption in the projection's launch)."""
    n_tok = x.shape[0]
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    if block_table.shape[0] != B:
        raise ValueError("the block table's rows and the query batch must agree")
    if workspace is None:
        workspace = _workspace(mla_cache_append_workspace_bytes(dims, n_tok), x.device)
    st = lib().mla_cache_append_absorb_q(
        ctypes.byref(dims), n_tok, _ptr(x), _ptr(seq_idx), _ptr(pos), _ptr(w_dkv), _ptr(gamma),
        _ptr(w_kr), _ptr(block_table), B, block_table.shape[1], num_blocks, _ptr(latent_cache),
        _ptr(workspace), workspace.numel(), s_q, _ptr(q_nope), _ptr(q_pe), _ptr(q_pos),
        _ptr(w_uk), _ptr(q_abs), _stream())
    _check(st, "mla_cache_append_absorb_q")


def mla_query_project_workspace_bytes(dims, n_tok, d_q) -> int:
    return lib().mla_query_project_workspace_bytes(ctypes.byref(dims), n_tok, d_q)


def mla_output_project_workspace_bytes(dims, n_tok) -> int:
    return lib().mla_output_project_workspace_bytes(ctypes.byref(dims), n_tok)


def mla_query_project(dims, x, w_dq, gamma_q, w_uq, w_qr, q_nope, q_pe, workspace=None):
    n_tok, d_q = x.shape[0], w_dq.shape[1]
    if workspace is None:
        workspace = _workspace(mla_query_project_workspace_bytes(dims, n_tok, d_q), x.device)
    st = lib().mla_query_project(ctypes.byref(dims), n_tok, d_q, _ptr(x), _ptr(w_dq),
                                 _ptr(gamma_q), _ptr(w_uq), _ptr(w_qr), _ptr(q_nope), _ptr(q_pe),
                                 _ptr(workspace), workspace.numel(), _stream())
    _check(st, "mla_query_project")


def mla_output_project(dims, o, w_o, b_o, y, workspace=None):
    n_tok = o.shape[0]
    if workspace is None:
        workspace = _workspace(mla_output_project_workspace_bytes(dims, n_tok), o.device)
    st = lib().mla_output_project(ctypes.byref(dims), n_tok, _ptr(o), _ptr(w_o), _ptr(b_o),
                                  _ptr(y), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "mla_output_project")


def mla_absorb_q(dims, q_nope, q_pe, q_pos, w_uk, q_abs):
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    st = lib().mla_absorb_q(ctypes.byref(dims), B, s_q, _ptr(q_nope), _ptr(q_pe), _ptr(q_pos),
                            _ptr(w_uk), _ptr(q_abs), _stream())
    _check(st, "mla_absorb_q")


def mla_auto_split(dims, batch, s_q, max_blocks) -> int:
    return lib().mla_auto_split(ctypes.byref(dims), batch, s_q, max_blocks)


MLA_PATH_ABSORBED, MLA_PATH_GQA = 0, 1


def mla_select_path(dims, s_q, context, hbm_bytes_per_s=0.0, flops_per_s=0.0):
    """(path, t_absorbed, t_gqa): the cheaper decode path by the roofline of each, and both
    times in seconds per query step of one sequence. Rates 0, 0 mean MI355X."""
    ta, tg = ctypes.c_double(), ctypes.c_double()
    r = lib().mla_select_path(ctypes.byref(dims), s_q, context, hbm_bytes_per_s, flops_per_s,
                              ctypes.byref(ta), ctypes.byref(tg))
    _check(r if r < 0 else 0, "mla_select_path")
    return r, ta.value, tg.value


def mla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks) -> int:
    return lib().mla_decode_workspace_bytes(ctypes.byref(dims), batch, s_q, n_split, max_blocks)


def mla_decode(dims, q_abs, latent_cache, block_table, seq_lens, w_uv, out, lse=None,
               n_split=0, workspace=None):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    mb = block_table.shape[1]
    if workspace is None:
        workspace = _workspace(mla_decode_workspace_bytes(dims, B, s_q, n_split, mb), q_abs.device)
    st = lib().mla_decode(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(latent_cache),
                          latent_cache.shape[0], _ptr(block_table), mb, _ptr(seq_lens),
                          _ptr(w_uv), n_split, _ptr(workspace), workspace.numel(), _ptr(out),
                          _ptr(lse), _stream())
    _check(st, "mla_decode")


def mla_decode_noalloc(dims, q_abs, latent_cache, block_table, seq_lens, w_uv, out, lse=None,
                       n_split=0):
    """mla_decode with its partials in the library's own device array (no workspace)."""
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    st = lib().mla_decode_noalloc(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(latent_cache),
                                  latent_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                  _ptr(seq_lens), _ptr(w_uv), n_split, _ptr(out), _ptr(lse),
                                  _stream())
    _check(st, "mla_decode_noalloc")


def mla_decode_step_workspace_bytes(dims, batch, s_q, n_split, max_blocks) -> int:
    return lib().mla_decode_step_workspace_bytes(ctypes.byref(dims), batch, s_q, n_split,
                                                 max_blocks)


def mla_decode_step(dims, x, w_dkv, gamma, w_kr, q_nope, q_pe, w_uk, w_uv, latent_cache,
                    block_table, seq_lens, out, lse=None, n_split=0, workspace=None):
    """One decode step: append the s_q new tokens of every sequence (its last s_q positions),
    absorb their queries, decode; out [B, s_q, H, D_v]."""
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    mb = block_table.shape[1]
    if x.shape[0] != B * s_q or block_table.shape[0] != B:
        raise ValueError("x must hold B * s_q tokens and the block table B rows")
    if workspace is None:
        workspace = _workspace(mla_decode_step_workspace_bytes(dims, B, s_q, n_split, mb),
                               x.device)
    st = lib().mla_decode_step(ctypes.byref(dims), B, s_q, _ptr(x), _ptr(w_dkv), _ptr(gamma),
                               _ptr(w_kr), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
                               _ptr(latent_cache), latent_cache.shape[0], _ptr(block_table), mb,
                               _ptr(seq_lens), n_split, _ptr(workspace), workspace.numel(),
                               _ptr(out), _ptr(lse), _stream())
    _check(st, "mla_decode_step")


def mla_decode_step_fp8(dims, x, w_dkv, gamma, w_kr, q_nope, q_pe, w_uk, w_uv, cache_fp8,
                        cache_scale, block_table, seq_lens, out, lse=None, n_split=0,
                        workspace=None):
    """mla_decode_step over an e4m3 cache (bytes [num_blocks, bs, d_c + d_r], scales
    [num_blocks, bs])."""
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    mb = block_table.shape[1]
    if x.shape[0] != B * s_q or block_table.shape[0] != B:
        raise ValueError("x must hold B * s_q tokens and the block table B rows")
    if workspace is None:
        workspace = _workspace(mla_decode_step_workspace_bytes(dims, B, s_q, n_split, mb),
                               x.device)
    st = lib().mla_decode_step_fp8(ctypes.byref(dims), B, s_q, _ptr(x), _ptr(w_dkv), _ptr(gamma),
                                   _ptr(w_kr), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
                                   _ptr(cache_fp8), _ptr(cache_scale), cache_fp8.shape[0],
                                   _ptr(block_table), mb, _ptr(seq_lens), n_split,
                                   _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                   _stream())
    _check(st, "mla_decode_step_fp8")


def mla_decode_splitk(dims, q_abs, latent_cache, block_table, seq_lens, n_split, workspace):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    st = lib().mla_decode_splitk(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(latent_cache),
                                 latent_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                 _ptr(seq_lens), n_split, _ptr(workspace), workspace.numel(),
                                 _stream())
    _check(st, "mla_decode_splitk")


def mla_decode_merge(dims, q_abs, latent_cache, block_table, seq_lens, w_uv, out, lse, n_split,
                     workspace):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    st = lib().mla_decode_merge(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(latent_cache),
                                latent_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                _ptr(seq_lens), _ptr(w_uv), n_split, _ptr(workspace),
                                workspace.numel(), _ptr(out), _ptr(lse), _stream())
    _check(st, "mla_decode_merge")


# ---- e4m3 latent cache: uint8 rows [num_blocks, bs, d_c + d_r] and fp32 scales [num_blocks, bs]
def mla_cache_quantize_fp8(dims, rows, rows_fp8, row_scale):
    """bf16 rows [..., d_c + d_r] to e4m3 bytes of the same shape and one scale per row."""
    n = row_scale.numel()
    if rows.numel() != n * (dims.d_c + dims.d_r) or rows_fp8.numel() != rows.numel():
        raise ValueError("rows, rows_fp8 and row_scale disagree")
    st = lib().mla_cache_quantize_fp8(ctypes.byref(dims), n, _ptr(rows), _ptr(rows_fp8),
                                      _ptr(row_scale), _stream())
    _check(st, "mla_cache_quantize_fp8")


def mla_cache_append_fp8(dims, x, seq_idx, pos, w_dkv, gamma, w_kr, block_table, num_blocks,
                         cache_fp8, cache_scale, workspace=None):
    n_tok = x.shape[0]
    if workspace is None:
        workspace = _workspace(mla_cache_append_workspace_bytes(dims, n_tok), x.device)
    st = lib().mla_cache_append_fp8(
        ctypes.byref(dims), n_tok, _ptr(x), _ptr(seq_idx), _ptr(pos), _ptr(w_dkv), _ptr(gamma),
        _ptr(w_kr), _ptr(block_table), block_table.shape[0], block_table.shape[1], num_blocks,
        _ptr(cache_fp8), _ptr(cache_scale), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "mla_cache_append_fp8")


def mla_cache_append_absorb_q_fp8(dims, x, seq_idx, pos, w_dkv, gamma, w_kr, block_table,
                                  num_blocks, cache_fp8, cache_scale, q_nope, q_pe, q_pos, w_uk,
                                  q_abs, workspace=None):
    n_tok = x.shape[0]
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    if block_table.shape[0] != B:
        raise ValueError("the block table's rows and the query batch must agree")
    if workspace is None:
        workspace = _workspace(mla_cache_append_workspace_bytes(dims, n_tok), x.device)
    st = lib().mla_cache_append_absorb_q_fp8(
        ctypes.byref(dims), n_tok, _ptr(x), _ptr(seq_idx), _ptr(pos), _ptr(w_dkv), _ptr(gamma),
        _ptr(w_kr), _ptr(block_table), B, block_table.shape[1], num_blocks, _ptr(cache_fp8),
        _ptr(cache_scale), _ptr(workspace), workspace.numel(), s_q, _ptr(q_nope), _ptr(q_pe),
        _ptr(q_pos), _ptr(w_uk), _ptr(q_abs), _stream())
    _check(st, "mla_cache_append_absorb_q_fp8")


def mla_decode_fp8(dims, q_abs, cache_fp8, cache_scale, block_table, seq_lens, w_uv, out,
                   lse=None, n_split=0, workspace=None):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    mb = block_table.shape[1]
    if workspace is None:
        workspace = _workspace(mla_decode_workspace_bytes(dims, B, s_q, n_split, mb), q_abs.device)
    st = lib().mla_decode_fp8(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(cache_fp8),
                              _ptr(cache_scale), cache_fp8.shape[0], _ptr(block_table), mb,
                              _ptr(seq_lens), _ptr(w_uv), n_split, _ptr(workspace),
                              workspace.numel(), _ptr(out), _ptr(lse), _stream())
    _check(st, "mla_decode_fp8")


def mla_decode_fp8_splitk(dims, q_abs, cache_fp8, cache_scale, block_table, seq_lens, n_split,
                          workspace):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    st = lib().mla_decode_fp8_splitk(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(cache_fp8),
                                     _ptr(cache_scale), cache_fp8.shape[0], _ptr(block_table),
                                     block_table.shape[1], _ptr(seq_lens), n_split,
                                     _ptr(workspace), workspace.numel(), _stream())
    _check(st, "mla_decode_fp8_splitk")


def mla_decode_fp8_merge(dims, q_abs, cache_fp8, cache_scale, block_table, seq_lens, w_uv, out,
                         lse, n_split, workspace):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    st = lib().mla_decode_fp8_merge(ctypes.byref(dims), B, s_q, _ptr(q_abs), _ptr(cache_fp8),
                                    _ptr(cache_scale), cache_fp8.shape[0], _ptr(block_table),
                                    block_table.shape[1], _ptr(seq_lens), _ptr(w_uv), n_split,
                                    _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                    _stream())
    _check(st, "mla_decode_fp8_merge")


def gqla_expand(dims, latent_cache, block_table, seq_lens, w_uk, w_uv, gqa_cache,
                start_pos=None):
    st = lib().gqla_expand(ctypes.byref(dims), block_table.shape[0], _ptr(latent_cache),
                           latent_cache.shape[0], _ptr(block_table), block_table.shape[1],
                           _ptr(seq_lens), _ptr(start_pos), _ptr(w_uk), _ptr(w_uv),
                           _ptr(gqa_cache), _stream())
    _check(st, "gqla_expand")


def gqla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks) -> int:
    return lib().gqla_decode_workspace_bytes(ctypes.byref(dims), batch, s_q, n_split, max_blocks)


def gqla_decode(dims, q_nope, q_pe, q_pos, gqa_cache, block_table, seq_lens, out, lse=None,
                n_split=0, workspace=None):
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    mb = block_table.shape[1]
    if workspace is None:
        workspace = _workspace(gqla_decode_workspace_bytes(dims, B, s_q, n_split, mb),
                               q_nope.device)
    st = lib().gqla_decode(ctypes.byref(dims), B, s_q, _ptr(q_nope), _ptr(q_pe), _ptr(q_pos),
                           _ptr(gqa_cache), gqa_cache.shape[0], _ptr(block_table), mb,
                           _ptr(seq_lens), n_split, _ptr(workspace), workspace.numel(),
                           _ptr(out), _ptr(lse), _stream())
    _check(st, "gqla_decode")


def mla_prefill_workspace_bytes(dims, batch, s_q, num_blocks, max_blocks) -> int:
    return lib().mla_prefill_workspace_bytes(ctypes.byref(dims), batch, s_q, num_blocks,
                                             max_blocks)


def mla_prefill(dims, q_nope, q_pe, q_pos, latent_cache, block_table, seq_lens, w_uk, w_uv,
                out, lse=None, workspace=None):
    B, s_q = q_nope.shape[0], q_nope.shape[1]
    nb, mb = latent_cache.shape[0], block_table.shape[1]
    if workspace is None:
        workspace = _workspace(mla_prefill_workspace_bytes(dims, B, s_q, nb, mb), q_nope.device)
    st = lib().mla_prefill(ctypes.byref(dims), B, s_q, _ptr(q_nope), _ptr(q_pe), _ptr(q_pos),
                           _ptr(latent_cache), nb, _ptr(block_table), mb, _ptr(seq_lens),
                           _ptr(w_uk), _ptr(w_uv), _ptr(workspace), workspace.numel(),
                           _ptr(out), _ptr(lse), _stream())
    _check(st, "mla_prefill")


def mla_validate_block_table(dims, table_host: torch.Tensor, seq_lens_host: torch.Tensor,
                             num_blocks: int) -> int:
    """Host check of a CPU int32 block table; returns the status code."""
    t = table_host.contiguous()
    s = seq_lens_host.contiguous()
    return lib().mla_validate_block_table(ctypes.byref(dims), t.data_ptr(), t.shape[0],
                                          t.shape[1], s.data_ptr(), num_blocks)


def status_string(st: int) -> str:
    return lib().mla_status_string(st).decode()
