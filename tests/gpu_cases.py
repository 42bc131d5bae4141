"""Shared builders for the GPU parity tests: seeded inputs (workloads), library calls through
the C ABI (binding) and expected values from the oracle, on the same input bits."""
import os

import numpy as np
import torch

import oracle as O
import workloads as W
from mla_latent_kv_21_amd import binding as M

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str):
    print(f"[case] {msg}", flush=True)


def stream_tag(w) -> int:
    """A small per-workload number that keeps the case generators' random streams apart."""
    return w.seed % 100


def rel_err(y, ref) -> float:
    """Normwise error max|y - ref| / max|ref| over a whole tensor."""
    y, ref = O.f64(y), O.f64(ref)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), "non-finite values in the GPU result"
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-30))


def row_errors(y, ref) -> np.ndarray:
    """Per-row error max_j|y_j - ref_j| / max_j|ref_j| over the last axis (one row per query
    and head of an output, or per position of cache rows)."""
    y, ref = O.f64(y), O.f64(ref)
    num = np.max(np.abs(y - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return num / den


def check(y, ref, tol: float, what: str = "") -> float:
    """Assert the normwise error of y against ref is within tol, and print it with the worst
    row's error and index so that the margin under the bound is on record."""
    err = rel_err(y, ref)
    rows = row_errors(y, ref)
    worst = np.unravel_index(int(np.argmax(rows)), rows.shape) if rows.size else ()
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    print(f"[err] {test} {what} normwise={err:.3e} worst_row={float(np.max(rows)):.3e} "
          f"at {tuple(int(i) for i in worst)} tol={tol:.0e}", flush=True)
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol}"
    return err


def check_lse(got, ref, tol: float, what: str = "lse") -> float:
    """Absolute error of log-sum-exps (natural log), printed and held to tol."""
    got, ref = O.f64(got), O.f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = float(np.max(np.abs(got - ref)))
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    print(f"[err] {test} {what} abs={err:.3e} tol={tol:.0e}", flush=True)
    assert err <= tol, f"{what}: error {err:.3e} > {tol}"
    return err


def check_per_seq(y, ref, tol: float, what: str = "out"):
    """check() on each sequence (axis 0) of a batch separately."""
    for b in range(len(ref)):
        check(y[b], ref[b], tol, f"{what}[seq {b}]")


def dev(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(t)).to(DEV)


# ----------------------------------------------------------------------------- decode cases
def decode_case(w, lens, s_q=1, random_table=True, poison=True, extra=0, max_blocks=None):
    lens = np.asarray(lens, np.int32)
    wq = w.replace(batch=len(lens), s_q=s_q)
    table, nb = W.block_table(wq, lens, random=random_table, max_blocks=max_blocks)
    pool = W.cache_pool(wq, nb, extra=extra)
    if poison:
        mask = O.owned_slot_mask(table, lens, nb, w.block_size)
        pool.view(-1, w.row)[torch.from_numpy(~mask)] = float("nan")
    return dict(w=wq, lens=lens, table=table, nb=nb, pool=pool, q_abs=W.absorbed_queries(wq),
                w_uv=W.weights(wq)["w_uv"])


def decode_ws_layout(c, n_split):
    w = c["w"]
    rows = w.batch * w.s_q * w.n_heads * n_split
    al = lambda x: (x + 255) // 256 * 256
    off_flags = al(rows * w.d_c * w.elt) + al(rows * 4)  # partial rows at the cache dtype
    return off_flags, w.batch * w.s_q * n_split


PLAN_SLOTS, PLAN_BYTES = 256, 1024   # the length-balanced plan's slots and workspace reserve


def planned_layout(c):
    """(byte offset, count) of the recompute flags of a planned decode's workspace."""
    w = c["w"]
    rows = PLAN_SLOTS * w.n_heads
    al = lambda x: (x + 255) // 256 * 256
    return PLAN_BYTES + al(rows * w.d_c * w.elt) + al(rows * 4), PLAN_SLOTS


def run_decode(c, n_split=0, generic=False, gpu=None, planned=False, ws_out=None):
    """mla_decode on the GPU; returns (out, lse, recompute flags) on the host. planned: pass
    n_split = 0 through, so that the library plans the splits from the lengths (the flags
    returned are those of the plan's slots)."""
    w = c["w"]
    d = M.dims_of(w, generic=generic)
    g = gpu or {}
    q = g.get("q") if "q" in g else dev(c["q_abs"])
    pool = g.get("pool") if "pool" in g else dev(c["pool"])
    tab = dev(c["table"])
    lens = dev(c["lens"])
    wuv = dev(c["w_uv"])
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    lse = torch.empty(w.batch, w.s_q, w.n_heads, dtype=torch.float32, device=DEV)
    ns = 0 if planned else n_split or M.mla_auto_split(d, w.batch, w.s_q, c["table"].shape[1])
    ws = torch.zeros(M.mla_decode_workspace_bytes(d, w.batch, w.s_q, ns, c["table"].shape[1]),
                     dtype=torch.uint8, device=DEV)
    M.mla_decode(d, q, pool, tab, lens, wuv, out, lse, n_split=ns, workspace=ws)
    torch.cuda.synchronize()
    if ws_out is not None:
        ws_out.append(ws.cpu())
    off, n = planned_layout(c) if planned else decode_ws_layout(c, ns)
    if off + 4 * n > ws.numel():  # n_split = 0 took the uniform split: no planned flags
        return out.cpu(), lse.cpu(), np.zeros(0, np.int32)
    flags = ws[off:off + 4 * n].view(torch.int32).cpu().numpy().copy()
    return out.cpu(), lse.cpu(), flags


def oracle_decode(c, seqs=None, heads=None):
    """Expected (out [b, s_q, h, D_v], lse) of the absorbed definition, from the same bits."""
    w = c["w"]
    seqs = range(w.batch) if seqs is None else seqs
    scale = O.softmax_scale(w.d_nope, w.d_r)
    outs, lses = [], []
    for b in seqs:
        rows = O.gather_rows(c["pool"], c["table"], b, int(c["lens"][b]))
        o_lat, lse = O.decode_absorbed_latent(c["q_abs"][b], rows, w.d_c, scale, heads=heads)
        outs.append(O.project_values(o_lat, c["w_uv"], w.n_groups, w.d_v, n_heads=w.n_heads,
                                     heads=heads))
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def pick(t, seqs, heads):
    t = O.f64(t)
    t = t[list(seqs)]
    return t[:, :, list(heads)] if heads is not None else t
