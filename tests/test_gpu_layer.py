"""GPU parity of the decode layer around the attention path: mla_query_project (query_down,
query_norm, query_up, query_rope) and mla_output_project (proj) against the oracle, and the
whole layer x -> q -> absorb -> append -> decode -> proj against the oracle's reconstruction."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_cases import (DEV, TOL, check, dev, note)
from mla_latent_kv_21_amd import binding as M

pytestmark = pytest.mark.gpu

BASE, EPS = 10000.0, 1e-6


def store(a, w):
    return O.round_storage(a, w.dtype)


def gpu_query_project(w, x, lw):
    n = x.shape[0]
    d = M.dims_of(w)
    q_nope = torch.empty(n, w.n_heads, w.d_nope, dtype=w.torch_dtype, device=DEV)
    q_pe = torch.empty(n, w.n_heads, w.d_r, dtype=w.torch_dtype, device=DEV)
    M.mla_query_project(d, dev(x), dev(lw["w_dq"]), dev(lw["gamma_q"]), dev(lw["w_uq"]),
                        dev(lw["w_qr"]), q_nope, q_pe)
    return q_nope, q_pe


@pytest.mark.parametrize("wl", ["smallem-fp32", "mid-bf16", "dsv3-paged"])
@pytest.mark.parametrize("n_tok", [1, 5, 33])
def test_query_project_matches_oracle(wl, n_tok):
    w = W.WORKLOADS[wl]
    x = W.tokens(w, n_tok, extra=7)
    lw = W.layer_weights(w)
    note(f"query project {wl} n_tok={n_tok}")
    q_nope, q_pe = gpu_query_project(w, x, lw)
    torch.cuda.synchronize()
    rn, rp = O.query_project(x, lw["w_dq"], lw["gamma_q"], lw["w_uq"], lw["w_qr"], EPS,
                             round_cq=lambda a: store(a, w))
    check(q_nope.cpu().view(n_tok, -1), rn, TOL[w.dtype])
    check(q_pe.cpu().view(n_tok, -1), rp, TOL[w.dtype])


@pytest.mark.parametrize("wl", ["smallem-fp32", "mid-bf16", "dsv3-paged"])
@pytest.mark.parametrize("n_tok,bias", [(1, True), (4, False), (40, True)])
def test_output_project_matches_oracle(wl, n_tok, bias):
    w = W.WORKLOADS[wl]
    o = W.head_outputs(w, n_tok)
    lw = W.layer_weights(w)
    b = lw["b_o"] if bias else None
    d = M.dims_of(w)
    y = torch.empty(n_tok, w.d_model, dtype=w.torch_dtype, device=DEV)
    note(f"output project {wl} n_tok={n_tok} bias={bias}")
    M.mla_output_project(d, dev(o), dev(lw["w_o"]), None if b is None else dev(b), y)
    torch.cuda.synchronize()
    check(y.cpu(), O.output_project(o, lw["w_o"], b), TOL[w.dtype])


@pytest.mark.parametrize("wl,lens,s_q", [("smallem-fp32", [40, 17], 1), ("dsv3-paged", [70, 33], 1),
                                         ("gqla-g8", [50, 9], 2)])
def test_decode_layer_matches_reconstructed_oracle(wl, lens, s_q):
    """The new tokens' x feeds both the cache append and the query side; the layer's output
    y = proj(attention) against the oracle, with the tensors stored between calls (c_q, q_nope,
    q_pe, the cache rows, the heads' outputs) rounded like the GPU stores them."""
    w = W.WORKLOADS[wl].replace(batch=len(lens), s_q=s_q)
    lens = np.asarray(lens, np.int32)
    table, nb = W.block_table(w, lens)
    seq = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    x = W.tokens(w, len(seq), extra=8)
    wts, lw = W.weights(w, random_gamma=True), W.layer_weights(w)
    d = M.dims_of(w)
    note(f"decode layer {wl} lens={lens.tolist()} s_q={s_q}")
    # the step's new tokens: the last s_q positions of each sequence, in (b, i) order
    new = np.concatenate([np.flatnonzero(seq == b)[-s_q:] for b in range(len(lens))])
    cache = torch.full((nb, w.block_size, w.row), float("nan"), dtype=w.torch_dtype, device=DEV)
    M.mla_cache_append(d, dev(x), dev(seq), dev(pos), dev(wts["w_dkv"]), dev(wts["gamma"]),
                       dev(wts["w_kr"]), dev(table), nb, cache)
    q_nope, q_pe = gpu_query_project(w, x[torch.from_numpy(new)], lw)
    qpos = dev(pos[new].reshape(len(lens), s_q))
    q_abs = torch.empty(len(lens), s_q, w.n_heads, w.row, dtype=w.torch_dtype, device=DEV)
    M.mla_absorb_q(d, q_nope.view(len(lens), s_q, w.n_heads, w.d_nope),
                   q_pe.view(len(lens), s_q, w.n_heads, w.d_r), qpos, dev(wts["w_uk"]), q_abs)
    out = torch.empty(len(lens), s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    M.mla_decode(d, q_abs, cache, dev(table), dev(lens), dev(wts["w_uv"]), out)
    y = torch.empty(len(new), w.d_model, dtype=w.torch_dtype, device=DEV)
    M.mla_output_project(d, out.view(len(new), -1), dev(lw["w_o"]), dev(lw["b_o"]), y)
    torch.cuda.synchronize()

    rows = store(O.latent_rows(x, wts["w_dkv"], wts["gamma"], wts["w_kr"], pos, BASE, EPS), w)
    rn, rp = O.query_project(x[torch.from_numpy(new)], lw["w_dq"], lw["gamma_q"], lw["w_uq"], lw["w_qr"], EPS,
                             round_cq=lambda a: store(a, w))
    rn = store(rn, w).reshape(len(lens), s_q, w.n_heads, w.d_nope)
    rp = store(rp, w).reshape(len(lens), s_q, w.n_heads, w.d_r)
    heads = []
    k = 0
    for b, L in enumerate(lens):
        o_b, _ = O.decode_reconstructed(rn[b], rp[b], pos[new].reshape(len(lens), s_q)[b],
                                        rows[k:k + L], wts["w_uk"], wts["w_uv"], w.n_groups,
                                        w.d_c, w.d_v, BASE)
        heads.append(store(o_b, w).reshape(s_q, -1))
        k += L
    ref = O.output_project(np.concatenate(heads), lw["w_o"], lw["b_o"])
    check(y.cpu(), ref, TOL[w.dtype])
