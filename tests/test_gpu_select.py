"""mla_select_path against the chip: on the GQLA workload at full size (32 sequences x 32,768
positions, H = 128, G = 8) both decode paths are timed at s_q = 1, 2, 4 and 8 (the absorbed
path with the balanced split plan, the GQA path on the expanded cache with the library's split
count, as the benchmark runs them), and wherever one is more than 15 % faster the selector's
default choice must be that one ([GQLA] summary, section 2, "Sélection du chemin")."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import DEV, dev, note
from mla_latent_kv_21_amd import binding as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def median_ms(fn, reps=7):
    fn()
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    s = torch.cuda.current_stream()
    for a, b in evs:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def test_selector_picks_the_faster_path():
    w = W.WORKLOADS["gqla-g8"]
    lens = W.seq_lens(w)
    table, nb = W.block_table(w, lens)
    cache = W.cache_pool_device(w, nb, DEV)
    wts = {k: dev(v) for k, v in W.weights(w).items()}
    tab, lens_d = dev(table), dev(lens)
    d = M.dims_of(w)
    gqa = torch.empty(nb, w.block_size, w.n_groups * (w.d_nope + w.d_v) + w.d_r,
                      dtype=w.torch_dtype, device=DEV)
    M.gqla_expand(d, cache, tab, lens_d, wts["w_uk"], wts["w_uv"], gqa)
    for s_q in (1, 2, 4, 8):
        ws_ = w.replace(s_q=s_q)
        d = M.dims_of(ws_)
        q_abs = dev(W.absorbed_queries(ws_))
        q = {k: dev(v) for k, v in W.queries(ws_).items()}
        qpos = dev(W.query_positions(ws_, lens))
        out = torch.empty(w.batch, s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
        wsa = torch.empty(M.mla_decode_workspace_bytes(d, w.batch, s_q, 0, table.shape[1]),
                          dtype=torch.uint8, device=DEV)
        t_abs = median_ms(lambda: M.mla_decode(d, q_abs, cache, tab, lens_d, wts["w_uv"], out,
                                               n_split=0, workspace=wsa))
        ns = M.mla_auto_split(d, w.batch, s_q, table.shape[1])
        wsg = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, s_q, ns, table.shape[1]),
                          dtype=torch.uint8, device=DEV)
        t_gqa = median_ms(lambda: M.gqla_decode(d, q["q_nope"], q["q_pe"], qpos, gqa, tab,
                                                lens_d, out, n_split=ns, workspace=wsg))
        path, _, _ = M.mla_select_path(d, s_q, int(np.max(lens)))
        chosen = "gqa" if path == M.MLA_PATH_GQA else "absorbed"
        note(f"select s_q={s_q}: absorbed {t_abs:.3f} ms, GQA {t_gqa:.3f} ms -> {chosen}")
        if t_abs < t_gqa / 1.15:
            assert chosen == "absorbed", (s_q, t_abs, t_gqa)
        elif t_gqa < t_abs / 1.15:
            assert chosen == "gqa", (s_q, t_abs, t_gqa)
