#!/usr/bin/env python3
"""Benchmark of one absorbed MLA decode step on one MI355X.

A step is one pass of the whole decode path over one batch: append the step's new positions to
the paged latent cache (W_DKV projection, RMSNorm, RoPE on k_r), carry the queries into latent
space (W_UK absorption + RoPE), the split-K attention core over [c || k_r], and the log-sum-exp
merge with the W_UV projection. Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line: tokens/s (query tokens per second, one layer), the dominant kernel's
roofline (the split-K core, timed with HIP events on the stream it runs on) and the CPU
oracle's throughput on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
SELECT_HBM_BPS = 6.0e12           # stream-read rate reached on the chip
SELECT_SUSTAINED_FLOPS = 1.0e15   # bf16 rate the absorbed split-K core sustains
SPLITK_SRC = os.path.join(ROOT, "mla_latent_kv_21_amd", "csrc", "decode_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_traffic.json")


def kernel_hash() -> str:
    return hashlib.sha256(open(SPLITK_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the split-K kernel from committed rocprofv3 counter runs, or
    None when they were taken on different kernel source or another workload."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, lens, budget_s: float):
    """The oracle's reconstructed-K/V decode timed on host cores, head by head over the
    sequences at their full context (longest first), until the time budget is spent; scaled
    to the whole step by the positions the sample covered."""
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count()))
    ws = w.replace(batch=1)
    done, covered, t_run, seqs = 0, 0.0, 0.0, []
    for b in np.argsort(-lens, kind="stable"):
        L = int(lens[b])
        nb = (L + w.block_size - 1) // w.block_size
        rows = O.f64(W.cache_pool(ws, nb, extra=99 + int(b)).reshape(nb * w.block_size, w.row)[:L])
        q = W.queries(ws.replace(s_q=w.s_q))
        qpos = W.query_positions(ws.replace(s_q=w.s_q), np.array([L], np.int32))
        wts = W.weights(ws)
        seqs.append(L)
        t0 = time.perf_counter()
        for h in range(w.n_heads):
            O.decode_reconstructed(q["q_nope"][0], q["q_pe"][0], qpos[0], rows, wts["w_uk"],
                                   wts["w_uv"], w.n_groups, w.d_c, w.d_v, 10000.0, heads=[h])
            done += 1
            covered += L
            if t_run + time.perf_counter() - t0 > budget_s and done >= 2:
                break
        t_run += time.perf_counter() - t0
        del rows
        if t_run > budget_s:
            break
    # the step: every head of every sequence over its own length
    step_s = t_run * float(np.sum(lens)) * w.n_heads / covered
    return {"value": w.batch * w.s_q / step_s, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"reconstructed-K/V oracle (f64), {done} (sequence, head) passes over "
                      f"{len(seqs)} sequence(s) of lengths {seqs}, {t_run:.1f} s; scaled to "
                      f"all {w.n_heads} heads of all {w.batch} sequences by positions"}


def _time_calls(fn, reps: int, torch):
    """Median duration (ms) of fn() over reps launches, each bracketed by HIP events on the
    current stream, after two warm-up calls."""
    fn(); fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    stream = torch.cuda.current_stream()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def measure_rows(dev, torch):
    """The other rows of the path, each timed on its own workload: the absorbed decode on the
    DeepSeek-shaped paged workload (64 sequences, lengths 1,024..8,192, random block table),
    and on the GQLA workload (G = 8, 32 x 32,768) the absorbed decode, the GQA expansion and
    the GQA decode. Rates use each call's algorithmic bytes against 8 TB/s."""
    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    rows = {}

    def absorbed(name):
        w = W.WORKLOADS[name]
        lens = W.seq_lens(w)
        table, nb = W.block_table(w, lens)
        d = M.dims_of(w)
        cache = W.cache_pool_device(w, nb, dev)
        q_abs = g(W.absorbed_queries(w))
        wts = {k: g(v) for k, v in W.weights(w).items()}
        tab, lens_d = g(table), g(lens)
        out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=dev)
        ns = 0  # the library plans the splits from the lengths
        ws = torch.empty(M.mla_decode_workspace_bytes(d, w.batch, w.s_q, ns, table.shape[1]),
                         dtype=torch.uint8, device=dev)
        ms = _time_calls(lambda: M.mla_decode(d, q_abs, cache, tab, lens_d, wts["w_uv"], out,
                                              n_split=ns, workspace=ws), 20, torch)
        tr = A.decode_traffic(lens, w.s_q, w.n_heads, w.d_c, w.d_r, w.d_v, w.n_groups, w.elt)
        gbs = tr["bytes"] / (ms * 1e-3) / 1e9
        return {"workload": w.name, "call": "mla_decode", "ms": ms,
                "tokens_per_s": w.batch * w.s_q / (ms * 1e-3), "GBps": gbs,
                "frac_hbm": gbs / HBM_PEAK_GBS, "n_split": "planned"}, (w, lens, table, nb, cache, tab,
                                                                  lens_d, wts)

    rows["absorbed_dsv3_paged"], _ = absorbed("dsv3-paged")
    rows["absorbed_gqla_g8"], ctx = absorbed("gqla-g8")
    w, lens, table, nb, cache, tab, lens_d, wts = ctx
    d = M.dims_of(w)
    gqa = torch.empty(nb, w.block_size, w.n_groups * (w.d_nope + w.d_v) + w.d_r,
                      dtype=w.torch_dtype, device=dev)
    ms = _time_calls(lambda: M.gqla_expand(d, cache, tab, lens_d, wts["w_uk"], wts["w_uv"], gqa),
                     5, torch)
    L = int(np.sum(lens))
    eb = L * (A.latent_row_bytes(w.d_c, w.d_r, w.elt) + A.gqa_row_bytes(w.n_groups, w.d_nope,
                                                                        w.d_r, w.elt))
    rows["gqla_expand"] = {"workload": w.name, "call": "gqla_expand", "ms": ms,
                           "positions_per_s": L / (ms * 1e-3), "GBps": eb / (ms * 1e-3) / 1e9,
                           "frac_hbm": eb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    q = {k: g(v) for k, v in W.queries(w).items()}
    qpos = g(W.query_positions(w, lens))
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=dev)
    ns = M.mla_auto_split(d, w.batch, w.s_q, table.shape[1])
    ws = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, w.s_q, ns, table.shape[1]),
                     dtype=torch.uint8, device=dev)
    ms = _time_calls(lambda: M.gqla_decode(d, q["q_nope"], q["q_pe"], qpos, gqa, tab, lens_d, out,
                                           n_split=ns, workspace=ws), 5, torch)
    tr = A.gqa_decode_traffic(lens, w.s_q, w.n_heads, w.n_groups, w.d_nope, w.d_r, w.elt)
    rows["gqla_decode"] = {"workload": w.name, "call": "gqla_decode", "ms": ms,
                           "tokens_per_s": w.batch * w.s_q / (ms * 1e-3),
                           "GBps": tr["bytes"] / (ms * 1e-3) / 1e9,
                           "frac_hbm": tr["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    rows["path_select"] = select_paths(dev, torch, w, lens, table, cache, gqa, tab, lens_d, wts)
    del cache, gqa
    rows["prefill"] = measure_prefill(dev, torch)
    return rows


def measure_prefill(dev, torch):
    """Prefill of two 4,096-token prompts (every position a query, H = 128, one key and value
    per head): mla_prefill, and its two parts (gqla_expand of the latents into every head's
    K and V, then the concatenated-score attention) timed alone. Rates in FLOP: the
    expansion's 2 d_c G (D + D_v) per position and the attention's 2 (D + d_r) + 2 D_v per
    head per visible (query, position) pair, against the bf16 matrix-core peak."""
    import workloads as W
    from mla_latent_kv_21_amd import binding as M
    w = W.WORKLOADS["prefill-4k"]
    lens = W.seq_lens(w)
    table, nb = W.block_table(w, lens)
    d = M.dims_of(w)
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    cache = W.cache_pool_device(w, nb, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    shp = (w.batch, w.s_q, w.n_heads)
    q_nope = torch.randn(shp + (w.d_nope,), generator=gen, device=dev).to(w.torch_dtype)
    q_pe = torch.randn(shp + (w.d_r,), generator=gen, device=dev).to(w.torch_dtype)
    qpos = g(W.query_positions(w, lens))
    wts = {k: g(v) for k, v in W.weights(w).items()}
    tab, lens_d = g(table), g(lens)
    out = torch.empty(shp + (w.d_v,), dtype=w.torch_dtype, device=dev)
    ws = torch.empty(M.mla_prefill_workspace_bytes(d, w.batch, w.s_q, nb, table.shape[1]),
                     dtype=torch.uint8, device=dev)
    ms = _time_calls(lambda: M.mla_prefill(d, q_nope, q_pe, qpos, cache, tab, lens_d,
                                           wts["w_uk"], wts["w_uv"], out, workspace=ws),
                     10, torch)
    kv = ws[:nb * w.block_size * (w.n_groups * (w.d_nope + w.d_v) + w.d_r) * w.elt]
    kv = kv.view(w.torch_dtype).view(nb, w.block_size, -1)
    ms_x = _time_calls(lambda: M.gqla_expand(d, cache, tab, lens_d, wts["w_uk"], wts["w_uv"], kv),
                       10, torch)
    dws = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, w.s_q, 0, table.shape[1]),
                      dtype=torch.uint8, device=dev)
    ms_a = _time_calls(lambda: M.gqla_decode(d, q_nope, q_pe, qpos, kv, tab, lens_d, out,
                                             workspace=dws), 10, torch)
    L = lens.astype(np.int64)
    pairs = int(np.sum(w.s_q * (L - w.s_q) + w.s_q * (w.s_q + 1) // 2))
    f_attn = pairs * w.n_heads * (2 * (w.d_nope + w.d_r) + 2 * w.d_v)
    f_exp = int(L.sum()) * 2 * w.d_c * w.n_groups * (w.d_nope + w.d_v)
    tf = lambda f, t: f / (t * 1e-3) / 1e12
    return {"workload": w.name, "call": "mla_prefill", "ms": ms,
            "tokens_per_s": w.batch * w.s_q / (ms * 1e-3),
            "flop": f_attn + f_exp, "TFLOPs": tf(f_attn + f_exp, ms),
            "frac_mfma": tf(f_attn + f_exp, ms) / BF16_PEAK_TFLOPS,
            "expand_ms": ms_x, "expand_TFLOPs": tf(f_exp, ms_x),
            "attention_ms": ms_a, "attention_TFLOPs": tf(f_attn, ms_a),
            "attention_frac_mfma": tf(f_attn, ms_a) / BF16_PEAK_TFLOPS}


def measure_layer(w, d, step, x_new, dev, torch):
    """The whole decode layer on the bench workload: the query side (mla_query_project) and
    the output projection (mla_output_project) around the step, each call's weight bytes
    against 8 TB/s, and the layer's tokens/s."""
    import workloads as W
    from mla_latent_kv_21_amd import binding as M
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    n = w.batch * w.s_q
    lw = {k: g(v) for k, v in W.layer_weights(w).items()}
    x = x_new[:n]
    q_nope = torch.empty(n, w.n_heads, w.d_nope, dtype=w.torch_dtype, device=dev)
    q_pe = torch.empty(n, w.n_heads, w.d_r, dtype=w.torch_dtype, device=dev)
    o = g(W.head_outputs(w, n))
    y = torch.empty(n, w.d_model, dtype=w.torch_dtype, device=dev)
    wsq = torch.empty(M.mla_query_project_workspace_bytes(d, n, w.d_q), dtype=torch.uint8,
                      device=dev)
    wso = torch.empty(M.mla_output_project_workspace_bytes(d, n), dtype=torch.uint8, device=dev)
    qp = lambda: M.mla_query_project(d, x, lw["w_dq"], lw["gamma_q"], lw["w_uq"], lw["w_qr"],
                                     q_nope, q_pe, workspace=wsq)
    op = lambda: M.mla_output_project(d, o, lw["w_o"], lw["b_o"], y, workspace=wso)
    ms_q = _time_calls(qp, 20, torch)
    ms_o = _time_calls(op, 20, torch)

    def layer():
        qp()
        step()
        op()
    ms_l = _time_calls(layer, 20, torch)
    e = w.elt
    bq = (w.d_model * w.d_q + w.d_q + w.d_q * w.n_heads * (w.d_nope + w.d_r)) * e
    bo = (w.n_heads * w.d_v * w.d_model + w.d_model) * e
    return {"workload": w.name, "calls": "mla_query_project, then the step, then mla_output_project",
            "d_q": w.d_q, "ms": ms_l, "tokens_per_s": n / (ms_l * 1e-3),
            "query_project_ms": ms_q, "query_project_weight_GBps": bq / (ms_q * 1e-3) / 1e9,
            "output_project_ms": ms_o, "output_project_weight_GBps": bo / (ms_o * 1e-3) / 1e9}


def select_paths(dev, torch, w, lens, table, cache, gqa, tab, lens_d, wts):
    """Both decode paths of the GQLA workload timed at s_q = 1, 2, 4, 8 (the absorbed one with
    planned splits, the GQA one with the automatic split count), beside mla_select_path's
    choice and model times for MI355X: the choice should be the faster measured path."""
    import workloads as W
    from mla_latent_kv_21_amd import binding as M
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    res = []
    for s_q in (1, 2, 4, 8):
        ws_ = w.replace(s_q=s_q)
        d = M.dims_of(ws_)
        q_abs = g(W.absorbed_queries(ws_))
        out = torch.empty(w.batch, s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=dev)
        wsa = torch.empty(M.mla_decode_workspace_bytes(d, w.batch, s_q, 0, table.shape[1]),
                          dtype=torch.uint8, device=dev)
        ms_abs = _time_calls(lambda: M.mla_decode(d, q_abs, cache, tab, lens_d, wts["w_uv"], out,
                                                  n_split=0, workspace=wsa), 10, torch)
        q = {k: g(v) for k, v in W.queries(ws_).items()}
        qpos = g(W.query_positions(ws_, lens))
        ns = M.mla_auto_split(d, w.batch, s_q, table.shape[1])
        wsg = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, s_q, ns, table.shape[1]),
                          dtype=torch.uint8, device=dev)
        ms_gqa = _time_calls(lambda: M.gqla_decode(d, q["q_nope"], q["q_pe"], qpos, gqa, tab,
                                                   lens_d, out, n_split=ns, workspace=wsg),
                             5, torch)
        path, ta, tg = M.mla_select_path(d, s_q, int(np.max(lens)))
        chosen = "gqa" if path == M.MLA_PATH_GQA else "absorbed"
        # the same model at the rate the absorbed split-K core's matrix cores sustain (its
        # MFMA-busy counters: ~0.96 PFLOP/s) instead of the chip's peak
        path_c, _, _ = M.mla_select_path(d, s_q, int(np.max(lens)), SELECT_HBM_BPS,
                                         SELECT_SUSTAINED_FLOPS)
        chosen_c = "gqa" if path_c == M.MLA_PATH_GQA else "absorbed"
        res.append({"s_q": s_q, "absorbed_ms": ms_abs, "gqa_ms": ms_gqa,
                    "model_absorbed_ms": ta * w.batch * 1e3, "model_gqa_ms": tg * w.batch * 1e3,
                    "selected": chosen,
                    "selected_is_faster": (ms_abs <= ms_gqa) == (chosen == "absorbed"),
                    "selected_sustained_rate": chosen_c,
                    "sustained_rate_is_faster": (ms_abs <= ms_gqa) == (chosen_c == "absorbed")})
    return {"workload": w.name, "call": "mla_select_path", "cases": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long-128k",
                    help="workload name (default long-128k: H=128, d_c=512, 4 x 131,072 context)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip timing the path's other rows on their own workloads")
    ap.add_argument("--rows", choices=("all", "layer", "prefill", "none"), default="all",
                    help="rows timed after the step: all of them, only the decode layer, only "
                         "the prefill, or none")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, copy a bf16 buffer of this many MiB three "
                         "times (a plain copy of known size for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is a design note, not part of this build)", flush=True)
        sys.exit(2)

    import torch

    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M

    if not os.path.exists(M.LIB_PATH):
        from mla_latent_kv_21_amd.build import build
        build()
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    lens = W.seq_lens(w)
    table, nb = W.block_table(w, lens)
    B, s_q, H = w.batch, w.s_q, w.n_heads
    d = M.dims_of(w)
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)

    cache = W.cache_pool_device(w, nb, dev)
    wts = {k: g(v) for k, v in W.weights(w).items()}
    x_new = g(W.tokens(w, B * s_q, extra=1))
    seq_idx = g(np.repeat(np.arange(B, dtype=np.int32), s_q))
    qpos_np = W.query_positions(w, lens)
    pos_new = g(qpos_np.reshape(-1))
    q = {k: g(v) for k, v in W.queries(w).items()}
    q_pos = g(qpos_np)
    tab, lens_d = g(table), g(lens)
    q_abs = torch.empty(B, s_q, H, w.row, dtype=w.torch_dtype, device=dev)
    out = torch.empty(B, s_q, H, w.d_v, dtype=w.torch_dtype, device=dev)
    lse = torch.empty(B, s_q, H, dtype=torch.float32, device=dev)
    ns = w.n_split or M.mla_auto_split(d, B, s_q, table.shape[1])
    ws = torch.empty(M.mla_decode_workspace_bytes(d, B, s_q, ns, table.shape[1]),
                     dtype=torch.uint8, device=dev)
    ws_app = torch.empty(max(M.mla_cache_append_workspace_bytes(d, B * s_q), 256),
                         dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    n_steps = args.steps
    # The split-K core is bracketed by events on every kCoreEvery-th timed step only: each
    # event record is a barrier packet on the stream that costs the step a few microseconds.
    kCoreEvery = 8
    core_steps = set(range(0, n_steps, kCoreEvery))
    ev_core = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for i in core_steps}

    def step(i=None):
        M.mla_cache_append(d, x_new, seq_idx, pos_new, wts["w_dkv"], wts["gamma"], wts["w_kr"],
                           tab, nb, cache, workspace=ws_app)
        M.mla_absorb_q(d, q["q_nope"], q["q_pe"], q_pos, wts["w_uk"], q_abs)
        if i in core_steps:
            ev_core[i][0].record(stream)
        M.mla_decode_splitk(d, q_abs, cache, tab, lens_d, ns, ws)
        if i in core_steps:
            ev_core[i][1].record(stream)
        M.mla_decode_merge(d, q_abs, cache, tab, lens_d, wts["w_uv"], out, lse, ns, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(n_steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / n_steps
    core_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_core.values()]))
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite decode output")

    tr = A.decode_traffic(lens, s_q, H, w.d_c, w.d_r, w.d_v, w.n_groups, w.elt)
    core_bytes = tr["core_bytes"]
    achieved = core_bytes / (core_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    tokens_per_s = B * s_q / (ms_step * 1e-3)
    rec = {
        "metric": "MLA decode tokens/s, latent-cache GB/s & % roofline (H=128, d_c=512)",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded latent cache and weights, shapes of the workload)",
        "config": {"workload": w.name, "batch": B, "s_q": s_q, "heads": H, "groups": w.n_groups,
                   "d_c": w.d_c, "d_r": w.d_r, "context": int(lens.max()),
                   "context_total": int(lens.sum()), "block_size": w.block_size,
                   "n_split": ns, "d_model": w.d_model},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_mfma_kernel (split-K core)", "launch_ms": core_ms,
                     "algorithmic_bytes_per_launch": core_bytes},
        "latent_cache_GBps": tr["cache_bytes"] / (core_ms * 1e-3) / 1e9,
        "step_latent_cache_GBps": tr["cache_bytes"] / (ms_step * 1e-3) / 1e9,
        "wall_s": wall,
    }
    rows = "none" if args.no_rows else args.rows
    if rows != "none":
        rec["rows"] = measure_rows(dev, torch) if rows == "all" else {}
        if rows == "prefill":
            rec["rows"]["prefill"] = measure_prefill(dev, torch)
        else:
            rec["rows"]["decode_layer"] = measure_layer(w, d, step, x_new, dev, torch)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.randn(n, device=dev).to(torch.bfloat16)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)  # one elementwise kernel: reads and writes 2n bytes
        torch.cuda.synchronize()
        rec["copy_calibration"] = {"bytes_read": 2 * n, "bytes_written": 2 * n, "launches": 3,
                                   "kernel": "torch elementwise neg (bf16)"}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, lens, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
