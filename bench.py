#!/usr/bin/env python3
"""Benchmark of one absorbed MLA decode step on one MI355X.

A step is one pass of the whole decode path over one batch: append the step's new positions to
the paged latent cache (W_DKV projection, RMSNorm, RoPE on k_r) and carry the queries into latent
space (W_UK absorption + RoPE), the absorption sharing the projection's launch; the split-K
attention core over [c || k_r];
and the log-sum-exp merge with the W_UV projection. Inputs are seeded synthetic tensors already resident in HBM.

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
# the split-K core's source and the headers it includes
SPLITK_SRC = [os.path.join(ROOT, "mla_latent_kv_21_amd", "csrc", f)
              for f in ("decode_mfma.hip", "mfma_util.hpp", "common.hpp", "plan.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_traffic.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in SPLITK_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


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


def _time_calls(fn, reps: int, torch, stats: bool = False):
    """Duration (ms) of fn(i) over reps launches, each bracketed by HIP events on the current
    stream, after two warm-up calls: the median, or with stats the mean, median, p10 and p90.
    fn receives the call's index (callers rotate over copies of their inputs with it)."""
    fn(0); fn(1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    stream = torch.cuda.current_stream()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    if not stats:
        return float(np.median(ms))
    return {"mean_ms": float(np.mean(ms)), "median_ms": float(np.median(ms)),
            "p10_ms": float(np.percentile(ms, 10)), "p90_ms": float(np.percentile(ms, 90)),
            "launches": reps}


def _interleaved(fa, fb, n: int, rounds: int, torch):
    """Mean per-call ms of fa and of fb, each run n times back to back (one event pair around
    the n calls) in `rounds` alternating rounds, so that clock and power drift cancel."""
    stream = torch.cuda.current_stream()
    ta, tb = [], []
    for _ in range(rounds):
        for fn, acc in ((fa, ta), (fb, tb)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            acc.append(e0.elapsed_time(e1) / n)
    return float(np.mean(ta)), float(np.mean(tb))


ROTATE_BYTES = 1 << 30   # caches smaller than the 256 MB MALL are rotated over >= 1 GiB


def _copies(cache_bytes: int) -> int:
    """Independent cache copies to rotate through so that >= 1 GiB separates two reads of one
    copy (none needed for caches of 1 GiB or more)."""
    return max(1, -(-ROTATE_BYTES // cache_bytes))


def _smi_sample():
    """(socket power W, mean gfx clock MHz) from one amd-smi reading, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"],
                           capture_output=True, text=True, timeout=5)
        j = json.loads(r.stdout)
        g = j["gpu_data"][0] if isinstance(j, dict) else j[0]
        pw = float(g["power"]["socket_power"]["value"])
        clks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                if k.startswith("gfx") and isinstance(v, dict) and "clk" in v]
        return pw, (sum(clks) / len(clks) if clks else None)
    except Exception:  # amd-smi missing or its output changed: no reading
        return None


def power_sample(fn, seconds: float, torch):
    """Board power and shader clock while fn() (the split-K core) runs back to back for about
    `seconds`, from amd-smi readings taken every ~50 ms by a helper thread, beside the idle
    reading before it. The core's mean launch time over the window comes from two events."""
    import threading
    idle = [x for x in (_smi_sample() for _ in range(3)) if x]
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            x = _smi_sample()
            if x:
                samples.append(x)
            time.sleep(0.05)
    fn(); torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    th = threading.Thread(target=sampler)
    th.start()
    time.sleep(0.2)
    n, t0 = 0, time.perf_counter()
    a.record(torch.cuda.current_stream())
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn()
        n += 50
        torch.cuda.synchronize()
    b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    stop.set()
    th.join()
    busy = samples[len(samples) // 4:]   # readings lag the load by a few samples
    if not idle or not busy:
        return None
    return {"idle_W": float(np.mean([x[0] for x in idle])),
            "busy_W": float(np.mean([x[0] for x in busy])),
            "busy_gfx_clock_MHz": float(np.mean([x[1] for x in busy if x[1]])),
            "launches": n, "mean_launch_ms": a.elapsed_time(b) / n,
            "readings": len(busy), "source": "amd-smi metric -p -c, every ~50 ms"}


def fp8_caches(w, nb, n, dev, torch):
    """n e4m3 caches (codes, scales) of workload w, each the library's quantisation of a
    seeded bf16 cache_pool_device draw."""
    import workloads as W
    from mla_latent_kv_21_amd import binding as M
    d = M.dims_of(w)
    out = []
    for k in range(n):
        bf = W.cache_pool_device(w, nb, dev, extra=k)
        codes = torch.empty(bf.shape, dtype=torch.uint8, device=dev)
        scales = torch.empty(bf.shape[:2], dtype=torch.float32, device=dev)
        M.mla_cache_quantize_fp8(d, bf, codes, scales)
        torch.cuda.synchronize()
        del bf
        out.append((codes, scales))
    return out


def absorbed_row(dev, torch, w, planned=True, reps=20, fp8=False):
    """mla_decode (split-K core + merge + W_UV) on workload w, timed with HIP events over
    reps calls that rotate over enough cache copies to keep the MALL from serving them, with
    the call's algorithmic bytes and FLOPs priced against the binding roofline. fp8: the same
    over an e4m3 cache (mla_decode_fp8, 580 bytes per position)."""
    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    lens = W.seq_lens(w)
    table, nb = W.block_table(w, lens)
    d = M.dims_of(w)
    row_b = A.fp8_row_bytes(w.d_c, w.d_r) if fp8 else w.row * w.elt
    n_copies = _copies(nb * w.block_size * row_b)
    if fp8:
        caches = fp8_caches(w, nb, n_copies, dev, torch)
    else:
        caches = [W.cache_pool_device(w, nb, dev, extra=k) for k in range(n_copies)]
    q_abs = g(W.absorbed_queries(w))
    wts = {k: g(v) for k, v in W.weights(w).items()}
    tab, lens_d = g(table), g(lens)
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=dev)
    ns = 0 if planned else (w.n_split or M.mla_auto_split(d, w.batch, w.s_q, table.shape[1]))
    ws = torch.empty(M.mla_decode_workspace_bytes(d, w.batch, w.s_q, ns, table.shape[1]),
                     dtype=torch.uint8, device=dev)
    if fp8:
        call = lambda i: M.mla_decode_fp8(d, q_abs, *caches[i % n_copies], tab, lens_d,
                                          wts["w_uv"], out, n_split=ns, workspace=ws)
    else:
        call = lambda i: M.mla_decode(d, q_abs, caches[i % n_copies], tab, lens_d, wts["w_uv"],
                                      out, n_split=ns, workspace=ws)
    ms = _time_calls(call, reps, torch)
    tr = A.decode_traffic(lens, w.s_q, w.n_heads, w.d_c, w.d_r, w.d_v, w.n_groups, w.elt,
                          row_bytes=row_b)
    row = {"workload": w.name, "call": "mla_decode_fp8" if fp8 else "mla_decode",
           "cache": "e4m3 + fp32 scale per position" if fp8 else w.dtype,
           "batch": w.batch, "s_q": w.s_q,
           "heads": w.n_heads, "context_max": int(lens.max()), "ms": ms,
           "tokens_per_s": w.batch * w.s_q / (ms * 1e-3),
           "GBps": tr["bytes"] / (ms * 1e-3) / 1e9,
           "latent_cache_GBps": tr["cache_bytes"] / (ms * 1e-3) / 1e9,
           "n_split": "planned" if planned else ns, "cache_copies_rotated": n_copies}
    row.update(A.binding_roofline(tr["bytes"], tr["flops"], ms))
    del caches
    return row, (lens, table, nb, tab, lens_d, wts)


def measure_rows(dev, torch):
    """The other rows of the path, each timed on its own workload: the absorbed decode on the
    mid-size (H = 32, 16 x 4,096) and DeepSeek-shaped paged workloads (64 sequences, lengths
    1,024..8,192, random block table), an H = 128 context sweep (8K, 32K, 128K positions per
    sequence at 524,288 cached positions in all), and on the GQLA workload (G = 8,
    32 x 32,768) the absorbed decode, the GQA expansion and the GQA decode. Every row carries
    its binding roofline: the larger of its HBM and bf16 matrix-core times at the published
    peaks."""
    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M
    rows = {}
    rows["absorbed_mid_bf16"], _ = absorbed_row(dev, torch, W.WORKLOADS["mid-bf16"])
    rows["absorbed_dsv3_paged"], _ = absorbed_row(dev, torch, W.WORKLOADS["dsv3-paged"])
    sweep = []
    base = W.WORKLOADS["long-128k"]
    for B, L in ((64, 8192), (16, 32768), (4, 131072)):
        r, _ = absorbed_row(dev, torch, base.replace(name=f"h128-ctx{L // 1024}k", batch=B,
                                                     ctx=L, n_split=0))
        sweep.append(r)
    rows["absorbed_h128_context_sweep"] = sweep
    # the same over e4m3 caches (half the cache bytes, the same matrix-core work)
    rows["fp8_dsv3_paged"], _ = absorbed_row(dev, torch, W.WORKLOADS["dsv3-paged"], fp8=True)
    sweep = []
    for B, L in ((64, 8192), (16, 32768), (4, 131072)):
        r, _ = absorbed_row(dev, torch, base.replace(name=f"h128-ctx{L // 1024}k", batch=B,
                                                     ctx=L, n_split=0), fp8=True)
        sweep.append(r)
    rows["fp8_h128_context_sweep"] = sweep
    w = W.WORKLOADS["gqla-g8"]
    rows["absorbed_gqla_g8"], ctx = absorbed_row(dev, torch, w)
    lens, table, nb, tab, lens_d, wts = ctx
    d = M.dims_of(w)
    rows["gqla_expand"], cache, gqa = expand_row(dev, torch, w, ctx)
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    q = {k: g(v) for k, v in W.queries(w).items()}
    qpos = g(W.query_positions(w, lens))
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=dev)
    ns = M.mla_auto_split(d, w.batch, w.s_q, table.shape[1])
    ws = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, w.s_q, ns, table.shape[1]),
                     dtype=torch.uint8, device=dev)
    ms = _time_calls(lambda i: M.gqla_decode(d, q["q_nope"], q["q_pe"], qpos, gqa, tab, lens_d,
                                             out, n_split=ns, workspace=ws), 5, torch)
    tr = A.gqa_decode_traffic(lens, w.s_q, w.n_heads, w.n_groups, w.d_nope, w.d_r, w.elt)
    rows["gqla_decode"] = {"workload": w.name, "call": "gqla_decode", "ms": ms,
                           "tokens_per_s": w.batch * w.s_q / (ms * 1e-3),
                           "GBps": tr["bytes"] / (ms * 1e-3) / 1e9}
    rows["gqla_decode"].update(A.binding_roofline(tr["bytes"], tr["flops"], ms))
    rows["path_select"] = select_paths(dev, torch, w, lens, table, cache, gqa, tab, lens_d, wts)
    del cache, gqa
    rows["prefill"] = measure_prefill(dev, torch)
    return rows


def expand_row(dev, torch, w, ctx=None, reps=5):
    """gqla_expand of every cached position of workload w into the expanded GQA cache, timed
    with HIP events over reps calls, priced in bytes (latent rows read, expanded rows written)
    and FLOPs (2 d_c G (D + D_v) per position) against the binding roofline. ctx: the
    workload's (lens, table, nb, tab, lens_d, wts) when the caller already has them on the
    device. Returns the row, the latent cache and the expanded cache."""
    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M
    if ctx is None:
        g = lambda a: (a if isinstance(a, torch.Tensor)
                       else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
        lens = W.seq_lens(w)
        table, nb = W.block_table(w, lens)
        ctx = (lens, table, nb, g(table), g(lens), {k: g(v) for k, v in W.weights(w).items()})
    lens, table, nb, tab, lens_d, wts = ctx
    d = M.dims_of(w)
    cache = W.cache_pool_device(w, nb, dev)
    gqa = torch.empty(nb, w.block_size, w.n_groups * (w.d_nope + w.d_v) + w.d_r,
                      dtype=w.torch_dtype, device=dev)
    ms = _time_calls(lambda i: M.gqla_expand(d, cache, tab, lens_d, wts["w_uk"], wts["w_uv"], gqa),
                     reps, torch)
    L = int(np.sum(lens))
    eb = L * (A.latent_row_bytes(w.d_c, w.d_r, w.elt) + A.gqa_row_bytes(w.n_groups, w.d_nope,
                                                                        w.d_r, w.elt))
    ef = L * 2 * w.d_c * w.n_groups * (w.d_nope + w.d_v)
    row = {"workload": w.name, "call": "gqla_expand", "ms": ms,
           "positions_per_s": L / (ms * 1e-3), "GBps": eb / (ms * 1e-3) / 1e9,
           "TFLOPs": ef / (ms * 1e-3) / 1e12}
    row.update(A.binding_roofline(eb, ef, ms))
    return row, cache, gqa


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
    ms = _time_calls(lambda i: M.mla_prefill(d, q_nope, q_pe, qpos, cache, tab, lens_d,
                                           wts["w_uk"], wts["w_uv"], out, workspace=ws),
                     10, torch)
    kv = ws[:nb * w.block_size * (w.n_groups * (w.d_nope + w.d_v) + w.d_r) * w.elt]
    kv = kv.view(w.torch_dtype).view(nb, w.block_size, -1)
    ms_x = _time_calls(lambda i: M.gqla_expand(d, cache, tab, lens_d, wts["w_uk"], wts["w_uv"], kv),
                       10, torch)
    dws = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, w.s_q, 0, table.shape[1]),
                      dtype=torch.uint8, device=dev)
    ms_a = _time_calls(lambda i: M.gqla_decode(d, q_nope, q_pe, qpos, kv, tab, lens_d, out,
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


def measure_fp8_step(w, d, lens, cache, tab, lens_d, nb, ns, step_args, n_steps, dev, torch):
    """The bench step over an e4m3 copy of its cache (mla_decode_step_fp8: the projection with
    the absorption, the e4m3 split-K core quantising the new rows, the merge), timed like the
    bf16 step, with the e4m3 split-K core in a loop of its own against the binding roofline
    (580 bytes per position)."""
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M
    x_new, seq_idx, pos_new, wts, q, q_pos, q_abs, out, lse, ws, ws_app, ws_step = step_args
    codes = torch.empty(cache.shape, dtype=torch.uint8, device=dev)
    scales = torch.empty(cache.shape[:2], dtype=torch.float32, device=dev)
    M.mla_cache_quantize_fp8(d, cache, codes, scales)

    def step8():
        M.mla_decode_step_fp8(d, x_new, wts["w_dkv"], wts["gamma"], wts["w_kr"], q["q_nope"],
                              q["q_pe"], wts["w_uk"], wts["w_uv"], codes, scales, tab, lens_d,
                              out, lse, n_split=ns, workspace=ws_step)
    for _ in range(5):
        step8()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n_steps):
        step8()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n_steps
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite fp8 decode output")
    # the absorbed queries, for the core on its own
    M.mla_cache_append_absorb_q_fp8(d, x_new, seq_idx, pos_new, wts["w_dkv"], wts["gamma"],
                                    wts["w_kr"], tab, nb, codes, scales, q["q_nope"], q["q_pe"],
                                    q_pos, wts["w_uk"], q_abs, workspace=ws_app)
    core8 = lambda: M.mla_decode_fp8_splitk(d, q_abs, codes, scales, tab, lens_d, ns, ws)
    core = _time_calls(lambda i: core8(), max(20, n_steps), torch, stats=True)
    bb_step, bb_core = _interleaved(step8, core8, 10, 5, torch)
    tr = A.decode_traffic(lens, w.s_q, w.n_heads, w.d_c, w.d_r, w.d_v, w.n_groups, w.elt,
                          row_bytes=A.fp8_row_bytes(w.d_c, w.d_r))
    r = {"workload": w.name, "cache": "e4m3 + fp32 scale per position",
         "calls": "mla_decode_step_fp8 (project_absorb, decode_mfma_kernel<4, true, true, NT>, "
                  "merge_project_kernel)",
         "ms_per_step": ms, "tokens_per_s": w.batch * w.s_q / (ms * 1e-3),
         "core_launch_stats": core, "core_bytes_per_launch": tr["core_bytes"],
         "core_GBps": tr["core_bytes"] / (core["mean_ms"] * 1e-3) / 1e9,
         "step_outside_core_ms": bb_step - bb_core,
         "back_to_back_ms": {"step": bb_step, "core": bb_core}}
    r["core_roofline"] = A.binding_roofline(tr["core_bytes"], tr["core_flops"], core["mean_ms"])
    del codes, scales
    return r


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
    ms_q = _time_calls(lambda i: qp(), 20, torch)
    ms_o = _time_calls(lambda i: op(), 20, torch)

    def layer():
        qp()
        step()
        op()
    ms_l = _time_calls(lambda i: layer(), 20, torch)
    e = w.elt
    bq = (w.d_model * w.d_q + w.d_q + w.d_q * w.n_heads * (w.d_nope + w.d_r)) * e
    bo = (w.n_heads * w.d_v * w.d_model + w.d_model) * e
    return {"workload": w.name, "calls": "mla_query_project, then the step, then mla_output_project",
            "d_q": w.d_q, "ms": ms_l, "tokens_per_s": n / (ms_l * 1e-3),
            "query_project_ms": ms_q, "query_project_weight_GBps": bq / (ms_q * 1e-3) / 1e9,
            "output_project_ms": ms_o, "output_project_weight_GBps": bo / (ms_o * 1e-3) / 1e9}


def mtp_rows(dev, torch, reps=5):
    """The absorbed decode (mla_decode, planned splits) on gqla-g8 at s_q = 1, 2 and 4: the
    s_q query tokens of a sequence attend over one cache, so the HBM bytes of the cache stay
    those of one read while the FLOPs grow with s_q. Each row carries its binding roofline;
    under a counter pass (FETCH_SIZE) the launches run in this order, reps + 2 per s_q."""
    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
    from mla_latent_kv_21_amd import binding as M
    g = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(dev)
    w = W.WORKLOADS["gqla-g8"]
    lens = W.seq_lens(w)
    table, nb = W.block_table(w, lens)
    cache = W.cache_pool_device(w, nb, dev)
    tab, lens_d = g(table), g(lens)
    w_uv = g(W.weights(w)["w_uv"])
    res = []
    for s_q in (1, 2, 4):
        ws_ = w.replace(s_q=s_q)
        d = M.dims_of(ws_)
        q_abs = g(W.absorbed_queries(ws_))
        out = torch.empty(w.batch, s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=dev)
        wsa = torch.empty(M.mla_decode_workspace_bytes(d, w.batch, s_q, 0, table.shape[1]),
                          dtype=torch.uint8, device=dev)
        ms = _time_calls(lambda i: M.mla_decode(d, q_abs, cache, tab, lens_d, w_uv, out,
                                              n_split=0, workspace=wsa), reps, torch)
        tr = A.decode_traffic(lens, s_q, w.n_heads, w.d_c, w.d_r, w.d_v, w.n_groups, w.elt)
        row = {"s_q": s_q, "ms": ms, "tokens_per_s": w.batch * s_q / (ms * 1e-3),
               "cache_bytes": tr["cache_bytes"], "core_bytes": tr["core_bytes"],
               "flops": tr["flops"], "launches": reps + 2}
        row.update(A.binding_roofline(tr["bytes"], tr["flops"], ms))
        res.append(row)
    return {"workload": w.name, "call": "mla_decode (planned splits)", "cases": res}


def select_paths(dev, torch, w, lens, table, cache, gqa, tab, lens_d, wts):
    """Both decode paths of the GQLA workload timed at s_q = 1, 2, 4, 8 (the absorbed one with
    planned splits, the GQA one with the automatic split count), beside mla_select_path's
    default choice and model times for MI355X (the rates its kernels sustain): the choice
    should be the faster measured path. Each path's binding roofline fraction is reported,
    and the choice the model would make at the chip's published peak rates."""
    import workloads as W
    from mla_latent_kv_21_amd import accounting as A
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
        ms_abs = _time_calls(lambda i: M.mla_decode(d, q_abs, cache, tab, lens_d, wts["w_uv"], out,
                                                  n_split=0, workspace=wsa), 10, torch)
        q = {k: g(v) for k, v in W.queries(ws_).items()}
        qpos = g(W.query_positions(ws_, lens))
        ns = M.mla_auto_split(d, w.batch, s_q, table.shape[1])
        wsg = torch.empty(M.gqla_decode_workspace_bytes(d, w.batch, s_q, ns, table.shape[1]),
                          dtype=torch.uint8, device=dev)
        ms_gqa = _time_calls(lambda i: M.gqla_decode(d, q["q_nope"], q["q_pe"], qpos, gqa, tab,
                                                   lens_d, out, n_split=ns, workspace=wsg),
                             5, torch)
        path, ta, tg = M.mla_select_path(d, s_q, int(np.max(lens)))
        chosen = "gqa" if path == M.MLA_PATH_GQA else "absorbed"
        # the same model at the chip's published peaks (8 TB/s, 2.5 PFLOP/s bf16)
        path_p, _, _ = M.mla_select_path(d, s_q, int(np.max(lens)), HBM_PEAK_GBS * 1e9,
                                         BF16_PEAK_TFLOPS * 1e12)
        tra = A.decode_traffic(lens, s_q, w.n_heads, w.d_c, w.d_r, w.d_v, w.n_groups, w.elt)
        trg = A.gqa_decode_traffic(lens, s_q, w.n_heads, w.n_groups, w.d_nope, w.d_r, w.elt)
        ra = A.binding_roofline(tra["bytes"], tra["flops"], ms_abs)
        rg = A.binding_roofline(trg["bytes"], trg["flops"], ms_gqa)
        res.append({"s_q": s_q, "absorbed_ms": ms_abs, "gqa_ms": ms_gqa,
                    "absorbed_bound": ra["bound"], "absorbed_frac": ra["frac"],
                    "gqa_bound": rg["bound"], "gqa_frac": rg["frac"],
                    "model_absorbed_ms": ta * w.batch * 1e3, "model_gqa_ms": tg * w.batch * 1e3,
                    "selected": chosen,
                    "selected_is_faster": (ms_abs <= ms_gqa) == (chosen == "absorbed"),
                    "selected_at_peak_rates": "gqa" if path_p == M.MLA_PATH_GQA else "absorbed"})
    return {"workload": w.name, "call": "mla_select_path", "cases": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long-128k",
                    help="workload name (default long-128k: H=128, d_c=512, 4 x 131,072 context)")
    ap.add_argument("--s-q", type=int, default=0,
                    help="query tokens per sequence in the step (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip timing the path's other rows on their own workloads")
    ap.add_argument("--rows", choices=("all", "layer", "prefill", "expand", "mtp", "none"),
                    default="all",
                    help="rows timed after the step: all of them, only the decode layer, only "
                         "the prefill, only the GQA expansion (gqla-g8), only the absorbed "
                         "decode of gqla-g8 at s_q = 1, 2, 4, or none")
    ap.add_argument("--power-seconds", type=float, default=2.0,
                    help="run the split-K core back to back for this long while sampling board "
                         "power and shader clock with amd-smi (0: skip)")
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
    if args.s_q > 0:
        w = w.replace(s_q=args.s_q)
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
    # the workload's split count, else 0: the library's choice (the length-balanced plan
    # where it applies, as the rows below time it)
    ns = w.n_split
    ws = torch.empty(M.mla_decode_workspace_bytes(d, B, s_q, ns, table.shape[1]),
                     dtype=torch.uint8, device=dev)
    ws_app = torch.empty(max(M.mla_cache_append_workspace_bytes(d, B * s_q), 256),
                         dtype=torch.uint8, device=dev)
    ws_step = torch.empty(M.mla_decode_step_workspace_bytes(d, B, s_q, ns, table.shape[1]),
                          dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    n_steps = args.steps

    def step():
        # append the B * s_q new tokens (each sequence's last s_q positions), absorb their
        # queries, split-K core (which forms the new rows), merge + W_UV
        M.mla_decode_step(d, x_new, wts["w_dkv"], wts["gamma"], wts["w_kr"], q["q_nope"],
                          q["q_pe"], wts["w_uk"], wts["w_uv"], cache, tab, lens_d, out, lse,
                          n_split=ns, workspace=ws_step)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(n_steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / n_steps
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite decode output")
    # the absorbed queries the step forms inside its workspace, for the core on its own
    M.mla_cache_append_absorb_q(d, x_new, seq_idx, pos_new, wts["w_dkv"], wts["gamma"],
                                wts["w_kr"], tab, nb, cache, q["q_nope"], q["q_pe"], q_pos,
                                wts["w_uk"], q_abs, workspace=ws_app)
    # The split-K core (the dominant kernel) in a loop of its own, every launch bracketed by
    # HIP events on the stream it runs on (an event pair inside the step would add its own
    # barrier packets to the step time).
    core = _time_calls(lambda i: M.mla_decode_splitk(d, q_abs, cache, tab, lens_d, ns, ws),
                       max(20, n_steps), torch, stats=True)
    core_ms = core["mean_ms"]
    # the step and the core alone, both back to back, in alternating rounds: what the step
    # spends outside the core
    bb_step, bb_core = _interleaved(
        step, lambda: M.mla_decode_splitk(d, q_abs, cache, tab, lens_d, ns, ws), 10, 5, torch)

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
                   "n_split": ns if ns else "planned", "d_model": w.d_model},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_mfma_kernel (split-K core)", "launch_ms": core_ms,
                     "launch_stats": core,
                     "algorithmic_bytes_per_launch": core_bytes,
                     "algorithmic_flops_per_launch": tr["core_flops"],
                     "frac_mfma": tr["core_flops"] / (core_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "step_outside_core_ms": bb_step - bb_core,
        "back_to_back_ms": {"step": bb_step, "core": bb_core, "rounds": 5, "calls_per_round": 10},
        "latent_cache_GBps": tr["cache_bytes"] / (core_ms * 1e-3) / 1e9,
        "step_latent_cache_GBps": tr["cache_bytes"] / (ms_step * 1e-3) / 1e9,
        "wall_s": wall,
    }
    if args.power_seconds > 0:
        rec["roofline"]["power"] = power_sample(
            lambda: M.mla_decode_splitk(d, q_abs, cache, tab, lens_d, ns, ws), args.power_seconds,
            torch)
    rows = "none" if args.no_rows else args.rows
    if rows != "none":
        rec["rows"] = {}
        if rows == "all":
            rec["rows"]["fp8_step"] = measure_fp8_step(
                w, d, lens, cache, tab, lens_d, nb, ns,
                (x_new, seq_idx, pos_new, wts, q, q_pos, q_abs, out, lse, ws, ws_app, ws_step),
                n_steps,
                dev, torch)
            rec["rows"].update(measure_rows(dev, torch))
        if rows == "prefill":
            rec["rows"]["prefill"] = measure_prefill(dev, torch)
        elif rows == "expand":
            rec["rows"]["gqla_expand"], _, _ = expand_row(dev, torch, W.WORKLOADS["gqla-g8"])
        elif rows == "mtp":
            rec["rows"]["absorbed_mtp"] = mtp_rows(dev, torch)
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
