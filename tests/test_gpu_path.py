"""GPU parity of mla_cache_append, mla_absorb_q, gqla_expand and gqla_decode, and of the whole
decode step end to end, against the oracle's reconstructed-K/V answer.

Integer work is checked bit-exactly: the set of cache slots the append writes equals the
oracle's slot set (every other slot keeps its NaN sentinel), and appending in chunks writes
the same bytes as appending at once.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_cases import (DEV, TOL, check, check_lse, check_per_seq, decode_case, dev, note)
from mla_latent_kv_21_amd import binding as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BASE, EPS = 10000.0, 1e-6


def ulp_close(gpu, ref, dtype):
    """Each stored value within one storage ulp of the oracle's f64 value plus the fp32
    accumulation error of its row (1e-5 of the row's largest magnitude): values that cancel
    to near zero have tiny ulps but carry the absolute error of their fp32 sums."""
    g, ref = O.f64(gpu), O.f64(ref)
    slack = 1e-5 * np.max(np.abs(ref), axis=-1, keepdims=True)
    if dtype == "bf16":
        _, e = np.frexp(np.abs(ref))
        ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
        return bool(np.all(np.abs(g - ref) <= ulp + slack))
    return bool(np.all(np.abs(g - ref) <= 1e-6 * np.abs(ref) + slack))


def append_case(w, lens, n_tok_extra=0):
    """History of every sequence appended token by token from seeded x; returns GPU cache."""
    lens = np.asarray(lens, np.int32)
    table, nb = W.block_table(w.replace(batch=len(lens)), lens)
    seq = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    x = W.tokens(w, len(seq), extra=n_tok_extra)
    wts = W.weights(w, random_gamma=True)
    return dict(lens=lens, table=table, nb=nb, seq=seq, pos=pos, x=x, wts=wts)


def gpu_append(w, a, chunks=1):
    d = M.dims_of(w)
    cache = torch.full((a["nb"], w.block_size, w.row), float("nan"), dtype=w.torch_dtype,
                       device=DEV)
    tab = dev(a["table"])
    n = len(a["seq"])
    edges = np.linspace(0, n, chunks + 1).astype(int)
    for lo, hi in zip(edges[:-1], edges[1:]):
        M.mla_cache_append(d, dev(a["x"][lo:hi]), dev(a["seq"][lo:hi]), dev(a["pos"][lo:hi]),
                           dev(a["wts"]["w_dkv"]), dev(a["wts"]["gamma"]), dev(a["wts"]["w_kr"]),
                           tab, a["nb"], cache)
    torch.cuda.synchronize()
    return cache.cpu()


@pytest.mark.parametrize("wl,lens", [("smallem-fp32", [512]), ("mid-bf16", [40, 130]),
                                     ("dsv3-paged", [3, 70]), ("gqla-g8", [65])])
def test_append_matches_oracle(wl, lens):
    w = W.WORKLOADS[wl]
    a = append_case(w, lens)
    note(f"append {wl} lens={lens}")
    cache = gpu_append(w, a)
    ref = O.latent_rows(a["x"], a["wts"]["w_dkv"], a["wts"]["gamma"], a["wts"]["w_kr"], a["pos"],
                        BASE, EPS)
    flat = cache.view(-1, w.row)
    k = 0
    for b, L in enumerate(a["lens"]):
        got = O.gather_rows(cache, a["table"], b, int(L))
        assert ulp_close(got, ref[k:k + L], w.dtype)
        k += L
    # integer addressing, bit-exact: exactly the oracle's slots were written
    owned = O.owned_slot_mask(a["table"], a["lens"], a["nb"], w.block_size)
    written = ~torch.isnan(flat.float()).all(dim=1).numpy()
    assert np.array_equal(written, owned)


def test_chunked_append_is_bit_exact():
    w = W.WORKLOADS["dsv3-paged"]
    a = append_case(w, [100, 37])
    note("append bulk vs 3 chunks")
    one = gpu_append(w, a, chunks=1)
    three = gpu_append(w, a, chunks=3)
    assert torch.equal(one.view(torch.int16), three.view(torch.int16))


APPEND_SHAPES = [
    ("dsv3-paged", {}),
    # latent width 160: the third 64-column block holds latent and rotary columns
    ("gqla-g8", dict(d_model=512, d_c=160, d_r=32, n_groups=8)),
]


@pytest.mark.parametrize("wl,kw", APPEND_SHAPES, ids=[s[0] + ("-dc160" if s[1] else "")
                                                     for s in APPEND_SHAPES])
def test_appends_of_any_size_write_the_same_bytes(wl, kw):
    """Appending 20 tokens one call at a time, then 13 and 7 at a time, through one reused
    workspace, writes exactly the bytes that one call with all 20 writes (a row depends only
    on its own token: fixed split-K ranges summed in a fixed order, and the sum of squares of
    the latent part taken per 64-column block in a fixed order), and those are within one
    storage ulp of the oracle's rows."""
    w = W.WORKLOADS[wl].replace(**kw)
    a = append_case(w, [12, 8])
    d = M.dims_of(w)
    n = len(a["seq"])
    assert n == 20
    bulk = gpu_append(w, a)
    ws = torch.empty(M.mla_cache_append_workspace_bytes(d, 16), dtype=torch.uint8, device=DEV)
    for sizes in ([1] * 20, [13, 7]):
        note(f"append {wl} {kw} in calls of {sizes[:3]}...")
        cache = torch.full((a["nb"], w.block_size, w.row), float("nan"), dtype=w.torch_dtype,
                           device=DEV)
        lo = 0
        for k in sizes:
            hi = lo + k
            M.mla_cache_append(d, dev(a["x"][lo:hi]), dev(a["seq"][lo:hi]), dev(a["pos"][lo:hi]),
                               dev(a["wts"]["w_dkv"]), dev(a["wts"]["gamma"]),
                               dev(a["wts"]["w_kr"]), dev(a["table"]), a["nb"], cache,
                               workspace=ws)
            lo = hi
        torch.cuda.synchronize()
        assert torch.equal(cache.cpu().view(torch.int16), bulk.view(torch.int16))
    ref = O.latent_rows(a["x"], a["wts"]["w_dkv"], a["wts"]["gamma"], a["wts"]["w_kr"], a["pos"],
                        BASE, EPS)
    k = 0
    for b, L in enumerate(a["lens"]):
        got = O.gather_rows(bulk, a["table"], b, int(L))
        assert ulp_close(got, ref[k:k + L], w.dtype)
        k += L


@pytest.mark.parametrize("wl,s_q", [("long-128k", 1), ("gqla-g8", 4), ("mid-bf16", 1)])
def test_append_absorb_in_one_launch(wl, s_q):
    """mla_cache_append_absorb_q (the absorption in the projection's launch) writes the same
    cache rows and absorbed queries, bit for bit, as mla_cache_append followed by mla_absorb_q
    (a decode step's first two calls)."""
    w = W.WORKLOADS[wl].replace(batch=4, s_q=s_q)
    lens = np.array([70, 129, 64, 3 + s_q], np.int32)
    table, nb = W.block_table(w, lens)
    seq = np.repeat(np.arange(w.batch, dtype=np.int32), s_q)
    qpos = W.query_positions(w, lens)
    pos = qpos.reshape(-1).astype(np.int32)
    x = W.tokens(w, len(seq), extra=3)
    wts = W.weights(w, random_gamma=True)
    q = W.queries(w)
    d = M.dims_of(w)
    outs = []
    for fused in (False, True):
        note(f"append+absorb {wl} s_q={s_q} fused={fused}")
        cache = torch.full((nb, w.block_size, w.row), float("nan"), dtype=w.torch_dtype,
                           device=DEV)
        q_abs = torch.full((w.batch, s_q, w.n_heads, w.row), float("nan"), dtype=w.torch_dtype,
                           device=DEV)
        args = (dev(x), dev(seq), dev(pos), dev(wts["w_dkv"]), dev(wts["gamma"]),
                dev(wts["w_kr"]), dev(table), nb, cache)
        if fused:
            M.mla_cache_append_absorb_q(d, *args, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos),
                                        dev(wts["w_uk"]), q_abs)
        else:
            M.mla_cache_append(d, *args)
            M.mla_absorb_q(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), dev(wts["w_uk"]),
                           q_abs)
        torch.cuda.synchronize()
        outs.append((cache.cpu(), q_abs.cpu()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
    ref = O.absorb_query(q["q_nope"], q["q_pe"], qpos, wts["w_uk"], w.n_groups, BASE)
    check(outs[1][1], ref, 4e-3, "q_abs")
    rows = O.latent_rows(x, wts["w_dkv"], wts["gamma"], wts["w_kr"], pos, BASE, EPS)
    flat = outs[1][0].view(-1, w.row)
    slots = np.array([O.slot(table, int(b), int(p), w.block_size) for b, p in zip(seq, pos)])
    assert ulp_close(flat[torch.from_numpy(slots)], rows, w.dtype)


@pytest.mark.parametrize("wl", ["long-128k", "dsv3-paged"])
def test_append_at_long_context_positions(wl):
    """Positions 131,000 .. 131,071 (the last 72 of a 131,072-position context) appended to a
    paged cache: the rotary angles pos * theta_j reach 1.3e5 rad there, so the rows are only
    right if the angle is reduced in double precision. Only the two logical blocks these
    positions fall in are mapped (to physical blocks 1 and 0 of a three-block cache; every
    other table entry is -1), and every slot the oracle does not own keeps its NaN."""
    w = W.WORKLOADS[wl]
    bs = w.block_size
    pos = np.arange(131000, 131072, dtype=np.int32)
    mb = 131072 // bs
    table = np.full((1, mb), -1, np.int32)
    table[0, 131000 // bs] = 1
    table[0, 131071 // bs] = 0
    nb = 3
    seq = np.zeros(len(pos), np.int32)
    x = W.tokens(w, len(pos), extra=7)
    wts = W.weights(w, random_gamma=True)
    d = M.dims_of(w)
    cache = torch.full((nb, bs, w.row), float("nan"), dtype=w.torch_dtype, device=DEV)
    note(f"append {wl} at positions {pos[0]}..{pos[-1]}")
    M.mla_cache_append(d, dev(x), dev(seq), dev(pos), dev(wts["w_dkv"]), dev(wts["gamma"]),
                       dev(wts["w_kr"]), dev(table), nb, cache)
    torch.cuda.synchronize()
    cache = cache.cpu()
    ref = O.latent_rows(x, wts["w_dkv"], wts["gamma"], wts["w_kr"], pos, BASE, EPS)
    flat = cache.view(-1, w.row)
    slots = np.array([O.slot(table, 0, int(p), bs) for p in pos])
    got = flat[torch.from_numpy(slots)]
    assert ulp_close(got, ref, w.dtype)
    check(got, ref, 4e-3, "rows")
    # the rotary part alone, where the angle matters
    check(got[:, w.d_c:], ref[:, w.d_c:], 4e-3, "k_r")
    written = ~torch.isnan(flat.float()).all(dim=1).numpy()
    expect = np.zeros(nb * bs, bool)
    expect[slots] = True
    assert np.array_equal(written, expect)


@pytest.mark.parametrize("wl,s_q", [("smallem-fp32", 1), ("mid-bf16", 1), ("dsv3-paged", 1),
                                    ("gqla-g8", 4)])
def test_absorb_matches_oracle(wl, s_q):
    w = W.WORKLOADS[wl].replace(batch=3, s_q=s_q)
    q = W.queries(w)
    lens = np.array([5000, 17, 131000], np.int32)[:w.batch]
    qpos = W.query_positions(w, lens)
    wts = W.weights(w)
    d = M.dims_of(w)
    out = torch.empty(w.batch, s_q, w.n_heads, w.row, dtype=w.torch_dtype, device=DEV)
    note(f"absorb {wl} s_q={s_q}")
    M.mla_absorb_q(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), dev(wts["w_uk"]), out)
    torch.cuda.synchronize()
    ref = O.absorb_query(q["q_nope"], q["q_pe"], qpos, wts["w_uk"], w.n_groups, BASE)
    check(out.cpu(), ref, (1e-5 if w.dtype == "f32" else 4e-3))


@pytest.mark.parametrize("wl,lens,s_q", [("smallem-fp32", [512], 1), ("mid-bf16", [300, 45], 1),
                                         ("gqla-g8", [200], 2), ("dsv3-paged", [129, 1], 1)])
def test_end_to_end_matches_reconstructed_oracle(wl, lens, s_q):
    """x -> append -> absorb -> decode on the GPU versus keys and values rebuilt explicitly."""
    w = W.WORKLOADS[wl].replace(batch=len(lens), s_q=s_q)
    a = append_case(w, lens)
    note(f"end to end {wl} lens={lens} s_q={s_q}")
    cache = gpu_append(w, a)
    q = W.queries(w)
    qpos = W.query_positions(w, a["lens"])
    d = M.dims_of(w)
    q_abs = torch.empty(w.batch, s_q, w.n_heads, w.row, dtype=w.torch_dtype, device=DEV)
    M.mla_absorb_q(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), dev(a["wts"]["w_uk"]), q_abs)
    out = torch.empty(w.batch, s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    lse = torch.empty(w.batch, s_q, w.n_heads, dtype=torch.float32, device=DEV)
    M.mla_decode(d, q_abs, dev(cache), dev(a["table"]), dev(a["lens"]), dev(a["wts"]["w_uv"]),
                 out, lse)
    torch.cuda.synchronize()
    rows_all = O.round_storage(O.latent_rows(a["x"], a["wts"]["w_dkv"], a["wts"]["gamma"],
                                             a["wts"]["w_kr"], a["pos"], BASE, EPS), w.dtype)
    k = 0
    tol = TOL[w.dtype]
    for b, L in enumerate(a["lens"]):
        ref, ref_lse = O.decode_reconstructed(q["q_nope"][b], q["q_pe"][b], qpos[b],
                                              rows_all[k:k + L], a["wts"]["w_uk"],
                                              a["wts"]["w_uv"], w.n_groups, w.d_c, w.d_v, BASE)
        k += L
        check(out[b].cpu(), ref, tol)
        check_lse(lse[b].cpu().double().numpy(), ref_lse, tol)


def gqa_cache_empty(w, nb):
    return torch.full((nb, w.block_size, w.n_groups * (w.d_nope + w.d_v) + w.d_r), float("nan"),
                      dtype=w.torch_dtype, device=DEV)


def test_gqla_expand_matches_oracle():
    w = W.WORKLOADS["gqla-g8"]
    c = decode_case(w, [70, 129], extra=21)
    wts = W.weights(c["w"])
    start = np.array([0, 64], np.int32)   # second sequence: only positions 64.. are expanded
    d = M.dims_of(c["w"])
    g = gqa_cache_empty(w, c["nb"])
    note("gqla_expand with a start offset")
    M.gqla_expand(d, dev(c["pool"]), dev(c["table"]), dev(c["lens"]), dev(wts["w_uk"]),
                  dev(wts["w_uv"]), g, start_pos=dev(start))
    torch.cuda.synchronize()
    g = g.cpu()
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        ref = O.gqa_expand_rows(rows, wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c, w.d_nope, w.d_v)
        got = O.gather_rows(g, c["table"], b, int(L))
        s = int(start[b])
        if not ulp_close(got[s:], ref[s:], w.dtype):
            check(got[s:], ref[s:], 4e-3, "rows beyond one ulp")
        assert np.isnan(got[:s]).all()                   # prefix left untouched


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d_c", [128, 160])
def test_gqla_expand_ragged_shapes(dtype, d_c):
    """Expansion where the expanded width (3 groups x (24 + 16) = 120 columns) fills part of
    a column tile, d_c = 128 spans four 32-row latent chunks and d_c = 160 an odd number (five,
    the last after the two-chunk loop), and the lengths leave ragged position tiles (1, 255,
    257 and 600 positions, block size 16); bf16 runs on the matrix cores, fp32 on the portable
    kernel."""
    w = W.WORKLOADS["gqla-g8"].replace(n_groups=3, n_heads=6, d_nope=24, d_v=16, d_c=d_c, d_r=16,
                             block_size=16, dtype=dtype)
    c = decode_case(w, [1, 255, 257, 600], extra=23)
    wts = W.weights(c["w"])
    d = M.dims_of(c["w"])
    g = gqa_cache_empty(w, c["nb"])
    note(f"gqla_expand ragged shapes {dtype} d_c {d_c}")
    M.gqla_expand(d, dev(c["pool"]), dev(c["table"]), dev(c["lens"]), dev(wts["w_uk"]),
                  dev(wts["w_uv"]), g)
    torch.cuda.synchronize()
    g = g.cpu()
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        ref = O.gqa_expand_rows(rows, wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c, w.d_nope, w.d_v)
        got = O.gather_rows(g, c["table"], b, int(L))
        if dtype == "bf16":
            if not ulp_close(got, ref, w.dtype):
                check(got, ref, 4e-3, "rows beyond one ulp")
        else:
            check(got, ref, TOL["f32"])


@pytest.mark.parametrize("s_q", [1, 2, 4])
def test_gqla_paths_agree_with_oracle(s_q):
    """GQA path (expand once, then grouped decode) and absorbed path on the same weights and
    latents: both match the reconstructed oracle and each other."""
    w = W.WORKLOADS["gqla-g8"].replace(s_q=s_q)
    c = decode_case(w, [s_q, 333, 1100], s_q=s_q, extra=22)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    d = M.dims_of(c["w"])
    note(f"gqla both paths s_q={s_q}")
    g = gqa_cache_empty(w, c["nb"])
    M.gqla_expand(d, dev(c["pool"]), dev(c["table"]), dev(c["lens"]), dev(wts["w_uk"]),
                  dev(wts["w_uv"]), g)
    out_g = torch.empty(c["w"].batch, s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    lse_g = torch.empty(c["w"].batch, s_q, w.n_heads, dtype=torch.float32, device=DEV)
    M.gqla_decode(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), g, dev(c["table"]),
                  dev(c["lens"]), out_g, lse_g)
    q_abs = torch.empty(c["w"].batch, s_q, w.n_heads, w.row, dtype=w.torch_dtype, device=DEV)
    M.mla_absorb_q(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), dev(wts["w_uk"]), q_abs)
    out_a = torch.empty_like(out_g)
    M.mla_decode(d, q_abs, dev(c["pool"]), dev(c["table"]), dev(c["lens"]), dev(wts["w_uv"]), out_a)
    torch.cuda.synchronize()
    out_g, out_a = out_g.cpu(), out_a.cpu()
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        ref, ref_lse = O.decode_reconstructed(q["q_nope"][b], q["q_pe"][b], qpos[b], rows,
                                              wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c,
                                              w.d_v, BASE)
        check(out_g[b], ref, TOL["bf16"])
        check(out_a[b], ref, TOL["bf16"])
        check_lse(lse_g[b].cpu().double().numpy(), ref_lse, TOL["bf16"])
    check_per_seq(out_g, out_a.double(), TOL["bf16"], "GQA vs absorbed")


@pytest.mark.parametrize("s_q,n_split,bs,generic", [(1, 0, 64, False), (3, 7, 32, False),
                                                    (8, 64, 32, False), (2, 5, 32, True)])
def test_gqa_decode_matches_oracle(s_q, n_split, bs, generic):
    """gqla_decode alone, on an expanded cache written from the oracle's expansion (stored
    as bf16), against the oracle's grouped-query decode of those same rows: lengths from
    s_q to past several tiles and splits, few and many (mostly empty) splits, up to 64 query
    rows per group (H / G = 8 heads x s_q = 8), block sizes 32 and 64, and the portable
    kernel on the same case."""
    w = W.WORKLOADS["gqla-g8"].replace(n_heads=32, n_groups=4, block_size=bs, s_q=s_q)
    c = decode_case(w, [s_q, 31 + s_q, 33, 700], s_q=s_q, extra=24)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    d = M.dims_of(c["w"], generic=generic)
    gw = w.n_groups * (w.d_nope + w.d_v) + w.d_r
    g = torch.full((c["nb"] * bs, gw), float("nan"), dtype=torch.float64)
    rows_of = []
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        e = torch.from_numpy(O.gqa_expand_rows(rows, wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c,
                                               w.d_nope, w.d_v)).to(torch.bfloat16)
        rows_of.append(e.double().numpy())
        g[torch.from_numpy(O.seq_slots(c["table"], b, int(L), bs))] = e.double()
    g = g.to(torch.bfloat16).view(c["nb"], bs, gw)
    note(f"gqa decode s_q={s_q} n_split={n_split} bs={bs} generic={generic}")
    out = torch.empty(c["w"].batch, s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    lse = torch.empty(c["w"].batch, s_q, w.n_heads, dtype=torch.float32, device=DEV)
    M.gqla_decode(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), dev(g), dev(c["table"]),
                  dev(c["lens"]), out, lse, n_split=n_split)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu().double().numpy()
    for b in range(len(c["lens"])):
        ref, ref_lse = O.decode_gqa(q["q_nope"][b], q["q_pe"][b], qpos[b], rows_of[b], w.n_groups,
                                    w.d_v, BASE)
        check(out[b], ref, TOL["bf16"])
        check_lse(lse[b], ref_lse, TOL["bf16"])


@pytest.mark.parametrize("s_q", [1, 2, 4])
def test_gqla_full_size_sampled(s_q):
    """The GQLA workload at full size (32 sequences x 32,768 positions, G = 8), in the launch
    configuration the benchmark times (expansion of the whole cache, GQA decode with the
    library's automatic split count; from s_q = 4 on, 64 query rows per group, the shared-tile
    kernel with its split partials merged): the expanded rows of sampled positions and the
    outputs of sampled sequences, queries and heads against the oracle, computed one sequence
    at a time."""
    w = W.WORKLOADS["gqla-g8"].replace(s_q=s_q)
    lens = W.seq_lens(w)
    c = decode_case(w, lens, s_q=s_q, extra=25, poison=False)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    d = M.dims_of(c["w"])
    ns = M.mla_auto_split(d, w.batch, s_q, c["table"].shape[1])
    note(f"gqla full size B={w.batch} L={int(lens[0])} s_q={s_q} n_split={ns}")
    g = torch.empty(c["nb"], w.block_size, w.n_groups * (w.d_nope + w.d_v) + w.d_r,
                    dtype=w.torch_dtype, device=DEV)
    M.gqla_expand(d, dev(c["pool"]), dev(c["table"]), dev(c["lens"]), dev(wts["w_uk"]),
                  dev(wts["w_uv"]), g)
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    lse = torch.empty(w.batch, w.s_q, w.n_heads, dtype=torch.float32, device=DEV)
    M.gqla_decode(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), g, dev(c["table"]),
                  dev(c["lens"]), out, lse, n_split=ns)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu().double().numpy()
    heads = [0, 77, w.n_heads - 1]
    gflat = g.view(-1, g.shape[-1])
    for b in (0, w.batch - 1):
        L = int(c["lens"][b])
        rows = O.gather_rows(c["pool"], c["table"], b, L)
        slots = O.seq_slots(c["table"], b, L, w.block_size)
        pick_pos = np.array([0, 1, 31, 32, 4095, L // 2, L - 1])
        ref_rows = O.gqa_expand_rows(rows[pick_pos], wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c,
                                     w.d_nope, w.d_v)
        got = gflat[torch.from_numpy(slots[pick_pos])].cpu()
        if not ulp_close(got, ref_rows, w.dtype):
            check(got, ref_rows, 4e-3, "rows beyond one ulp")
        # decode of the sampled heads over the GPU-expanded rows (isolates the decode error)
        exp_rows = O.f64(gflat[torch.from_numpy(slots)].cpu())
        ref, ref_lse = O.decode_gqa(q["q_nope"][b], q["q_pe"][b], qpos[b], exp_rows, w.n_groups,
                                    w.d_v, BASE, heads=heads)
        check(out[b][:, heads], ref, TOL["bf16"])
        check_lse(lse[b][:, heads], ref_lse, TOL["bf16"])
