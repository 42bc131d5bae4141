"""GPU parity of mla_prefill: attention of many new tokens per sequence over the latent cache
in the expanded, concatenated-score form of the no-cache pass (Smallem article 13, "Le code"
and "Deux produits ou une concaténation ?"), against the oracle's reconstructed attention
(every head's K and V rebuilt from the latents), which is the prefill written out."""
import pytest
import torch

import oracle as O
import workloads as W
from gpu_cases import (DEV, TOL, check, check_lse, decode_case, dev, note)
from mla_latent_kv_21_amd import binding as M

pytestmark = pytest.mark.gpu

BASE = 10000.0


def run_prefill(c, q, qpos, wts):
    w = c["w"]
    d = M.dims_of(w)
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    lse = torch.empty(w.batch, w.s_q, w.n_heads, dtype=torch.float32, device=DEV)
    M.mla_prefill(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), dev(c["pool"]),
                  dev(c["table"]), dev(c["lens"]), dev(wts["w_uk"]), dev(wts["w_uv"]), out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# (workload, lengths, s_q): a full prefill beside a chunk appended to 53 cached positions
# (MLA, one key and value per head); the GQLA grouping (G = 8) with two chunks of 260 over
# 300 and 260 positions; the Smallem shape (fp32, H 8, D 64, d_r 32, portable kernels) at
# 128 new tokens; single-token steps (one query row per head, split-K partials merged); and
# 200 new tokens per head (a full and a ragged block of 128 query rows in the prefill kernel)
CASES = [("dsv3-paged", [150, 97], 97), ("gqla-g8", [300, 260], 260),
         ("smallem-fp32", [128, 200], 128), ("dsv3-paged", [5, 300], 1),
         ("dsv3-paged", [300, 200], 200)]


@pytest.mark.parametrize("wl,lens,s_q", CASES)
def test_prefill_matches_reconstructed_oracle(wl, lens, s_q):
    w = W.WORKLOADS[wl].replace(s_q=s_q)
    c = decode_case(w, lens, s_q=s_q, extra=41)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    note(f"mla_prefill {wl} lens={lens} s_q={s_q}")
    out, lse = run_prefill(c, q, qpos, wts)
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        ref, ref_lse = O.decode_reconstructed(q["q_nope"][b], q["q_pe"][b], qpos[b], rows,
                                              wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c,
                                              w.d_v, BASE)
        check(out[b], ref, TOL[w.dtype])
        check_lse(lse[b].double().numpy(), ref_lse, TOL[w.dtype])


def test_prefill_4k_sampled_rows():
    """The full prefill workload (two 4,096-token prompts, H = 128, every position a query) in
    the launch configuration the benchmark times, checked on sampled (query, head) outputs the
    oracle computes one by one: the first and last queries, either side of a 32-row block
    boundary and the middle, on three heads of each sequence; every output finite."""
    w = W.WORKLOADS["prefill-4k"]
    lens = W.seq_lens(w)
    c = decode_case(w, lens, s_q=w.s_q, extra=42)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    note("mla_prefill prefill-4k sampled rows")
    out, lse = run_prefill(c, q, qpos, wts)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    heads = [0, 37, 127]
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        for i in (0, 31, 32, 2047, int(L) - 1):
            n = int(L) - w.s_q + i + 1   # positions query i sees
            ref, ref_lse = O.decode_reconstructed(q["q_nope"][b][i:i + 1], q["q_pe"][b][i:i + 1],
                                                  qpos[b][i:i + 1], rows[:n], wts["w_uk"],
                                                  wts["w_uv"], w.n_groups, w.d_c, w.d_v, BASE,
                                                  heads=heads)
            got = out[b, i, heads]
            check(got, ref[0], TOL[w.dtype], f"(b, i) = {(b, i)}")
            check_lse(lse[b, i, heads].double().numpy(), ref_lse[0], TOL[w.dtype])


def test_prefill_equals_expand_then_grouped_decode():
    """mla_prefill is gqla_expand of the sequences' positions then gqla_decode over them: the
    two ways give the same bits."""
    w = W.WORKLOADS["gqla-g8"].replace(s_q=200)
    c = decode_case(w, [200, 333], s_q=200, extra=43)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    d = M.dims_of(c["w"])
    note("mla_prefill against expand + gqla_decode")
    out, lse = run_prefill(c, q, qpos, wts)
    g = torch.empty(c["nb"], w.block_size, w.n_groups * (w.d_nope + w.d_v) + w.d_r,
                    dtype=w.torch_dtype, device=DEV)
    M.gqla_expand(d, dev(c["pool"]), dev(c["table"]), dev(c["lens"]), dev(wts["w_uk"]),
                  dev(wts["w_uv"]), g)
    out2 = torch.empty(c["w"].batch, 200, w.n_heads, w.d_v, dtype=w.torch_dtype, device=DEV)
    M.gqla_decode(d, dev(q["q_nope"]), dev(q["q_pe"]), dev(qpos), g, dev(c["table"]),
                  dev(c["lens"]), out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2.cpu())


def test_prefill_kernel_block_size_32_and_eight_heads_per_group():
    """The prefill kernel (one split: B s_q >= 256) with 32-position cache blocks, so every tile
    is a whole block, and 8 heads per group, so a 32-row block mixes query tokens and heads
    (row n -> token n / 8, head n % 8); lengths leave ragged last blocks."""
    w = W.WORKLOADS["gqla-g8"].replace(n_heads=32, n_groups=4, block_size=32, s_q=100)
    c = decode_case(w, [100, 177, 300], s_q=100, extra=44)
    wts = W.weights(c["w"])
    q = W.queries(c["w"])
    qpos = W.query_positions(c["w"], c["lens"])
    note("mla_prefill bs 32, H 32, G 4, s_q 100")
    out, lse = run_prefill(c, q, qpos, wts)
    for b, L in enumerate(c["lens"]):
        rows = O.gather_rows(c["pool"], c["table"], b, int(L))
        ref, ref_lse = O.decode_reconstructed(q["q_nope"][b], q["q_pe"][b], qpos[b], rows,
                                              wts["w_uk"], wts["w_uv"], w.n_groups, w.d_c,
                                              w.d_v, BASE)
        check(out[b], ref, TOL[w.dtype])
        check_lse(lse[b].double().numpy(), ref_lse, TOL[w.dtype])
