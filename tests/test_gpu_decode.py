"""GPU parity of mla_decode (split-K core + log-sum-exp combine + W_UV) against the oracle.

Inputs are seeded synthetic latent rows in a paged cache whose unowned slots hold NaN, so a
read past a sequence end or through a wrong block id poisons the result. Both the MFMA kernel
and the portable kernel are checked; the MFMA path must not have needed its recompute
fallback (its flags are read back from the workspace). Tolerances: normwise 2e-2 for bf16 and
1e-4 for fp32 outputs, lse within the same bound.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import (PLAN_SLOTS, TOL, check_lse, check_per_seq, decode_case, note,
                       oracle_decode, pick, run_decode, stream_tag)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    # (name, workload, lens, s_q, n_split)
    ("smallem-f32", "smallem-fp32", [512], 1, 0),
    ("smallem-f32-ragged", "smallem-fp32", [1, 77, 300], 1, 3),
    ("mid-h32", "mid-bf16", [1, 65, 1000], 1, 0),
    ("mid-h32-split7", "mid-bf16", [700, 2049], 1, 7),
    ("paged-h128-ragged", "dsv3-paged", [64, 33, 2600], 1, 0),
    ("paged-h128-split1", "dsv3-paged", [1500], 1, 1),
    ("long-h128-many-splits", "long-128k", [4096, 100], 1, 64),
    ("gqla-g8-sq2", "gqla-g8", [2, 300], 2, 0),
    ("gqla-g8-sq4", "gqla-g8", [4, 257, 1030], 4, 5),
]


@pytest.mark.parametrize("name,wl,lens,s_q,n_split", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("generic", [False, True], ids=["mfma", "portable"])
def test_decode_matches_oracle(name, wl, lens, s_q, n_split, generic):
    w = W.WORKLOADS[wl]
    c = decode_case(w, lens, s_q=s_q, extra=stream_tag(w))
    note(f"decode {name} generic={generic} lens={lens} s_q={s_q} n_split={n_split}")
    out, lse, flags = run_decode(c, n_split=n_split, generic=generic)
    ref, ref_lse = oracle_decode(c)
    tol = TOL[w.dtype]
    check_per_seq(out, ref, tol)
    check_lse(lse.double().numpy(), ref_lse, tol)
    if not generic and w.dtype == "bf16":
        assert not flags.any(), "MFMA kernel fell back to the portable kernel"


def test_split_count_invariance():
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [3000, 200], extra=11)
    ref, _ = oracle_decode(c)
    outs = []
    for ns in (1, 2, 7, 64):
        note(f"decode split invariance n_split={ns}")
        out, _, _ = run_decode(c, n_split=ns)
        check_per_seq(out, ref, TOL["bf16"])
        outs.append(out.double())
    for o in outs[1:]:
        check_per_seq(o, outs[0], TOL["bf16"])


def test_block_permutation_is_bit_exact():
    """Renumbering physical blocks (same logical content) leaves every output bit unchanged."""
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [1000, 257, 64], extra=12, poison=False)
    note("decode block permutation (original ids)")
    out_a, lse_a, _ = run_decode(c, n_split=5)
    nb, bs, row = c["pool"].shape
    perm = np.random.default_rng(5).permutation(nb)
    pool_b = torch.empty_like(c["pool"])
    pool_b[torch.from_numpy(perm)] = c["pool"]          # block i moves to perm[i]
    table_b = c["table"].copy()
    used = table_b >= 0
    table_b[used] = perm[table_b[used]]
    c2 = dict(c, pool=pool_b, table=table_b)
    note("decode block permutation (renumbered ids)")
    out_b, lse_b, _ = run_decode(c2, n_split=5)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_a, lse_b)


def test_recompute_fallback_for_outgrown_reference():
    """A late position whose score beats the split's first tile by far more than 2^64 (log2)
    is flagged by the MFMA kernel and recomputed exactly by the portable kernel."""
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [2048], extra=13, random_table=False, poison=False)
    q = c["q_abs"][0, 0].float()
    # position 1500 of sequence 0 (identity table, block 23, row 28): 4x the query of head 5
    c["pool"][1500 // 64, 1500 % 64] = (4.0 * q[5]).to(torch.bfloat16)
    note("decode outgrown reference -> recompute")
    out, lse, flags = run_decode(c, n_split=2)
    assert flags.any(), "expected the MFMA kernel to flag the split"
    ref, ref_lse = oracle_decode(c)
    check_per_seq(out, ref, TOL["bf16"])
    check_lse(lse.double().numpy(), ref_lse, TOL["bf16"])


def test_single_position_and_minimum_lengths():
    """L = 1 (out = that position's value projection) and L = s_q for multi-token steps."""
    for wl, lens, s_q in (("dsv3-paged", [1, 1], 1), ("gqla-g8", [4, 4], 4), ("mid-bf16", [2], 2)):
        w = W.WORKLOADS[wl]
        c = decode_case(w, lens, s_q=s_q, extra=14)
        note(f"decode minimum lengths {wl} lens={lens} s_q={s_q}")
        out, lse, _ = run_decode(c)
        ref, ref_lse = oracle_decode(c)
        check_per_seq(out, ref, TOL[w.dtype])


def test_unused_table_entries_and_spare_capacity():
    """max_blocks larger than any sequence needs; entries past ceil(L/bs) hold -1."""
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [130, 64], extra=15, max_blocks=40)
    assert (c["table"][:, 3:] == -1).all()
    note("decode spare table capacity")
    out, _, _ = run_decode(c)
    ref, _ = oracle_decode(c)
    check_per_seq(out, ref, TOL["bf16"])


FULL_SIZE = [
    # (workload, s_q, planned): the split scheme each workload's benchmark row uses
    ("dsv3-paged", 1, True),     # balanced plan over 64 mixed lengths
    ("long-128k", 1, False),     # 64 uniform splits of 2,048 positions
    ("gqla-g8", 1, True),
    ("gqla-g8", 2, True),
    ("gqla-g8", 4, True),
]


@pytest.mark.parametrize("wl,s_q,planned", FULL_SIZE, ids=[f"{w}-sq{s}" for w, s, _ in FULL_SIZE])
def test_full_size_sampled(wl, s_q, planned):
    """Full workload shapes, in the launch configuration the benchmark times, checked on a
    sample of sequences and heads that the oracle computes one by one."""
    w = W.WORKLOADS[wl].replace(s_q=s_q)
    lens = W.seq_lens(w)
    c = decode_case(w, lens, s_q=s_q, extra=16, poison=False)
    note(f"decode full size {wl} s_q={s_q} planned={planned} B={w.batch} "
         f"sum(L)={int(lens.sum())}")
    out, lse, flags = run_decode(c, n_split=w.n_split, planned=planned)
    assert not flags.any()
    seqs = sorted({0, w.batch - 1, int(np.argmax(lens))})
    heads = [0, 37, w.n_heads - 1]
    ref, ref_lse = oracle_decode(c, seqs=seqs, heads=heads)
    check_per_seq(pick(out, seqs, heads), ref, TOL["bf16"])
    check_lse(pick(lse, seqs, heads), ref_lse, TOL["bf16"])


def test_mid_bf16_full_size():
    """The mid-size workload whole (16 sequences x 4,096 positions, H = 32), every sequence
    and head against the oracle, with the balanced plan and with the library's uniform
    split count."""
    w = W.WORKLOADS["mid-bf16"]
    lens = W.seq_lens(w)
    c = decode_case(w, lens, extra=17, poison=False)
    ref, ref_lse = oracle_decode(c)
    for planned in (True, False):
        note(f"decode mid-bf16 full size planned={planned}")
        out, lse, flags = run_decode(c, planned=planned)
        assert not flags.any()
        check_per_seq(out, ref, TOL["bf16"], f"out planned={planned}")
        check_lse(lse.double().numpy(), ref_lse, TOL["bf16"])


# ---- length-balanced split plan (n_split = 0 on the matrix-core path)

def expected_plan(lens, s_q, capacity, slots=PLAN_SLOTS, cap=64, align=64):
    """The plan's rule on the host: the smallest chunk (a multiple of `align`) for which the
    rows (b, i) need at most `slots` splits in all and at most `cap` each; row m takes
    ceil(lim_m / chunk) splits, numbered in row order."""
    lims = [max(0, min(L - s_q + i + 1, capacity)) for L in lens for i in range(s_q)]
    up = lambda x: -(-x // align) * align
    chunk = up(max(-(-sum(lims) // slots), -(-max(lims) // cap), 1))
    while sum(-(-l // chunk) for l in lims) > slots:
        chunk += align
    counts = [-(-l // chunk) for l in lims]
    return chunk, sum(counts), np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


PLAN_CASES = [
    # (name, workload, lens, s_q)
    ("paged-mixed", "dsv3-paged", [64, 33, 2600, 1, 5000, 1024], 1),
    ("paged-one-long", "dsv3-paged", [8000, 1, 2, 3], 1),
    ("mid-h32-mixed", "mid-bf16", [1, 65, 1000, 4096], 1),
    ("gqla-g8-sq4", "gqla-g8", [4, 257, 1030, 3000], 4),
    ("long-h128", "long-128k", [20000, 300], 1),
]


@pytest.mark.parametrize("name,wl,lens,s_q", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_planned_decode_matches_oracle(name, wl, lens, s_q):
    """n_split = 0: the library cuts mixed-length rows into chunks of one size chosen on the
    device; outputs match the oracle, the stored plan matches the host rule exactly, and no
    split needed the recompute."""
    w = W.WORKLOADS[wl]
    c = decode_case(w, lens, s_q=s_q, extra=40 + stream_tag(w))
    note(f"planned decode {name} lens={lens} s_q={s_q}")
    wss = []
    out, lse, flags = run_decode(c, planned=True, ws_out=wss)
    ref, ref_lse = oracle_decode(c)
    check_per_seq(out, ref, TOL["bf16"])
    check_lse(lse.double().numpy(), ref_lse, TOL["bf16"])
    plan = wss[0][:1024].view(torch.int32).numpy()
    rows = len(lens) * s_q
    chunk, total, first = expected_plan(c["lens"], s_q, c["table"].shape[1] * w.block_size)
    assert plan[0] == chunk and plan[1] == total
    assert np.array_equal(plan[2:2 + rows + 1], first)
    assert total <= PLAN_SLOTS
    assert not flags[:total].any()


def test_planned_recompute_fallback():
    """The recompute of a flagged split follows the plan's chunk and slot layout. The plan cuts
    these rows into 64-position splits; position 1530 lies in the second tile of its split
    (1472 .. 1535), after the tile that set the split's reference."""
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [2048, 300], extra=45, random_table=False, poison=False)
    chunk, _, _ = expected_plan(c["lens"], 1, c["table"].shape[1] * w.block_size)
    assert chunk == 64
    q = c["q_abs"][0, 0].float()
    c["pool"][1530 // 64, 1530 % 64] = (4.0 * q[5]).to(torch.bfloat16)
    note("planned decode outgrown reference -> recompute")
    out, lse, flags = run_decode(c, planned=True)
    assert flags.any(), "expected the MFMA kernel to flag a split"
    ref, ref_lse = oracle_decode(c)
    check_per_seq(out, ref, TOL["bf16"])
    check_lse(lse.double().numpy(), ref_lse, TOL["bf16"])


def test_planned_matches_uniform_and_falls_back_past_128_rows():
    """Planned and uniform splits agree; a batch of more than 128 query rows takes the
    uniform split even with n_split = 0."""
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [3000, 200, 64], extra=46)
    note("planned vs uniform")
    out_p, _, _ = run_decode(c, planned=True)
    out_u, _, _ = run_decode(c, n_split=7)
    check_per_seq(out_p, out_u.double(), TOL["bf16"])
    lens = (np.arange(130) * 37) % 500 + 1
    c2 = decode_case(w, lens, extra=47)
    note("planned request with 130 rows")
    out, _, _ = run_decode(c2, planned=True)
    ref, _ = oracle_decode(c2, seqs=[0, 64, 129], heads=[0, 127])
    check_per_seq(pick(out, [0, 64, 129], [0, 127]), ref, TOL["bf16"])


@pytest.mark.parametrize("generic", [False, True], ids=["mfma", "portable"])
@pytest.mark.parametrize("lens,s_q,n_split", [([1, 65, 1000], 1, 0), ([700, 2049, 33], 2, 7)],
                         ids=["planned", "sq2-split7"])
def test_decode_h64_matches_oracle(lens, s_q, n_split, generic):
    """H = 64 (two blocks of 32 heads, each block's scores formed by two of the four waves)."""
    w = W.WORKLOADS["mid-bf16"].replace(n_heads=64, n_groups=64)
    c = decode_case(w, lens, s_q=s_q, extra=stream_tag(w) + 3)
    note(f"decode h64 generic={generic} lens={lens} s_q={s_q} n_split={n_split}")
    out, lse, flags = run_decode(c, n_split=n_split, generic=generic)
    ref, ref_lse = oracle_decode(c)
    check_per_seq(out, ref, TOL[w.dtype])
    check_lse(lse.double().numpy(), ref_lse, TOL[w.dtype])
    if not generic:
        assert not flags.any(), "MFMA kernel fell back to the portable kernel"


@pytest.mark.parametrize("heads", [32, 64])
def test_small_head_counts_on_ragged_lengths(heads):
    """H = 32 (the score contraction split over four waves) and H = 64 (two waves per head
    block) over lengths around the 32-position tile and 64-position block edges, planned and
    uniform splits, s_q = 1 and 3."""
    w = W.WORKLOADS["mid-bf16"].replace(n_heads=heads, n_groups=heads)
    lens = [1, 2, 31, 32, 33, 64, 65, 97, 160, 1000]
    for s_q, n_split in ((1, 0), (1, 7), (3, 0)):
        ls = [max(L, s_q) for L in lens]
        c = decode_case(w, ls, s_q=s_q, extra=stream_tag(w) + 5 + s_q)
        note(f"decode H={heads} ragged s_q={s_q} n_split={n_split}")
        out, lse, flags = run_decode(c, n_split=n_split)
        ref, ref_lse = oracle_decode(c)
        check_per_seq(out, ref, TOL[w.dtype])
        check_lse(lse.double().numpy(), ref_lse, TOL[w.dtype])
        assert not flags.any(), "MFMA kernel fell back to the portable kernel"


@pytest.mark.parametrize("bs", [32, 128])
@pytest.mark.parametrize("wl", ["dsv3-paged", "mid-bf16"])
def test_block_sizes_and_long_splits(wl, bs):
    """Cache blocks of 32 and 128 positions, with single-split sequences long enough (5,000
    positions: 157 blocks of 32) that a workgroup walks past its first 64 block ids and reloads
    them, and planned splits; H = 128 and H = 32."""
    w = W.WORKLOADS[wl].replace(block_size=bs)
    c = decode_case(w, [5000, 2100, 33], extra=stream_tag(w) + bs)
    ref, ref_lse = oracle_decode(c)
    for n_split in (1, 0):
        note(f"decode {wl} block_size={bs} n_split={n_split}")
        out, lse, flags = run_decode(c, n_split=n_split)
        check_per_seq(out, ref, TOL[w.dtype])
        check_lse(lse.double().numpy(), ref_lse, TOL[w.dtype])
        assert not flags.any(), "MFMA kernel fell back to the portable kernel"


@pytest.mark.parametrize("wl", ["dsv3-paged", "mid-bf16"])
def test_the_largest_split_count(wl):
    """n_split = 256 (the most the library takes): 20,000 positions in 64-position splits
    beside a 70-position sequence whose splits are nearly all empty (weight zero)."""
    w = W.WORKLOADS[wl]
    c = decode_case(w, [20000, 70], extra=stream_tag(w) + 256)
    note(f"decode {wl} n_split=256")
    out, lse, flags = run_decode(c, n_split=256)
    ref, ref_lse = oracle_decode(c)
    check_per_seq(out, ref, TOL[w.dtype])
    check_lse(lse.double().numpy(), ref_lse, TOL[w.dtype])
    assert not flags.any(), "MFMA kernel fell back to the portable kernel"


@pytest.mark.parametrize("generic", [False, True], ids=["mfma", "portable"])
@pytest.mark.parametrize("n_split", [0, 3])
def test_queries_with_nothing_visible(n_split, generic):
    """A sequence of length 0 (its query sees no position) gets out = 0 and lse = -inf, as the
    header states, beside an ordinary sequence, on either split layout."""
    w = W.WORKLOADS["dsv3-paged"]
    c = decode_case(w, [0, 300, 0], extra=stream_tag(w) + 40)
    note(f"decode nothing visible n_split={n_split} generic={generic}")
    out, lse, _ = run_decode(c, n_split=n_split, generic=generic)
    for b in (0, 2):
        assert torch.equal(out[b].float(), torch.zeros_like(out[b].float())), f"sequence {b}"
        assert bool(torch.isinf(lse[b]).all()) and bool((lse[b] < 0).all())
    ref, ref_lse = oracle_decode(c, seqs=[1])
    check_per_seq(out[1:2], ref, TOL[w.dtype])
    check_lse(lse[1:2].double().numpy(), ref_lse, TOL[w.dtype])
