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
from gpu_cases import TOL, decode_case, note, oracle_decode, pick, rel_err, run_decode

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    # (name, config, lens, s_q, n_split)
    ("c1-f32", 1, [512], 1, 0),
    ("c1-f32-ragged", 1, [1, 77, 300], 1, 3),
    ("c2-h32", 2, [1, 65, 1000], 1, 0),
    ("c2-h32-split7", 2, [700, 2049], 1, 7),
    ("c3-h128-ragged", 3, [64, 33, 2600], 1, 0),
    ("c3-h128-split1", 3, [1500], 1, 1),
    ("c4-h128-many-splits", 4, [4096, 100], 1, 64),
    ("c5-g8-sq2", 5, [2, 300], 2, 0),
    ("c5-g8-sq4", 5, [4, 257, 1030], 4, 5),
]


@pytest.mark.parametrize("name,cfg,lens,s_q,n_split", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("generic", [False, True], ids=["mfma", "portable"])
def test_decode_matches_oracle(name, cfg, lens, s_q, n_split, generic):
    w = W.CONFIGS[cfg]
    c = decode_case(w, lens, s_q=s_q, extra=cfg)
    note(f"decode {name} generic={generic} lens={lens} s_q={s_q} n_split={n_split}")
    out, lse, flags = run_decode(c, n_split=n_split, generic=generic)
    ref, ref_lse = oracle_decode(c)
    tol = TOL[w.dtype]
    assert rel_err(out, ref) <= tol
    assert np.max(np.abs(lse.double().numpy() - ref_lse)) <= tol
    if not generic and w.dtype == "bf16":
        assert not flags.any(), "MFMA kernel fell back to the portable kernel"


def test_split_count_invariance():
    w = W.CONFIGS[3]
    c = decode_case(w, [3000, 200], extra=11)
    ref, _ = oracle_decode(c)
    outs = []
    for ns in (1, 2, 7, 64):
        note(f"decode split invariance n_split={ns}")
        out, _, _ = run_decode(c, n_split=ns)
        assert rel_err(out, ref) <= TOL["bf16"]
        outs.append(out.double())
    for o in outs[1:]:
        assert rel_err(o, outs[0]) <= TOL["bf16"]


def test_block_permutation_is_bit_exact():
    """Renumbering physical blocks (same logical content) leaves every output bit unchanged."""
    w = W.CONFIGS[3]
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
    w = W.CONFIGS[3]
    c = decode_case(w, [2048], extra=13, random_table=False, poison=False)
    q = c["q_abs"][0, 0].float()
    # position 1500 of sequence 0 (identity table, block 23, row 28): 4x the query of head 5
    c["pool"][1500 // 64, 1500 % 64] = (4.0 * q[5]).to(torch.bfloat16)
    note("decode outgrown reference -> recompute")
    out, lse, flags = run_decode(c, n_split=2)
    assert flags.any(), "expected the MFMA kernel to flag the split"
    ref, ref_lse = oracle_decode(c)
    assert rel_err(out, ref) <= TOL["bf16"]
    assert np.max(np.abs(lse.double().numpy() - ref_lse)) <= TOL["bf16"]


def test_single_position_and_minimum_lengths():
    """L = 1 (out = that position's value projection) and L = s_q for multi-token steps."""
    for cfg, lens, s_q in ((3, [1, 1], 1), (5, [4, 4], 4), (2, [2], 2)):
        w = W.CONFIGS[cfg]
        c = decode_case(w, lens, s_q=s_q, extra=14)
        note(f"decode minimum lengths cfg={cfg} lens={lens} s_q={s_q}")
        out, lse, _ = run_decode(c)
        ref, ref_lse = oracle_decode(c)
        assert rel_err(out, ref) <= TOL[w.dtype]


def test_unused_table_entries_and_spare_capacity():
    """max_blocks larger than any sequence needs; entries past ceil(L/bs) hold -1."""
    w = W.CONFIGS[3]
    c = decode_case(w, [130, 64], extra=15, max_blocks=40)
    assert (c["table"][:, 3:] == -1).all()
    note("decode spare table capacity")
    out, _, _ = run_decode(c)
    ref, _ = oracle_decode(c)
    assert rel_err(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("cfg,s_q", [(3, 1), (4, 1), (5, 1), (5, 4)])
def test_full_size_sampled(cfg, s_q):
    """Full workload shapes, in the launch configuration the benchmark times, checked on a
    sample of sequences and heads that the oracle computes one by one."""
    w = W.CONFIGS[cfg].replace(s_q=s_q)
    lens = W.seq_lens(w)
    c = decode_case(w, lens, s_q=s_q, extra=16, poison=False)
    note(f"decode full size cfg={cfg} s_q={s_q} B={w.batch} sum(L)={int(lens.sum())}")
    out, lse, flags = run_decode(c, n_split=w.n_split)
    assert not flags.any()
    seqs = sorted({0, w.batch - 1, int(np.argmax(lens))})
    heads = [0, 37, w.n_heads - 1]
    ref, ref_lse = oracle_decode(c, seqs=seqs, heads=heads)
    assert rel_err(pick(out, seqs, heads), ref) <= TOL["bf16"]
    assert np.max(np.abs(pick(lse, seqs, heads) - ref_lse)) <= TOL["bf16"]
