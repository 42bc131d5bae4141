"""Pins that tie the CPU oracle to something other than itself (no GPU needed).

* brute force: a pure-Python loop re-derivation (tests/bruteforce.py), the way the Smallem
  article checks its layer, on tiny shapes, agrees to 1e-12;
* library / textbook special cases: torch's float32->bfloat16 cast, complex-number
  rotation, torch's scaled_dot_product_attention in f64;
* closed special cases: one position gives that position's value exactly, a zero query
  gives the plain mean of the values;
* invariants: shifting every position leaves the output unchanged (relative RoPE), a
  multi-token step equals single-token steps at the matching lengths (causality), the
  absorbed and GQA forms equal the reconstructed one to 1e-11 (the pages' own agreement
  bound for the hand-written layer, Smallem "Vérifier une couche compliquée"), replicating
  group weights per head turns GQLA into MLA;
* planted mistakes: each plausible slip (wrong scale, reversed rotation, wrong group map,
  off-by-one visibility, dropped rotary term, mean vs sum in the norm) makes at least one
  of the pins above fail.
"""
import math

import numpy as np
import pytest
import torch

import bruteforce as BF
import oracle as O
from oracle import mla_oracle as OM

BASE = 10000.0
EPS = 1e-6


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch_cast_on_f32_values():
    r = np.random.default_rng(1)
    a = np.concatenate([
        r.standard_normal(200_000).astype(np.float32) * np.float32(1e3),
        r.standard_normal(1000).astype(np.float32) * np.float32(1e-38),   # subnormal range
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.3895e38, 0.0, 2 ** -133],
                 np.float32)])
    mine = O.round_bf16(a.astype(np.float64))
    ref = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, ref)


def test_round_bf16_single_rounding_of_f64():
    # just above a tie: the correct result rounds up; a double rounding through float32
    # would first land on the tie and then go to even (down)
    x = 1 + 2 ** -8 + 2 ** -40
    assert O.round_bf16(np.array([x]))[0] == 1 + 2 ** -7
    assert O.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0          # tie -> even
    assert O.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6  # tie -> even (up)
    assert np.isinf(O.round_bf16(np.array([2.0 ** 128]))[0])


# ----------------------------------------------------------------------------- RoPE / RMSNorm
def test_rope_is_complex_rotation():
    r = np.random.default_rng(2)
    v = r.standard_normal((5, 8))
    pos = np.array([0, 1, 7, 1000, 131071])
    out = O.rope(v, pos, BASE)
    z = v[:, 0::2] + 1j * v[:, 1::2]
    theta = BASE ** (-np.arange(4) * 2.0 / 8)
    w = z * np.exp(1j * pos[:, None] * theta)
    assert np.allclose(out[:, 0::2], w.real, rtol=0, atol=1e-12)
    assert np.allclose(out[:, 1::2], w.imag, rtol=0, atol=1e-12)
    assert np.array_equal(O.rope(v[:1], np.array([0]), BASE), v[:1])
    # first pair has frequency 1: (1, 0) at position 1 goes to (cos 1, sin 1)
    e = np.zeros(8); e[0] = 1
    assert np.allclose(O.rope(e, 1, BASE)[:2], [math.cos(1), math.sin(1)], atol=1e-15)
    assert np.allclose(np.linalg.norm(out, axis=1), np.linalg.norm(v, axis=1), atol=1e-12)


def test_rope_scores_depend_on_offset_only():
    r = np.random.default_rng(3)
    q, k = r.standard_normal(16), r.standard_normal(16)
    s0 = O.rope(q, 40, BASE) @ O.rope(k, 13, BASE)
    for shift in (1, 77, 5000):
        s1 = O.rope(q, 40 + shift, BASE) @ O.rope(k, 13 + shift, BASE)
        assert abs(s1 - s0) < 1e-10


def test_rms_norm_closed_forms():
    r = np.random.default_rng(4)
    y = r.standard_normal((3, 32))
    n = O.rms_norm(y, np.ones(32), 0.0)
    assert np.allclose(np.mean(n * n, axis=1), 1.0, atol=1e-14)
    assert np.allclose(O.rms_norm(7.5 * y, np.ones(32), 0.0), n, atol=1e-14)
    g = r.standard_normal(32)
    assert np.allclose(O.rms_norm(y, g, 0.0), n * g, atol=1e-14)


# ----------------------------------------------------------------------------- tiny problems
def tiny_problem(seed, H=4, G=2, D=4, Dv=3, d_c=4, d_r=2, C=6, L=5, s_q=1, gamma_random=True):
    r = np.random.default_rng(seed)
    p = dict(
        x=r.standard_normal((L, C)),
        w_dkv=r.standard_normal((C, d_c)) / math.sqrt(C),
        gamma=(1 + 0.3 * r.standard_normal(d_c)) if gamma_random else np.ones(d_c),
        w_kr=r.standard_normal((C, d_r)) / math.sqrt(C),
        w_uk=r.standard_normal((d_c, G * D)) / math.sqrt(d_c),
        w_uv=r.standard_normal((d_c, G * Dv)) / math.sqrt(d_c),
        q_nope=r.standard_normal((s_q, H, D)),
        q_pe=r.standard_normal((s_q, H, d_r)),
        q_pos=np.array([L - s_q + i for i in range(s_q)]),
        pos=np.arange(L),
    )
    p.update(H=H, G=G, D=D, Dv=Dv, d_c=d_c, d_r=d_r, L=L, s_q=s_q)
    return p


def oracle_decode(p, hist=None, fn=None):
    fn = fn or O.decode_reconstructed
    if hist is None:
        hist = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
    return fn(p["q_nope"], p["q_pe"], p["q_pos"], hist, p["w_uk"], p["w_uv"], p["G"], p["d_c"],
              p["Dv"], BASE)


def brute_decode(p):
    tolist = lambda a: np.asarray(a).tolist()
    hist = [BF.cache_row(tolist(p["x"][t]), tolist(p["w_dkv"]), tolist(p["gamma"]),
                         tolist(p["w_kr"]), int(p["pos"][t]), BASE, EPS) for t in range(p["L"])]
    out, lse = BF.decode(tolist(p["q_nope"]), tolist(p["q_pe"]), tolist(p["q_pos"]), hist,
                         tolist(p["w_uk"]), tolist(p["w_uv"]), p["G"], p["d_c"], p["Dv"], BASE)
    return np.array(hist), np.array(out), np.array(lse)


TINY = [
    dict(H=1, G=1, D=2, Dv=2, d_c=3, d_r=2, L=1),
    dict(H=2, G=1, D=4, Dv=3, d_c=3, d_r=2, L=2),
    dict(H=4, G=2, D=4, Dv=4, d_c=4, d_r=2, L=5),
    dict(H=4, G=4, D=2, Dv=3, d_c=4, d_r=2, L=5, s_q=2),
    dict(H=4, G=2, D=4, Dv=2, d_c=3, d_r=4, L=7, s_q=3),
]


def check_core_pins(seed=0):
    """Run the brute-force pins; return a list of failure strings (empty = all hold)."""
    bad = []
    for k, shp in enumerate(TINY):
        p = tiny_problem(seed + k, **shp)
        hist_b, out_b, lse_b = brute_decode(p)
        hist_o = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
        out_o, lse_o = oracle_decode(p, hist_o)
        if rel(hist_o, hist_b) > 1e-12:
            bad.append(f"cache rows {shp}: {rel(hist_o, hist_b)}")
        if rel(out_o, out_b) > 1e-12:
            bad.append(f"out {shp}: {rel(out_o, out_b)}")
        if np.max(np.abs(lse_o - lse_b)) > 1e-12:
            bad.append(f"lse {shp}")
    return bad


def test_oracle_matches_bruteforce():
    assert check_core_pins() == []


def check_form_agreement(seed=10):
    bad = []
    for k, shp in enumerate(TINY[1:]):
        p = tiny_problem(seed + k, **shp)
        hist = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
        ref, lse_ref = oracle_decode(p, hist)
        ab, lse_ab = oracle_decode(p, hist, O.decode_absorbed)
        rows = O.gqa_expand_rows(hist, p["w_uk"], p["w_uv"], p["G"], p["d_c"], p["D"], p["Dv"])
        gq, lse_gq = O.decode_gqa(p["q_nope"], p["q_pe"], p["q_pos"], rows, p["G"], p["Dv"], BASE)
        for name, o, l in (("absorbed", ab, lse_ab), ("gqa", gq, lse_gq)):
            if rel(o, ref) > 1e-11 or np.max(np.abs(l - lse_ref)) > 1e-11:
                bad.append(f"{name} {shp}")
    return bad


def test_absorbed_and_gqa_forms_equal_reconstructed():
    assert check_form_agreement() == []


def test_one_position_returns_its_value_exactly():
    p = tiny_problem(20, H=3, G=3, L=1)
    hist = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
    out, lse = oracle_decode(p, hist)
    c = hist[0, :p["d_c"]]
    for h in range(p["H"]):
        v = c @ p["w_uv"][:, h * p["Dv"]:(h + 1) * p["Dv"]]
        assert np.array_equal(out[0, h], v)


def test_zero_query_gives_mean_of_values():
    p = tiny_problem(21, H=2, G=1, L=6)
    p["q_nope"][:] = 0
    p["q_pe"][:] = 0
    hist = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
    out, lse = oracle_decode(p, hist)
    V = hist[:, :p["d_c"]] @ p["w_uv"][:, :p["Dv"]]
    assert np.allclose(out[0, 0], V.mean(axis=0), atol=1e-14)
    assert abs(lse[0, 0] - math.log(6)) < 1e-14


def test_single_head_identity_weights_is_textbook_attention():
    r = np.random.default_rng(22)
    d, L = 8, 9
    hist = r.standard_normal((L, d))
    q = r.standard_normal((1, 1, d))
    eye = np.eye(d)
    out, _ = O.decode_reconstructed(q, np.zeros((1, 1, 0)), [L - 1], hist, eye, eye, 1, d, d, BASE)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q).view(1, 1, 1, d), t(hist).view(1, 1, L, d), t(hist).view(1, 1, L, d))
    assert np.allclose(out[0, 0], ref.view(d).numpy(), atol=1e-14)


def test_group_weights_replicated_per_head_is_mla():
    p = tiny_problem(23, H=4, G=2, L=6)
    hist = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
    ref, _ = oracle_decode(p, hist)
    D, Dv = p["D"], p["Dv"]
    per = p["H"] // p["G"]
    uk = np.concatenate([p["w_uk"][:, (h // per) * D:(h // per + 1) * D] for h in range(p["H"])], 1)
    uv = np.concatenate([p["w_uv"][:, (h // per) * Dv:(h // per + 1) * Dv] for h in range(p["H"])], 1)
    mla, _ = O.decode_reconstructed(p["q_nope"], p["q_pe"], p["q_pos"], hist, uk, uv, p["H"],
                                    p["d_c"], Dv, BASE)
    assert rel(mla, ref) < 1e-14
    # one group: every head shares keys and values (MQA); equal queries give equal outputs
    q = tiny_problem(24, H=3, G=1, L=4)
    q["q_nope"][:, 1:] = q["q_nope"][:, :1]
    q["q_pe"][:, 1:] = q["q_pe"][:, :1]
    o, _ = oracle_decode(q)
    assert np.array_equal(o[0, 1], o[0, 0]) and np.array_equal(o[0, 2], o[0, 0])


def check_invariants(seed=30):
    bad = []
    # shift every position (cache keys and queries) by the same amount
    p = tiny_problem(seed, H=4, G=2, L=6, s_q=2)
    ref, _ = oracle_decode(p)
    for s in (3, 1000):
        q = dict(p); q["pos"] = p["pos"] + s; q["q_pos"] = p["q_pos"] + s
        o, _ = oracle_decode(q)
        if rel(o, ref) > 1e-9:
            bad.append(f"shift {s}: {rel(o, ref)}")
    # a multi-token step equals single-token steps at the matching lengths
    hist = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
    multi, lse_m = oracle_decode(p, hist)
    for i in range(p["s_q"]):
        n = p["L"] - p["s_q"] + i + 1
        one, lse_1 = O.decode_reconstructed(p["q_nope"][i:i + 1], p["q_pe"][i:i + 1],
                                            p["q_pos"][i:i + 1], hist[:n], p["w_uk"], p["w_uv"],
                                            p["G"], p["d_c"], p["Dv"], BASE)
        if rel(one[0], multi[i]) > 1e-14:
            bad.append(f"causal {i}")
    return bad


def test_invariants():
    assert check_invariants() == []


def test_softmax_weights_sum_to_one_and_lse():
    r = np.random.default_rng(40)
    K, V, q = r.standard_normal((50, 6)), np.eye(50)[:, :50], r.standard_normal(6)
    p, lse = O.attend(q, K, np.eye(50), 0.3)
    assert abs(math.fsum(p) - 1) < 1e-15 and np.all(p > 0)
    z = 0.3 * (K @ q)
    assert abs(lse - math.log(math.fsum(math.exp(v) for v in z))) < 1e-13


def test_bulk_and_chunked_rows_agree():
    p = tiny_problem(41, L=9)
    whole = O.latent_rows(p["x"], p["w_dkv"], p["gamma"], p["w_kr"], p["pos"], BASE, EPS)
    parts = np.concatenate([O.latent_rows(p["x"][a:b], p["w_dkv"], p["gamma"], p["w_kr"],
                                          p["pos"][a:b], BASE, EPS) for a, b in ((0, 4), (4, 9))])
    assert rel(parts, whole) < 1e-15


def test_paging_slots():
    table = np.array([[5, 2, -1], [0, 3, 1]], dtype=np.int32)
    bs = 4
    assert O.slot(table, 0, 0, bs) == 20 and O.slot(table, 0, 5, bs) == 9
    assert O.slot(table, 1, 11, bs) == 7
    assert list(O.seq_slots(table, 1, 6, bs)) == [0, 1, 2, 3, 12, 13]
    m = O.owned_slot_mask(table, [6, 9], num_blocks=6, bs=bs)
    assert m.sum() == 15 and not m[16:20].any()


# ----------------------------------------------------------------------------- planted mistakes
def _wrong_scale(d_nope, d_r):
    return 1.0 / math.sqrt(d_nope + d_r + 1)


def _reversed_rope(v, pos, base):
    return OM.__dict__["_orig_rope"](v, -np.asarray(pos, dtype=np.float64), base)


def _wrong_group(h, H, G):
    return h % G


def _off_by_one(L, s_q):
    return [L - s_q + i for i in range(s_q)]


def _no_rotary(v, pos, base):
    return np.zeros_like(np.asarray(v, dtype=np.float64))


def _rms_sum(y, gamma, eps):
    return y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + eps) * gamma


@pytest.mark.parametrize("name,fn", [
    ("softmax_scale", _wrong_scale), ("rope", _reversed_rope), ("group_of", _wrong_group),
    ("visible_lengths", _off_by_one), ("rope", _no_rotary), ("rms_norm", _rms_sum)])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setitem(OM.__dict__, "_orig_rope", OM.rope)
    monkeypatch.setattr(OM, name, fn)
    failures = []
    for check in (check_core_pins, check_invariants):
        try:
            failures += check()
        except (ValueError, IndexError, ZeroDivisionError) as e:   # a crash is a catch too
            failures.append(repr(e))
    assert failures, f"planted mistake in {name} went unnoticed"


def test_planted_transpose_in_absorb_is_caught(monkeypatch):
    orig = OM.absorb_query

    def transposed(q_nope, q_pe, q_pos, w_uk, n_groups, base):
        wk = np.asarray(w_uk)
        d_c, GD = wk.shape
        # read the projection with its latent index reversed: a plausible layout slip
        return orig(q_nope, q_pe, q_pos, wk[::-1], n_groups, base)

    monkeypatch.setattr(OM, "absorb_query", transposed)
    assert check_form_agreement()
