"""Pins of the oracle's layer projections (query side and output projection), CPU only:
pure-Python loops on tiny shapes, closed forms with identity weights, the affine property of
the output projection, and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import bruteforce as BF
import oracle as O

EPS = 1e-6


def rand(rng, *shape):
    return rng.standard_normal(size=shape)


@pytest.mark.parametrize("C,d_q,H,D,d_r", [(6, 5, 2, 3, 2), (4, 7, 3, 2, 0), (8, 4, 1, 4, 4)])
def test_query_project_matches_loops(C, d_q, H, D, d_r):
    rng = np.random.default_rng([31, C, d_q, H])
    n = 3
    x, w_dq, g = rand(rng, n, C), rand(rng, C, d_q), 1 + 0.3 * rand(rng, d_q)
    w_uq, w_qr = rand(rng, d_q, H * D), rand(rng, d_q, H * d_r)
    qn, qp = O.query_project(x, w_dq, g, w_uq, w_qr, EPS)
    for i in range(n):
        bn, bp = BF.query_project(list(x[i]), w_dq.tolist(), list(g), w_uq.tolist(),
                                  w_qr.tolist(), EPS)
        assert np.max(np.abs(qn[i] - np.array(bn))) <= 1e-12 * max(1.0, np.max(np.abs(bn)))
        if d_r:
            assert np.max(np.abs(qp[i] - np.array(bp))) <= 1e-12 * max(1.0, np.max(np.abs(bp)))
        else:
            assert qp.shape[1] == 0


@pytest.mark.parametrize("bias", [False, True])
def test_output_project_matches_loops(bias):
    rng = np.random.default_rng([32, bias])
    o, w_o = rand(rng, 4, 6), rand(rng, 6, 5)
    b = rand(rng, 5) if bias else None
    y = O.output_project(o, w_o, b)
    for i in range(4):
        ref = BF.output_project(list(o[i]), w_o.tolist(), None if b is None else list(b))
        assert np.max(np.abs(y[i] - np.array(ref))) <= 1e-12


def test_identity_weights_give_the_normalised_input():
    """W_DQ = I, gamma_q = 1, W_UQ = I: q_nope = x / rms(x), the textbook RMSNorm."""
    rng = np.random.default_rng(33)
    x = rand(rng, 2, 8)
    qn, _ = O.query_project(x, np.eye(8), np.ones(8), np.eye(8), np.zeros((8, 0)), 0.0)
    ref = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    assert np.max(np.abs(qn - ref)) <= 1e-14


def test_output_projection_is_affine():
    rng = np.random.default_rng(34)
    o1, o2, w_o, b = rand(rng, 3, 6), rand(rng, 3, 6), rand(rng, 6, 4), rand(rng, 4)
    y12 = O.output_project(o1 + o2, w_o, b)
    assert np.max(np.abs(y12 - (O.output_project(o1, w_o, b) + O.output_project(o2, w_o, None)))) <= 1e-12
    assert np.max(np.abs(O.output_project(np.zeros((1, 6)), w_o, b) - b)) == 0.0


def test_storage_rounding_of_the_query_latent():
    """round_cq applies between the two products: with bf16 rounding the result equals the
    exact product of the rounded latent."""
    rng = np.random.default_rng(35)
    x, w_dq, g, w_uq, w_qr = rand(rng, 2, 6), rand(rng, 6, 5), np.ones(5), rand(rng, 5, 4), rand(rng, 5, 2)
    qn, qp = O.query_project(x, w_dq, g, w_uq, w_qr, EPS, round_cq=O.round_bf16)
    c = O.round_bf16(O.rms_norm(x @ w_dq, g, EPS))
    assert np.array_equal(qn, c @ w_uq) and np.array_equal(qp, c @ w_qr)


def _transposed_up(x, w_dq, g, w_uq, w_qr, eps, round_cq=None):
    c = O.rms_norm(x @ w_dq, g, eps)
    return c @ w_uq.T, c @ w_qr


def _no_norm(x, w_dq, g, w_uq, w_qr, eps, round_cq=None):
    c = (x @ w_dq) * g
    return c @ w_uq, c @ w_qr


def _no_gain(x, w_dq, g, w_uq, w_qr, eps, round_cq=None):
    c = O.rms_norm(x @ w_dq, np.ones_like(g), eps)
    return c @ w_uq, c @ w_qr


def _norm_width_off_by_one(x, w_dq, g, w_uq, w_qr, eps, round_cq=None):
    y = x @ w_dq
    c = y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) / (y.shape[-1] - 1) + eps) * g
    return c @ w_uq, c @ w_qr


@pytest.mark.parametrize("bad", [_transposed_up, _no_norm, _no_gain, _norm_width_off_by_one])
def test_planted_mistakes_are_caught(bad):
    rng = np.random.default_rng(36)
    C, d_q, H, D = 5, 4, 1, 4
    x, w_dq, g = rand(rng, 1, C), rand(rng, C, d_q), 1 + 0.3 * rand(rng, d_q)
    w_uq, w_qr = rand(rng, d_q, H * D), rand(rng, d_q, 2)
    qn, _ = bad(x, w_dq, g, w_uq, w_qr, EPS)
    bn, _ = BF.query_project(list(x[0]), w_dq.tolist(), list(g), w_uq.tolist(), w_qr.tolist(), EPS)
    assert np.max(np.abs(qn[0] - np.array(bn))) > 1e-6


def test_planted_missing_bias_is_caught():
    rng = np.random.default_rng(37)
    o, w_o, b = rand(rng, 1, 6), rand(rng, 6, 5), rand(rng, 5)
    ref = BF.output_project(list(o[0]), w_o.tolist(), list(b))
    assert np.max(np.abs(O.output_project(o, w_o, None)[0] - np.array(ref))) > 1e-6
    assert np.max(np.abs(O.output_project(o, w_o, b)[0] - np.array(ref))) <= 1e-12
