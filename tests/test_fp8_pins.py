"""Pins of the oracle's FP8 (OCP E4M3) latent rows against things other than itself.

The pages fix no FP8 format (they name quantisation among the ways to shrink a cache entry:
[KV-cache] "Les trois dimensions de compression"; [Slides] trainer notes on the INT8 check).
The oracle's reading is OCP E4M3 with one power-of-two scale per row; these tests tie it to
the format's published extremes, to torch's own float8_e4m3fn conversions (a library routine
written independently of the oracle), and to hand-worked scale cases.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

torch_e4m3 = getattr(torch, "float8_e4m3fn", None)
needs_torch_fp8 = pytest.mark.skipif(torch_e4m3 is None, reason="torch has no float8_e4m3fn")


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch_e4m3).double().numpy()


def torch_encode(v: np.ndarray) -> np.ndarray:
    # float32 input (exact for every value used here), round to nearest even in torch
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch_e4m3).view(
        torch.uint8).numpy()


def test_extremes_of_the_format():
    v = O.e4m3_values()
    assert v[0x7E] == 448.0                       # largest finite: 0 1111 110
    assert v[0x08] == 2.0 ** -6                   # smallest normal: 0 0001 000
    assert v[0x07] == 0.875 * 2.0 ** -6           # largest subnormal: 0 0000 111
    assert v[0x01] == 2.0 ** -9                   # smallest subnormal
    assert v[0x38] == 1.0                         # exponent field 7 = bias
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2               # no infinities, two NaN codes
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.all(np.diff(v[:0x7F]) > 0)          # positive codes in increasing order
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


@needs_torch_fp8
def test_value_table_matches_torch():
    codes = np.arange(256)
    assert np.array_equal(O.e4m3_values(), torch_decode(codes), equal_nan=True)


@needs_torch_fp8
def test_encode_matches_torch_on_ties_and_random_values():
    mags = O.e4m3_values()[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2             # every tie between neighbouring codes
    rng = np.random.default_rng(7)
    rand = rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 9, 200_000))
    rand = rand[np.abs(rand) <= 448].astype(np.float32).astype(np.float64)
    for v in (mids, -mids, rand, mags, -mags):
        assert np.array_equal(O.e4m3_encode(v), torch_encode(v))


def test_ties_go_to_the_even_code():
    mags = O.e4m3_values()[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2
    codes = O.e4m3_encode(mids).astype(int)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0x7E)) | (codes == np.arange(1, 0x7F)))
    # 1 + 1/16 sits between 1 (0x38) and 1.125 (0x39): the even code is 0x38
    assert O.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert O.e4m3_encode(np.array([1.1875]))[0] == 0x3A  # between 0x39 and 0x3A


def test_every_code_round_trips_and_signs_are_kept():
    v = O.e4m3_values()
    fin = np.flatnonzero(~np.isnan(v))
    assert np.array_equal(O.e4m3_encode(v[fin]), fin.astype(np.uint8))
    assert O.e4m3_encode(np.array([-1e-30]))[0] == 0x80   # negative values round to -0
    assert O.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00  # half the smallest subnormal: tie
    assert O.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02  # 1.5 subnormal steps -> even
    assert O.e4m3_encode(np.array([3 * 2.0 ** -11]))[0] == 0x01  # 0.75 of a step -> 1
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([449.0]))


def test_row_scale_hand_cases():
    assert O.e4m3_row_scale(0.0) == 1.0
    assert O.e4m3_row_scale(448.0) == 1.0
    assert O.e4m3_row_scale(448.0 * (1 + 2.0 ** -20)) == 2.0
    assert O.e4m3_row_scale(224.0) == 0.5          # 224 = 448 / 2 fits exactly
    assert O.e4m3_row_scale(1.0) == 2.0 ** -8      # 1 <= 1.75, 1 > 0.875
    assert O.e4m3_row_scale(0.875) == 2.0 ** -9    # 0.875 = 448 * 2^-9 exactly
    assert O.e4m3_row_scale(3.0e38) == 2.0 ** 120  # 3e38 / 448 = 6.7e35, 2^119 = 6.6e35
    rng = np.random.default_rng(3)
    for amax in np.exp2(rng.uniform(-120, 120, 2000)):
        s = O.e4m3_row_scale(amax)
        assert math.frexp(s)[0] == 0.5             # a power of two
        assert amax <= 448.0 * s and amax > 224.0 * s


def test_quantised_rows_within_half_a_step():
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((64, 576)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    rows[:, 512:] *= 0.01                           # a small rotary part shares the row's scale
    rows[5] = 0.0                                   # an all-zero row
    rows = O.round_bf16(rows)
    codes, scales = O.quantize_rows_e4m3(rows)
    assert codes.dtype == np.uint8 and codes.shape == rows.shape
    assert scales[5] == 1.0 and np.all(codes[5] == 0)
    deq = O.dequantize_rows_e4m3(codes, scales)
    amax = np.max(np.abs(rows), axis=1)
    assert np.all(np.max(np.abs(deq), axis=1) <= 448.0 * scales)
    assert np.all(amax[amax > 0] > 224.0 * scales[amax > 0])
    bound = np.maximum(2.0 ** -4 * np.abs(rows), 2.0 ** -10 * scales[:, None])
    assert np.all(np.abs(deq - rows) <= bound)
    # dequantised values are exact in bf16: byte x power of two
    assert np.array_equal(O.round_bf16(deq), deq)


@needs_torch_fp8
def test_quantised_rows_match_torch_per_row():
    rng = np.random.default_rng(5)
    rows = O.round_bf16(rng.standard_normal((32, 576)) * 3.0)
    codes, scales = O.quantize_rows_e4m3(rows)
    for r in range(rows.shape[0]):
        assert np.array_equal(codes[r], torch_encode(rows[r] / scales[r]))


def _pins_hold(values, encode, row_scale) -> bool:
    """The pins above, as one predicate over a (value table, encoder, row scale) triple."""
    v = values()
    if not (v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x38] == 1.0):
        return False
    mags = v[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2
    if not np.all(encode(mids).astype(int) % 2 == 0):
        return False
    if not (row_scale(1.0) == 2.0 ** -8 and row_scale(448.0) == 1.0 and row_scale(224.0) == 0.5):
        return False
    return True


def test_planted_mistakes_fail_the_pins():
    """Mistakes planted in copies of the oracle's FP8 functions: a wrong exponent bias, ties
    rounded away from zero, a scale twice too large. Each must break a pin; the real
    functions must pass."""
    assert _pins_hold(O.e4m3_values, O.e4m3_encode, O.e4m3_row_scale)

    def biased_values():
        return O.e4m3_values() / 2.0              # bias 8 instead of 7

    def ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        mags = O.e4m3_values()[:0x7F]
        a = np.abs(x)
        hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)
        lo = np.maximum(hi - 1, 0)
        pick_hi = (mags[hi] - a) <= (a - mags[lo])  # a tie goes up, whatever the code
        return np.where(pick_hi, hi, lo).astype(np.uint8) | (np.signbit(x).astype(np.uint8) << 7)

    def double_scale(amax):
        return 2.0 * O.e4m3_row_scale(amax)

    assert not _pins_hold(biased_values, O.e4m3_encode, O.e4m3_row_scale)
    assert not _pins_hold(O.e4m3_values, ties_away, O.e4m3_row_scale)
    assert not _pins_hold(O.e4m3_values, O.e4m3_encode, double_scale)
