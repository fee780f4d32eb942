"""Pins of the oracle's layer-stack step (no GPU): the input of the next layer
is x + y, summed in float32 and rounded to nearest even for bf16 activations.
The rounding is checked against nearest-value selection done in float64
(a different derivation from the oracle's bit manipulation), and against
worked cases: exact values, ties to even both ways, overflow, NaN."""

import numpy as np

from oracle import moe_oracle as O


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_rounding_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.0e38)]
    got = O.bf16_round_bits(f)
    # the two bf16 neighbours of each value, compared by distance in float64
    lo = (f.view(np.uint32) >> 16).astype(np.uint16)
    a = _bf16_to_f64(lo)
    b = _bf16_to_f64((lo.astype(np.uint32) + 1).astype(np.uint16))
    x = f.astype(np.float64)
    da, db = np.abs(x - a), np.abs(b - x)
    want = np.where(da < db, lo, (lo.astype(np.uint32) + 1).astype(np.uint16))
    tie = da == db
    want = np.where(tie, np.where(lo % 2 == 0, lo, (lo.astype(np.uint32) + 1).astype(np.uint16)), want)
    assert np.array_equal(got, want)


def test_bf16_rounding_worked_cases():
    one = np.float32(1.0)
    cases = [
        (one, 0x3F80),                                   # exact
        (np.float32(1.0 + 2.0 ** -8), 0x3F80),           # halfway, even below
        (np.float32(1.0 + 3 * 2.0 ** -8), 0x3F82),       # halfway, odd below: up to even
        (np.float32(1.0 + 2.0 ** -8 + 2.0 ** -20), 0x3F81),   # just past halfway
        (np.float32(-2.5), 0xC020),                      # exact negative
        (np.float32(3.4028235e38), 0x7F80),              # rounds up to infinity
    ]
    for v, bits in cases:
        assert int(O.bf16_round_bits(np.array([v]))[0]) == bits, (v, hex(bits))
    nan = O.bf16_round_bits(np.array([np.float32("nan")]))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_residual_next_sums_in_float32():
    x = np.array([0x3F80, 0x3F80, 0xC020, 0x0000], dtype=np.uint16)      # 1, 1, -2.5, 0
    y = np.array([2.0 ** -8, 3 * 2.0 ** -8, 2.5, -0.0], dtype=np.float32)
    assert O.residual_next(x, y, "bf16").tolist() == [0x3F80, 0x3F82, 0x0000, 0x0000]
    xf = np.array([1.0, 1e8, -3.0], dtype=np.float32)
    yf = np.array([2.0 ** -30, 1.0, 3.0], dtype=np.float32)
    got = O.residual_next(xf, yf, "f32")
    assert got.dtype == np.float32
    assert got.tolist() == [1.0, 1e8, 0.0]        # float32 sums: the small terms vanish
