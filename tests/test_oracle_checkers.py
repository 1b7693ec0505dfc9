"""Pins of the oracle's acceptance metrics, the functions every GPU comparison runs
through: e4m3_code_distance (with _grid_index) and y_row_error.

The e4m3 grid is the OCP e4m3fn format of chenxutan.com/d/1930 section 4.1 (1 sign,
4 exponent, 3 mantissa bits, bias 7; 0x7F/0xFF NaN), each value carried by the UE8M0
block scale of section 11.1's per-block scaling (byte b = 2^(b-127), 255 NaN). The
expected values below are worked out by hand from that definition, and two brute-force
checks recount the same distances by sorting and counting the grid points, with no
searchsorted and no half-index arithmetic."""
import numpy as np
import pytest

import oracle

INF = float("inf")

# (code a, scale byte a, code b, scale byte b, expected distance), worked by hand:
# 0x38 = 1.0, 0x39 = 1.125, 0x3A = 1.25, 0x37 = 0.9375 (the largest value below 1),
# 0x30 = 0.5, 0x31 = 0.5625, 0x01 = 2^-9 (the smallest subnormal), 0x07 = 7/8 * 2^-6 (the
# largest subnormal), 0x08 = 2^-6 (the smallest normal), 0x09 = 1.125 * 2^-6,
# 0x7E = 448, 0x7D = 416, 0x80 = -0, 0x81 = -2^-9, 0xB8 = -1.0. The positive values in
# code order are the grid positions: code c (c < 0x7F) sits at position c.
HAND_CASES = [
    (0x38, 127, 0x38, 127, 0.0),      # identical
    (0x38, 127, 0x39, 127, 1.0),      # neighbours
    (0x39, 127, 0x38, 127, 1.0),      # symmetric
    (0x38, 127, 0x3A, 127, 2.0),      # two steps
    (0x37, 127, 0x38, 127, 1.0),      # across a binade boundary
    (0x07, 127, 0x08, 127, 1.0),      # largest subnormal to smallest normal
    (0x01, 127, 0x00, 127, 1.0),      # smallest subnormal to zero
    (0x01, 127, 0x81, 127, 2.0),      # +min, 0, -min
    (0x00, 127, 0x80, 127, 0.0),      # +0 and -0 are one value
    (0x38, 127, 0xB8, 127, 112.0),    # +1 and -1: 56 positions each side of zero
    (0x7E, 127, 0x7D, 127, 1.0),      # the top of the grid
    (0x38, 0, 0x39, 0, 1.0),          # the smallest scale byte
    (0x38, 254, 0x39, 254, 1.0),      # the largest finite scale byte
    # different scale bytes: both values are placed on the grid of the coarser scale
    (0x38, 127, 0x30, 128, 0.0),      # 1.0 and 0.5 * 2: one value at two scales
    (0x38, 127, 0x31, 128, 1.0),      # 1.0 and 1.125 (= 0.5625 * 2): 0.5, 0.5625 at 2^1
    (0x01, 127, 0x00, 128, 0.5),      # 2^-9 is 2^-10 at 2^1: half way between 0 and 2^-9
    (0x01, 127, 0x01, 128, 0.5),      # 2^-10 and 2^-9 on the 2^1 grid
    (0x08, 127, 0x09, 130, 8.0),      # 2^-6 is 2^-9 (position 1) at 2^3; 1.125*2^-6 is 0x09 (9).
                                      # On the finer 2^0 grid they would be 25 apart
    (0x38, 127, 0x39, 131, 33.0),     # 1/16 (0x18, 24) and 1.125 (0x39, 57) at 2^4
    # NaN codes and the NaN scale byte are never acceptable
    (0x7F, 127, 0x7E, 127, INF),
    (0xFF, 127, 0xFE, 127, INF),
    (0x38, 127, 0x7F, 127, INF),
    (0x38, 255, 0x38, 255, INF),
    (0x38, 127, 0x38, 255, INF),
    (0x00, 255, 0x00, 127, INF),
]


def test_code_distance_hand_cases():
    a, sa, b, sb, want = (np.array(v) for v in zip(*HAND_CASES))
    got = oracle.e4m3_code_distance(a, sa, b, sb)
    for case, g in zip(HAND_CASES, got):
        assert g == case[4], f"{case}: got {g}"


def _finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)])


def _rank_by_sorting(values: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Position of each value on a sorted grid of distinct values, counted: points strictly
    below plus points at or below, minus one, halved (a grid point gets its index, a value
    between two points the midpoint of theirs)."""
    below = (grid[None, :] < values[:, None]).sum(axis=1)
    at_or_below = (grid[None, :] <= values[:, None]).sum(axis=1)
    return (below + at_or_below - 1) / 2.0


def _signed_grid():
    vals = np.array([oracle.e4m3_value(c) for c in _finite_codes()])
    return np.unique(vals)          # sorted distinct values; +0 and -0 are one point


def test_code_distance_same_scale_is_rank_difference():
    """Every pair of finite codes at one scale byte: the distance is the difference of the
    two values' ranks among the sorted distinct grid values."""
    codes = _finite_codes()
    grid = _signed_grid()
    rank = _rank_by_sorting(np.array([oracle.e4m3_value(c) for c in codes]), grid)
    a = np.repeat(codes, len(codes))
    b = np.tile(codes, len(codes))
    want = np.abs(np.repeat(rank, len(codes)) - np.tile(rank, len(codes)))
    for byte in (0, 120, 127, 254):
        sc = np.full(a.shape, byte)
        got = oracle.e4m3_code_distance(a, sc, b, sc)
        assert np.array_equal(got, want), byte


def test_code_distance_across_scales_by_counting():
    """Random pairs of finite codes with scale bytes up to 14 apart: both values are placed
    on the grid of the coarser scale by counting that grid's points below them."""
    rng = np.random.default_rng(7)
    codes = _finite_codes()
    n = 4000
    a = rng.choice(codes, n)
    b = rng.choice(codes, n)
    sa = rng.integers(100, 140, n)
    sb = sa + rng.integers(-14, 15, n)
    grid = _signed_grid()
    va = np.array([oracle.e4m3_value(c) for c in a]) * np.ldexp(1.0, sa - 127)
    vb = np.array([oracle.e4m3_value(c) for c in b]) * np.ldexp(1.0, sb - 127)
    coarse = np.ldexp(1.0, np.maximum(sa, sb) - 127)
    ra = np.array([_rank_by_sorting(np.array([v / c]), grid)[0] for v, c in zip(va, coarse)])
    rb = np.array([_rank_by_sorting(np.array([v / c]), grid)[0] for v, c in zip(vb, coarse)])
    got = oracle.e4m3_code_distance(a, sa, b, sb)
    assert np.array_equal(got, np.abs(ra - rb))
    assert (got % 1 == 0.5).any()     # the sample reaches values between coarse grid points


def _bf16(vals):
    """bf16 bit patterns of values that bf16 holds exactly (checked)."""
    f = np.asarray(vals, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), vals
    return bits


def test_y_row_error_hand_cases():
    # exact row
    assert oracle.y_row_error(_bf16([[1.0, -2.0, 0.5]]), np.array([[1.0, -2.0, 0.5]]))[0] == 0.0
    # one bf16 step (2^-6 at magnitude 2) off the row's largest element: 2^-6 / 2
    assert oracle.y_row_error(_bf16([[1.0, -2.015625, 0.5]]),
                              np.array([[1.0, -2.0, 0.5]]))[0] == 2.0 ** -7
    # the worst element counts, not the mean: errors 2^-7 (at 0.5) and 2^-6 (at -2)
    assert oracle.y_row_error(_bf16([[1.0, -2.015625, 0.5078125, 0.25]]),
                              np.array([[1.0, -2.0, 0.5, 0.25]]))[0] == 2.0 ** -7
    # the denominator is the row's largest reference magnitude, not the element's own:
    # 2^-9 off at 0.25 in a row whose largest element is 2
    assert oracle.y_row_error(_bf16([[0.251953125, -2.0]]), np.array([[0.25, -2.0]]))[0] == 2.0 ** -10
    # rows are independent
    e = oracle.y_row_error(_bf16([[1.0, 1.0], [4.0, 4.0625]]), np.array([[1.0, 1.0], [4.0, 4.0]]))
    assert e[0] == 0.0 and e[1] == 2.0 ** -6
    # an all-zero reference row: exactly zero (either sign) passes, anything else is inf
    zero = np.zeros((1, 2))
    assert oracle.y_row_error(np.array([[0x0000, 0x8000]], dtype=np.uint16), zero)[0] == 0.0
    assert oracle.y_row_error(np.array([[0x0001, 0x0000]], dtype=np.uint16), zero)[0] == INF
    # a NaN or an infinity on the GPU side is never acceptable
    ref = np.array([[1.0, 2.0]])
    assert oracle.y_row_error(np.array([[0x7FC0, 0x4000]], dtype=np.uint16), ref)[0] == INF
    assert oracle.y_row_error(np.array([[0x3F80, 0x7F80]], dtype=np.uint16), ref)[0] == INF
    assert oracle.y_row_error(np.array([[0xFF80, 0x4000]], dtype=np.uint16), ref)[0] == INF
