"""Pins for the oracle's codecs and rounding rules (CPU only).

Each check compares the oracle with something other than itself: torch's own
float8_e4m3fn / float8_e8m0fnu / bfloat16 conversions (library routines), the
E2M1 codebook written out, or invariants that the rounding definitions fix.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_TABLE
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert set(np.nonzero(nan_ref)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    # signed zero
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_closed_form_points():
    v = oracle.e4m3_value
    assert v(0x7E) == 448.0            # largest finite: 2^8 * 1.75
    assert v(0x01) == 2.0 ** -9        # smallest subnormal
    assert v(0x08) == 2.0 ** -6        # smallest normal
    assert v(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert v(0x38) == 1.0 and v(0xB8) == -1.0
    assert v(0x30) == 0.5 and v(0x40) == 2.0
    with pytest.raises(oracle.OracleInputError):
        oracle.decode_e4m3(np.array([0x7F], dtype=np.uint8))


def test_e2m1_codebook():
    # OCP MX E2M1: codes 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 their negatives
    book = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert oracle.e2m1_value(c) == book[c]
        assert oracle.e2m1_value(c + 8) == -book[c]
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0
    assert max(abs(oracle.e2m1_value(c)) for c in range(16)) == 6.0   # range +-6


def test_e2m1_nibble_order():
    # element 2i is the low nibble of byte i
    packed = np.array([[0x21, 0x7F]], dtype=np.uint8)
    vals = oracle.E2M1_TABLE[oracle.unpack_e2m1(packed)]
    assert vals.tolist() == [[0.5, 1.0, -6.0, 6.0]]


def test_ue8m0_matches_torch():
    b = torch.arange(255, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(ref, oracle.UE8M0_TABLE[:255])
    assert oracle.ue8m0_value(127) == 1.0
    assert math.isnan(oracle.ue8m0_value(255))
    assert math.isnan(torch.tensor([255], dtype=torch.uint8).view(torch.float8_e8m0fnu).float().item())
    with pytest.raises(oracle.OracleInputError):
        oracle.decode_ue8m0(np.array([255], dtype=np.uint8))


def _e4m3_sweep():
    mags = sorted(set(abs(oracle.e4m3_value(c)) for c in range(0x7F)))
    vals = []
    for i, m in enumerate(mags):
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
        if i + 1 < len(mags):
            mid = np.float32((m + mags[i + 1]) / 2)
            vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    rng = np.random.default_rng(0)
    vals += list(rng.uniform(0, 448, 20000).astype(np.float32))
    vals += list((2.0 ** rng.uniform(-12, 8.8, 20000)).astype(np.float32))
    v = np.array([x for x in vals if x <= 448.0], dtype=np.float32)
    return np.concatenate([v, -v])


def test_e4m3_encoder_matches_torch_rne():
    v = _e4m3_sweep()
    ours = oracle.encode_e4m3_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps -0 for tiny negatives, as do we
    assert np.array_equal(ours, ref), np.nonzero(ours != ref)[0][:10]


def test_e4m3_encoder_ties_to_even():
    enc = oracle.encode_e4m3_rne
    assert enc(np.array([272.0]))[0] == 0x78    # between 256 (0x78) and 288 (0x79)
    assert enc(np.array([304.0]))[0] == 0x7A    # between 288 (0x79) and 320 (0x7A)
    assert enc(np.array([1.0625]))[0] == 0x38   # between 1.0 and 1.125
    assert enc(np.array([1.1875]))[0] == 0x3A   # between 1.125 and 1.25 -> 1.25
    assert enc(np.array([2.0 ** -10]))[0] == 0x00   # half of the smallest subnormal -> 0
    assert enc(np.array([3 * 2.0 ** -10]))[0] == 0x02   # 1.5 quanta -> 2 (even)


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    f = np.concatenate([rng.standard_normal(50000), rng.standard_normal(50000) * 1e6,
                        rng.standard_normal(1000) * 1e-30]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.bf16_rne_bits(f.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_rounding_single_rounding_from_fp64():
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); a hair above goes up.
    assert oracle.bf16_rne_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.bf16_rne_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert oracle.bf16_rne_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82   # tie -> even
    assert oracle.bf16_rne_bits(np.array([-131072.0]))[0] == 0xC800
    assert oracle.bf16_rne_bits(np.array([0.0]))[0] == 0x0000


def test_pow2_scale_rule_invariants():
    rng = np.random.default_rng(2)
    amax = np.abs(rng.standard_normal(100000)) * 2.0 ** rng.integers(-60, 60, 100000)
    s = oracle.pow2_scale_exponent(amax)
    r = amax * np.ldexp(1.0, -s)
    assert np.all(r <= 448.0) and np.all(r > 224.0)      # least such s
    # boundary: amax = 448*2^s exactly stays at s, the next double up goes to s+1
    for e in range(-20, 20):
        a = 448.0 * 2.0 ** e
        assert oracle.pow2_scale_exponent(np.array([a]))[0] == e
        assert oracle.pow2_scale_exponent(np.array([np.nextafter(a, np.inf)]))[0] == e + 1
    assert oracle.pow2_scale_exponent(np.array([0.0]))[0] == 0
    # E2M1 maximum 6
    assert oracle.pow2_scale_exponent(np.array([6.0]), 6.0)[0] == 0
    assert oracle.pow2_scale_exponent(np.array([6.5]), 6.0)[0] == 1


def test_requant_grid_roundtrip_and_clamp():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, (4, 256)).astype(np.uint8)
    codes[:, 0] = 0x7E          # each block reaches 448 so the block scale is the given one
    codes[:, 128] = 0x7E
    sb = rng.integers(100, 150, (4, 2))
    vals = oracle.E4M3_TABLE[codes] * np.repeat(np.ldexp(1.0, sb - 127), 128, axis=1)
    q, sf, deq = oracle.requant_fp8_1x128(vals)
    assert np.array_equal(sf.astype(np.int64), sb)
    assert np.array_equal(q, codes)
    assert np.array_equal(deq, vals)
    # a block far below 448*2^-127 clamps at byte 0
    tiny = np.full((1, 128), 2.0 ** -140)
    q, sf, deq = oracle.requant_fp8_1x128(tiny)
    assert sf[0, 0] == 0
    assert np.all(deq == 0.0)   # 2^-140 * 2^127 = 2^-13 rounds to 0 on the e4m3 grid
    # zero block: byte 127, codes 0
    q, sf, _ = oracle.requant_fp8_1x128(np.zeros((1, 128)))
    assert sf[0, 0] == 127 and np.all(q == 0)


def test_requant_codes_match_torch_cast():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((64, 512)) * 2.0 ** rng.integers(-10, 10, (64, 1))
    q, sf, _ = oracle.requant_fp8_1x128(h)
    h32 = h.astype(np.float32)
    scale = np.repeat(np.ldexp(1.0, sf.astype(np.int64) - 127), 128, axis=1)
    ref = torch.from_numpy((h32 / scale).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_requant_decides_on_fp32_value():
    # fp64 h just above the 272 tie (between e4m3 256 and 288 at scale 2^5); its fp32
    # rounding is the tie itself, which goes to the even code 0x78 (256).
    h = np.zeros((1, 128))
    h[0, 0] = 8192.0
    h[0, 1] = 8704.0 * (1.0 + 2.0 ** -30)
    q, sf, _ = oracle.requant_fp8_1x128(h)
    assert sf[0, 0] == 132
    assert q[0, 1] == 0x78
