"""Pins of the GEMM and cast oracle (oracle/gemm_oracle.py) against what the pages and the
mathematics fix: exact rational sums written element by element, closed forms, the round
trip of values already on the FP8 grid, torch's float8_e4m3fn cast, and invariants."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E2M1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _rand_fp8(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    return c


def _rand_gemm(rng, M, N, K, sa=(118, 136), sb=(118, 136)):
    a = _rand_fp8(rng, (M, K))
    a_sf = np.zeros((M, 4 * ((K + 511) // 512)), np.uint8)
    a_sf[:, : K // 128] = rng.integers(*sa, size=(M, K // 128))
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    b_sf = rng.integers(*sb, size=(N, K // 32)).astype(np.uint8)
    return a, a_sf, b, b_sf


def _e4m3_fraction(code):
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _e2m1_fraction(nib):
    return (-1 if nib & 8 else 1) * Fraction(E2M1[nib & 7]).limit_denominator(2)


def _pow2(b):
    return Fraction(2) ** (int(b) - 127)


def test_gemm_equals_exact_rational_sum():
    rng = np.random.default_rng(0)
    M, N, K = 3, 4, 256
    a, a_sf, b, b_sf = _rand_gemm(rng, M, N, K)
    r = oracle.fp8_fp4_gemm(a, a_sf, b, b_sf, K)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            absum = Fraction(0)
            for c in range(K):
                va = _e4m3_fraction(int(a[m, c])) * _pow2(a_sf[m, c // 128])
                nib = (int(b[n, c // 2]) >> (4 * (c % 2))) & 0xF
                vb = _e2m1_fraction(nib) * _pow2(b_sf[n, c // 32])
                tot += va * vb
                absum += abs(va * vb)
            assert abs(Fraction(r["exact"][m, n]) - tot) <= Fraction(2) ** -50 * absum
            assert r["bits"][m, n] == oracle.bf16_rne_bits(np.array([float(tot)]))[0]
            g = (K - 1) * 2.0 ** -24
            assert r["bound"][m, n] >= g * float(absum) * (1 - 1e-12)


def test_gemm_one_hot_selects_a_column_of_b():
    """A = one-hot rows (value 1.0 at column c_m, scale 2^0): D[m, n] = B[n, c_m] exactly."""
    rng = np.random.default_rng(1)
    M, N, K = 5, 6, 384
    cols = [0, 31, 32, 255, 383]
    a = np.zeros((M, K), np.uint8)
    for m, c in enumerate(cols):
        a[m, c] = 0x38                        # e4m3 1.0: exponent 7, mantissa 0
    a_sf = np.zeros((M, 4), np.uint8)
    a_sf[:, :3] = 127
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    b_sf = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    r = oracle.fp8_fp4_gemm(a, a_sf, b, b_sf, K)
    for m, c in enumerate(cols):
        for n in range(N):
            nib = (int(b[n, c // 2]) >> (4 * (c % 2))) & 0xF
            want = float(_e2m1_fraction(nib) * _pow2(b_sf[n, c // 32]))
            assert r["exact"][m, n] == want
            assert r["bound"][m, n] == 0.0 or abs(want) > 0


def test_gemm_scale_bytes_scale_the_output():
    rng = np.random.default_rng(2)
    a, a_sf, b, b_sf = _rand_gemm(rng, 4, 8, 512)
    r = oracle.fp8_fp4_gemm(a, a_sf, b, b_sf, 512)
    a2 = a_sf.copy()
    a2[:, :4] += 1
    r2 = oracle.fp8_fp4_gemm(a, a2, b, b_sf, 512)
    assert np.array_equal(r2["exact"], 2 * r["exact"])
    r3 = oracle.fp8_fp4_gemm(a, a_sf, b, b_sf + 3, 512)
    assert np.array_equal(r3["exact"], 8 * r["exact"])
    # one scale block of one B row: only that row's column changes, by the block's part
    b4 = b_sf.copy()
    b4[5, 7] += 1
    r4 = oracle.fp8_fp4_gemm(a, a_sf, b, b4, 512)
    assert np.array_equal(np.delete(r4["exact"], 5, axis=1), np.delete(r["exact"], 5, axis=1))
    assert not np.array_equal(r4["exact"][:, 5], r["exact"][:, 5])


def test_fp32_sums_fall_within_the_bound():
    """Any FP32 order of the same products lands within the bound, and the bound is not
    vacuous: an FP32 sum differs from exact, at least somewhere, by a visible fraction of it."""
    rng = np.random.default_rng(3)
    M, N, K = 6, 16, 2048
    a, a_sf, b, b_sf = _rand_gemm(rng, M, N, K)
    r = oracle.fp8_fp4_gemm(a, a_sf, b, b_sf, K)
    A = oracle.dequant_fp8_rows(a, a_sf, K)
    B = oracle.dequant_fp4_rows(b, b_sf, K)
    worst = 0.0
    for order in (slice(None), slice(None, None, -1)):
        terms = (A[:, None, order] * B[None, :, order]).astype(np.float32)
        s = np.zeros((M, N), np.float32)
        for c in range(K):
            s = s + terms[:, :, c]
        err = np.abs(s.astype(np.float64) - r["exact"])
        assert np.all(err <= r["bound"])
        worst = max(worst, float((err / r["bound"]).max()))
        d = oracle.bf16_rne_bits(s.astype(np.float64))
        assert oracle.gemm_bf16_within_bound(d, r["exact"], r["bound"]).all()
    assert worst > 1e-3
    # a value off by one bf16 step past the bound fails the check
    d = r["bits"].copy().astype(np.int64)
    far = np.abs(r["exact"]) > 1e3 * r["bound"]
    d[far] += 2
    assert not oracle.gemm_bf16_within_bound(d.astype(np.uint16), r["exact"], r["bound"])[far].any()


def test_contiguous_layout_matches_rows_of_dense():
    rng = np.random.default_rng(4)
    G, N, K, M = 3, 8, 256, 23
    a, a_sf, _, _ = _rand_gemm(rng, M, N, K)
    bs = [_rand_gemm(rng, 1, N, K)[2:] for _ in range(G)]
    b = np.stack([x[0] for x in bs])
    b_sf = np.stack([x[1] for x in bs])
    grp = np.array([0] * 5 + [-1] * 2 + [2] * 7 + [1] * 3 + [-1] + [2] * 5, np.int32)
    r = oracle.m_grouped_gemm_contiguous(a, a_sf, grp, b, b_sf, K)
    assert np.array_equal(r["valid"], grp >= 0)
    for m in range(M):
        if grp[m] < 0:
            continue
        d = oracle.fp8_fp4_gemm(a[m:m + 1], a_sf[m:m + 1], b[grp[m]], b_sf[grp[m]], K)
        assert np.array_equal(r["exact"][m], d["exact"][0])
    # rows are independent: reordering rows reorders outputs
    p = rng.permutation(M)
    r2 = oracle.m_grouped_gemm_contiguous(a[p], a_sf[p], grp[p], b, b_sf, K)
    assert np.array_equal(r2["exact"], r["exact"][p])
    with pytest.raises(oracle.OracleInputError):
        oracle.m_grouped_gemm_contiguous(a, a_sf, np.full(M, 3, np.int32), b, b_sf, K)


def test_masked_layout_counts():
    rng = np.random.default_rng(5)
    G, max_m, N, K = 4, 9, 8, 256
    a = np.stack([_rand_gemm(rng, max_m, N, K)[0] for _ in range(G)])
    a_sf = np.stack([_rand_gemm(rng, max_m, N, K)[1] for _ in range(G)])
    bs = [_rand_gemm(rng, 1, N, K)[2:] for _ in range(G)]
    b = np.stack([x[0] for x in bs])
    b_sf = np.stack([x[1] for x in bs])
    masked = np.array([0, 9, 4, 100], np.int32)
    r = oracle.m_grouped_gemm_masked(a, a_sf, masked, b, b_sf, K)
    assert r["valid"].sum(axis=1).tolist() == [0, 9, 4, 9]
    for g in range(G):
        c = min(int(masked[g]), max_m)
        if c:
            d = oracle.fp8_fp4_gemm(a[g, :c], a_sf[g, :c], b[g], b_sf[g], K)
            assert np.array_equal(r["exact"][g, :c], d["exact"])
        assert not r["exact"][g, c:].any()
    r2 = oracle.m_grouped_gemm_masked(a, a_sf, np.array([-3, 0, 0, 0]), b, b_sf, K)
    assert not r2["valid"].any()


# ---------------------------------------------------------------------------- cast


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_cast_round_trips_values_on_the_grid():
    """Blocks built as e4m3 value x 2^(byte-127), with the block's largest magnitude in
    (224, 448], come back as the same codes and bytes (the rule picks that byte)."""
    rng = np.random.default_rng(6)
    R, C = 16, 640
    nb = C // 128
    codes = _rand_fp8(rng, (R, C))
    byte = rng.integers(100, 150, size=(R, nb))
    for r in range(R):
        for k in range(nb):
            j = rng.integers(0, 128)
            # codes 0x77..0x7E are 240..448: the block's largest magnitude is in (224, 448]
            codes[r, 128 * k + j] = rng.integers(0x77, 0x7F) | (0x80 if rng.random() < 0.5 else 0)
    vals = oracle.decode_e4m3(codes) * np.repeat(np.ldexp(1.0, byte - 127), 128, axis=1)
    bits = _bf16_bits(vals)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), vals)      # exact in bf16
    c2, sf = oracle.cast_to_fp8(bits)
    assert sf.shape == (R, 4 * ((C + 511) // 512))
    assert np.array_equal(sf[:, :nb], byte.astype(np.uint8))
    assert not sf[:, nb:].any()
    # codes agree wherever the value is not zero (+0 and -0 encode the sign)
    assert np.array_equal(c2, codes)


def test_cast_matches_torch_float8_cast():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((32, 512)) * np.exp(rng.uniform(-8, 8, size=(32, 1)))).astype(np.float32)
    bits = _bf16_bits(x)
    codes, sf = oracle.cast_to_fp8(bits)
    xb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    scale = torch.from_numpy(np.ldexp(1.0, -(sf[:, :4].astype(np.int64) - 127))).float()
    ref = (xb.view(32, 4, 128) * scale[:, :, None]).reshape(32, 512).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())


def test_cast_edge_blocks():
    C = 256
    x = np.zeros((4, C), np.float32)
    x[1, :128] = 448.0                       # exactly 448 * 2^0: byte 127
    x[1, 128] = np.float32(448.0) * 2.0      # 896 = 448 * 2^1: byte 128
    x[2, 0] = 2.0 ** -133                    # bf16's smallest subnormal: s = -141, byte 0
    x[2, 128] = 3.0 * 2 ** 125               # 1.5 * 2^126: s = 118, code of 384
    x[3, :] = -0.0
    x[3, 128] = 449.0                        # rounds to bf16 448: byte 127
    x[3, 129] = 450.0                        # bf16 450 > 448: byte 128
    bits = _bf16_bits(x)
    codes, sf = oracle.cast_to_fp8(bits)
    assert sf.tolist() == [[127, 127, 0, 0], [127, 128, 0, 0], [0, 245, 0, 0], [127, 128, 0, 0]]
    assert codes[0].tolist() == [0] * C
    assert codes[1, :128].tolist() == [0x7E] * 128 and codes[1, 128] == 0x7E
    assert codes[2, 0] == 0x08                # 2^-133 * 2^127 = 2^-6: the first normal code
    assert codes[2, 128] == 0x7C              # 384 = 1.5 * 2^8: exponent field 15, mantissa 4
    assert codes[3, 0] == 0x80                # -0 keeps its sign
    with pytest.raises(oracle.OracleInputError):
        oracle.cast_to_fp8(_bf16_bits(np.full((1, 128), np.inf, np.float32)))
    with pytest.raises(oracle.OracleInputError):
        oracle.cast_to_fp8(bits[:, :100])
