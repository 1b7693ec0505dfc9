"""Plain fp64 CPU oracle of the FP8 x FP4 block-scaled GEMMs and of the FP8 cast (numpy).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU-baseline
leg may use this module. It shares no code with the HIP path and imports nothing
from it; it builds on the decoders and rounding rules of moe_oracle.

Sources (the pages are cited by address and section):
  [P1] chenxutan.com/d/1930 -- 4.3 (the FP8 x FP4 GEMM call: A FP8 [M, K] with block
       scales, B FP4 [N, K] two per byte with UE8M0 scales, output bf16 [M, N]), 4.2
       (FP32 accumulation), 9.2 (input preparation: a bf16 activation is cast to FP8 codes
       plus scale factors before the MoE call), 11.1 (per-block scale = block amax /
       format max).
  [P2] zevenfang.github.io 2026/04/23 DeepGEMM review -- 二 (the GEMM family: dense,
       M-axis grouped, and masked grouped GEMM for decoding under graph capture, where the
       host does not know each expert's row count).
  [P4] juejin.cn/post/7631516744872673307 -- "MoE模型专属优化" (contiguous layout: the
       rows of all experts back to back, one grouped GEMM; masked layout for decoding).

Readings (the pages do not spell these out): the cast takes bf16 input and uses the
same per-1x128 scale rule and rounding as the intermediate's requantisation; the bytes
of the last 32-bit scale word past the row's last 128-block are 0. In the contiguous
layout every row names its group (-1: a padding row, not computed), with no alignment
required. In the masked layout group g's rows are A[g, :masked_m[g]] (count clamped
to [0, max_m]); other rows are not computed.

Parity pins: tests/test_oracle_gemm.py (exact rational sums, closed forms, the
grid round trip of the cast, torch's float8_e4m3fn cast, invariants).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .moe_oracle import (OracleInputError, bf16_bits_to_f64, bf16_rne_bits, dequant_fp4_rows,
                         dequant_fp8_rows, requant_fp8_1x128)

# unit roundoff of FP32
_U32 = 2.0 ** -24


def cast_to_fp8(x_bf16_bits: np.ndarray):
    """bf16 activations (bit patterns u16 [R, C], C a multiple of 128, finite) -> e4m3
    codes u8 [R, C] and UE8M0 bytes u8 [R, 4*ceil(C/512)] (byte j of word w = block
    4w+j). Per 1x128 block: byte = max(s + 127, 0) with s the least integer such that
    amax <= 448 * 2^s (s = 0 for an all-zero block); code = e4m3 RNE of x * 2^-(byte-127)
    [P1 9.2; P1 11.1]. bf16 -> fp64 is exact, so nothing rounds before the decision."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    R, C = bits.shape
    if C % 128:
        raise OracleInputError("cast: columns must be a multiple of 128")
    x = bf16_bits_to_f64(bits)
    if not np.all(np.isfinite(x)):
        raise OracleInputError("cast: non-finite input")
    codes, sf, _ = requant_fp8_1x128(x)
    out_sf = np.zeros((R, 4 * ((C + 511) // 512)), dtype=np.uint8)
    out_sf[:, : C // 128] = sf
    return codes, out_sf


def fp8_fp4_gemm(a: np.ndarray, a_sf: np.ndarray, b: np.ndarray, b_sf: np.ndarray, K: int):
    """D = A . B^T  [P1 4.3].

    A: e4m3 codes u8 [M, K], UE8M0 per 1x128 along K, u8 [M, 4*ceil(K/512)].
    B: E2M1 two per byte u8 [N, K/2] (element 2i low nibble), UE8M0 per 1x32, u8 [N, K/32].
    Returns dict: exact (fp64 [M, N]; every product is exact, the sum is fp64),
    bits (bf16 RNE of exact, u16 [M, N]), bound (gamma_{K-1} * sum_c |a_c b_c|: how far
    any FP32 summation order of the same products can land from exact [P1 4.2])."""
    A = dequant_fp8_rows(np.asarray(a), np.asarray(a_sf), K)
    B = dequant_fp4_rows(np.asarray(b), np.asarray(b_sf), K)
    exact = A @ B.T
    gamma = (K - 1) * _U32 / (1.0 - (K - 1) * _U32)
    bound = gamma * (np.abs(A) @ np.abs(B).T)
    return {"exact": exact, "bits": bf16_rne_bits(exact), "bound": bound}


def m_grouped_gemm_contiguous(a, a_sf, group_of_row, b, b_sf, K: int):
    """Contiguous layout [P4 "MoE模型专属优化"; P2 二]: row r of A uses B[group_of_row[r]]
    (b [G, N, K/2], b_sf [G, N, K/32]); rows with group -1 are padding. Returns dict as
    fp8_fp4_gemm over all rows, plus valid (bool [M]); padding rows hold 0 / NaN bound."""
    group_of_row = np.asarray(group_of_row)
    M = group_of_row.shape[0]
    G, N = b.shape[0], b.shape[1]
    if np.any((group_of_row < -1) | (group_of_row >= G)):
        raise OracleInputError("contiguous: group id out of range")
    exact = np.zeros((M, N))
    bound = np.zeros((M, N))
    for g in range(G):
        rows = np.nonzero(group_of_row == g)[0]
        if len(rows) == 0:
            continue
        r = fp8_fp4_gemm(np.asarray(a)[rows], np.asarray(a_sf)[rows], b[g], b_sf[g], K)
        exact[rows] = r["exact"]
        bound[rows] = r["bound"]
    return {"exact": exact, "bits": bf16_rne_bits(exact), "bound": bound,
            "valid": group_of_row >= 0}


def m_grouped_gemm_masked(a, a_sf, masked_m, b, b_sf, K: int) -> Dict[str, np.ndarray]:
    """Masked layout [P2 二; P4 "MoE模型专属优化"]: a [G, max_m, K], a_sf [G, max_m, sfw];
    group g computes rows i < clamp(masked_m[g], 0, max_m) against B[g]. Returns dict
    with exact / bits / bound [G, max_m, N] and valid (bool [G, max_m])."""
    a = np.asarray(a)
    G, max_m = a.shape[0], a.shape[1]
    N = b.shape[1]
    exact = np.zeros((G, max_m, N))
    bound = np.zeros((G, max_m, N))
    valid = np.zeros((G, max_m), dtype=bool)
    for g in range(G):
        c = int(min(max(int(masked_m[g]), 0), max_m))
        valid[g, :c] = True
        if c == 0:
            continue
        r = fp8_fp4_gemm(a[g, :c], np.asarray(a_sf)[g, :c], b[g], b_sf[g], K)
        exact[g, :c] = r["exact"]
        bound[g, :c] = r["bound"]
    return {"exact": exact, "bits": bf16_rne_bits(exact), "bound": bound, "valid": valid}


def gemm_bf16_within_bound(d_bits: np.ndarray, exact: np.ndarray, bound: np.ndarray) -> np.ndarray:
    """Per element: can d be bf16_RNE(s) for some s with |s - exact| <= bound? Holds
    when |d - exact| <= bound + half an ulp of bf16 at max(|exact| + bound), i.e.
    2^-8 * (|exact| + bound) (bf16 keeps 8 significant bits)."""
    d = bf16_bits_to_f64(d_bits)
    return np.abs(d - exact) <= bound + 2.0 ** -8 * (np.abs(exact) + bound) + 2.0 ** -134
