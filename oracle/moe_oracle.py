"""Plain, slow, fp64 CPU oracle of the one-GPU Mega MoE forward (numpy).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU-baseline
leg may use this module. It shares no code with the HIP path and imports nothing
from it.

Sources (the pages are cited by address and section):
  [P1] chenxutan.com/d/1930, "DeepSeek DeepGEMM 2026年4月重磅更新" -- section 3.1 (the
       five steps of an MoE layer: dispatch, Linear1, SwiGLU, Linear2, combine),
       3.2 (the five steps fused), 3.3 (call sequence and tensor shapes), 4.1
       (E4M3 and E2M1 formats), 4.2 (UE8M0 scale factors, FP32 accumulation),
       9.2 (router: top-k then softmax over the chosen logits), 11.1
       (per-block scale = block amax / format max).
  [P2] zevenfang.github.io 2026/04/23 DeepGEMM review -- section 4 (SM100 scale
       factors are packed UE8M0, four per 32-bit int), section 5 (Mega MoE =
       dispatch, Linear1 FP8xFP4, SwiGLU, Linear2 FP8xFP4, combine).
  [P4] juejin.cn/post/7631516744872673307 -- "MoE模型专属优化" (contiguous-layout
       grouped GEMM with block-aligned expert groups).

Readings of points the pages leave open (each listed with its reason in the
design notes): FP8 = OCP e4m3fn (max 448, codes 0x7F/0xFF NaN, no inf); E2M1 =
the OCP MX codebook with element 2i in the low nibble; UE8M0 byte b = 2^(b-127),
255 = NaN; activations and the intermediate are scaled per 1x128 along K, weights
per 1x32; W1 holds 2I rows, gate rows first; the power-of-two block scale is
rounded up (smallest s with amax <= 448*2^s) and elements are rounded to nearest
even; silu(g)*u with silu(v) = v/(1+exp(-v)); top-k weights are applied at the
combine, on the Linear2 output, summed over slots j = 0..k-1 in order; idx -1 is
an unused slot, other ids outside [0,E) are counted and skipped; experts' rows
are kept in ascending (token, slot) order and each expert's group is padded to a
multiple of BM rows.

Precision: decode is exact; Linear1/Linear2 accumulate in fp64; SwiGLU in fp64.
The requantisation decision (block scale and e4m3 code) is taken on the fp32
rounding of h, the precision the GPU kernel decides in. The output is rounded
once, fp64 -> bf16, round to nearest even.

Parity pins: every function here is checked in tests/ against library decoders
(torch float8_e4m3fn / float8_e8m0fnu), exhaustive codebooks, closed-form worked
examples (tests/golden), exact rational arithmetic, brute force and invariants.
Every function is pinned. No pin can reach DeepGEMM's own output: the pages print
no numeric example of the fused operator, so where they leave a step open the
readings are checked against their definitions and the mathematics, not against
upstream numbers.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# O1. Element and scale codecs  [P1 4.1, P1 4.2, P2 4]
# ----------------------------------------------------------------------------


def e4m3_value(code: int) -> float:
    """FP8 E4M3 (1 sign, 4 exponent, 3 mantissa bits; bias 7) [P1 4.1].
    Normal: (-1)^s 2^(E-7) (1+m/8); E=0: (-1)^s 2^-6 (m/8); 0x7F/0xFF: NaN."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m / 8.0, -6)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


def e2m1_value(code: int) -> float:
    """FP4 E2M1 (1 sign, 2 exponent, 1 mantissa bit; bias 1; range +-6) [P1 4.1].
    E=0: (-1)^s (m/2); else (-1)^s 2^(E-1) (1+m/2)."""
    code = int(code) & 0xF
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * (m / 2.0)
    return s * math.ldexp(1.0 + m / 2.0, e - 1)


def ue8m0_value(byte: int) -> float:
    """UE8M0 scale factor: an unsigned 8-bit exponent, value 2^(b-127); 255 is NaN
    [P1 4.2; P2 4]."""
    b = int(byte) & 0xFF
    if b == 255:
        return math.nan
    return math.ldexp(1.0, b - 127)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
UE8M0_TABLE = np.array([ue8m0_value(b) for b in range(256)], dtype=np.float64)


class OracleInputError(ValueError):
    pass


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    if np.any((codes & 0x7F) == 0x7F):
        raise OracleInputError("e4m3 NaN code in input")
    return E4M3_TABLE[codes]


def decode_ue8m0(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    if np.any(b == 255):
        raise OracleInputError("UE8M0 NaN scale byte in input")
    return UE8M0_TABLE[b]


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """u8 [..., K/2] -> nibble codes u8 [..., K]; element 2i is the low nibble of byte i."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant_fp8_rows(codes: np.ndarray, sf: np.ndarray, K: int) -> np.ndarray:
    """x[r, c] = e4m3(codes[r, c]) * 2^(sf[r, c // 128] - 127)  [P1 11.1; per 1x128]."""
    R = codes.shape[0]
    vals = decode_e4m3(codes[:, :K]).reshape(R, K // 128, 128)
    scale = decode_ue8m0(sf[:, : K // 128])
    return (vals * scale[:, :, None]).reshape(R, K)


# value pair of each packed byte: (element 2i = low nibble, element 2i+1 = high nibble)
_E2M1_PAIRS = np.stack([E2M1_TABLE[np.arange(256) & 0x0F], E2M1_TABLE[np.arange(256) >> 4]], axis=1)


def dequant_fp4_rows(packed: np.ndarray, sf: np.ndarray, K: int, out=None) -> np.ndarray:
    """w[n, c] = e2m1(nibble(n, c)) * 2^(sf[n, c // 32] - 127)  [P1 11.1; per 1x32].
    `out` (optional, f64 [R, K]) is filled and returned."""
    R = packed.shape[0]
    if out is None:
        out = np.empty((R, K), dtype=np.float64)
    np.take(_E2M1_PAIRS, np.asarray(packed, dtype=np.uint8)[:, : K // 2], axis=0,
            out=out.reshape(R, K // 2, 2))
    scale = decode_ue8m0(sf[:, : K // 32])
    v = out.reshape(R, K // 32, 32)
    np.multiply(v, scale[:, :, None], out=v)
    return out


# ----------------------------------------------------------------------------
# Rounding helpers (definitions written out)
# ----------------------------------------------------------------------------


def encode_e4m3_rne(v: np.ndarray) -> np.ndarray:
    """Round each value to the nearest e4m3fn value, ties to the even code.
    |v| must be <= 448 (the block scale guarantees it). Returns u8 codes."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > 448.0) or np.any(~np.isfinite(v)):
        raise OracleInputError("e4m3 encode input out of range")
    sign = np.signbit(v).astype(np.uint8) << 7
    # subnormal range: a < 2^-6, quantum 2^-9; q == 8 lands on the first normal code 0x08
    q_sub = np.rint(a * 512.0)
    # normal range: a = m * 2^e with m in [1, 2); quantum 2^(e-3)
    m, e = np.frexp(np.where(a > 0, a, 1.0))   # m in [0.5, 1)
    e = e - 1
    m = m * 2.0
    q = np.rint((m - 1.0) * 8.0)               # 0..8, half to even
    carry = q == 8
    q = np.where(carry, 0, q)
    e = np.where(carry, e + 1, e)
    code_norm = ((e + 7) << 3).astype(np.int64) + q.astype(np.int64)
    code = np.where(a < 2.0 ** -6, q_sub.astype(np.int64), code_norm)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def round_f32(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp32, round to nearest even (IEEE conversion)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def bf16_rne_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns (u16), rounding the fp64 value once to 8 significant
    bits, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                       # |v| = m 2^e, m in [0.5, 1)
    qexp = np.maximum(e - 8, -133)           # bf16: 8 significant bits; subnormal quantum 2^-133
    r = np.ldexp(np.rint(np.ldexp(v, -qexp)), qexp)
    f = r.astype(np.float32)                 # exact: r has <= 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# O5. Block scale rule  [P1 11.1: scale = block amax / format max; UE8M0 forces a power of 2]
# ----------------------------------------------------------------------------


def pow2_scale_exponent(amax: np.ndarray, qmax: float = 448.0) -> np.ndarray:
    """Least integer s with amax <= qmax * 2^s (0 where amax == 0). Exact: from the
    binary exponent of amax, amax = m 2^E with m in [1,2)."""
    amax = np.asarray(amax, dtype=np.float64)
    qm, qe = np.frexp(qmax)
    qm, qe = qm * 2.0, qe - 1                # qmax = qm 2^qe, qm in [1,2)  (448 = 1.75 2^8)
    m, e = np.frexp(np.where(amax > 0, amax, 1.0))
    m, e = m * 2.0, e - 1
    s = e - qe + (m > qm).astype(np.int64)
    return np.where(amax > 0, s, 0).astype(np.int64)


def requant_fp8_1x128(h: np.ndarray):
    """Per 1x128 block of each row: byte = max(s + 127, 0) with s the least integer such
    that amax <= 448 * 2^s; codes = e4m3 RNE of h * 2^-(byte-127). The decision is
    taken on float32(h). Returns (codes u8 [R, N], sf u8 [R, N/128], dequantised f64)."""
    h32 = round_f32(h).astype(np.float64)
    R, N = h32.shape
    assert N % 128 == 0
    blocks = h32.reshape(R, N // 128, 128)
    amax = np.abs(blocks).max(axis=-1)
    s = pow2_scale_exponent(amax)
    byte = np.maximum(s + 127, 0)
    codes = encode_e4m3_rne(blocks * np.ldexp(1.0, -(byte - 127))[..., None]).reshape(R, N)
    sf = byte.astype(np.uint8)
    deq = E4M3_TABLE[codes] * np.repeat(np.ldexp(1.0, byte - 127), 128, axis=1)
    return codes, sf, deq


# ----------------------------------------------------------------------------
# O2. Dispatch / routing  [P1 3.1 step 1; P4 contiguous layout, block-aligned groups]
# ----------------------------------------------------------------------------


def route(topk_idx: np.ndarray, E: int, BM: int) -> Dict[str, np.ndarray]:
    """Group the (token, slot) assignments by expert, stable in ascending (t, j).

    counts[e]   = number of slots with idx == e
    offsets[e]  = sum over e' < e of ceil(counts[e'] / BM) * BM   (E+1 entries)
    perm[p]     = t*k + j for the rows of each expert's group in (t, j) order, -1 on padding
    inv[t*k+j]  = position of that slot in perm, -1 for skipped slots
    tile_expert / tile_row0: one entry per BM-row tile, experts in order
    num_invalid = ids outside [-1, E)  (-1 marks an unused slot and is not counted)
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    groups = [[] for _ in range(E)]
    invalid = 0
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j])
            if 0 <= e < E:
                groups[e].append(t * k + j)
            elif e != -1:
                invalid += 1
    counts = np.array([len(g) for g in groups], dtype=np.int32)
    padded = [((c + BM - 1) // BM) * BM for c in counts]
    offsets = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + padded[e]
    perm = np.full(int(offsets[E]), -1, dtype=np.int32)
    for e in range(E):
        perm[offsets[e]: offsets[e] + counts[e]] = groups[e]
    inv = np.full(T * k, -1, dtype=np.int32)
    for p, s in enumerate(perm):
        if s >= 0:
            inv[s] = p
    tile_expert, tile_row0 = [], []
    for e in range(E):
        for m in range(padded[e] // BM):
            tile_expert.append(e)
            tile_row0.append(int(offsets[e]) + m * BM)
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv,
                tile_expert=np.array(tile_expert, dtype=np.int32),
                tile_row0=np.array(tile_row0, dtype=np.int32),
                num_invalid=np.int32(invalid))


# ----------------------------------------------------------------------------
# O3-O7. The expert FFN and the combine
# ----------------------------------------------------------------------------


def linear1(xr: np.ndarray, w1e: np.ndarray, w1e_sf: np.ndarray, row_chunk: int = 1024,
            abs_sums: bool = False):
    """G = xr . W1_gate^T, U = xr . W1_up^T for one expert, fp64 [P1 3.1 step 2; 4.2].
    xr: dequantised activation rows [R, H]; w1e u8 [2I, H/2]; w1e_sf u8 [2I, H/32].
    With abs_sums, also returns |xr| . |W1_gate|^T and |xr| . |W1_up|^T (the sums of the
    magnitudes of the products, used by accumulation_error_bound)."""
    R, H = xr.shape
    I = w1e.shape[0] // 2
    G = np.empty((R, I))
    U = np.empty((R, I))
    AG = np.empty((R, I)) if abs_sums else None
    AU = np.empty((R, I)) if abs_sums else None
    xa = np.abs(xr) if abs_sums else None
    buf = np.empty((min(row_chunk, I), H))                                # reused: bounds memory
    for r0 in range(0, I, row_chunk):
        r1 = min(I, r0 + row_chunk)
        Wg = dequant_fp4_rows(w1e[r0:r1], w1e_sf[r0:r1], H, out=buf[: r1 - r0])
        G[:, r0:r1] = xr @ Wg.T
        if abs_sums:
            AG[:, r0:r1] = xa @ np.abs(Wg).T
        Wu = dequant_fp4_rows(w1e[I + r0:I + r1], w1e_sf[I + r0:I + r1], H, out=buf[: r1 - r0])
        U[:, r0:r1] = xr @ Wu.T
        if abs_sums:
            AU[:, r0:r1] = xa @ np.abs(Wu).T
    if abs_sums:
        return G, U, AG, AU
    return G, U


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(gate) * up, silu(v) = v / (1 + exp(-v))  [P1 3.1 step 3; P2 5]."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


# Largest slope of silu(v) = v * sigmoid(v) over the reals (about 1.0998, at v ~ 2.40).
SILU_LIPSCHITZ = 1.1
# Unit roundoff used for FP32 arithmetic of unknown order and rounding mode: 2^-23 covers
# rounding by truncation as well as round-to-nearest (2^-24).
FP32_UNIT = 2.0 ** -23


def accumulation_error_bound(g: np.ndarray, u: np.ndarray, ag: np.ndarray, au: np.ndarray,
                             K: int) -> np.ndarray:
    """Bound on |h32 - h| for h = silu(g) * u, where h32 is computed from g32 and u32, FP32
    accumulations of the same K exact products in any order, and the SwiGLU is then
    evaluated in FP32.

    A sum of K terms accumulated in floating point with unit roundoff eps is within
    gamma_{K-1} * sum|terms| of the exact sum, gamma_n = n*eps / (1 - n*eps) (the standard
    forward error bound of recursive summation; it holds for every summation order). With
    dg, du those bounds for g and u (ag, au are the sums of |product|):
        |silu(g32) u32 - silu(g) u| <= L dg (|u| + du) + |silu(g)| du,   L = SILU_LIPSCHITZ,
    and evaluating silu(g32) * u32 in FP32 (exponential, reciprocal, three products, one
    sum: a few units each) adds at most (16 + |g|) eps of the result (the |g| term is the
    rounding of the exponential's argument)."""
    n = max(K - 1, 1)
    gamma = n * FP32_UNIT / (1.0 - n * FP32_UNIT)
    dg = gamma * ag
    du = gamma * au
    with np.errstate(over="ignore"):
        sg = g / (1.0 + np.exp(-g))
    acc = SILU_LIPSCHITZ * dg * (np.abs(u) + du) + np.abs(sg) * du
    h_mag = (np.abs(sg) + SILU_LIPSCHITZ * dg) * (np.abs(u) + du)
    return acc + (16.0 + np.abs(g) + dg) * FP32_UNIT * h_mag


def forward(x_fp8, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf,
            tokens: Optional[Sequence[int]] = None, cols: Optional[Sequence[int]] = None,
            row_chunk: int = 1024, keep_intermediates: bool = True,
            keep_bounds: bool = False):
    """The Mega MoE forward of one device's local experts [P1 3.1-3.3; P2 5].

    Shapes: x_fp8 u8 [T,H]; x_sf u8 [T, >=H/128]; topk_idx i32 [T,k]; topk_weights
    f32 [T,k]; w1 u8 [E,2I,H/2] (gate rows 0..I-1, up rows I..2I-1); w1_sf u8
    [E,2I,H/32]; w2 u8 [E,H,I/2]; w2_sf u8 [E,H,I/32].

    tokens: optional subset of token ids (tokens are independent given the routing);
    cols: optional subset of output columns. Returns a dict with
      y_bits  u16 [len(tokens), len(cols)]  bf16 bit patterns of y
      y       f64 (y before the bf16 rounding)
      h8      {slot: e4m3 codes [I]}, h_sf {slot: UE8M0 bytes [I/128]}   (if kept)
      h, h_bound  {slot: fp64 h [I]}, {slot: accumulation_error_bound of h [I]}
                  (if keep_bounds; otherwise empty)
    Steps, per expert e and each of its slots (t, j):
      O3  g = x[t] . W1[e, n],  u = x[t] . W1[e, I+n]        (fp64)        [P1 3.1 step 2; 4.2]
      O4  h = silu(g) * u                                                  [P1 3.1 step 3]
      O5  (q, sf) = requant per 1x128 of h; h' = dequant(q, sf)            [P1 11.1]
    then, on every slot's h' (linear2_combine):
      O6  o = h' . W2[e, m]                                                [P1 3.1 step 4]
      O7  y[t, m] = bf16( sum_j  w[t, j] * o[t, j, m] )                    [P1 3.1 step 5; 9.2]
    """
    x_fp8 = np.asarray(x_fp8)
    T, H = x_fp8.shape
    topk_idx = np.asarray(topk_idx)
    k = topk_idx.shape[1]
    E, twoI, _ = w1.shape
    I = twoI // 2
    assert w2.shape[0] == E and w2.shape[1] == H and w2.shape[2] * 2 == I
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    tok_pos = {int(t): i for i, t in enumerate(toks)}

    h8, hsf, hdeq, h64, hbound = {}, {}, {}, {}, {}
    xd_all = dequant_fp8_rows(x_fp8[toks], np.asarray(x_sf)[toks], H)   # [len(toks), H]
    for e in range(E):
        slots = [(int(t), j) for t in toks for j in range(k) if int(topk_idx[t, j]) == e]
        if not slots:
            continue
        xr = np.stack([xd_all[tok_pos[t]] for t, _ in slots])            # [R, H]
        if keep_bounds:
            G, U, AG, AU = linear1(xr, w1[e], w1_sf[e], row_chunk, abs_sums=True)
        else:
            G, U = linear1(xr, w1[e], w1_sf[e], row_chunk)
        h = swiglu(G, U)
        hb = accumulation_error_bound(G, U, AG, AU, H) if keep_bounds else None
        q, sf, hd = requant_fp8_1x128(h)
        for r, (t, j) in enumerate(slots):
            hdeq[t * k + j] = hd[r]
            if keep_intermediates:
                h8[t * k + j] = q[r]
                hsf[t * k + j] = sf[r]
            if keep_bounds:
                h64[t * k + j] = h[r]
                hbound[t * k + j] = hb[r]
    out = linear2_combine(hdeq, topk_idx, topk_weights, w2, w2_sf, tokens=toks, cols=cols,
                          row_chunk=row_chunk)
    return dict(y=out["y"], y_bits=out["y_bits"], h8=h8, h_sf=hsf, h=h64, h_bound=hbound,
                tokens=toks, cols=out["cols"])


def linear2_combine(hdeq: Dict[int, np.ndarray], topk_idx, topk_weights, w2, w2_sf,
                    tokens: Optional[Sequence[int]] = None, cols: Optional[Sequence[int]] = None,
                    row_chunk: int = 1024):
    """O6 and O7 on a given requantised intermediate [P1 3.1 steps 4-5; P2 5].

    hdeq: {slot t*k+j: fp64 h' [I]}, the dequantised intermediate of every valid slot of
    the given tokens (forward() passes its own; a test may pass another device's, decoded
    exactly). For each valid slot, o = h' . W2[e]^T (fp64); then
    y[t] = bf16( sum over j = 0..k-1 of w[t, j] * o[t, j] ) in fp64, slot order, skipped
    slots adding 0. Returns y (fp64 before rounding), y_bits (bf16), cols."""
    topk_idx = np.asarray(topk_idx)
    topk_weights = np.asarray(topk_weights, dtype=np.float32)
    T, k = topk_idx.shape
    E, H, _ = w2.shape
    I = 2 * w2.shape[2]
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    cols_arr = np.arange(H) if cols is None else np.asarray(cols, dtype=np.int64)
    tok_pos = {int(t): i for i, t in enumerate(toks)}

    contrib = np.zeros((len(toks), k, len(cols_arr)), dtype=np.float64)   # w[t,j] * o[t,j,:]
    for e in range(E):
        slots = [(int(t), j) for t in toks for j in range(k) if int(topk_idx[t, j]) == e]
        if not slots:
            continue
        hd = np.stack([hdeq[t * k + j] for t, j in slots])                 # [R, I]
        O = np.empty((len(slots), len(cols_arr)))                          # [R, len(cols)]
        buf = np.empty((min(row_chunk, len(cols_arr)), I))
        for c0 in range(0, len(cols_arr), row_chunk):
            cc = cols_arr[c0:c0 + row_chunk]
            W2c = dequant_fp4_rows(w2[e][cc], w2_sf[e][cc], I, out=buf[: len(cc)])
            O[:, c0:c0 + len(cc)] = hd @ W2c.T
        for r, (t, j) in enumerate(slots):
            contrib[tok_pos[t], j] = float(topk_weights[t, j]) * O[r]
    # O7: the combine sums the slots in order j = 0..k-1 (skipped slots add 0)
    acc = np.zeros((len(toks), len(cols_arr)), dtype=np.float64)
    for j in range(k):
        acc += contrib[:, j]
    return dict(y=acc, y_bits=bf16_rne_bits(acc), cols=cols_arr)


def forward_inputs(inp: dict, **kw):
    """forward() on a dict with keys x_fp8, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf."""
    return forward(inp["x_fp8"], inp["x_sf"], inp["topk_idx"], inp["topk_weights"],
                   inp["w1"], inp["w1_sf"], inp["w2"], inp["w2_sf"], **kw)


# ----------------------------------------------------------------------------
# Acceptance metrics
# ----------------------------------------------------------------------------


def y_row_error(y_bits_gpu: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per row: max_m |y_gpu - y_ref| / max_m |y_ref| (the largest error in the row over
    the row's largest reference magnitude). A row whose reference is all zero gives 0 only
    if y_gpu is exactly zero there (either sign), else inf. A row holding a NaN or an
    infinity on the GPU side gives inf."""
    yg = bf16_bits_to_f64(y_bits_gpu)
    yr = np.asarray(y_ref, dtype=np.float64)
    bad = ~np.isfinite(yg).all(axis=1)
    num = np.abs(np.where(np.isfinite(yg), yg, 0.0) - yr).max(axis=1)
    den = np.abs(yr).max(axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num == 0, 0.0, np.inf))
    return np.where(bad, np.inf, out)


def e4m3_code_distance(a: np.ndarray, sa: np.ndarray, b: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """Distance, in steps of the e4m3 grid at the coarser of the two block scales,
    between two requantised values (codes a, b with UE8M0 scale bytes sa, sb). A value
    that lies between two grid points of the coarser scale (a fine-scale subnormal) sits
    half way between their positions. A NaN code (0x7F, 0xFF) or a NaN scale byte (255)
    on either side gives inf: such a value is never an acceptable requantisation."""
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    sa = np.asarray(sa, dtype=np.int64)
    sb = np.asarray(sb, dtype=np.int64)
    invalid = np.isnan(E4M3_TABLE[a]) | np.isnan(E4M3_TABLE[b]) | (sa == 255) | (sb == 255)
    s = np.maximum(sa, sb) - 127
    # both values on the coarser scale's grid: e4m3 value times 2^(own scale - coarser scale)
    ia = _grid_index(np.where(invalid, 0.0, E4M3_TABLE[a]) * np.ldexp(1.0, sa - 127 - s))
    ib = _grid_index(np.where(invalid, 0.0, E4M3_TABLE[b]) * np.ldexp(1.0, sb - 127 - s))
    return np.where(invalid, np.inf, np.abs(ia - ib))


_POS_VALUES = np.array([e4m3_value(c) for c in range(0x7F)])   # ascending magnitudes 0..448


def _grid_index(v: np.ndarray) -> np.ndarray:
    """Signed position of v on the e4m3 grid (between-grid values get a half index)."""
    a = np.abs(v)
    i = np.searchsorted(_POS_VALUES, a)
    i = np.clip(i, 0, len(_POS_VALUES) - 1)
    exact = _POS_VALUES[i] == a
    idx = np.where(exact, i.astype(np.float64), i - 0.5)
    return np.where(np.signbit(v) & (a > 0), -idx, idx)
