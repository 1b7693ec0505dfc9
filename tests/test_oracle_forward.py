"""Pins for the oracle's expert FFN and combine (CPU only).

- the hand-derived closed-form example (tests/golden/closed_form_ffn.json)
- exact rational arithmetic for Linear1 on tiny shapes
- a single expert with k=1, w=1 reduces to a dense FFN computed with torch fp64
  matmul, torch's silu and torch's e4m3 cast
- invariants: token order, expert relabelling, weight doubling, scale shifts,
  w=0 vs unused slot, empty experts, token/column sampling
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import MoEConfig, make_inputs
from closed_form import build_closed_form_inputs, expected_y_bits


def _small(T=6, E=3, k=2, H=256, I=256, seed=0, routing="uniform"):
    cfg = MoEConfig("small", T=T, E=E, k=k, H=H, I=I, routing=routing)
    return make_inputs(cfg, seed=seed).numpy()


def test_closed_form_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "closed_form_ffn.json")))
    inp = build_closed_form_inputs()
    r = oracle.forward_inputs(inp)
    assert np.array_equal(r["y_bits"], expected_y_bits())
    for slot, code in g["expected"]["h8"].items():
        assert np.all(r["h8"][int(slot)] == int(code, 16)), slot
    for slot, b in g["expected"]["h_sf"].items():
        assert r["h_sf"][int(slot)].tolist() == [b], slot
    ro = oracle.route(inp["topk_idx"], 2, 16)
    exp = g["expected"]["route_BM16"]
    assert ro["counts"].tolist() == exp["counts"]
    assert ro["offsets"].tolist() == exp["offsets"]
    assert ro["inv"].tolist() == exp["inv"]
    for p, s in exp["perm_head"].items():
        assert ro["perm"][int(p)] == s


def test_linear2_combine_on_hand_derived_intermediates():
    """Linear2 and the combine alone, fed the dequantised intermediates the worked example
    derives by hand (h' = 8192 for slot 0, -8192 for slot 1, -3072 for slot 2), give the
    example's y; a token subset and a column subset give the matching part of it."""
    inp = build_closed_form_inputs()
    hd = {0: np.full(128, 8192.0), 1: np.full(128, -8192.0), 2: np.full(128, -3072.0)}
    r = oracle.linear2_combine(hd, inp["topk_idx"], inp["topk_weights"], inp["w2"], inp["w2_sf"])
    assert np.array_equal(r["y_bits"], expected_y_bits())
    r1 = oracle.linear2_combine({2: hd[2]}, inp["topk_idx"], inp["topk_weights"], inp["w2"],
                                inp["w2_sf"], tokens=[1], cols=[0, 5])
    assert r1["y_bits"].tolist() == [[0xC8C0, 0xC840]]
    # one element of slot 0 one code up (0x79 at scale 2^5: 9216): o_m grows by 1024 * W2[0][m][0],
    # so y[0, 1] = 524288 + 0.75 * 1024 = 525056, which bf16 (step 4096 there) rounds back to 2^19,
    # and y[0, 0] = -131072 + 0.75 * 512 = -130688, which rounds to -130560 (step 512 below 2^17)
    hd1 = dict(hd)
    hd1[0] = hd[0].copy()
    hd1[0][0] = 9216.0
    r2 = oracle.linear2_combine(hd1, inp["topk_idx"], inp["topk_weights"], inp["w2"], inp["w2_sf"])
    assert r2["y"][0, 0] == -130688.0 and r2["y"][0, 1] == 525056.0
    assert r2["y_bits"][0, 0] == 0xC7FF and r2["y_bits"][0, 1] == 0x4900


def test_closed_form_catches_gate_up_swap_and_nibble_order():
    # the example distinguishes silu(g)*u from silu(u)*g and the nibble order
    inp = build_closed_form_inputs()
    swapped = dict(inp)
    w1 = inp["w1"].copy()
    I = w1.shape[1] // 2
    swapped["w1"] = np.concatenate([w1[:, I:], w1[:, :I]], axis=1)
    assert not np.array_equal(oracle.forward_inputs(swapped)["y_bits"], expected_y_bits())
    nib = dict(inp)
    nib["w1"] = ((inp["w1"] >> 4) | (inp["w1"] << 4)).astype(np.uint8)
    assert not np.array_equal(oracle.forward_inputs(nib)["y_bits"], expected_y_bits())


def test_linear1_exact_rational():
    inp = _small(T=3, E=2, k=1, H=256, I=128, seed=5)
    x = inp["x_fp8"]
    xs = inp["x_sf"]
    for e in range(2):
        xr = oracle.dequant_fp8_rows(x, xs, 256)
        G, U = oracle.linear1(xr, inp["w1"][e], inp["w1_sf"][e])
        codes = oracle.unpack_e2m1(inp["w1"][e])
        for t in range(3):
            for n in (0, 5, 127, 128, 200, 255):
                acc = Fraction(0)
                for c in range(256):
                    xv = Fraction(oracle.e4m3_value(x[t, c])) * Fraction(2) ** (int(xs[t, c // 128]) - 127)
                    wv = Fraction(oracle.e2m1_value(codes[n, c])) * Fraction(2) ** (int(inp["w1_sf"][e][n, c // 32]) - 127)
                    acc += xv * wv
                got = G[t, n] if n < 128 else U[t, n - 128]
                assert Fraction(got) == acc      # products are dyadic; the fp64 sum is exact here


_BOOK = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], dtype=torch.float64)


def _torch_decode_fp8(codes, sf, K):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.from_numpy(sf[:, :K // 128].copy()).view(torch.float8_e8m0fnu).to(torch.float64)
    return (v * sc.repeat_interleave(128, dim=1)).numpy()


def _torch_decode_fp4(packed, sf):
    p = torch.from_numpy(packed).to(torch.int64)
    codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1)
    sc = torch.from_numpy(sf.copy()).view(torch.float8_e8m0fnu).to(torch.float64)
    return (_BOOK[codes] * sc.repeat_interleave(32, dim=1)).numpy()


def _torch_dense_ffn(x, W1, W2):
    """Dense FFN for one expert with torch fp64 ops; requant via torch's e4m3 cast."""
    xt = torch.from_numpy(x)
    I = W1.shape[0] // 2
    g = xt @ torch.from_numpy(W1[:I]).T
    u = xt @ torch.from_numpy(W1[I:]).T
    h = (torch.nn.functional.silu(g) * u).to(torch.float32)
    hb = h.view(h.shape[0], -1, 128)
    amax = hb.abs().amax(-1, keepdim=True).to(torch.float64)
    # scale: smallest power of two 2^s with amax <= 448 * 2^s, by search over s
    s = torch.ceil(torch.log2(amax / 448.0))
    s = torch.where(amax * 2.0 ** (-s) > 448.0, s + 1, s)
    s = torch.where(amax * 2.0 ** (-(s - 1)) <= 448.0, s - 1, s)
    s = torch.where(amax == 0, torch.zeros_like(s), s).clamp(min=-127)
    q = (hb.to(torch.float64) * 2.0 ** (-s)).to(torch.float8_e4m3fn).to(torch.float64)
    hd = (q * 2.0 ** s).view(h.shape[0], -1)
    return (hd @ torch.from_numpy(W2).T).numpy()


def test_single_expert_reduces_to_dense_ffn():
    inp = _small(T=16, E=1, k=1, H=256, I=512, seed=7)
    inp["topk_idx"][:] = 0
    inp["topk_weights"][:] = 1.0
    r = oracle.forward_inputs(inp)
    # decode with torch's float8_e4m3fn / float8_e8m0fnu and an explicit E2M1 codebook
    x = _torch_decode_fp8(inp["x_fp8"], inp["x_sf"], 256)
    W1 = _torch_decode_fp4(inp["w1"][0], inp["w1_sf"][0])
    W2 = _torch_decode_fp4(inp["w2"][0], inp["w2_sf"][0])
    ref = _torch_dense_ffn(x, W1, W2)
    ref_bits = torch.from_numpy(ref).to(torch.bfloat16)   # torch fp64 -> bf16
    ours = oracle.bf16_bits_to_f64(r["y_bits"])
    assert np.allclose(ours, ref_bits.to(torch.float64).numpy(), rtol=2 ** -8, atol=0)
    # before the final rounding the two agree to fp64 rounding
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-30)


def test_token_order_equivariance():
    inp = _small(T=9, E=3, k=2, seed=1)
    r = oracle.forward_inputs(inp)
    perm = np.random.default_rng(0).permutation(9)
    p = dict(inp)
    for key in ("x_fp8", "x_sf", "topk_idx", "topk_weights"):
        p[key] = inp[key][perm]
    rp = oracle.forward_inputs(p)
    assert np.array_equal(rp["y_bits"], r["y_bits"][perm])


def test_expert_relabelling():
    inp = _small(T=9, E=4, k=2, seed=2)
    r = oracle.forward_inputs(inp)
    sigma = np.array([2, 0, 3, 1])          # new expert id of old expert e
    p = dict(inp)
    p["topk_idx"] = sigma[inp["topk_idx"]].astype(np.int32)
    invs = np.argsort(sigma)
    for key in ("w1", "w1_sf", "w2", "w2_sf"):
        p[key] = inp[key][invs]
    assert np.array_equal(oracle.forward_inputs(p)["y_bits"], r["y_bits"])


def test_weight_doubling_and_scale_shifts():
    inp = _small(T=8, E=2, k=2, seed=3)
    r = oracle.forward_inputs(inp)
    y = oracle.bf16_bits_to_f64(r["y_bits"])
    p = dict(inp)
    p["topk_weights"] = inp["topk_weights"] * 2
    assert np.array_equal(oracle.bf16_bits_to_f64(oracle.forward_inputs(p)["y_bits"]), 2 * y)
    p = dict(inp)
    p["w2_sf"] = inp["w2_sf"] + 1            # every W2 doubled
    assert np.array_equal(oracle.bf16_bits_to_f64(oracle.forward_inputs(p)["y_bits"]), 2 * y)
    p = dict(inp)
    I = inp["w1"].shape[1] // 2
    sf = inp["w1_sf"].copy()
    sf[:, I:] += 1                           # up half doubled: h doubles exactly
    p["w1_sf"] = sf
    rp = oracle.forward_inputs(p)
    for s in r["h8"]:
        assert np.array_equal(rp["h8"][s], r["h8"][s])
        assert np.array_equal(rp["h_sf"][s].astype(int), r["h_sf"][s].astype(int) + 1)
    assert np.array_equal(oracle.bf16_bits_to_f64(rp["y_bits"]), 2 * y)


def test_zero_weight_equals_unused_slot_and_empty_experts():
    inp = _small(T=8, E=3, k=2, seed=4)
    a = dict(inp)
    a["topk_weights"] = inp["topk_weights"].copy()
    a["topk_weights"][:, 1] = 0.0
    b = dict(inp)
    b["topk_idx"] = inp["topk_idx"].copy()
    b["topk_idx"][:, 1] = -1
    ya = oracle.bf16_bits_to_f64(oracle.forward_inputs(a)["y_bits"])
    yb = oracle.bf16_bits_to_f64(oracle.forward_inputs(b)["y_bits"])
    assert np.array_equal(ya, yb)
    # an extra expert nobody routes to changes nothing
    c = dict(inp)
    for key in ("w1", "w1_sf", "w2", "w2_sf"):
        c[key] = np.concatenate([inp[key], inp[key][:1] ^ np.uint8(0x11) if key in ("w1", "w2") else inp[key][:1]], axis=0)
    assert np.array_equal(oracle.forward_inputs(c)["y_bits"], oracle.forward_inputs(inp)["y_bits"])


def test_unrouted_token_gives_positive_zero():
    inp = _small(T=4, E=2, k=2, seed=6)
    inp["topk_idx"][2, :] = -1
    r = oracle.forward_inputs(inp)
    assert np.all(r["y_bits"][2] == 0)


def test_sampling_matches_full():
    inp = _small(T=10, E=3, k=2, seed=8)
    full = oracle.forward_inputs(inp)
    toks = [7, 1, 4]
    cols = [0, 3, 100, 255]
    part = oracle.forward_inputs(inp, tokens=toks, cols=cols)
    assert np.array_equal(part["y_bits"], full["y_bits"][np.ix_(toks, cols)])
    for s in part["h8"]:
        assert np.array_equal(part["h8"][s], full["h8"][s])


def test_invalid_ids_are_skipped():
    inp = _small(T=6, E=3, k=2, seed=9)
    a = dict(inp)
    a["topk_idx"] = inp["topk_idx"].copy()
    a["topk_idx"][1, 0] = 7
    a["topk_idx"][3, 1] = -5
    b = dict(inp)
    b["topk_idx"] = a["topk_idx"].copy()
    b["topk_idx"][1, 0] = -1
    b["topk_idx"][3, 1] = -1
    assert np.array_equal(oracle.forward_inputs(a)["y_bits"], oracle.forward_inputs(b)["y_bits"])


def _fp32_sums(p64: np.ndarray):
    """FP32 accumulations of the exact products p64 [..., K] in several orders and two
    rounding modes: sequential, reversed, pairwise (numpy), blocks of 128 then across
    blocks, and sequential with rounding toward zero."""
    p32 = p64.astype(np.float32)
    assert np.array_equal(p32.astype(np.float64), p64)           # the products are exact
    K = p64.shape[-1]
    out = []
    acc = np.zeros(p64.shape[:-1], np.float32)
    for c in range(K):
        acc = acc + p32[..., c]
    out.append(acc)
    acc = np.zeros(p64.shape[:-1], np.float32)
    for c in reversed(range(K)):
        acc = acc + p32[..., c]
    out.append(acc)
    out.append(np.sum(p32, axis=-1, dtype=np.float32))
    blocks = [np.sum(p32[..., b:b + 128], axis=-1, dtype=np.float32) for b in range(0, K, 128)]
    acc = np.zeros(p64.shape[:-1], np.float32)
    for b in blocks:
        acc = acc + b
    out.append(acc)
    acc = np.zeros(p64.shape[:-1], np.float32)
    for c in range(K):
        v = acc.astype(np.float64) + p64[..., c]
        r = v.astype(np.float32)
        over = np.abs(r.astype(np.float64)) > np.abs(v)
        acc = np.where(over, np.nextafter(r, np.float32(0)), r)
    out.append(acc)
    return out


def _bound_ratios(pg, pu, g, u):
    """|h32 - h| / bound for every FP32 summation variant of the products pg, pu."""
    K = pg.shape[-1]
    h = oracle.swiglu(g, u)
    bound = oracle.accumulation_error_bound(g, u, np.abs(pg).sum(-1), np.abs(pu).sum(-1), K)
    out = []
    for g32, u32 in zip(_fp32_sums(pg), _fp32_sums(pu)):
        one = np.float32(1)
        h32 = (g32 / (one + np.exp(-g32)) * u32).astype(np.float64)
        out.append(np.abs(h32 - h) / bound)
    return np.max(out, axis=0), bound, h


def test_accumulation_error_bound_on_the_path_operands():
    """The bound holds for products of e4m3 activations and E2M1 weights as the path
    makes them, summed in FP32 in several orders and rounding modes, then an FP32 SwiGLU;
    and it stays far below the size of h."""
    K, R, N = 512, 16, 16
    inp = _small(T=R, E=1, k=1, H=K, I=128, seed=3)
    x = oracle.dequant_fp8_rows(inp["x_fp8"], inp["x_sf"], K)                  # [R, K]
    w = oracle.dequant_fp4_rows(inp["w1"][0], inp["w1_sf"][0], K)             # [256, K]
    pg = x[:, None, :] * w[None, :N, :]
    pu = x[:, None, :] * w[None, 128:128 + N, :]
    ratio, bound, h = _bound_ratios(pg, pu, pg.sum(-1), pu.sum(-1))
    assert np.all(ratio <= 1.0), ratio.max()
    assert np.median(bound) < 1e-3 * np.abs(h).max()


def test_accumulation_error_bound_is_sharp_on_adversarial_sums():
    """The bound covers arbitrary FP32 terms (it is a statement about any exactly
    representable products), and adversarial sums come within a small factor of it, so
    that neither of its two error paths nor the growth with K can be dropped. Columns 0-3
    cancel in the up projection, columns 4-7 in the gate projection: positive terms in
    [0.5, 1) on the first K half and the same terms negated on the second, so a sequential
    sum climbs to its largest value before cancelling to an exact 0 and keeps the rounding
    errors of the climb (most of all when rounding toward zero)."""
    K, R, N = 512, 4, 8
    rng = np.random.default_rng(11)
    half = K // 2
    pg = rng.standard_normal((R, N, K)).astype(np.float32).astype(np.float64)
    pu = rng.standard_normal((R, N, K)).astype(np.float32).astype(np.float64)
    for p, cols in ((pu, slice(0, 4)), (pg, slice(4, 8))):
        pos = rng.uniform(0.5, 1.0, (R, 4, half)).astype(np.float32).astype(np.float64)
        p[:, cols, :half] = pos
        p[:, cols, half:] = -pos
    g = np.array([[math.fsum(v) for v in row] for row in pg])
    u = np.array([[math.fsum(v) for v in row] for row in pu])
    assert np.all(u[:, :4] == 0) and np.all(g[:, 4:] == 0)
    ratio, _, _ = _bound_ratios(pg, pu, g, u)
    assert np.all(ratio <= 1.0), ratio.max()
    # u = 0 leaves silu(g) * du; g = 0 leaves silu'(0) * dg * u
    assert ratio[:, :4].max() > 0.02 and ratio[:, 4:].max() > 0.02, ratio.max(axis=0)
