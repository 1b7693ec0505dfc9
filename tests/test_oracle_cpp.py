"""Pins of the plain C++ oracle (oracle/ref_forward.cpp), a second, independently written
form of the forward oracle that the benchmark times as its CPU baseline.

It must reproduce the hand-derived worked example (tests/golden/closed_form_ffn.json), the
one-expert case reduced to a dense FFN computed with torch fp64 ops and torch's own e4m3
cast, and the numpy oracle bit for bit (y, every requantised code and scale byte) on
seeded workloads that include unused (-1) and out-of-range expert ids, a token subset, H
and I that are odd multiples of 128, and a Zipf-routed case; its result must not depend
on its thread count."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from closed_form import build_closed_form_inputs, expected_y_bits
from oracle import ref_cpp
from synth import MoEConfig, make_inputs
from test_oracle_forward import _torch_decode_fp4, _torch_decode_fp8, _torch_dense_ffn


def _inputs(T, E, k, H, I, seed, routing="uniform"):
    return make_inputs(MoEConfig("cpp", T=T, E=E, k=k, H=H, I=I, routing=routing), seed=seed).numpy()


def _same(a, b):
    assert np.array_equal(a["y_bits"], b["y_bits"])
    assert sorted(a["h8"]) == sorted(b["h8"])
    for s in a["h8"]:
        assert np.array_equal(a["h8"][s], b["h8"][s]), s
        assert np.array_equal(a["h_sf"][s], b["h_sf"][s]), s


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_cpp_closed_form_example(lib=None):
    g = json.load(open(os.path.join(GOLDEN, "closed_form_ffn.json")))
    r = ref_cpp.forward_cpp(build_closed_form_inputs(), threads=2, lib=lib)
    assert np.array_equal(r["y_bits"], expected_y_bits())
    for slot, code in g["expected"]["h8"].items():
        assert np.all(r["h8"][int(slot)] == int(code, 16)), slot
    for slot, b in g["expected"]["h_sf"].items():
        assert r["h_sf"][int(slot)].tolist() == [b], slot
    assert sorted(r["h8"]) == [0, 1, 2]        # token 1's second slot is unused (-1)


def test_cpp_single_expert_reduces_to_dense_ffn(lib=None):
    inp = _inputs(16, 1, 1, 256, 512, seed=7)
    inp["topk_idx"][:] = 0
    inp["topk_weights"][:] = 1.0
    r = ref_cpp.forward_cpp(inp, threads=3, lib=lib)
    x = _torch_decode_fp8(inp["x_fp8"], inp["x_sf"], 256)
    W1 = _torch_decode_fp4(inp["w1"][0], inp["w1_sf"][0])
    W2 = _torch_decode_fp4(inp["w2"][0], inp["w2_sf"][0])
    ref = _torch_dense_ffn(x, W1, W2)
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-30)
    ref_bits = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.allclose(oracle.bf16_bits_to_f64(r["y_bits"]), ref_bits, rtol=2 ** -8, atol=0)


@pytest.mark.parametrize("T,E,k,H,I,seed,routing", [
    (64, 4, 2, 256, 512, 0, "uniform"),      # the tiny workload's shape
    (40, 3, 3, 384, 128, 1, "uniform"),      # H, I odd multiples of 128
    (50, 6, 4, 640, 384, 2, "zipf"),         # skewed routing, scale words with unused bytes
])
def test_cpp_matches_numpy_oracle(T, E, k, H, I, seed, routing, lib=None):
    inp = _inputs(T, E, k, H, I, seed, routing)
    # unused slots and out-of-range ids are skipped by both
    inp["topk_idx"][1, 0] = -1
    inp["topk_idx"][3, k - 1] = E + 5
    inp["topk_idx"][4, :] = -1
    _same(ref_cpp.forward_cpp(inp, threads=4, lib=lib), oracle.forward_inputs(inp))
    assert np.all(ref_cpp.forward_cpp(inp, threads=2, lib=lib)["y_bits"][4] == 0)


def _boundary_inputs():
    """One token, one expert, H = I = 128, every value 1.0 or 0 (scale bytes 127): x = 1;
    gate rows hold 1.0 in their first 64 columns, up rows in their first 112, so
    g = 64 (silu(64) = 64 in fp64: e^-64 < 2^-53), u = 112 and every h = 7168 = 448 * 2^4,
    exactly on the scale rule's boundary: s = 4 (byte 131), code 448 (0x7E). W2 is all 1.0,
    so o = 128 * 7168 = 917504 = 1.75 * 2^19, bf16 0x4960."""
    H = I = 128
    x = np.full((1, H), 0x38, dtype=np.uint8)
    x_sf = np.zeros((1, 4), dtype=np.uint8)
    x_sf[0, 0] = 127
    w1c = np.zeros((1, 2 * I, H), dtype=np.uint8)
    w1c[0, :I, :64] = 2
    w1c[0, I:, :112] = 2
    w2c = np.full((1, H, I), 2, dtype=np.uint8)
    pack = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return dict(x_fp8=x, x_sf=x_sf, topk_idx=np.zeros((1, 1), dtype=np.int32),
                topk_weights=np.ones((1, 1), dtype=np.float32), w1=pack(w1c),
                w1_sf=np.full((1, 2 * I, H // 32), 127, dtype=np.uint8), w2=pack(w2c),
                w2_sf=np.full((1, H, I // 32), 127, dtype=np.uint8))


def test_scale_rule_boundary_example(lib=None):
    inp = _boundary_inputs()
    for r in (ref_cpp.forward_cpp(inp, lib=lib), oracle.forward_inputs(inp)):
        assert r["h_sf"][0].tolist() == [131]
        assert np.all(r["h8"][0] == 0x7E)
        assert np.all(r["y_bits"] == 0x4960)


# (id, text to replace in ref_forward.cpp, replacement, pins that must fail)
CPP_MUTANTS = [
    ("nibble_order", "(c % 2 == 0) ? (byte & 15) : (byte >> 4)", "(c % 2 == 0) ? (byte >> 4) : (byte & 15)",
     ["golden", "dense", "numpy0"]),
    ("fp4_scale_wrong_block", "const double s = ue8m0_value(sf[c / 32]);",
     "const double s = ue8m0_value(sf[(c / 32) ^ 1]);", ["dense", "numpy0"]),
    ("fp8_scale_off_by_one", "ue8m0_value(x_sf[(size_t)t * x_sf_stride + c / 128])",
     "2.0 * ue8m0_value(x_sf[(size_t)t * x_sf_stride + c / 128])", ["golden", "dense", "numpy0"]),
    ("e4m3_ties_away", "double q = std::nearbyint((2.0 * m - 1.0) * 8.0);",
     "double q = std::floor((2.0 * m - 1.0) * 8.0 + 0.5);", ["golden"]),   # random data holds no exact tie
    ("e4m3_subnormal_quantum", "const double q = std::nearbyint(a * 512.0);",
     "const double q = 2.0 * std::nearbyint(a * 256.0);", ["numpy0"]),
    ("scale_rule_tie", "(2.0 * m > 1.75 ? 1 : 0)", "(2.0 * m >= 1.75 ? 1 : 0)", ["boundary"]),
    ("gate_up_swap", "const double h = G[n] / (1.0 + std::exp(-G[n])) * U[n];",
     "const double h = U[n] / (1.0 + std::exp(-U[n])) * G[n];", ["golden", "dense", "numpy0"]),
    ("silu_sign", "(1.0 + std::exp(-G[n]))", "(1.0 + std::exp(G[n]))", ["golden", "dense", "numpy0"]),
    ("topk_weight_dropped", "(double)topk_w[(size_t)toks[i] * k + j] * o", "o", ["golden", "numpy0"]),
    ("combine_drops_last_slot", "for (int j = 0; j < k; ++j) acc +=", "for (int j = 0; j + 1 < k; ++j) acc +=",
     ["golden", "numpy0"]),
    ("bf16_truncates", "std::nearbyint(std::ldexp(v, -q))", "std::trunc(std::ldexp(v, -q))",
     ["dense", "numpy0"]),
    ("requant_skipped", "Hq[(size_t)r * I + b * 128 + q] = e4m3_value(code) * scale;",
     "Hq[(size_t)r * I + b * 128 + q] = h32[q];", ["dense", "numpy0"]),
]


@pytest.mark.parametrize("mid,old,new,catchers", CPP_MUTANTS, ids=[m[0] for m in CPP_MUTANTS])
def test_cpp_planted_mistake_is_caught(tmp_path, mid, old, new, catchers):
    src = open(ref_cpp.SRC).read()
    assert src.count(old) == 1, mid
    lib = ref_cpp.load(ref_cpp.build_from_source(src.replace(old, new), str(tmp_path / f"lib_{mid}.so")))
    pins = {"golden": lambda: test_cpp_closed_form_example(lib),
            "dense": lambda: test_cpp_single_expert_reduces_to_dense_ffn(lib),
            "numpy0": lambda: test_cpp_matches_numpy_oracle(64, 4, 2, 256, 512, 0, "uniform", lib),
            "boundary": lambda: test_scale_rule_boundary_example(lib)}
    failed = []
    for name in catchers:
        try:
            pins[name]()
        except (AssertionError, RuntimeError):
            failed.append(name)
    assert failed == catchers, f"{mid}: pins that still pass: {sorted(set(catchers) - set(failed))}"


def test_cpp_token_subset_and_thread_count():
    inp = _inputs(48, 5, 2, 256, 256, seed=3)
    toks = [0, 7, 8, 31, 47]
    a = ref_cpp.forward_cpp(inp, tokens=toks, threads=1)
    b = ref_cpp.forward_cpp(inp, tokens=toks, threads=5)
    _same(a, b)
    assert np.array_equal(a["y"], b["y"])
    full = ref_cpp.forward_cpp(inp, threads=3)
    assert np.array_equal(a["y_bits"], full["y_bits"][toks])
    _same(a, oracle.forward_inputs(inp, tokens=toks))


def test_cpp_rejects_nan_codes():
    inp = _inputs(4, 2, 1, 256, 256, seed=4)
    inp["x_fp8"][2, 5] = 0x7F
    with pytest.raises(RuntimeError):
        ref_cpp.forward_cpp(inp)
    inp = _inputs(4, 2, 1, 256, 256, seed=4)
    inp["w2_sf"][inp["topk_idx"][0, 0], 3, 1] = 255
    with pytest.raises(RuntimeError):
        ref_cpp.forward_cpp(inp)
