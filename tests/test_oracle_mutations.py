"""The oracle's pins have teeth: plant one plausible mistake at a time in a copy of the oracle's
source (on the CPU), rerun the existing pins against that copy, and require that the pins named
for the mistake fail.

Each mistake is a text edit of oracle/moe_oracle.py or oracle/gemm_oracle.py that must match
exactly once (the MUTANTS table): codec mistakes (nibble order, scale exponents off by one,
a scale read from the wrong block, ties rounded away from even, the subnormal quantum, the
scale rule's tie, the byte clamp, bf16 rounded to 9 bits or truncated), routing mistakes
(padding dropped from the scan, the stable order transposed, unused slots counted as
invalid), FFN and combine mistakes (gate and up swapped, a sign flip in silu, the
requantisation skipped or decided on fp64, the top-k weight dropped, a slot left out), error
bounds that lose a term or their growth with K, and GEMM/cast layout mistakes (the masked
count unclamped, padding rows marked valid, scale bytes in the wrong order). The unedited
copy must pass every pin, so a failure comes from the planted mistake and not from the way
the copy is loaded.

The copies are loaded as modules of their own; the `oracle` package's names are pointed at
them for the duration of one check and restored afterwards (monkeypatch)."""
import inspect
import os
import sys
import types

import pytest

import oracle
import test_oracle_checkers as P_checkers
import test_oracle_codecs as P_codecs
import test_oracle_forward as P_forward
import test_oracle_gemm as P_gemm
import test_oracle_route as P_route

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _pins():
    """name -> zero-argument callable, one per pin (parametrised pins once per case)."""
    pins = {}
    for mod in (P_checkers, P_codecs, P_forward, P_gemm, P_route):
        short = mod.__name__.replace("test_oracle_", "")
        for name, fn in vars(mod).items():
            if not (name.startswith("test_") and inspect.isfunction(fn)):
                continue
            params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
            args = list(inspect.signature(fn).parameters)
            if params:
                argnames = [a.strip() for a in params[0].args[0].split(",")]
                for vals in params[0].args[1]:
                    vals = vals if isinstance(vals, tuple) else (vals,)
                    kw = dict(zip(argnames, vals))
                    pins[f"{short}.{name}[{'-'.join(map(str, vals))}]"] = (
                        lambda fn=fn, kw=kw: fn(**kw))
            elif args == ["golden_dir"]:
                pins[f"{short}.{name}"] = lambda fn=fn: fn(GOLDEN)
            else:
                assert not args, f"{name}: unexpected arguments {args}"
                pins[f"{short}.{name}"] = fn
    return pins


PINS = _pins()


def _load(name, src):
    mod = types.ModuleType(f"oracle.{name}")
    mod.__package__ = "oracle"
    mod.__file__ = os.path.join(ORACLE_DIR, name + ".py")
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


def _source(name):
    with open(os.path.join(ORACLE_DIR, name + ".py")) as f:
        return f.read()


def _install_copy(monkeypatch, target=None, old=None, new=None):
    """Load fresh copies of both oracle modules, with `old` replaced by `new` in `target`,
    and point the oracle package (and sys.modules, which the relative imports of the
    GEMM module resolve through) at them until the test ends."""
    srcs = {n: _source(n) for n in ("moe_oracle", "gemm_oracle")}
    if target is not None:
        assert srcs[target].count(old) == 1, f"mutation site not unique in {target}: {old!r}"
        srcs[target] = srcs[target].replace(old, new)
    moe = _load("moe_oracle", srcs["moe_oracle"])
    monkeypatch.setitem(sys.modules, "oracle.moe_oracle", moe)
    gemm = _load("gemm_oracle", srcs["gemm_oracle"])         # binds the copied moe_oracle
    monkeypatch.setitem(sys.modules, "oracle.gemm_oracle", gemm)
    for mod in (moe, gemm):
        for k, v in vars(mod).items():
            if not k.startswith("__") and hasattr(oracle, k):
                monkeypatch.setattr(oracle, k, v)


def _failing(names):
    failed = []
    for n in names:
        try:
            PINS[n]()
        except Exception:          # an assertion, or any error the mistake provokes
            failed.append(n)
    return failed


# (id, module, text to replace, replacement, pins that must fail)
MUTANTS = [
    ('nibble_order', 'moe_oracle',
     'E2M1_TABLE[np.arange(256) & 0x0F], E2M1_TABLE[np.arange(256) >> 4]',
     'E2M1_TABLE[np.arange(256) >> 4], E2M1_TABLE[np.arange(256) & 0x0F]',
     ['forward.test_closed_form_example',
      'forward.test_closed_form_catches_gate_up_swap_and_nibble_order',
      'forward.test_linear1_exact_rational',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_gemm_equals_exact_rational_sum',
      'gemm.test_gemm_one_hot_selects_a_column_of_b']),
    ('unpack_nibble_order', 'moe_oracle',
     'out[..., 0::2] = packed & 0x0F\n    out[..., 1::2] = packed >> 4',
     'out[..., 0::2] = packed >> 4\n    out[..., 1::2] = packed & 0x0F',
     ['codecs.test_e2m1_nibble_order',
      'forward.test_linear1_exact_rational']),
    ('fp8_scale_off_by_one', 'moe_oracle',
     'scale = decode_ue8m0(sf[:, : K // 128])',
     'scale = 2.0 * decode_ue8m0(sf[:, : K // 128])',
     ['forward.test_closed_form_example',
      'forward.test_linear1_exact_rational',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_gemm_equals_exact_rational_sum',
      'gemm.test_gemm_one_hot_selects_a_column_of_b']),
    ('fp4_scale_wrong_block', 'moe_oracle',
     'np.multiply(v, scale[:, :, None], out=v)',
     'np.multiply(v, scale[:, ::-1, None], out=v)',
     ['forward.test_linear1_exact_rational',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_gemm_equals_exact_rational_sum',
      'gemm.test_gemm_one_hot_selects_a_column_of_b']),
    ('fp4_scale_off_by_one', 'moe_oracle',
     'scale = decode_ue8m0(sf[:, : K // 32])',
     'scale = 0.5 * decode_ue8m0(sf[:, : K // 32])',
     ['forward.test_closed_form_example',
      'forward.test_linear1_exact_rational',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_gemm_equals_exact_rational_sum',
      'gemm.test_gemm_one_hot_selects_a_column_of_b']),
    ('e4m3_ties_away', 'moe_oracle',
     'q = np.rint((m - 1.0) * 8.0)',
     'q = np.floor((m - 1.0) * 8.0 + 0.5)',
     ['codecs.test_e4m3_encoder_matches_torch_rne',
      'codecs.test_e4m3_encoder_ties_to_even',
      'codecs.test_requant_decides_on_fp32_value',
      'forward.test_closed_form_example',
      'gemm.test_cast_matches_torch_float8_cast']),
    ('e4m3_subnormal_quantum', 'moe_oracle',
     'q_sub = np.rint(a * 512.0)',
     'q_sub = 2 * np.rint(a * 256.0)',
     ['codecs.test_e4m3_encoder_matches_torch_rne',
      'codecs.test_requant_grid_roundtrip_and_clamp',
      'codecs.test_requant_codes_match_torch_cast',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_cast_round_trips_values_on_the_grid']),
    ('scale_rule_tie', 'moe_oracle',
     's = e - qe + (m > qm).astype(np.int64)',
     's = e - qe + (m >= qm).astype(np.int64)',
     ['codecs.test_pow2_scale_rule_invariants',
      'codecs.test_requant_grid_roundtrip_and_clamp',
      'gemm.test_cast_round_trips_values_on_the_grid',
      'gemm.test_cast_edge_blocks']),
    ('requant_on_fp64', 'moe_oracle',
     'h32 = round_f32(h).astype(np.float64)',
     'h32 = np.asarray(h, dtype=np.float64)',
     ['codecs.test_requant_decides_on_fp32_value']),
    ('byte_clamp_dropped', 'moe_oracle',
     'byte = np.maximum(s + 127, 0)',
     'byte = s + 127',
     ['codecs.test_requant_grid_roundtrip_and_clamp',
      'gemm.test_cast_edge_blocks']),
    ('scan_no_padding', 'moe_oracle',
     'offsets[e + 1] = offsets[e] + padded[e]',
     'offsets[e + 1] = offsets[e] + counts[e]',
     ['forward.test_closed_form_example',
      'route.test_route_hand_worked_example',
      'route.test_route_synthetic_configs[c0-256]',
      'route.test_route_synthetic_configs[c1-64]',
      'route.test_route_synthetic_configs[c3-256]',
      'route.test_route_synthetic_configs[c3e-128]',
      'route.test_route_synthetic_configs[c4-256]',
      'route.test_route_edge_cases']),
    ('route_order_transposed', 'moe_oracle',
     '    for t in range(T):\n        for j in range(k):\n            e = int(topk_idx[t, j])',
     '    for j in range(k):\n        for t in range(T):\n            e = int(topk_idx[t, j])',
     ['forward.test_closed_form_example',
      'route.test_route_hand_worked_example',
      'route.test_route_synthetic_configs[c0-256]',
      'route.test_route_synthetic_configs[c1-64]',
      'route.test_route_synthetic_configs[c3-256]',
      'route.test_route_synthetic_configs[c3e-128]',
      'route.test_route_synthetic_configs[c4-256]',
      'route.test_route_edge_cases']),
    ('unused_counted_invalid', 'moe_oracle',
     'elif e != -1:',
     'else:',
     ['route.test_route_hand_worked_example',
      'route.test_route_edge_cases']),
    ('gate_up_swap', 'moe_oracle',
     'h = swiglu(G, U)',
     'h = swiglu(U, G)',
     ['forward.test_closed_form_example',
      'forward.test_closed_form_catches_gate_up_swap_and_nibble_order',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'forward.test_weight_doubling_and_scale_shifts']),
    ('silu_sign', 'moe_oracle',
     'return g / (1.0 + np.exp(-g)) * u',
     'return g / (1.0 + np.exp(g)) * u',
     ['forward.test_closed_form_example',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'forward.test_accumulation_error_bound_on_the_path_operands']),
    ('requant_skipped', 'moe_oracle',
     'hdeq[t * k + j] = hd[r]',
     'hdeq[t * k + j] = h[r]',
     ['forward.test_single_expert_reduces_to_dense_ffn']),
    ('topk_weight_dropped', 'moe_oracle',
     'contrib[tok_pos[t], j] = float(topk_weights[t, j]) * O[r]',
     'contrib[tok_pos[t], j] = O[r]',
     ['forward.test_closed_form_example',
      'forward.test_weight_doubling_and_scale_shifts',
      'forward.test_zero_weight_equals_unused_slot_and_empty_experts']),
    ('combine_drops_last_slot', 'moe_oracle',
     '    for j in range(k):\n        acc += contrib[:, j]',
     '    for j in range(k - 1):\n        acc += contrib[:, j]',
     ['forward.test_closed_form_example',
      'forward.test_single_expert_reduces_to_dense_ffn']),
    ('bf16_nine_bits', 'moe_oracle',
     'qexp = np.maximum(e - 8, -133)',
     'qexp = np.maximum(e - 9, -133)',
     ['codecs.test_bf16_rounding_matches_torch_on_fp32_values',
      'codecs.test_bf16_rounding_single_rounding_from_fp64',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_fp32_sums_fall_within_the_bound']),
    ('bf16_truncates', 'moe_oracle',
     'r = np.ldexp(np.rint(np.ldexp(v, -qexp)), qexp)',
     'r = np.ldexp(np.trunc(np.ldexp(v, -qexp)), qexp)',
     ['codecs.test_bf16_rounding_matches_torch_on_fp32_values',
      'codecs.test_bf16_rounding_single_rounding_from_fp64',
      'forward.test_single_expert_reduces_to_dense_ffn',
      'gemm.test_fp32_sums_fall_within_the_bound']),
    ('swiglu_bound_drops_du_term', 'moe_oracle',
     'acc = SILU_LIPSCHITZ * dg * (np.abs(u) + du) + np.abs(sg) * du',
     'acc = SILU_LIPSCHITZ * dg * (np.abs(u) + du)',
     ['forward.test_accumulation_error_bound_is_sharp_on_adversarial_sums']),
    ('swiglu_bound_drops_dg_term', 'moe_oracle',
     'acc = SILU_LIPSCHITZ * dg * (np.abs(u) + du) + np.abs(sg) * du',
     'acc = np.abs(sg) * du',
     ['forward.test_accumulation_error_bound_is_sharp_on_adversarial_sums']),
    ('swiglu_bound_gamma_no_K', 'moe_oracle',
     'gamma = n * FP32_UNIT / (1.0 - n * FP32_UNIT)',
     'gamma = FP32_UNIT',
     ['forward.test_accumulation_error_bound_is_sharp_on_adversarial_sums']),
    ('gemm_bound_abs_of_sum', 'gemm_oracle',
     'bound = gamma * (np.abs(A) @ np.abs(B).T)',
     'bound = gamma * np.abs(A @ B.T)',
     ['gemm.test_gemm_equals_exact_rational_sum']),
    ('gemm_bound_gamma_no_K', 'gemm_oracle',
     'gamma = (K - 1) * _U32 / (1.0 - (K - 1) * _U32)',
     'gamma = _U32',
     ['gemm.test_gemm_equals_exact_rational_sum',
      'gemm.test_fp32_sums_fall_within_the_bound']),
    ('masked_unclamped', 'gemm_oracle',
     'c = int(min(max(int(masked_m[g]), 0), max_m))',
     'c = int(min(int(masked_m[g]), max_m))',
     ['gemm.test_masked_layout_counts']),
    ('padding_rows_valid', 'gemm_oracle',
     '"valid": group_of_row >= 0}',
     '"valid": group_of_row >= -1}',
     ['gemm.test_contiguous_layout_matches_rows_of_dense']),
    ('cast_sf_reversed', 'gemm_oracle',
     'out_sf[:, : C // 128] = sf',
     'out_sf[:, : C // 128] = sf[:, ::-1]',
     ['gemm.test_cast_round_trips_values_on_the_grid',
      'gemm.test_cast_matches_torch_float8_cast',
      'gemm.test_cast_edge_blocks']),
    ('gemm_a_scales_reversed', 'gemm_oracle',
     'A = dequant_fp8_rows(np.asarray(a), np.asarray(a_sf), K)',
     'A = dequant_fp8_rows(np.asarray(a), np.asarray(a_sf)[:, ::-1], K)',
     ['gemm.test_gemm_equals_exact_rational_sum',
      'gemm.test_gemm_one_hot_selects_a_column_of_b',
      'gemm.test_fp32_sums_fall_within_the_bound']),
]


# Mistakes in the acceptance metrics every GPU comparison runs through
CHECKER_PINS = ['checkers.test_code_distance_hand_cases',
                'checkers.test_code_distance_same_scale_is_rank_difference',
                'checkers.test_code_distance_across_scales_by_counting']
MUTANTS += [
    ('distance_on_finer_scale', 'moe_oracle',
     's = np.maximum(sa, sb) - 127',
     's = np.minimum(sa, sb) - 127',
     ['checkers.test_code_distance_hand_cases',
      'checkers.test_code_distance_across_scales_by_counting']),
    ('grid_index_no_half_step', 'moe_oracle',
     'idx = np.where(exact, i.astype(np.float64), i - 0.5)',
     'idx = np.where(exact, i.astype(np.float64), i - 1.0)',
     ['checkers.test_code_distance_hand_cases',
      'checkers.test_code_distance_across_scales_by_counting']),
    ('grid_index_half_step_up', 'moe_oracle',
     'idx = np.where(exact, i.astype(np.float64), i - 0.5)',
     'idx = np.where(exact, i.astype(np.float64), i + 0.5)',
     ['checkers.test_code_distance_hand_cases',
      'checkers.test_code_distance_across_scales_by_counting']),
    ('grid_index_unsigned', 'moe_oracle',
     'return np.where(np.signbit(v) & (a > 0), -idx, idx)',
     'return idx',
     CHECKER_PINS),
    ('grid_index_negative_zero_signed', 'moe_oracle',
     'return np.where(np.signbit(v) & (a > 0), -idx, idx)',
     'return np.where(np.signbit(v), -idx - 0.5, idx)',
     ['checkers.test_code_distance_hand_cases',
      'checkers.test_code_distance_same_scale_is_rank_difference']),
    ('distance_nan_scale_accepted', 'moe_oracle',
     ' | (sa == 255) | (sb == 255)',
     '',
     ['checkers.test_code_distance_hand_cases']),
    ('distance_nan_code_accepted', 'moe_oracle',
     'invalid = np.isnan(E4M3_TABLE[a]) | np.isnan(E4M3_TABLE[b]) |',
     'invalid =',
     ['checkers.test_code_distance_hand_cases']),
    ('y_error_mean_not_max', 'moe_oracle',
     'num = np.abs(np.where(np.isfinite(yg), yg, 0.0) - yr).max(axis=1)',
     'num = np.abs(np.where(np.isfinite(yg), yg, 0.0) - yr).mean(axis=1)',
     ['checkers.test_y_row_error_hand_cases']),
    ('y_error_mean_denominator', 'moe_oracle',
     'den = np.abs(yr).max(axis=1)',
     'den = np.abs(yr).mean(axis=1)',
     ['checkers.test_y_row_error_hand_cases']),
    ('y_error_zero_row_lenient', 'moe_oracle',
     'np.where(num == 0, 0.0, np.inf))',
     '0.0)',
     ['checkers.test_y_row_error_hand_cases']),
    ('y_error_nan_passes', 'moe_oracle',
     'return np.where(bad, np.inf, out)',
     'return out',
     ['checkers.test_y_row_error_hand_cases']),
]


def test_pin_registry_is_complete():
    # every pin function of the four pin modules is in the registry
    assert len(PINS) >= 40
    assert "forward.test_closed_form_example" in PINS
    assert "route.test_route_synthetic_configs[c0-256]" in PINS


def test_unmutated_copy_passes_every_pin(monkeypatch):
    _install_copy(monkeypatch)
    assert oracle.forward is sys.modules["oracle.moe_oracle"].forward
    assert _failing(PINS) == []


@pytest.mark.parametrize("mid,target,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, mid, target, old, new, catchers):
    _install_copy(monkeypatch, target, old, new)
    assert catchers, mid
    failed = _failing(catchers)
    assert failed == catchers, f"{mid}: pins that still pass: {sorted(set(catchers) - set(failed))}"
