"""GPU parity: the HIP path through the C ABI against the oracle, on the same seeded bytes.

Routing/permutation/counts/tile list: bit-exact. Requantised FP8 intermediates: at most
0.1 % differ, each by one code on the e4m3 grid of the coarser block scale; an element more
than one code off passes only if it lies at most 1/16 of its block's largest |h| and is
explained by the FP32 accumulation bound, and such elements are capped at a rate of 1e-5,
rounded up (gpu_helpers.check_intermediates). Samples under 10 000 elements, too small to estimate a
0.1 % rate, need every difference explained by the FP32 bound, and their pooled rate is
checked over the whole tiny-shape sweep. y: max |y_gpu - y_ref| / max |y_ref| <= 2e-2 per
row, rows the oracle gives as exactly 0 are exactly 0.
"""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from synth import CONFIGS, MoEConfig, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import oracle  # noqa: E402
from gpu_helpers import (FAR_EXCUSED_MAX_RATE, OFF_BY_ONE_MAX, RATE_MIN_ELEMENTS, Run,  # noqa: E402
                         check_intermediates, check_routing, check_y)


def _full_check(cfg: MoEConfig, seed=0, tokens=None, cols=None, max_tokens=None, stats=None):
    print(f"[parity] {cfg} seed={seed}", flush=True)
    inp = make_inputs(cfg, seed=seed, device="cuda")
    run = Run(inp, max_tokens=max_tokens)
    y = run.forward()
    idx = inp.topk_idx.cpu().numpy()
    got = run.routing()
    check_routing(got, idx, cfg.E)
    host = inp.numpy()
    ref = oracle.forward_inputs(host, tokens=tokens, cols=cols, keep_bounds=True)
    frac = check_intermediates(run, ref, got["inv"], stats=stats)
    err = check_y(y, ref, tokens=ref["tokens"] if tokens is not None else None, cols=cols,
                  run=run, inv=got["inv"], host=host)
    print(f"[parity] {cfg.name}: block_m={got['block_m']} tiles={got['meta'][0]} "
          f"off-by-one={frac:.2e} max row err={err:.3e}", flush=True)
    return run, ref


def test_tiny_c0():
    _full_check(CONFIGS["c0"])


@pytest.mark.parametrize("T,E,k,H,I,seed", [
    (150, 2, 1, 512, 256, 5),      # 64-row tiles, two tiles per expert, ragged tail
    (300, 5, 3, 512, 384, 1),      # 128-row tiles, ragged tails
    (700, 3, 2, 256, 640, 2),      # medium class, I not a multiple of 512
    (1200, 2, 2, 768, 256, 3),     # large class, K steps not a multiple of 4
    (1, 4, 2, 256, 256, 4),        # one token
    (200, 3, 2, 384, 128, 6),      # H an odd multiple of 128 (Linear2's last column tile half
                                   # empty), I = 128 (Linear2 has one K step)
    (40, 2, 2, 128, 256, 7),       # H = 128: Linear1 has one K step, Linear2 one half tile
    (1100, 2, 2, 640, 384, 8),     # 256-row tiles and second launch with H = 640
    (300, 4, 3, 128, 128, 9),      # H = I = 128 with rows read through the row list (top-3)
    (150, 4, 2, 512, 1024, 10),    # 64-row tiles, experts of one and two row tiles, K = 1024
    (90, 8, 4, 1024, 2048, 11),    # 64-row tiles, rows through the row list (top-4)
    (12, 24, 1, 1536, 1024, 12),   # mostly empty experts
])
def test_small_shapes(T, E, k, H, I, seed):
    _full_check(MoEConfig("small", T=T, E=E, k=k, H=H, I=I), seed=seed)


TINY_SWEEP = [(T, E, k) for T in (2, 5) for E in (1, 2, 3) for k in range(1, E + 1)]


@pytest.mark.parametrize("T,E,k", TINY_SWEEP)
def test_tiny_shape_sweep(T, E, k):
    """Every (E, k) with k <= E <= 3 at two and five tokens (one 64-row tile per expert,
    most of it padding), full parity."""
    _full_check(MoEConfig("tiny", T=T, E=E, k=k, H=256, I=256), seed=T * 10 + E * 3 + k)


def test_tiny_shape_sweep_pooled_rate():
    """Each case of the tiny sweep compares fewer than 10 000 intermediates, too few to
    estimate a 0.1 % rate on its own; pooled over the whole sweep they are enough, and the
    pooled fraction of differing intermediates must stay within 0.1 %."""
    stats = {}
    for T, E, k in TINY_SWEEP:
        _full_check(MoEConfig("tiny", T=T, E=E, k=k, H=256, I=256), seed=T * 10 + E * 3 + k,
                    stats=stats)
    rate = stats["differing"] / stats["n"]
    print(f"[parity] tiny sweep pooled: {stats['differing']} of {stats['n']} intermediates differ "
          f"({rate:.2e}); excused far elements {stats['excused']}", flush=True)
    assert stats["n"] >= RATE_MIN_ELEMENTS
    assert rate <= OFF_BY_ONE_MAX
    assert stats["excused"] <= int(np.ceil(FAR_EXCUSED_MAX_RATE * stats["n"]))
