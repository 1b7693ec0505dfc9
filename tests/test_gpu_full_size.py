"""GPU parity at the full workload sizes, in the launch configuration bench.py times
(one moe_forward on a workspace sized for exactly T tokens, tile class chosen by the
library).

At these sizes the oracle cannot run every token, so each case checks
  * the whole routing (counts, padded offsets, perm, inv, tile list) bit-exactly,
  * every y row is written (the poisoned output holds no NaN afterwards), and tokens with
    no valid slot are exactly +0,
  * y and the requantised intermediates of a token sample against the oracle: for every
    non-empty expert the first and the last token routed to it (the last one sits in the
    ragged tail tile of that expert), plus random tokens.
"""
import dataclasses

import numpy as np
import pytest
import torch

from conftest import gpu_available
from synth import CONFIGS, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import oracle  # noqa: E402
from gpu_helpers import Run, check_intermediates, check_routing, check_y  # noqa: E402


def sample_tokens(idx: np.ndarray, E: int, n_random: int, seed: int):
    T, k = idx.shape
    toks = set()
    for e in range(E):
        hit = np.nonzero((idx == e).any(axis=1))[0]
        if len(hit):
            toks.add(int(hit[0]))
            toks.add(int(hit[-1]))
    rng = np.random.default_rng(seed)
    toks.update(int(t) for t in rng.choice(T, size=min(n_random, T), replace=False))
    return sorted(toks)


@pytest.mark.parametrize("name", ["c1", "c3", "c3e", "c4", "c2"])
def test_full_size_sampled(name):
    cfg = CONFIGS[name]
    print(f"[full] {name}: {cfg}", flush=True)
    inp = make_inputs(cfg, seed=0, device="cuda")
    run = Run(inp)
    y = run.forward(poison=True)
    idx = inp.topk_idx.cpu().numpy()
    got = run.routing()
    check_routing(got, idx, cfg.E)
    yv = torch.from_numpy(y.astype(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.isfinite(yv).all(), "a y row was not written"
    toks = sample_tokens(idx, cfg.E, n_random=8, seed=1)
    host = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v)
            for k, v in dataclasses.asdict(inp).items() if k != "cfg"}
    ref = oracle.forward_inputs(host, tokens=toks, keep_bounds=True)
    frac = check_intermediates(run, ref, got["inv"])
    err = check_y(y, ref, tokens=toks)
    print(f"[full] {name}: block_m={got['block_m']} tiles={got['meta'][0]} sampled tokens="
          f"{len(toks)} off-by-one={frac:.2e} max row err={err:.3e}", flush=True)
