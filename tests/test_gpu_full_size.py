"""GPU parity at the full workload sizes, in the launch configuration bench.py times
(one moe_forward on a workspace sized for exactly T tokens, tile class chosen by the
library).

Each case checks
  * the whole routing (counts, padded offsets, perm, inv, tile list) bit-exactly,
  * every y row is written (the poisoned output holds no NaN afterwards), and tokens with
    no valid slot are exactly +0,
  * y and the requantised intermediates against the oracle: every token of the decode
    share (T=128) and of both skewed-routing workloads (T=4096); for the two largest
    workloads (T=8192, top-2 and T=32768, top-8), whose full oracle run would take many
    minutes, a seeded stratified sample of at least 512 tokens holding at least 8 tokens of
    every non-empty expert, among them its first and its last token (the last one sits in
    that expert's ragged tail tile).

c4_wide is the T=32768 top-8 workload grown to T=40960: its 4.7 GB staging buffer is past
4 GiB, where Linear2 stores through 64-bit addresses instead of 32-bit buffer offsets.
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


def stratified_tokens(idx: np.ndarray, E: int, per_expert: int, total: int, seed: int):
    """At least `per_expert` tokens routed to each non-empty expert (its first and last among
    them), then random tokens up to `total`; sorted."""
    T, k = idx.shape
    rng = np.random.default_rng(seed)
    toks = set()
    for e in range(E):
        hit = np.nonzero((idx == e).any(axis=1))[0]
        if not len(hit):
            continue
        toks.update((int(hit[0]), int(hit[-1])))
        have = sum(1 for t in hit if int(t) in toks)
        rest = np.array([t for t in hit if int(t) not in toks], dtype=np.int64)
        need = min(per_expert - have, len(rest))
        if need > 0:
            toks.update(int(t) for t in rng.choice(rest, size=need, replace=False))
    others = np.array([t for t in range(T) if t not in toks], dtype=np.int64)
    need = min(max(total - len(toks), 0), len(others))
    toks.update(int(t) for t in rng.choice(others, size=need, replace=False))
    return sorted(toks)


def expert_coverage(idx: np.ndarray, toks, E: int):
    """Per expert: (slots of sampled tokens routed to it, all slots routed to it)."""
    sub = idx[np.asarray(toks)]
    return [(int((sub == e).sum()), int((idx == e).sum())) for e in range(E)]


WORKLOADS = dict(CONFIGS, c4_wide=dataclasses.replace(CONFIGS["c4"], name="c4_wide", T=40960))
# workload -> tokens compared with the oracle (None: all of them)
FULL = {"c1": None, "c3": None, "c3e": None, "c4": 512, "c2": 512, "c4_wide": 512}
PER_EXPERT = 8


@pytest.mark.parametrize("name", list(FULL))
def test_full_size(name):
    cfg = WORKLOADS[name]
    print(f"[full] {name}: {cfg}", flush=True)
    if name == "c4_wide":
        assert cfg.T * cfg.k * cfg.H * 2 > 1 << 32
    inp = make_inputs(cfg, seed=0, device="cuda")
    run = Run(inp)
    y = run.forward(poison=True)
    idx = inp.topk_idx.cpu().numpy()
    got = run.routing()
    check_routing(got, idx, cfg.E)
    yv = torch.from_numpy(y.astype(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.isfinite(yv).all(), "a y row was not written"
    if FULL[name] is None:
        toks = list(range(cfg.T))
    else:
        toks = stratified_tokens(idx, cfg.E, PER_EXPERT, FULL[name], seed=1)
        assert len(toks) >= FULL[name]
    cov = expert_coverage(idx, toks, cfg.E)
    for e, (got_e, all_e) in enumerate(cov):
        assert got_e >= min(PER_EXPERT, all_e), f"expert {e}: {got_e} of {all_e} slots sampled"
    print(f"[full] {name}: {len(toks)} of {cfg.T} tokens against the oracle; slots checked per "
          f"expert (checked/all): " + " ".join(f"{a}/{b}" for a, b in cov), flush=True)
    host = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v)
            for k, v in dataclasses.asdict(inp).items() if k != "cfg"}
    ref = oracle.forward_inputs(host, tokens=None if FULL[name] is None else toks, keep_bounds=True)
    frac = check_intermediates(run, ref, got["inv"])
    err = check_y(y, ref, tokens=None if FULL[name] is None else toks, run=run, inv=got["inv"],
                  host=host)
    print(f"[full] {name}: block_m={got['block_m']} tiles={got['meta'][0]} "
          f"off-by-one={frac:.2e} max row err={err:.3e}", flush=True)
