"""Pins for the oracle's dispatch step (CPU only): a hand-worked example, a library
stable sort, and the invariants that define the permutation."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_routing


def test_route_hand_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_small.json")))
    r = oracle.route(np.array(g["topk_idx"], dtype=np.int32), g["E"], g["BM"])
    for key, val in g["expected"].items():
        assert np.array_equal(np.asarray(r[key]), np.asarray(val)), key


def check_route_invariants(r, topk_idx, E, BM):
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts, offsets, perm, inv = r["counts"], r["offsets"], r["perm"], r["inv"]
    assert counts.sum() == valid.sum()
    assert int(r["num_invalid"]) == int(((flat < -1) | (flat >= E)).sum())
    assert offsets[0] == 0 and np.all(offsets % BM == 0)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        c = counts[e]
        assert offsets[e + 1] - offsets[e] == ((c + BM - 1) // BM) * BM
        assert np.all(seg[c:] == -1)
        assert np.all(np.diff(seg[:c]) > 0)              # ascending (t, j)
        assert np.all(flat[seg[:c]] == e)
    real = perm[perm >= 0]
    assert np.array_equal(np.sort(real), np.nonzero(valid)[0])   # bijection onto valid slots
    assert np.all(inv[~valid] == -1)
    assert np.array_equal(perm[inv[valid]], np.nonzero(valid)[0])  # perm o inv = id
    ntiles = offsets[E] // BM
    assert len(r["tile_expert"]) == ntiles
    for i in range(ntiles):
        e = r["tile_expert"][i]
        r0 = r["tile_row0"][i]
        assert offsets[e] <= r0 < offsets[e + 1]


def stable_sort_route(topk_idx, E):
    """Library cross-check: a stable argsort of the expert ids gives the expert-major,
    (t, j)-ascending order of the valid slots."""
    flat = topk_idx.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < E))[0]
    order = np.argsort(flat[valid], kind="stable")
    return valid[order]


@pytest.mark.parametrize("cfg_name,BM", [("c0", 256), ("c1", 64), ("c3", 256), ("c3e", 128), ("c4", 256)])
def test_route_synthetic_configs(cfg_name, BM):
    cfg = CONFIGS[cfg_name]
    T = min(cfg.T, 4096)
    idx, _ = make_routing(cfg, seed=0, T=T)
    idx = idx.numpy()
    r = oracle.route(idx, cfg.E, BM)
    check_route_invariants(r, idx, cfg.E, BM)
    perm = r["perm"]
    assert np.array_equal(perm[perm >= 0], stable_sort_route(idx, cfg.E))


def test_route_edge_cases():
    rng = np.random.default_rng(0)
    cases = [
        (np.zeros((0, 2), dtype=np.int32), 4, 16),                         # no tokens
        (np.array([[3]], dtype=np.int32), 4, 16),                          # one token
        (np.zeros((37, 1), dtype=np.int32), 3, 16),                        # all to one expert
        (np.tile(np.arange(5, dtype=np.int32), (9, 1)), 5, 8),             # k = E
        (np.full((6, 3), -1, dtype=np.int32), 2, 4),                       # every slot unused
        (rng.integers(-3, 9, (50, 4)).astype(np.int32), 6, 16),            # invalid ids mixed in
        (np.array([[0, 0], [1, 1]], dtype=np.int32), 2, 4),                # duplicate ids in a token
    ]
    for idx, E, BM in cases:
        r = oracle.route(idx, E, BM)
        check_route_invariants(r, idx, E, BM)
        perm = r["perm"]
        assert np.array_equal(perm[perm >= 0], stable_sort_route(idx, E))


def test_generator_routing_properties():
    # uniform: k distinct experts per token; zipf c3e: four least popular experts empty
    for name in ("c1", "c3", "c3e"):
        cfg = CONFIGS[name]
        idx, w = make_routing(cfg, seed=0)
        idx = idx.numpy()
        assert idx.shape == (cfg.T, cfg.k)
        assert all(len(set(row)) == cfg.k for row in idx)
        assert np.allclose(w.sum(dim=1).numpy(), 1.0, atol=1e-6)
        if name == "c3e":
            assert np.all(idx < cfg.E - 4)
