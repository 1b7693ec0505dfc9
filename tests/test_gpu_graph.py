"""The forward under HIP graph capture: moe_forward launches kernels only (no host
synchronisation, no memset, no allocation), so a decode loop can capture it once and replay
it with new tokens written into the same buffers. Every replay must give the bytes an eager
call gives on the same inputs; replays alternate with eager work on the same stream."""
import dataclasses

import numpy as np
import pytest
import torch

from conftest import gpu_available
from synth import MoEConfig, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import block_scaled_fp8_dispatch_amd as moe  # noqa: E402
from gpu_helpers import Run  # noqa: E402


@pytest.mark.parametrize("cfg", [
    MoEConfig("graph128", T=600, E=6, k=2, H=512, I=384),      # 128-row tiles, dispatch copy
    MoEConfig("graph256", T=2048, E=4, k=2, H=512, I=256),     # 256-row tiles + tail launch
    MoEConfig("graph64k4", T=96, E=8, k=4, H=256, I=256),      # 64-row tiles, rows through perm
], ids=lambda c: c.name)
def test_forward_graph_replays_match_eager(cfg):
    print(f"[graph] {cfg}", flush=True)
    # three batches of tokens (activations and routing) for one set of weights
    trials = [make_inputs(cfg, seed=s, device="cuda") for s in (40, 41, 42)]
    base = trials[0]
    batches = [dataclasses.replace(base, x_fp8=t.x_fp8, x_sf=t.x_sf, topk_idx=t.topk_idx,
                                   topk_weights=t.topk_weights) for t in trials]
    # eager reference of each batch, through its own buffers
    eager = [Run(b).forward(poison=False).copy() for b in batches]
    assert not np.array_equal(eager[0], eager[1])

    # the buffers the captured forward reads; each replay first gets a batch copied in
    run = Run(base)
    buf = {k: getattr(base, k).clone() for k in ("x_fp8", "x_sf", "topk_idx", "topk_weights")}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        moe.moe_forward(run.y, buf["x_fp8"], buf["x_sf"], buf["topk_idx"], buf["topk_weights"], cfg.T,
                        run.shape, run.packed, run.ws)
    for i in (0, 1, 2, 1, 0):
        for k in buf:
            buf[k].copy_(getattr(batches[i], k))
        run.y.fill_(0x7FBF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = run.y[: cfg.T].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, eager[i]), f"replay with batch {i}"
        # eager work on the same buffers between replays
        moe.moe_forward(run.y, buf["x_fp8"], buf["x_sf"], buf["topk_idx"], buf["topk_weights"], cfg.T,
                        run.shape, run.packed, run.ws)
        torch.cuda.synchronize()
        assert np.array_equal(run.y[: cfg.T].cpu().numpy().view(np.uint16), eager[i])
