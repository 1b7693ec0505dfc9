"""moe_forward_noalloc: the forward with its workspace in the library's fixed per-GPU
scratch array. Its output must be byte-identical to moe_forward's with a caller-owned
workspace on the same inputs (the same kernels on the same rows; only the workspace
address differs), on two calls in a row, the second with fewer tokens than the first,
so that it runs on what the first call left in the scratch array. Calls too large for the
array are refused on the host."""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from synth import CONFIGS, MoEConfig, make_inputs

import block_scaled_fp8_dispatch_amd as moe  # noqa: E402


def _need_bytes(cfg, T):
    return moe.moe_workspace_bytes(moe.make_shape(cfg.E, cfg.H, cfg.I, cfg.k, T))


def test_noalloc_host_errors():
    """Host-detectable errors return before the device is touched (no GPU needed)."""
    s = moe.make_shape(8, 7168, 18432, 2, 8192)
    A = 0x10000
    call = lambda T=64, shape=s, **o: moe.moe_forward_noalloc_raw(
        o.get("y", A), o.get("x", A), A, A, A, T, shape, o.get("packed", A), None)
    # the T=8192, E=8, top-2 forward needs far more than the scratch array holds
    assert moe.moe_workspace_bytes(moe.make_shape(8, 7168, 18432, 2, 8192)) > moe.NOALLOC_SCRATCH_BYTES
    assert call(T=8192) == moe.MOE_ERR_SCRATCH
    assert call(y=None) == moe.MOE_ERR_NULL
    assert call(packed=None) == moe.MOE_ERR_NULL
    assert call(x=A + 4) == moe.MOE_ERR_ALIGN
    assert call(T=8193) == moe.MOE_ERR_TOKENS
    assert call(T=-1) == moe.MOE_ERR_TOKENS
    assert call(shape=moe.make_shape(8, 7000, 18432, 2, 8192)) == moe.MOE_ERR_SHAPE
    assert call(T=0) == moe.MOE_OK
    assert "scratch" in moe.moe_status_string(moe.MOE_ERR_SCRATCH)


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
@pytest.mark.parametrize("cfg,T1,T2", [
    (CONFIGS["c0"], 64, 37),                                   # 64-row tiles, top-2 dispatch copy
    (CONFIGS["c1"], 128, 50),                                  # decode share: top-8, rows through perm
    (MoEConfig("nb256", T=1300, E=2, k=2, H=512, I=256), 1300, 700),   # 256-row tiles + second launch
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_noalloc_matches_workspace_forward(cfg, T1, T2):
    from gpu_helpers import Run
    print(f"[noalloc] {cfg} T1={T1} T2={T2}", flush=True)
    assert _need_bytes(cfg, T1) <= moe.NOALLOC_SCRATCH_BYTES
    inp = make_inputs(cfg, seed=0, device="cuda")
    run = Run(inp)
    for T in (T1, T2):
        ref = run.forward(T=T).copy()           # moe_forward, poisoned caller workspace
        y = torch.full((T, cfg.H), 0x7FBF, dtype=torch.int16, device="cuda")
        moe.moe_forward_noalloc(y, inp.x_fp8, inp.x_sf, inp.topk_idx, inp.topk_weights, T,
                                run.shape, run.packed)
        torch.cuda.synchronize()
        got = y.cpu().numpy().view(np.uint16)
        diff = int(np.count_nonzero(got != ref))
        print(f"[noalloc] {cfg.name} T={T}: {diff} differing bf16 values of {got.size}", flush=True)
        assert diff == 0
