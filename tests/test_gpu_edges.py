"""GPU edge cases and exact invariants of the forward, through the C ABI.

Edge cases: zero tokens, fewer tokens than the workspace capacity, every slot on one
expert (with duplicate experts inside a token), k = E, the largest k (64), unused (-1) and
invalid expert ids with the diagnostic count (in the one-launch routing and over the chunks
of the three-launch routing), many experts with most of them empty.

Invariants that hold bit for bit on the GPU, whatever the tolerance against the oracle:
the same call twice gives the same bytes; permuting tokens permutes y; relabelling
experts leaves y unchanged; doubling the top-k weights doubles y; raising every W2 scale
byte by one doubles y; raising the scale bytes of W1's up rows by one leaves the h8 codes
unchanged, raises every h_sf byte by one and doubles y.
"""
import dataclasses

import numpy as np
import pytest
import torch

from conftest import gpu_available
from synth import MoEConfig, make_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import block_scaled_fp8_dispatch_amd as moe  # noqa: E402
import oracle  # noqa: E402
from gpu_helpers import Run, check_intermediates, check_routing, check_y  # noqa: E402


def _host(inp):
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v)
            for k, v in dataclasses.asdict(inp).items() if k != "cfg"}


def _parity(run: Run, inp, T=None):
    T = inp.x_fp8.shape[0] if T is None else T
    y = run.forward(T=T)
    idx = inp.topk_idx[:T].cpu().numpy()
    got = run.routing(T)
    ref_route = check_routing(got, idx, inp.cfg.E)
    host = _host(inp)
    for key in ("x_fp8", "x_sf", "topk_idx", "topk_weights"):
        host[key] = host[key][:T]
    ref = oracle.forward_inputs(host, keep_bounds=True)
    check_intermediates(run, ref, got["inv"])
    check_y(y, ref, run=run, inv=got["inv"], host=host)
    return y, ref, ref_route


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).astype(np.int16)).view(torch.bfloat16).float().numpy()


def test_zero_tokens_writes_nothing():
    cfg = MoEConfig("edge", T=64, E=4, k=2, H=256, I=256)
    print(f"[edge] zero tokens {cfg}", flush=True)
    inp = make_inputs(cfg, seed=11, device="cuda")
    run = Run(inp)
    run.y.fill_(0x1234)
    moe.moe_forward(run.y, inp.x_fp8, inp.x_sf, inp.topk_idx, inp.topk_weights, 0, run.shape,
                    run.packed, run.ws)
    torch.cuda.synchronize()
    assert bool((run.y == 0x1234).all())


def test_fewer_tokens_than_capacity():
    cfg = MoEConfig("edge", T=300, E=6, k=2, H=512, I=256)
    print(f"[edge] T=200 of capacity 512 {cfg}", flush=True)
    inp = make_inputs(cfg, seed=12, device="cuda")
    run = Run(inp, max_tokens=512)
    run.y = torch.empty(512, cfg.H, dtype=torch.int16, device="cuda")
    _parity(run, inp, T=200)
    assert bool((run.y[200:] == 0x7FBF).all()), "rows past num_tokens were written"


def test_all_slots_on_one_expert_with_duplicates():
    cfg = MoEConfig("edge", T=200, E=4, k=2, H=256, I=384)
    print(f"[edge] all slots on expert 2 {cfg}", flush=True)
    inp = make_inputs(cfg, seed=13, device="cuda")
    inp = dataclasses.replace(inp, topk_idx=torch.full_like(inp.topk_idx, 2))
    run = Run(inp)
    _, _, r = _parity(run, inp)
    assert list(r["counts"]) == [0, 0, 400, 0]


def test_k_equals_num_experts():
    cfg = MoEConfig("edge", T=96, E=3, k=3, H=256, I=256)
    print(f"[edge] k = E {cfg}", flush=True)
    inp = make_inputs(cfg, seed=14, device="cuda")
    run = Run(inp)
    _parity(run, inp)


def test_unused_and_invalid_slots():
    cfg = MoEConfig("edge", T=160, E=5, k=3, H=256, I=256)
    print(f"[edge] -1 and invalid ids {cfg}", flush=True)
    inp = make_inputs(cfg, seed=15, device="cuda")
    idx = inp.topk_idx.cpu().numpy().copy()
    rng = np.random.default_rng(0)
    idx[rng.random(idx.shape) < 0.2] = -1
    bad = rng.random(idx.shape) < 0.05
    idx[bad] = rng.choice(np.array([5, 6, 1000, -2, -7, 2**31 - 1], dtype=np.int64),
                          size=int(bad.sum())).astype(np.int32)
    idx[7, :] = -1                 # a token with no slot at all
    idx[9, :] = [5, -1, 1000]      # only invalid ids
    inp = dataclasses.replace(inp, topk_idx=torch.from_numpy(idx).cuda())
    run = Run(inp)
    y, ref, r = _parity(run, inp)
    assert (y[7] == 0).all() and (y[9] == 0).all(), "a token without valid slots is not +0"
    invalid, counts = moe.moe_read_diagnostics(run.shape, run.ws)
    assert invalid == int(r["num_invalid"]) == int(((idx < -1) | (idx >= cfg.E)).sum())
    assert counts == [int(c) for c in r["counts"]]


@pytest.mark.parametrize("T,k", [(4097, 1), (2049, 3), (1536, 8)])
def test_unused_and_invalid_slots_across_chunks(T, k):
    """The three-launch routing (more than 4096 slots, chunks of 2048): -1 and invalid ids
    scattered over every chunk, a chunk boundary inside a token's slots, a last chunk of one
    or three slots (4097 and 6147 slots) or none (12 288): routing bit-exact, parity, and the
    invalid-id count summed over the chunks."""
    cfg = MoEConfig("edge", T=T, E=9, k=k, H=256, I=256)
    print(f"[edge] -1 and invalid ids over chunks {cfg}", flush=True)
    inp = make_inputs(cfg, seed=31 + k, device="cuda")
    idx = inp.topk_idx.cpu().numpy().copy()
    rng = np.random.default_rng(k)
    idx[rng.random(idx.shape) < 0.1] = -1
    bad = rng.random(idx.shape) < 0.03
    idx[bad] = rng.choice(np.array([9, 11, 1000, -2, -9], dtype=np.int64),
                          size=int(bad.sum())).astype(np.int32)
    idx[-1, :] = 9                 # the last slot(s), alone in the last chunk, invalid
    inp = dataclasses.replace(inp, topk_idx=torch.from_numpy(idx).cuda())
    run = Run(inp)
    y, ref, r = _parity(run, inp)
    assert (y[-1] == 0).all(), "a token without valid slots is not +0"
    invalid, counts = moe.moe_read_diagnostics(run.shape, run.ws)
    assert invalid == int(r["num_invalid"]) == int(((idx < -1) | (idx >= cfg.E)).sum())
    assert counts == [int(c) for c in r["counts"]]


def test_largest_topk():
    """k = 64, the most slots per token the boundary accepts (64 distinct experts per token)."""
    cfg = MoEConfig("edge", T=40, E=80, k=64, H=256, I=256)
    print(f"[edge] k = 64 {cfg}", flush=True)
    inp = make_inputs(cfg, seed=18, device="cuda")
    run = Run(inp)
    _parity(run, inp)


def test_many_experts_mostly_empty():
    cfg = MoEConfig("edge", T=100, E=1024, k=8, H=256, I=256)
    print(f"[edge] E=1024 {cfg}", flush=True)
    inp = make_inputs(cfg, seed=16, device="cuda")
    run = Run(inp)
    _parity(run, inp)


# ---------------------------------------------------------------------------
# Exact invariants
# ---------------------------------------------------------------------------

CFG_INV = MoEConfig("inv", T=333, E=5, k=2, H=512, I=384)


def _run_once(inp):
    run = Run(inp)
    y = run.forward()
    return run, y


def test_half_tiles_of_several_sizes():
    """With 256-row tiles and K >= 4096, each expert's last tile of at most 128 rows (a half
    tile) runs in the second launch as a 128-row tile. Experts whose last tiles hold 40, 64,
    65 and 128 rows; the sampled tokens include the first and last rows of every half tile."""
    tails = [40, 64, 65, 128]
    counts = [512 + t for t in tails]
    T, E, H, I = sum(counts), 4, 4096, 4096
    cfg = MoEConfig("edge", T=T, E=E, k=1, H=H, I=I)
    print(f"[edge] half tiles of {tails} rows {cfg}", flush=True)
    inp = make_inputs(cfg, seed=21, device="cuda")
    idx = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    idx = np.random.default_rng(3).permutation(idx).reshape(T, 1)
    inp = dataclasses.replace(inp, topk_idx=torch.from_numpy(idx).cuda())
    run = Run(inp)
    y = run.forward(poison=True)
    got = run.routing()
    assert got["block_m"] == 256
    r = check_routing(got, idx, E)
    assert list(r["counts"]) == counts
    toks = set()
    for e in range(E):
        rows = np.nonzero(idx[:, 0] == e)[0]
        toks.update(int(t) for t in rows[-3:])              # the expert's last tile
        toks.update(int(t) for t in rows[511:513])         # last row of a full tile, first of the half tile
    toks.update(int(t) for t in np.random.default_rng(4).choice(T, 6, replace=False))
    toks = sorted(toks)
    host = _host(inp)
    ref = oracle.forward_inputs(host, tokens=toks, keep_bounds=True)
    check_intermediates(run, ref, got["inv"])
    check_y(y, ref, tokens=toks, run=run, inv=got["inv"], host=host)


@pytest.mark.parametrize("k,BMexp", [(2, 256), (8, 128)])
def test_dispatch_scale_copy(k, BMexp):
    """The gather's copy of each padded row's token scale row (xg_sf), read back from the
    workspace in the blocked scale layout (decoded by the test's own statement of it): equal
    to the token's x_sf row on every routed row and zero on padding rows, for a top-k with
    the dispatch copy of x (2) and one without (8, 128-row tiles; with 64-row tiles and a
    top-k above 2 nothing is copied, Linear1 reads x_sf through the row list)."""
    E = 8
    T = 2048 if k == 2 else 160
    cfg = MoEConfig("edge", T=T, E=E, k=k, H=1280, I=256)
    print(f"[edge] dispatch scale copy {cfg}", flush=True)
    inp = make_inputs(cfg, seed=23, device="cuda")
    run = Run(inp)
    run.forward(poison=True)
    got = run.routing()
    hb = got["block_m"]
    assert hb == BMexp
    L = run.layout()
    words = (cfg.H + 511) // 512
    rows = np.arange(int(got["meta"][0]) * hb)
    raw = run.ws[L["xg_sf"]: L["xg_sf"] + len(rows) * 4 * words].cpu().numpy()
    from gpu_helpers import blocked_scale_bytes
    nblocks = cfg.H // 128
    copied = raw[blocked_scale_bytes(rows, nblocks, words, hb)]          # [rows, H/128]
    perm = got["perm"][: len(rows)]
    x_sf = inp.x_sf.cpu().numpy()[:, :nblocks]
    valid = perm >= 0
    assert np.array_equal(copied[valid], x_sf[perm[valid] // k])
    assert not copied[~valid].any()


def test_deterministic():
    print(f"[inv] determinism {CFG_INV}", flush=True)
    inp = make_inputs(CFG_INV, seed=21, device="cuda")
    run = Run(inp)
    y1 = run.forward().copy()
    L = run.layout()
    h1 = run.ws[L["h8"]: L["stage"]].clone()
    y2 = run.forward()
    h2 = run.ws[L["h8"]: L["stage"]]
    assert np.array_equal(y1, y2)
    rows = int(run.routing()["offsets"][-1])
    I = CFG_INV.I
    assert torch.equal(h1[: rows * I], h2[: rows * I])


def test_token_permutation():
    print(f"[inv] token permutation {CFG_INV}", flush=True)
    inp = make_inputs(CFG_INV, seed=22, device="cuda")
    _, y = _run_once(inp)
    pi = torch.from_numpy(np.random.default_rng(3).permutation(CFG_INV.T)).cuda()
    inp2 = dataclasses.replace(inp, x_fp8=inp.x_fp8[pi].contiguous(), x_sf=inp.x_sf[pi].contiguous(),
                               topk_idx=inp.topk_idx[pi].contiguous(),
                               topk_weights=inp.topk_weights[pi].contiguous())
    _, y2 = _run_once(inp2)
    assert np.array_equal(y2, y[pi.cpu().numpy()])


def test_expert_relabelling():
    print(f"[inv] expert relabelling {CFG_INV}", flush=True)
    inp = make_inputs(CFG_INV, seed=23, device="cuda")
    _, y = _run_once(inp)
    sigma = np.array([3, 0, 4, 1, 2])           # old expert e becomes sigma[e]
    src = torch.from_numpy(np.argsort(sigma)).cuda()   # new slot e' holds old expert src[e']
    idx2 = torch.from_numpy(sigma[inp.topk_idx.cpu().numpy()].astype(np.int32)).cuda()
    inp2 = dataclasses.replace(inp, topk_idx=idx2, w1=inp.w1[src].contiguous(),
                               w1_sf=inp.w1_sf[src].contiguous(), w2=inp.w2[src].contiguous(),
                               w2_sf=inp.w2_sf[src].contiguous())
    _, y2 = _run_once(inp2)
    assert np.array_equal(y2, y)


def test_weight_and_scale_doubling():
    print(f"[inv] doubling {CFG_INV}", flush=True)
    inp = make_inputs(CFG_INV, seed=24, device="cuda")
    run, y = _run_once(inp)
    yf = _bf16(y)
    assert np.abs(yf).max() < 1e30
    # top-k weights x 2
    _, y_w = _run_once(dataclasses.replace(inp, topk_weights=inp.topk_weights * 2))
    assert np.array_equal(_bf16(y_w), 2 * yf)
    # every W2 scale byte + 1
    _, y_s = _run_once(dataclasses.replace(inp, w2_sf=inp.w2_sf + 1))
    assert np.array_equal(_bf16(y_s), 2 * yf)
    # W1 up rows' scale bytes + 1: same codes, h_sf + 1, y x 2
    I = CFG_INV.I
    w1_sf = inp.w1_sf.clone()
    w1_sf[:, I:, :] += 1
    run_u, y_u = _run_once(dataclasses.replace(inp, w1_sf=w1_sf))
    assert np.array_equal(_bf16(y_u), 2 * yf)
    rows = int(run.routing()["offsets"][-1])
    perm = run.routing()["perm"]
    valid = np.nonzero(perm >= 0)[0]
    h8a, sfa = run.intermediates(valid)
    h8b, sfb = run_u.intermediates(valid)
    assert rows == int(run_u.routing()["offsets"][-1])
    assert np.array_equal(h8a, h8b)
    assert np.array_equal(sfb.astype(np.int32), sfa.astype(np.int32) + 1)


def test_offsets_beyond_2gib():
    """x holds more than 2^31 bytes (T = 300000, H = 7168), so the rows of the last tokens
    sit at byte offsets past 2^31 in the GEMM's A loads; their outputs must still match."""
    cfg = MoEConfig("big", T=300000, E=4, k=1, H=7168, I=256)
    print(f"[edge] offsets past 2 GiB {cfg}", flush=True)
    inp = make_inputs(cfg, seed=17, device="cuda")
    assert inp.x_fp8.numel() > 2**31
    run = Run(inp)
    y = run.forward(poison=False)
    idx = inp.topk_idx.cpu().numpy()
    got = run.routing()
    check_routing(got, idx, cfg.E)
    toks = [0, 1, 299593, 299594, 299998, 299999]      # rows below and above byte 2^31
    assert 299594 * cfg.H >= 2**31
    host = _host(inp)
    ref = oracle.forward_inputs(host, tokens=toks, keep_bounds=True)
    check_intermediates(run, ref, got["inv"])
    check_y(y, ref, tokens=toks, run=run, inv=got["inv"], host=host)


def test_two_streams_two_workspaces():
    """Calls on different streams with different workspaces are independent: two forwards
    launched back to back on two streams give the bytes each gives alone."""
    cfg_a = MoEConfig("sa", T=900, E=6, k=2, H=512, I=384)
    cfg_b = MoEConfig("sb", T=700, E=3, k=3, H=256, I=640)
    print(f"[edge] two streams {cfg_a} {cfg_b}", flush=True)
    ia = make_inputs(cfg_a, seed=31, device="cuda")
    ib = make_inputs(cfg_b, seed=32, device="cuda")
    ra, rb = Run(ia), Run(ib)
    ya = ra.forward().copy()
    yb = rb.forward().copy()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        ra.y.fill_(0); rb.y.fill_(0)
        torch.cuda.synchronize()
        moe.moe_forward(ra.y, ia.x_fp8, ia.x_sf, ia.topk_idx, ia.topk_weights, cfg_a.T, ra.shape,
                        ra.packed, ra.ws, stream=sa)
        moe.moe_forward(rb.y, ib.x_fp8, ib.x_sf, ib.topk_idx, ib.topk_weights, cfg_b.T, rb.shape,
                        rb.packed, rb.ws, stream=sb)
        torch.cuda.synchronize()
        assert np.array_equal(ra.y[: cfg_a.T].cpu().numpy().view(np.uint16), ya)
        assert np.array_equal(rb.y[: cfg_b.T].cpu().numpy().view(np.uint16), yb)
