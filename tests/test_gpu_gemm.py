"""GPU parity of the standalone FP8 x FP4 GEMMs (dense, M-grouped contiguous, masked) and of
the FP8 cast, through the C ABI of include/fp8_fp4_gemm.h, against the oracle.

Acceptance: the cast is bit-exact (codes and scale bytes: integer outputs, decided in
exact arithmetic on both sides). Each GEMM output element must be the bf16 rounding of a
value within the FP32 accumulation error bound of the exact sum (oracle
gemm_bf16_within_bound); rows and columns that must not be written keep the poison value.
Rows of one output are independent of the row-tile size, so the masked GEMM gives the same
bytes whatever expected_m picks. Dense GEMMs with few output tiles split K over several
workgroups (g_split128, g_dense_decode); their sums are another FP32 order of the same
products, inside the same bound.
"""
import dataclasses

import numpy as np
import pytest
import torch

from conftest import gpu_available
from synth import GEMM_CONFIGS, GemmConfig, make_bf16_activations, make_gemm_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import block_scaled_fp8_dispatch_amd as moe  # noqa: E402
import oracle  # noqa: E402

POISON = 0x7FBF          # a bf16 NaN pattern the kernels never write


class GemmRun:
    def __init__(self, inp):
        c = inp.cfg
        self.inp, self.cfg = inp, c
        nb = moe.moe_gemm_packed_b_bytes(c.G, c.N, c.K)
        assert nb > 0
        self.packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
        moe.moe_gemm_prepare_b(c.G, c.N, c.K, inp.b, inp.b_sf, self.packed)
        self.ws = torch.empty(moe.moe_gemm_workspace_bytes(c.rows, c.G), dtype=torch.uint8, device="cuda")
        # one guard row past the end catches stores beyond the last row
        self.d = torch.empty(c.rows + 1, c.N, dtype=torch.int16, device="cuda")

    def run(self, expected_m=None):
        c, i = self.cfg, self.inp
        self.d.fill_(POISON)
        self.ws.fill_(0xFF)
        if c.layout == "dense":
            moe.moe_fp8_fp4_gemm(self.d, i.a, i.a_sf, c.M, c.N, c.K, self.packed, self.ws)
        elif c.layout == "contiguous":
            moe.moe_m_grouped_fp8_fp4_gemm_contiguous(self.d, i.a, i.a_sf, i.group_of_row, c.M, c.G,
                                                      c.N, c.K, self.packed, self.ws)
        else:
            moe.moe_m_grouped_fp8_fp4_gemm_masked(self.d, i.a, i.a_sf, i.masked_m, c.G, c.M,
                                                  c.expected_m if expected_m is None else expected_m,
                                                  c.N, c.K, self.packed, self.ws)
        torch.cuda.synchronize()
        out = self.d.cpu().numpy().view(np.uint16)
        assert (out[c.rows] == POISON).all(), "a store went past the last row"
        return out[: c.rows]


def _host(t):
    return t.cpu().numpy()


def _check_rows(d, rows, ref_rows, ref):
    """d[rows] against oracle results ref (exact/bits/bound) for the same rows."""
    ok = oracle.gemm_bf16_within_bound(d[rows], ref["exact"], ref["bound"])
    if not ok.all():
        r, c = np.argwhere(~ok)[0]
        got = oracle.bf16_bits_to_f64(d[rows][r, c])
        raise AssertionError(f"row {ref_rows[r]} col {c}: gpu {got} exact {ref['exact'][r, c]} "
                             f"bound {ref['bound'][r, c]} ({(~ok).sum()} elements off)")


@pytest.mark.parametrize("cfg", [
    GEMM_CONFIGS["g_tiny"],                                           # ragged M and N, K = 3 steps
    GemmConfig("g_mid", "dense", M=1000, N=528, K=1152),              # 256-row tiles + tail halves
    GemmConfig("g_one", "dense", M=1, N=16, K=128),                   # smallest shape: one K step
    GemmConfig("g_k128", "dense", M=300, N=272, K=128),               # one K step, 128-row tiles
    GemmConfig("g_split128", "dense", M=200, N=1040, K=4096),         # split K, 128-row tiles
    GEMM_CONFIGS["g_dense_decode"],                                   # split K, 64-row tiles
], ids=lambda c: c.name)
def test_dense_gemm(cfg):
    print(f"[gemm] dense {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=1, device="cuda")
    run = GemmRun(inp)
    d = run.run()
    assert np.array_equal(run.run(), d), "two calls gave different bytes"
    ref = oracle.fp8_fp4_gemm(_host(inp.a), _host(inp.a_sf), _host(inp.b[0]), _host(inp.b_sf[0]), cfg.K)
    rows = np.arange(cfg.M)
    _check_rows(d, rows, rows, ref)
    exact = (d == ref["bits"]).mean()
    print(f"[gemm] {cfg.name}: bf16 bits equal to the rounded exact sum: {100 * exact:.2f} %", flush=True)


def test_contiguous_gemm_unaligned_groups_and_skipped_rows():
    cfg = GemmConfig("g_contig_small", "contiguous", M=700, N=512, K=512, G=3)
    print(f"[gemm] contiguous {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=2, device="cuda")
    rng = np.random.default_rng(0)
    grp = rng.integers(0, 3, size=cfg.M).astype(np.int32)        # groups interleaved, unaligned
    grp[rng.random(cfg.M) < 0.1] = -1
    grp[[5, 6, 400]] = [7, -9, 3]                                 # ids outside [-1, G): skipped
    inp.group_of_row = torch.from_numpy(grp).cuda()
    d = GemmRun(inp).run()
    ref = oracle.m_grouped_gemm_contiguous(_host(inp.a), _host(inp.a_sf), np.where(
        (grp >= 0) & (grp < 3), grp, -1), _host(inp.b), _host(inp.b_sf), cfg.K)
    valid = np.nonzero(ref["valid"])[0]
    _check_rows(d, valid, valid, {k: ref[k][valid] for k in ("exact", "bound")})
    skipped = np.nonzero(~ref["valid"])[0]
    assert (d[skipped] == POISON).all(), "a skipped row was written"


def test_contiguous_gemm_full_size_sampled():
    cfg = GEMM_CONFIGS["g_contig4"]
    print(f"[gemm] contiguous {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=3, device="cuda")
    d = GemmRun(inp).run()
    grp = _host(inp.group_of_row)
    assert (d[grp < 0] == POISON).all()
    a, a_sf = _host(inp.a), _host(inp.a_sf)
    for g in range(cfg.G):
        rows = np.nonzero(grp == g)[0]
        pick = np.unique(np.concatenate([rows[:2], rows[-2:], np.random.default_rng(g).choice(rows, 4)]))
        ref = oracle.fp8_fp4_gemm(a[pick], a_sf[pick], _host(inp.b[g]), _host(inp.b_sf[g]), cfg.K)
        _check_rows(d, pick, pick, ref)


@pytest.mark.parametrize("cfg", [
    GemmConfig("g_masked_small", "masked", M=70, N=272, K=640, G=5, expected_m=32),
    GEMM_CONFIGS["g_masked_decode"],
], ids=lambda c: c.name)
def test_masked_gemm(cfg):
    print(f"[gemm] masked {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=4, device="cuda")
    if cfg.name == "g_masked_small":
        inp.masked_m = torch.tensor([0, 70, 33, 1, 200], dtype=torch.int32, device="cuda")
    run = GemmRun(inp)
    d = run.run().reshape(cfg.G, cfg.M, cfg.N)
    cnt = np.clip(_host(inp.masked_m), 0, cfg.M)
    a, a_sf = _host(inp.a), _host(inp.a_sf)
    for g in range(cfg.G):
        c = int(cnt[g])
        assert (d[g, c:] == POISON).all(), f"group {g}: a row past its count was written"
        if c == 0:
            continue
        ref = oracle.fp8_fp4_gemm(a[g, :c], a_sf[g, :c], _host(inp.b[g]), _host(inp.b_sf[g]), cfg.K)
        _check_rows(d[g], np.arange(c), np.arange(c), ref)
    # the row-tile size (picked from expected_m) does not change a single byte
    for em in (1, 200, 4096):
        d2 = run.run(expected_m=em).reshape(cfg.G, cfg.M, cfg.N)
        assert np.array_equal(d2, d), f"expected_m={em} changed the output"


def test_grouped_gemms_with_the_most_groups():
    """1024 groups (the most the boundary accepts), most of them tiny or empty."""
    G, N, K = 1024, 32, 256
    cfg = GemmConfig("g_masked_1024", "masked", M=3, N=N, K=K, G=G, expected_m=1)
    print(f"[gemm] {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=6, device="cuda")
    cnt = np.random.default_rng(1).integers(-1, 4, size=G).astype(np.int32)
    inp.masked_m = torch.from_numpy(cnt).cuda()
    d = GemmRun(inp).run().reshape(G, 3, N)
    a, a_sf, b, b_sf = _host(inp.a), _host(inp.a_sf), _host(inp.b), _host(inp.b_sf)
    ref = oracle.m_grouped_gemm_masked(a, a_sf, cnt, b, b_sf, K)
    v = ref["valid"]
    assert (d[~v] == POISON).all()
    ok = oracle.gemm_bf16_within_bound(d[v], ref["exact"][v], ref["bound"][v])
    assert ok.all(), f"{(~ok).sum()} elements off"
    # the same rows as a contiguous layout: row (g, i) belongs to group g when i < count
    cfg2 = GemmConfig("g_contig_1024", "contiguous", M=G * 3, N=N, K=K, G=G)
    inp2 = dataclasses.replace(inp, cfg=cfg2, a=inp.a.reshape(G * 3, K), a_sf=inp.a_sf.reshape(G * 3, -1),
                               masked_m=None)
    grp = np.where(v, np.arange(G)[:, None], -1).reshape(-1).astype(np.int32)
    inp2.group_of_row = torch.from_numpy(grp).cuda()
    d2 = GemmRun(inp2).run().reshape(G, 3, N)
    assert np.array_equal(d2, d), "contiguous and masked layouts of the same rows differ"


def test_masked_gemm_packed_b_beyond_4gb():
    """Packed B above 4 GB: the last groups lie past 4 GB from the start of the packed buffer
    (the kernels' 32-bit buffer offsets are relative to each tile's own B)."""
    G, N, K = 300, 4096, 7168
    cfg = GemmConfig("g_masked_4g", "masked", M=4, N=N, K=K, G=G, expected_m=2)
    assert moe.moe_gemm_packed_b_bytes(G, N, K) > 2 ** 32
    print(f"[gemm] {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=8, device="cuda")
    run = GemmRun(inp)
    d = run.run().reshape(G, cfg.M, N)
    cnt = np.clip(_host(inp.masked_m), 0, cfg.M)
    a, a_sf = _host(inp.a), _host(inp.a_sf)
    for g in (0, G // 2, G - 8, G - 1):
        c = int(cnt[g])
        assert (d[g, c:] == POISON).all()
        ref = oracle.fp8_fp4_gemm(a[g, :c], a_sf[g, :c], _host(inp.b[g]), _host(inp.b_sf[g]), K)
        _check_rows(d[g], np.arange(c), np.arange(c), ref)
    del run, inp
    torch.cuda.empty_cache()


def test_masked_gemm_graph_replays_follow_device_counts():
    """Captured once, replayed with counts changed on the device between replays: each replay
    computes the rows the counts name at that time (the host never reads them)."""
    cfg = GemmConfig("g_masked_graph", "masked", M=48, N=256, K=512, G=4, expected_m=24)
    print(f"[gemm] masked under graph capture {cfg}", flush=True)
    inp = make_gemm_inputs(cfg, seed=5, device="cuda")
    run = GemmRun(inp)
    counts = inp.masked_m
    eager = {}
    for trial in ([0, 48, 10, 3], [48, 1, 0, 20], [7, 7, 7, 7]):
        counts.copy_(torch.tensor(trial, dtype=torch.int32))
        eager[tuple(trial)] = run.run().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    run.d.fill_(POISON)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        moe.moe_m_grouped_fp8_fp4_gemm_masked(run.d, inp.a, inp.a_sf, counts, cfg.G, cfg.M,
                                              cfg.expected_m, cfg.N, cfg.K, run.packed, run.ws)
    for trial in ([0, 48, 10, 3], [48, 1, 0, 20], [7, 7, 7, 7], [0, 48, 10, 3]):
        counts.copy_(torch.tensor(trial, dtype=torch.int32))
        run.d.fill_(POISON)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = run.d.cpu().numpy().view(np.uint16)[: cfg.rows]
        assert np.array_equal(got, eager[tuple(trial)]), f"replay with counts {trial}"


# ---------------------------------------------------------------------------- cast


def _cast_gpu(x_bf16):
    R, C = x_bf16.shape
    q = torch.full((R, C), 0x55, dtype=torch.uint8, device="cuda")
    sf = torch.full((R, 4 * ((C + 511) // 512)), 0x55, dtype=torch.uint8, device="cuda")
    moe.moe_cast_to_fp8(x_bf16, R, C, q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def _bits(x_bf16):
    return x_bf16.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 640), (300, 7168), (5, 18432)])
def test_cast_bit_exact(rows, cols):
    print(f"[cast] {rows} x {cols}", flush=True)
    x = make_bf16_activations(rows, cols, seed=rows, device="cuda")
    # rows of very different magnitudes, a zero block and a block of tiny values
    x = x * torch.exp2(torch.linspace(-30, 30, rows, device="cuda")).to(torch.bfloat16)[:, None]
    x[0, :128] = 0
    if cols >= 256:
        x[0, 128:256] = x[0, 128:256] * 2.0 ** -120
    q, sf = _cast_gpu(x)
    rq, rsf = oracle.cast_to_fp8(_bits(x))
    assert np.array_equal(sf, rsf), np.argwhere(sf != rsf)[:4]
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:4]


def test_cast_edge_values():
    vals = np.zeros((4, 256), np.float32)
    vals[0, :128] = 448.0
    vals[0, 128] = 896.0
    vals[1, 0] = 2.0 ** -133                       # bf16 subnormal block: byte 0
    vals[1, 1] = -(2.0 ** -130)
    vals[1, 128] = 3.0 * 2 ** 125                  # near the top of bf16
    vals[1, 129] = -1e-30
    vals[2, :] = -0.0
    vals[2, 128:] = np.linspace(-447, 449, 128)
    vals[3, :] = np.float32(2.0 ** -10) * np.arange(256) / 64   # ties of the e4m3 subnormals
    vals[3, 0] = 448.0 * 2 ** 20
    x = torch.from_numpy(vals).to(torch.bfloat16).cuda()
    q, sf = _cast_gpu(x)
    rq, rsf = oracle.cast_to_fp8(_bits(x))
    assert np.array_equal(sf, rsf), (sf, rsf)
    assert np.array_equal(q, rq), np.argwhere(q != rq)[:8]


def test_cast_feeds_the_forward():
    """The cast's output is the forward's input: cast on the GPU, then forward, gives the
    same y bytes as the forward on the oracle's cast of the same bf16 rows."""
    from gpu_helpers import Run
    from synth import MoEConfig, make_inputs
    cfg = MoEConfig("castfwd", T=96, E=4, k=2, H=512, I=256)
    print(f"[cast] feeds the forward {cfg}", flush=True)
    inp = make_inputs(cfg, seed=6, device="cuda")
    x = make_bf16_activations(cfg.T, cfg.H, seed=7, device="cuda")
    q, sf = _cast_gpu(x)
    rq, rsf = oracle.cast_to_fp8(_bits(x))
    assert np.array_equal(q, rq) and np.array_equal(sf, rsf)
    inp.x_fp8 = torch.from_numpy(q).cuda()
    inp.x_sf = torch.from_numpy(sf).cuda()
    y = Run(inp).forward()
    import dataclasses
    host = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v)
            for k, v in dataclasses.asdict(inp).items() if k != "cfg"}
    ref = oracle.forward_inputs(host)
    from gpu_helpers import check_y
    check_y(y, ref)
