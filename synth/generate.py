"""Seeded input generators (torch; any device).

Workloads (T tokens, E local experts, top-k, hidden H, intermediate I):

  c0  T=64    E=4  k=2 H=256  I=512    uniform routing       tiny case
  c1  T=128   E=32 k=8 H=7168 I=2048   uniform routing       decode-sized share
  c2  T=8192  E=8  k=2 H=7168 I=18432  uniform routing       the explainer's worked shape
  c3  T=4096  E=32 k=8 H=7168 I=2048   Zipf(1.2) routing     skewed expert load
  c3e as c3 with the four least popular experts never chosen (empty experts)
  c4  T=32768 E=32 k=8 H=7168 I=2048   uniform routing       prefill share of a 256-expert layer

Distributions (the explainer's usage example, chenxutan.com/d/1930 section 3.3 and
section 9.2): x ~ N(0,1) cast to FP8 e4m3 with one UE8M0 scale per 1x128 block of
each row; W1 [E, 2I, H] (rows 0..I-1 gate, I..2I-1 up) and W2 [E, H, I] ~ N(0, 0.02)
cast to FP4 E2M1 with one UE8M0 scale per 1x32 block along K; router = top-k
experts then softmax over the k chosen logits (section 9.2's router lines).

The casts here are the producer step that sits before the path (the pages leave
it to the caller, e.g. a cast_to_fp8 call): block scale = the smallest power of
two 2^s with amax <= Qmax * 2^s (Qmax 448 for e4m3, 6 for E2M1), elements rounded
to nearest, ties to even. Each tensor draws from its own torch.Generator seeded
from (seed, tensor id), so a tensor does not change when another one's size does.
The same seed gives the same bytes on the same device type; CPU and GPU streams
differ, so a test always hands the same bytes to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    routing: str = "uniform"        # "uniform" | "zipf"
    zipf_s: float = 1.2
    zero_least_popular: int = 0     # c3e: experts with zero popularity

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def flop(self) -> float:
        # 2*P*H*(2I) for Linear1 plus 2*P*I*H for Linear2, valid slots only
        return 6.0 * self.T * self.k * self.H * self.I


CONFIGS = {
    "c0": MoEConfig("c0", T=64, E=4, k=2, H=256, I=512),
    "c1": MoEConfig("c1", T=128, E=32, k=8, H=7168, I=2048),
    "c2": MoEConfig("c2", T=8192, E=8, k=2, H=7168, I=18432),
    "c3": MoEConfig("c3", T=4096, E=32, k=8, H=7168, I=2048, routing="zipf"),
    "c3e": MoEConfig("c3e", T=4096, E=32, k=8, H=7168, I=2048, routing="zipf", zero_least_popular=4),
    "c4": MoEConfig("c4", T=32768, E=32, k=8, H=7168, I=2048),
}

# tensor ids for per-tensor seeding
_TID_X, _TID_ROUTE, _TID_LOGITS, _TID_W1, _TID_W2 = 1, 2, 3, 100, 200


def _gen(device, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 100003 + tid)
    return g


def _pow2_scale_exp(amax: torch.Tensor, qmax_mant: float, qmax_exp: int) -> torch.Tensor:
    """Smallest integer s with amax <= Qmax*2^s, where Qmax = qmax_mant*2^qmax_exp and
    qmax_mant in [1,2). amax == 0 gives s = 0. Exact: uses the binary exponent."""
    m, e = torch.frexp(amax)                 # amax = m * 2^e, m in [0.5, 1)
    m2 = m * 2.0                             # in [1, 2)
    e2 = e - 1
    s = e2 - qmax_exp + (m2 > qmax_mant).to(e2.dtype)
    return torch.where(amax == 0, torch.zeros_like(s), s)


def cast_fp8_blocks(x: torch.Tensor, block: int = 128):
    """fp32 [R, K] -> (e4m3 codes u8 [R, K], UE8M0 bytes u8 [R, 4*ceil(K/512)])."""
    R, K = x.shape
    assert K % block == 0
    xb = x.view(R, K // block, block)
    amax = xb.abs().amax(dim=-1)
    s = _pow2_scale_exp(amax, 1.75, 8)       # 448 = 1.75 * 2^8
    s = s.clamp(min=-127, max=127)
    scaled = torch.ldexp(xb, (-s).unsqueeze(-1).to(xb.dtype))
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).view(R, K)
    nsf = 4 * ((K + 511) // 512)
    sf = torch.zeros(R, nsf, dtype=torch.uint8, device=x.device)
    sf[:, : K // block] = (s + 127).to(torch.uint8)
    return codes, sf


# E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 ; round-to-nearest with ties to the even code.
# Boundaries between consecutive magnitudes are their midpoints; a value exactly on a
# midpoint goes to the neighbour whose code is even.
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (False, True, False, True, False, True, False)   # upper neighbour even?


def cast_fp4_blocks(w: torch.Tensor, block: int = 32):
    """fp32 [R, K] -> (E2M1 nibbles packed u8 [R, K/2], element 2i in the low nibble;
    UE8M0 bytes u8 [R, K/32])."""
    R, K = w.shape
    assert K % block == 0
    wb = w.view(R, K // block, block)
    amax = wb.abs().amax(dim=-1)
    s = _pow2_scale_exp(amax, 1.5, 2)        # 6 = 1.5 * 2^2
    s = s.clamp(min=-127, max=127)
    v = torch.ldexp(wb, (-s).unsqueeze(-1).to(wb.dtype)).view(R, K)
    a = v.abs()
    code = torch.zeros(a.shape, dtype=torch.uint8, device=w.device)
    for mid, up in zip(_E2M1_MID, _E2M1_TIE_UP):
        code += ((a > mid) | ((a == mid) & up)).to(torch.uint8)
    code |= (torch.signbit(v).to(torch.uint8) << 3)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    sf = (s + 127).to(torch.uint8)
    return packed.contiguous(), sf.contiguous()


def make_activations(cfg: MoEConfig, seed: int = 0, device="cpu", T: Optional[int] = None):
    T = cfg.T if T is None else T
    g = _gen(device, seed, _TID_X)
    x = torch.randn(T, cfg.H, generator=g, device=device, dtype=torch.float32)
    return cast_fp8_blocks(x)


def make_routing(cfg: MoEConfig, seed: int = 0, device="cpu", T: Optional[int] = None):
    """topk_idx int32 [T, k] (distinct experts per token) and topk_weights f32 [T, k]."""
    T = cfg.T if T is None else T
    g = _gen(device, seed, _TID_ROUTE)
    if cfg.routing == "uniform":
        keys = torch.rand(T, cfg.E, generator=g, device=device)
        idx = keys.argsort(dim=1)[:, : cfg.k]
    elif cfg.routing == "zipf":
        p = torch.arange(1, cfg.E + 1, device=device, dtype=torch.float64).pow(-cfg.zipf_s)
        if cfg.zero_least_popular:
            p[cfg.E - cfg.zero_least_popular:] = 0.0
        p = (p / p.sum()).to(torch.float32)
        # sequential weighted draws without replacement, one row per token
        idx = torch.multinomial(p.expand(T, cfg.E), cfg.k, replacement=False, generator=g)
    else:
        raise ValueError(cfg.routing)
    gl = _gen(device, seed, _TID_LOGITS)
    logits = torch.randn(T, cfg.k, generator=gl, device=device, dtype=torch.float32)
    w = torch.softmax(logits, dim=-1)
    return idx.to(torch.int32).contiguous(), w.contiguous()


def make_weights(cfg: MoEConfig, seed: int = 0, device="cpu", sigma: float = 0.02):
    """W1 packed u8 [E, 2I, H/2] + sf [E, 2I, H/32]; W2 packed u8 [E, H, I/2] + sf [E, H, I/32].
    Generated one expert (and, for big experts, one row chunk) at a time."""
    E, H, I = cfg.E, cfg.H, cfg.I
    w1 = torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, device=device)
    w1_sf = torch.empty(E, 2 * I, H // 32, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I // 2, dtype=torch.uint8, device=device)
    w2_sf = torch.empty(E, H, I // 32, dtype=torch.uint8, device=device)
    chunk = 8192
    for e in range(E):
        g1 = _gen(device, seed, _TID_W1 + e)
        for r0 in range(0, 2 * I, chunk):
            r1 = min(2 * I, r0 + chunk)
            w = torch.randn(r1 - r0, H, generator=g1, device=device) * sigma
            w1[e, r0:r1], w1_sf[e, r0:r1] = cast_fp4_blocks(w)
        g2 = _gen(device, seed, _TID_W2 + e)
        for r0 in range(0, H, chunk):
            r1 = min(H, r0 + chunk)
            w = torch.randn(r1 - r0, I, generator=g2, device=device) * sigma
            w2[e, r0:r1], w2_sf[e, r0:r1] = cast_fp4_blocks(w)
    return w1, w1_sf, w2, w2_sf


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    x_fp8: torch.Tensor       # u8 [T, H]
    x_sf: torch.Tensor        # u8 [T, 4*ceil(H/512)]
    topk_idx: torch.Tensor    # i32 [T, k]
    topk_weights: torch.Tensor  # f32 [T, k]
    w1: torch.Tensor
    w1_sf: torch.Tensor
    w2: torch.Tensor
    w2_sf: torch.Tensor

    def to(self, device) -> "MoEInputs":
        f = {k: (v.to(device) if isinstance(v, torch.Tensor) else v)
             for k, v in dataclasses.asdict(self).items() if k != "cfg"}
        return MoEInputs(cfg=self.cfg, **f)

    def numpy(self) -> dict:
        return {k: v.cpu().numpy() for k, v in dataclasses.asdict(self).items() if k != "cfg"}


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu") -> MoEInputs:
    x_fp8, x_sf = make_activations(cfg, seed, device)
    idx, w = make_routing(cfg, seed, device)
    w1, w1_sf, w2, w2_sf = make_weights(cfg, seed, device)
    return MoEInputs(cfg, x_fp8, x_sf, idx, w, w1, w1_sf, w2, w2_sf)


def custom_config(name="custom", **kw) -> MoEConfig:
    return MoEConfig(name, **kw)


# ---------------------------------------------------------------------------
# Inputs of the standalone FP8 x FP4 GEMMs and of the FP8 cast
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class GemmConfig:
    """One GEMM workload. layout: "dense" (M rows, one group), "contiguous" (M rows in G
    groups, each group's segment padded to a multiple of 128 rows with rows of group -1),
    "masked" (G groups of up to M = max_m rows, expected_m rows per group on average)."""
    name: str
    layout: str
    M: int
    N: int
    K: int
    G: int = 1
    expected_m: int = 0

    @property
    def rows(self) -> int:
        return self.G * self.M if self.layout == "masked" else self.M


# Shapes of the GEMM table on juejin.cn/post/7631516744872673307 (section "性能实测"): a
# decode-sized dense GEMM (M=64, N=2112, K=7168), a 4-group contiguous MoE GEMM (M=8192,
# N=4096; K not printed, taken as 7168) and a large dense GEMM (M=4096, K=16384; N not
# printed, taken as 4096). The masked case has no printed shape: it is the decode-sized
# share of c1 (32 groups of about 32 rows, N = 2*2048, K = 7168).
GEMM_CONFIGS = {
    "g_tiny": GemmConfig("g_tiny", "dense", M=77, N=272, K=384),
    "g_dense_decode": GemmConfig("g_dense_decode", "dense", M=64, N=2112, K=7168),
    "g_contig4": GemmConfig("g_contig4", "contiguous", M=8192, N=4096, K=7168, G=4),
    "g_dense_large": GemmConfig("g_dense_large", "dense", M=4096, N=4096, K=16384),
    "g_masked_decode": GemmConfig("g_masked_decode", "masked", M=64, N=4096, K=7168, G=32,
                                  expected_m=32),
}

_TID_GA, _TID_GB, _TID_GLAYOUT, _TID_BF16 = 300, 400, 500, 600


@dataclasses.dataclass
class GemmInputs:
    cfg: GemmConfig
    a: torch.Tensor            # u8 [rows, K] e4m3 (masked: [G, max_m, K])
    a_sf: torch.Tensor         # u8 [rows, 4*ceil(K/512)]
    b: torch.Tensor            # u8 [G, N, K/2] E2M1 pairs
    b_sf: torch.Tensor         # u8 [G, N, K/32]
    group_of_row: Optional[torch.Tensor] = None   # i32 [M] (contiguous)
    masked_m: Optional[torch.Tensor] = None       # i32 [G] (masked)


def make_gemm_inputs(cfg: GemmConfig, seed: int = 0, device="cpu", sigma: float = 0.02) -> GemmInputs:
    """A ~ N(0,1) cast to e4m3 per 1x128; B ~ N(0, sigma) cast to E2M1 per 1x32 (as the MoE
    activations and weights). Contiguous: group g owns segment g of M/G rows (the last one
    takes the remainder), whose last 0..127 rows are padding (-1). Masked: counts uniform in
    [expected_m/2, 3*expected_m/2], clamped to max_m."""
    rows, K, N, G = cfg.rows, cfg.K, cfg.N, cfg.G
    ga = _gen(device, seed, _TID_GA)
    a_parts, sf_parts = [], []
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        q, s = cast_fp8_blocks(torch.randn(r1 - r0, K, generator=ga, device=device))
        a_parts.append(q)
        sf_parts.append(s)
    a = torch.cat(a_parts) if a_parts else torch.empty(0, K, dtype=torch.uint8, device=device)
    a_sf = torch.cat(sf_parts) if sf_parts else torch.empty(0, 4 * ((K + 511) // 512), dtype=torch.uint8, device=device)
    b = torch.empty(G, N, K // 2, dtype=torch.uint8, device=device)
    b_sf = torch.empty(G, N, K // 32, dtype=torch.uint8, device=device)
    for g in range(G):
        gb = _gen(device, seed, _TID_GB + g)
        for r0 in range(0, N, 8192):
            r1 = min(N, r0 + 8192)
            b[g, r0:r1], b_sf[g, r0:r1] = cast_fp4_blocks(torch.randn(r1 - r0, K, generator=gb, device=device) * sigma)
    out = GemmInputs(cfg, a, a_sf, b, b_sf)
    gl = _gen("cpu", seed, _TID_GLAYOUT)
    if cfg.layout == "contiguous":
        grp = torch.full((cfg.M,), -1, dtype=torch.int32)
        seg = cfg.M // G
        for g in range(G):
            s0 = g * seg
            s1 = cfg.M if g == G - 1 else s0 + seg
            pad = int(torch.randint(0, 128, (1,), generator=gl))
            grp[s0:max(s0, s1 - pad)] = g
        out.group_of_row = grp.to(device)
    elif cfg.layout == "masked":
        e = max(cfg.expected_m, 1)
        cnt = torch.randint(e // 2, e + e // 2 + 1, (G,), generator=gl).clamp(max=cfg.M)
        out.masked_m = cnt.to(torch.int32).to(device)
        out.a = out.a.view(G, cfg.M, K)
        out.a_sf = out.a_sf.view(G, cfg.M, -1)
    return out


def make_bf16_activations(rows: int, cols: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """bf16 [rows, cols] ~ N(0, 1) (the activation of the explainer's usage example, section
    9.2, before it is cast to FP8)."""
    g = _gen(device, seed, _TID_BF16)
    return torch.randn(rows, cols, generator=g, device=device).to(torch.bfloat16)
