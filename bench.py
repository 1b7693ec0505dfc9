#!/usr/bin/env python3
"""Throughput of the one-GPU Mega MoE forward on MI355X.

One step = one moe_forward (dispatch -> Linear1 + SwiGLU + FP8 requant -> Linear2 +
top-k weighting -> combine) over one batch of seeded synthetic inputs already resident in
HBM; the weight transform (moe_prepare_weights) is done once beforehand, as the pages do
it. Default workload: T=8192 tokens, E=8 experts, top-2, H=7168, I=18432 (the
explainer's worked shape, chenxutan.com/d/1930 section 3.3).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2]

Other workloads (not the default line): --config g_dense_decode | g_contig4 | g_dense_large |
g_masked_decode times one call of the standalone FP8 x FP4 GEMM of that shape (section 4.3's
GEMM; the shapes of juejin.cn/post/7631516744872673307 "性能实测"), and --config cast times
the FP8 cast of 8192 x 7168 bf16 rows.

Prints one JSON line. FLOP = 6*T*k*H*I over valid slots only (2*P*H*2I for Linear1 plus
2*P*I*H for Linear2). The timed region holds K plain forwards between two events on the
launch stream; stage times come from a separate loop of forwards whose HIP events the
library records between its kernels; the roofline object is for Linear1, the dominant
kernel. The CPU baseline is the plain C++ fp64 oracle timed on a bounded token sample,
with the host's CPU model and core counts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused MoE FFN TFLOPS & % of MI355X FP8×FP4 MFMA peak; tokens/s (1 GPU)"
PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (FP8 x FP4 issues at the FP8 rate)
PEAK_HBM_GBS = 8000.0
GEMM_SRC = os.path.join(ROOT, "block_scaled_fp8_dispatch_amd", "csrc", "gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=384)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (for counter scaling)")
    return ap.parse_args()


def code_hash(text: str) -> str:
    """sha256 (first 16 hex) of C++ source with comments and whitespace removed: a change
    to the comments alone does not change the kernel the counters were taken on."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def gemm_source_hash() -> str:
    return code_hash(open(GEMM_SRC, encoding="utf-8").read())


def linear1_roofline(T: int, k: int, H: int, I: int, E: int, n_active: int, w1_bytes: float,
                     linear1_ms: float, traffic):
    """The roofline object of the Linear1 stage. Algorithmic bytes: W1 and its scales for the
    experts that receive a row, and per valid slot its x row, h8 row and h_sf bytes;
    algorithmic FLOP: 4*P*H*I. Below the ridge (peak FLOP/s over HBM bytes/s) the stage is
    priced against HBM bandwidth, else against the MFMA peak."""
    P = T * k
    flop = 4.0 * P * H * I
    nbytes = w1_bytes * n_active / E + P * (H + I + I // 128)
    kname = "Linear1 grouped GEMM with SwiGLU/requant epilogue (main + second launch)"
    if flop / nbytes < PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        gbs = nbytes / (linear1_ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    tflops = flop / (linear1_ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kname, "achieved": round(tflops, 2), "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4), "traffic": traffic}


def load_traffic(cfg_name: str):
    """HBM bytes per Linear1 launch from the committed counter summary, or None if the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"linear1_{cfg_name}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"gemm_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != gemm_source_hash():
        return None
    return float(m_bytes.group(1))


def host_cpu():
    """The host's CPU model, physical cores, logical CPUs, and the CPUs this process may run
    on (its affinity, capped by OMP_NUM_THREADS where that is set)."""
    model, cores = "unknown", set()
    try:
        phys = core = None
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name" and model == "unknown":
                model = val
            elif key == "physical id":
                phys = val
            elif key == "core id":
                core = val
            elif not key and phys is not None:
                cores.add((phys, core))
                phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    logical = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else logical
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        usable = min(usable, int(omp))
    return model, len(cores) or None, logical, usable


def cpu_baseline(inp_cpu: dict, cfg, n_tokens: int):
    """Time the plain C++ oracle (oracle/ref_forward.cpp: fp64, one ascending sum per dot
    product, std::thread over output rows, timed inside with std::chrono::steady_clock) on
    the first n_tokens tokens of the batch, with one thread per CPU this process may use.
    Every expert the sample routes to is decoded, so the sample carries the oracle's full
    per-expert cost."""
    import numpy as np
    from oracle import ref_cpp
    model, phys, logical, usable = host_cpu()
    idx = inp_cpu["topk_idx"]
    toks = list(range(min(n_tokens, idx.shape[0])))
    r = ref_cpp.forward_cpp(inp_cpu, tokens=toks, threads=usable, keep_intermediates=False)
    dt = r["seconds"]
    valid = (idx[toks] >= 0) & (idx[toks] < cfg.E)
    slots = int(np.sum(valid))
    experts = int(len(np.unique(idx[toks][valid])))
    flop = 6.0 * slots * cfg.H * cfg.I
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"first {len(toks)} tokens ({slots} slots over {experts} experts) of {cfg.name}, "
                      f"{dt:.1f} s; plain C++ fp64 oracle (no BLAS), {r['threads']} std::thread workers",
            "cpu_model": model, "physical_cores": phys, "logical_cpus": logical,
            "seconds": dt}


def _timed(call, steps, warmup):
    """Mean ms of `call` over `steps` calls between two events on the launch stream, after
    `warmup` untimed calls; synchronised on both sides."""
    import torch
    for _ in range(warmup):
        call()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - t0


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def bench_gemm(args, gcfg):
    """One standalone GEMM call per step (its layout or routing kernel plus the GEMM)."""
    import numpy as np
    import torch

    import block_scaled_fp8_dispatch_amd as moe
    from synth import make_gemm_inputs
    c = gcfg
    inp = make_gemm_inputs(c, seed=args.seed, device="cuda")
    packed = torch.empty(moe.moe_gemm_packed_b_bytes(c.G, c.N, c.K), dtype=torch.uint8, device="cuda")
    moe.moe_gemm_prepare_b(c.G, c.N, c.K, inp.b, inp.b_sf, packed)
    ws = torch.empty(moe.moe_gemm_workspace_bytes(c.rows, c.G), dtype=torch.uint8, device="cuda")
    d = torch.empty(c.rows, c.N, dtype=torch.int16, device="cuda")

    def call():
        if c.layout == "dense":
            moe.moe_fp8_fp4_gemm(d, inp.a, inp.a_sf, c.M, c.N, c.K, packed, ws)
        elif c.layout == "contiguous":
            moe.moe_m_grouped_fp8_fp4_gemm_contiguous(d, inp.a, inp.a_sf, inp.group_of_row, c.M, c.G,
                                                      c.N, c.K, packed, ws)
        else:
            moe.moe_m_grouped_fp8_fp4_gemm_masked(d, inp.a, inp.a_sf, inp.masked_m, c.G, c.M,
                                                  c.expected_m, c.N, c.K, packed, ws)

    ms, wall = _timed(call, args.steps, args.warmup)
    if c.layout == "dense":
        rows = c.M
    elif c.layout == "contiguous":
        rows = int((inp.group_of_row >= 0).sum())
    else:
        rows = int(inp.masked_m.clamp(0, c.M).sum())
    flop = 2.0 * rows * c.N * c.K
    tflops = flop / (ms * 1e-3) / 1e12
    # algorithmic bytes: B and its scales once, the computed A rows and scales, D rows
    alg = c.G * c.N * (c.K // 2 + c.K // 32) + rows * (c.K + 4 * ((c.K + 511) // 512)) + 2 * rows * c.N
    gbs = alg / (ms * 1e-3) / 1e9
    hbm_bound = flop / alg < PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4)} if hbm_bound else
            {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tflops / PEAK_TFLOPS, 4)})
    roof.update({"kernel": "one GEMM call (layout or routing kernel + grouped GEMM in plain mode)",
                 "traffic": None})
    out = {"metric": "FP8×FP4 GEMM TFLOPS & % of MI355X FP8 MFMA peak (1 GPU)", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8e4m3 x fp4e2m1 -> f32 accumulate, bf16 out",
           "data": "synthetic (seeded; A~N(0,1) FP8 1x128 UE8M0, B~N(0,0.02) FP4 1x32 UE8M0)",
           "config": {"workload": f"{c.name}: {c.layout} GEMM M={c.M} N={c.N} K={c.K} groups={c.G}"
                                  + (f" expected_m={c.expected_m}" if c.layout == "masked" else ""),
                      "layout": c.layout, "M": c.M, "N": c.N, "K": c.K, "groups": c.G, "rows_computed": rows},
           "alg_hbm_gbs": round(gbs, 1), "wall_s_timed": round(wall, 3), "roofline": roof, "cpu_baseline": None}
    if not args.no_cpu_baseline:
        import oracle   # the CPU baseline leg only
        # the oracle on the first rows of group 0 (about 10-30 s of CPU work is the aim)
        n = max(1, min(rows, int(6e10 / (2.0 * c.N * c.K))))
        a = inp.a.reshape(-1, c.K)[:n].cpu().numpy()
        a_sf = inp.a_sf.reshape(-1, inp.a_sf.shape[-1])[:n].cpu().numpy()
        b, b_sf = inp.b[0].cpu().numpy(), inp.b_sf[0].cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - t0 < 10.0:
            oracle.fp8_fp4_gemm(a, a_sf, b, b_sf, c.K)
            reps += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": reps * 2.0 * n * c.N * c.K / dt / 1e12, "unit": "TFLOP/s",
                               "cores": int(_threads()), "kind": "oracle",
                               "sample": f"{reps} x the first {n} rows against group 0's B, {dt:.1f} s; numpy fp64"}
    print(json.dumps(out), flush=True)


def bench_cast(args, rows=8192, cols=7168):
    import torch

    import block_scaled_fp8_dispatch_amd as moe
    from synth import make_bf16_activations
    x = make_bf16_activations(rows, cols, seed=args.seed, device="cuda")
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    sf = torch.empty(rows, 4 * ((cols + 511) // 512), dtype=torch.uint8, device="cuda")
    ms, wall = _timed(lambda: moe.moe_cast_to_fp8(x, rows, cols, q, sf), args.steps, args.warmup)
    alg = rows * cols * 3 + rows * sf.shape[1]
    gbs = alg / (ms * 1e-3) / 1e9
    out = {"metric": "FP8 cast GB/s (bf16 -> e4m3 + UE8M0 per 1x128, 1 GPU)", "value": round(gbs, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 -> fp8e4m3", "data": "synthetic (seeded; x~N(0,1) bf16)",
           "config": {"workload": f"cast: {rows} x {cols} bf16", "rows": rows, "cols": cols},
           "wall_s_timed": round(wall, 3),
           "roofline": {"bound": "hbm", "kernel": "cast_fp8_kernel", "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": None},
           "cpu_baseline": None}
    if not args.no_cpu_baseline:
        import oracle   # the CPU baseline leg only
        n = 1024
        bits = x[:n].view(torch.int16).cpu().numpy().view("uint16")
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.cast_to_fp8(bits)
            reps += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": reps * n * (cols * 3 + sf.shape[1]) / dt / 1e9, "unit": "GB/s",
                               "cores": int(_threads()), "kind": "oracle",
                               "sample": f"{reps} casts of the first {n} rows, {dt:.1f} s; numpy fp64"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "expert-parallel exchange is not part of it", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_scaled_fp8_dispatch_amd as moe
    from synth import CONFIGS, GEMM_CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load_library()
    if args.config in GEMM_CONFIGS:
        return bench_gemm(args, GEMM_CONFIGS[args.config])
    if args.config == "cast":
        return bench_cast(args)
    cfg = CONFIGS[args.config]
    dev = "cuda"
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    inp = make_inputs(cfg, seed=args.seed, device=dev)
    shape = moe.make_shape(cfg.E, cfg.H, cfg.I, cfg.k, cfg.T)
    packed = torch.empty(moe.moe_packed_weights_bytes(shape), dtype=torch.uint8, device=dev)
    moe.moe_prepare_weights(shape, inp.w1, inp.w1_sf, inp.w2, inp.w2_sf, packed)
    ws = torch.empty(moe.moe_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    y = torch.empty(cfg.T, cfg.H, dtype=torch.int16, device=dev)
    w1_bytes = inp.w1.numel() + inp.w1_sf.numel()
    w2_bytes = inp.w2.numel() + inp.w2_sf.numel()
    del inp.w1, inp.w1_sf, inp.w2, inp.w2_sf
    torch.cuda.synchronize()

    def step(events=None):
        if events is None:
            moe.moe_forward(y, inp.x_fp8, inp.x_sf, inp.topk_idx, inp.topk_weights, cfg.T, shape,
                            packed, ws)
        else:
            moe.moe_forward_events(y, inp.x_fp8, inp.x_sf, inp.topk_idx, inp.topk_weights, cfg.T,
                                   shape, packed, ws, events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # The timed region: K plain forwards between two events on the launch stream. The stage
    # split and the per-step spread come from two further loops of K forwards, so that no
    # event other than the two brackets sits inside the timed forwards (at T=128 the five
    # stage events of moe_forward_events add about 20 us to a 157 us forward).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    for e in [e for row in evs for e in row] + marks:   # create the HIP events beforehand
        e.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms = total_ms / K
    # per-step spread: one event between consecutive forwards
    marks[0].record()
    for i in range(K):
        step()
        marks[i + 1].record()
    # stage split: the library records its stage events between its own launches
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(K)])
    stage = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(K)])
    st_ms = stage.mean(axis=0)
    yv = y.view(torch.bfloat16).float()
    assert torch.isfinite(yv).all().item(), "non-finite output"

    flop = cfg.flop
    tflops = flop / (ms * 1e-3) / 1e12
    P = cfg.T * cfg.k
    traffic = load_traffic(cfg.name)
    ids = inp.topk_idx
    n_active = int(torch.unique(ids[(ids >= 0) & (ids < cfg.E)]).numel())   # experts with a row
    roof = linear1_roofline(cfg.T, cfg.k, cfg.H, cfg.I, cfg.E, n_active, w1_bytes, float(st_ms[1]), traffic)
    alg_bytes = (w1_bytes + w2_bytes + cfg.T * cfg.H + cfg.T * (4 * ((cfg.H + 511) // 512))
                 + 8 * P + 2 * cfg.T * cfg.H)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 -> f32 accumulate, bf16 out",
        "data": "synthetic (seeded; x~N(0,1) FP8 1x128 UE8M0, W~N(0,0.02) FP4 1x32 UE8M0)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} E={cfg.E} top-{cfg.k} H={cfg.H} I={cfg.I} "
                               f"{cfg.routing} routing", "T": cfg.T, "E": cfg.E, "k": cfg.k,
                   "H": cfg.H, "I": cfg.I, "routing": cfg.routing, "parallelism": "single GPU"},
        "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
        "pct_fp8xfp4_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "alg_hbm_gbs": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "stage_ms": {"dispatch": round(float(st_ms[0]), 4), "linear1": round(float(st_ms[1]), 4),
                     "linear2": round(float(st_ms[2]), 4), "combine": round(float(st_ms[3]), 4)},
        "wall_s_timed": round(wall, 3),
        "step_ms_p50": round(float(np.percentile(per_step, 50)), 4),
        "step_ms_p99": round(float(np.percentile(per_step, 99)), 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {args.cpu_sample_tokens} tokens ...", file=sys.stderr,
              flush=True)
        idx = inp.topk_idx.cpu().numpy()
        # host copies of what the sample needs: its tokens and the two experts' weights
        from synth import make_weights
        w1, w1_sf, w2, w2_sf = make_weights(cfg, seed=args.seed, device=dev)
        host = {"x_fp8": inp.x_fp8.cpu().numpy(), "x_sf": inp.x_sf.cpu().numpy(),
                "topk_idx": idx, "topk_weights": inp.topk_weights.cpu().numpy(),
                "w1": w1.cpu().numpy(), "w1_sf": w1_sf.cpu().numpy(),
                "w2": w2.cpu().numpy(), "w2_sf": w2_sf.cpu().numpy()}
        del w1, w1_sf, w2, w2_sf
        cb = cpu_baseline(host, cfg, args.cpu_sample_tokens)
        cb.pop("seconds")
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
