"""Benchmark of the fused SVDQuant linear layer on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: the
fused activation-quantization + low-rank down-projection kernel (with its
ordered Z reduction when the channel groups are split) followed by the fused
W4A4 GEMM + low-rank up-projection kernel -- exactly what ``svdq_linear``
launches.  The two halves are issued through their own C-ABI entry points so
that HIP events on the launch stream can bracket the GEMM kernel inside the
timed region.  Offline preparation (smoothing, SVD, residual quantization) is
done before timing and is not part of a step.

Prints ONE JSON line (see the keys below).  Default workload: the FLUX-shaped
fused QKV projection (b=4608 tokens, m=3072, n=9216, rank 32, group 64).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

I8_PEAK_TOPS = 5000.0      # MI355X dense i8 MFMA, TOP/s
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
METRIC = "fused W4A4+low-rank linear TOPS (2·b·m·n/s), FLUX shapes; % of i8 MFMA peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(b, m, n, r):
    """Bytes the two kernels must move (inputs once, outputs once, intermediates
    written and read once); Y as bf16."""
    G = m // 64
    k1 = 2 * b * m + b * m // 2 + 2 * b * G + 4 * b * r + 2 * m * r + 4 * m
    k2 = b * m // 2 + 2 * b * G + 4 * b * r + m * n // 2 + 2 * G * n + 2 * n * r + 2 * b * n
    return k1, k2


def cpu_baseline(inp, cfg, rows):
    """Time the oracle's linear on the first `rows` rows of the workload."""
    from oracle import svdq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    x = inp["x"]
    log(f"cpu_baseline: oracle preparation (ARPACK SVD) for {cfg.name}")
    lay = O.prepare_weights(inp["w"], O.act_amax(x), cfg.rank, svd="arpack")
    if cfg.lora_rank:
        l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], inp["lora_a"], inp["lora_b"],
                                 inp["lora_scale"])
        lay = dict(lay, l1=l1p, l2=l2p)
    xs = x[:rows]
    O.linear(xs[: min(rows, 64)], lay)  # warm-up
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        O.linear(xs, lay)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    ops = 2.0 * rows * cfg.m * cfg.n
    log(f"cpu_baseline: {rows} rows, median {dt:.2f} s of 3 runs, {threads} threads")
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle linear (numpy fp64: quantize, Z, dequantized dgemm, up-projection) on "
                      f"{rows} of {x.shape[0]} rows of {cfg.name}; median of 3 runs = {dt:.2f} s; "
                      f"oracle preparation (SVD) excluded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flux_qkv")
    ap.add_argument("--out", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--rank", type=int, default=None, help="override the SVD rank (0 = bare W4A4)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows for the oracle timing (0 = all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the layer shards "
              "over token rows with no communication; see DESIGN.md). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    cfg = workloads.CONFIGS[args.workload]
    log(f"bench: workload {cfg.name} b={cfg.rows or cfg.b} m={cfg.m} n={cfg.n}")
    inp = workloads.make_inputs(cfg)
    b = inp["x"].shape[0]
    m, n = cfg.m, cfg.n
    rank_svd = cfg.rank if args.rank is None else args.rank
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)

    # calibration statistic on the GPU, then host preparation in the library
    amax = S.svdq_calibrate_act_amax(x).cpu().numpy()
    t0 = time.perf_counter()
    host = S.svdq_prepare_weights(inp["w"], amax, rank_svd)
    prep_s = time.perf_counter() - t0
    if cfg.lora_rank and args.rank is None:
        l1p, l2p = S.svdq_append_lora(host["l1"], host["l2"], m, n, rank_svd, host["lambda"],
                                      inp["lora_a"], inp["lora_b"], inp["lora_scale"])
        host = dict(host, l1=l1p, l2=l2p, rank=rank_svd + cfg.lora_rank)
    r = int(host["rank"])
    log(f"bench: host preparation {prep_s:.1f} s (rank {r})")
    layer = S.DeviceLayer(host, device=dev)

    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    G = m // 64
    qx = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    asc = torch.empty((G, b), dtype=torch.float16, device=dev)
    z = torch.empty((b, max(r, 1)), dtype=torch.float32, device=dev) if r else None
    wsz = S.svdq_act_workspace_size(b, m, r)
    ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)
    y = torch.empty((b, n), dtype=out_dtype, device=dev)
    gws = torch.empty(max(S.svdq_gemm_workspace_size(b, n, m), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        S.svdq_quantize_act_lowrank_down(x, layer.smooth_inv, layer.l1, r, qx=qx, ascale=asc, z=z,
                                         workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        S.svdq_gemm_w4a4_lowrank_up(qx, asc, z, layer, b, out_dtype, y=y, workspace=gws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # timed region: barrier (single process) + synchronize on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    k2_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    ms_per_step = elapsed * 1e3 / args.steps

    # the same work through the one-call entry point, for reference
    ws_lin = torch.empty(max(S.svdq_linear_workspace_size(b, m, n, r), 1), dtype=torch.uint8, device=dev)
    for _ in range(3):
        S.svdq_linear(x, layer, out_dtype, y=y, workspace=ws_lin, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        S.svdq_linear(x, layer, out_dtype, y=y, workspace=ws_lin, stream=stream)
    torch.cuda.synchronize()
    linear_ms = (time.perf_counter() - t1) * 1e3 / args.steps

    ops = 2.0 * b * m * n
    value = ops / (ms_per_step * 1e-3) / 1e12
    k2_tops = ops / (k2_ms * 1e-3) / 1e12
    k1_bytes, k2_bytes = algorithmic_bytes(b, m, n, r)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "b": b, "m": m, "n": n, "rank": r, "group": 64,
                   "out": args.out, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(k2_tops, 2), "peak": I8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(k2_tops / I8_PEAK_TOPS, 4), "traffic": None},
        "kernels": {"act_quant_down_ms": round(k1_ms, 5), "gemm_w4a4_up_ms": round(k2_ms, 5),
                    "act_quant_down_GBs": round(k1_bytes / (k1_ms * 1e-3) / 1e9, 1),
                    "act_quant_down_hbm_frac": round(k1_bytes / (k1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "gemm_w4a4_up_TOPs": round(k2_tops, 2),
                    "gemm_algorithmic_bytes": k2_bytes, "act_algorithmic_bytes": k1_bytes,
                    "svdq_linear_ms": round(linear_ms, 5)},
        "prep_s": round(prep_s, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, cfg, min(args.cpu_rows, b) if args.cpu_rows else b)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
