"""Benchmark of the fused SVDQuant linear layer on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: the
fused activation-quantization + low-rank down-projection kernel (with its
ordered Z reduction when the channel groups are split) followed by the fused
W4A4 GEMM + low-rank up-projection kernel -- exactly what ``svdq_linear``
launches.  The two halves are issued through their own C-ABI entry points so
that HIP events on the launch stream can bracket the GEMM kernel inside the
timed region.  Offline preparation (smoothing, SVD, residual quantization) is
done before timing and is not part of a step.

Timed region ("cold"): the steps rotate over several independently seeded
input + weight sets whose footprint exceeds the 256 MB last-level cache, so a
step does not find its layer's weights or activations cached by the previous
step.  Between the warm-up steps and the timed region the layer's own steps
run untimed for about a quarter second, with no idle gap (``settle_steps``),
so that the timed steps see the GPU's sustained clock rather than its ramp
from idle; ``--no-settle`` times from idle instead.  Two HIP events per step
bracket the GEMM kernel.  Also reported: the same steps on one set ("warm"),
the low-rank overhead t(rank r) / t(rank 0, same codes and scales) - 1 from
rank-r and rank-0 steps interleaved on one set (median HIP-event step times),
the one-call ``svdq_linear`` entry point, and the GEMM's fractions of the i8
MFMA peak, of HBM bandwidth and of the fp32 FMA peak its scale epilogue needs.

Prints ONE JSON line.  Default workload: the FLUX-shaped fused QKV projection
(b=4608 tokens, m=3072, n=9216, rank 32, group 64).  The other FLUX- and
PixArt-shaped layers are timed by the same method in the same run and reported
under ``extra_configs`` (their cold sets are copies of one prepared set at
fresh addresses, which keeps the run short).

Extra modes (used with rocprofv3 runs):
  --copy-check               also run a plain device copy of known size, which
                             calibrates the FETCH_SIZE / WRITE_SIZE counters;
  --traffic-summary F W      turn two counter-collection directories (a
                             FETCH_SIZE run and a WRITE_SIZE run of the same
                             command) into the per-launch HBM traffic summary
                             read by the JSON line's roofline.traffic;
  --trace-summary DIR        summarize a --kernel-trace --stats run of this
                             script (same --workload/--steps/--warmup);
  --cpu-threads N            time the oracle baseline on at most N BLAS threads
                             (default: all the process may use);
  --prep-refine [WORKLOADS]  preparation with a search over migration
                             strengths and factor refinement against the
                             plain preparation: layer-output error on held-out
                             rows (one JSON line);
  --fusion-ab [RANKS]        time the fused layer against the unfused one
                             (separate down- and up-projection kernels, a
                             second b x n output and an addition) at each rank,
                             and print that table as one JSON line instead.
"""
from __future__ import annotations

import argparse
import ctypes
import functools
import glob
import csv
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

I8_PEAK_TOPS = 5000.0      # MI355X dense i8 MFMA, TOP/s
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 MFMA, TFLOP/s
FP32_FMA_PEAK_TFLOPS = 78.6  # MI355X fp32 FMA without packed math: 256 CUs x 64 lanes x 2 flops x 2.4 GHz
EXTRA_CONFIGS = "flux_fc2,flux_single_fc,flux_single_out,flux_single_fc_b256,flux_single_out_b256,pixart_fc1"
METRIC = "fused W4A4+low-rank linear TOPS (2·b·m·n/s), FLUX shapes; % of i8 MFMA peak"
GEMM_KERNEL = "gemm_w4a4_up_kernel"
# sources whose text defines the GEMM kernel and its launch plan
GEMM_SOURCES = ["w4a4_rank_corrected_amd/csrc/gemm_kernels.hip",
                "w4a4_rank_corrected_amd/csrc/device_common.h",
                "w4a4_rank_corrected_amd/csrc/internal.h",
                "w4a4_rank_corrected_amd/csrc/plan.cpp"]
COPY_BYTES = 256 << 20     # plain copy used to calibrate the byte counters
SETTLE_OPS = 2.5e14        # work of the clock-settling steps: about 0.25 s at 1 POP/s
COLD_BYTES = 512 << 20     # rotated footprint of the cold measurement


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{GEMM_KERNEL}_{workload}.json")


def algorithmic_bytes(b, m, n, r):
    """Bytes the two kernels must move (inputs once, outputs once, intermediates
    written and read once); Y as bf16."""
    G = m // 64
    k1 = 2 * b * m + b * m // 2 + 2 * b * G + 4 * b * r + 2 * m * r + 4 * m
    k2 = b * m // 2 + 2 * b * G + 4 * b * r + m * n // 2 + 2 * G * n + 2 * n * r + 2 * b * n
    return k1, k2


def settle_steps(b, m, n):
    """Untimed steps of the layer run right before its timed region, with no
    idle gap, so that the region measures the sustained engine clock.  From
    idle an MI355X raises its clock over about 40 ms of continuous work (the
    FLUX QKV GEMM falls from about 255 to 216.5 us per launch over its first
    150 launches and then holds that), and it drops back after about a second
    of idling, e.g. while the host prepares a layer.  The count is a function of
    the shape only (about 0.25 s of work at 1 POP/s, at least 50 steps and at
    most 5000), so that a kernel trace of the run can find the timed region."""
    return int(min(5000, max(50, math.ceil(SETTLE_OPS / (2.0 * b * m * n)))))


def compare_untimed_steps(b, m, n, args):
    """Untimed steps of the setting comparisons (--w8a8, --fp4): the warm-up,
    then the clock-settling steps; a step runs both settings' kernels, about
    twice one layer's work, so half of ``settle_steps``."""
    return max(50, args.warmup) + (0 if args.no_settle else settle_steps(b, m, n) // 2)


def set_plan(cfg, rank, out):
    """(bytes of one input+weight set, number of sets rotated by the cold timing)."""
    b, m, n = cfg.rows or cfg.b, cfg.m, cfg.n
    per_set = 2 * b * m + m * n // 2 + 2 * (m // 64) * n + 2 * rank * (m + n) + 4 * m + \
        (2 if out == "bf16" else 4) * b * n
    return per_set, max(3, math.ceil(COLD_BYTES / per_set))


# ---------------------------------------------------------------------------
# profile summaries (no GPU needed)
# ---------------------------------------------------------------------------

def trace_summary(prof_dir, cfg, args, rank):
    """Markdown summary of a ``rocprofv3 --kernel-trace --stats`` run of this
    script: per-kernel totals, and the mean duration of each kernel over the
    cold timed region (the dispatches after the warm-up, in launch order)."""
    import re
    import sqlite3
    dbs = glob.glob(os.path.join(prof_dir, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocpd database under {prof_dir}")
    c = sqlite3.connect(dbs[0])
    w8 = args.w8a8 is not None
    f4 = args.fp4 is not None
    cmp_mode = w8 or f4
    _, n_sets = set_plan(cfg, rank, args.out)
    b_rows = cfg.rows or cfg.b
    n_settle = 0 if cmp_mode or args.no_settle else settle_steps(b_rows, cfg.m, cfg.n)
    skip = compare_untimed_steps(b_rows, cfg.m, cfg.n, args) if cmp_mode else max(args.warmup, n_sets) + n_settle
    short = lambda nm: re.sub(r"\(.*", "", nm.replace("svdq::(anonymous namespace)::", "")
                              .replace("void ", "").replace("svdq::", ""))
    rows = list(c.execute("select name, start, end, grid_x, grid_y, workgroup_x, workgroup_y, vgpr_count, "
                          "accum_vgpr_count, lds_size, scratch_size from kernels order by start"))
    by = {}
    for nm, st, en, gx, gy, wx, wy, vg, ag, lds, scr in rows:
        wgs = (gx // max(wx, 1)) * (gy // max(wy, 1))
        by.setdefault(nm, []).append(((en - st) / 1e3, wgs, wx * wy, vg, ag, lds, scr))
    mode = f" --w8a8 {args.w8a8}" if w8 else (f" --fp4 {args.fp4}" if f4 else " --no-cpu-baseline --extra-configs ''")
    cmd = (f"rocprofv3 --kernel-trace --stats -d {prof_dir} -o run -- python3 bench.py --workload {cfg.name} "
           f"--steps {args.steps} --warmup {args.warmup}{mode}")
    if cmp_mode:
        other = "8-bit" if w8 else "NVFP4"
        region = (f"Timed region: {args.steps} steps after {skip} untimed ones; each step runs the INT4 "
                  f"activation kernel, the INT4 GEMM, the {other} activation kernel(s) and the {other} GEMM, "
                  f"all at rank {rank} on one input and weight set (warm).")
        title = f"# Kernel trace, {other} setting against INT4: {cfg.name}"
    else:
        region = (f"Timed region: {args.steps} steps after {skip} untimed ones ({max(args.warmup, n_sets)} "
                  f"warm-up and {n_settle} clock-settling steps), rotating over {n_sets} "
                  f"input+weight sets; the script then times warm steps, rank-r and rank-0 steps interleaved "
                  f"and the one-call entry point, which the all-dispatch columns include.")
        title = f"# Kernel trace: {cfg.name}"
    out = [f"{title} (b={cfg.rows or cfg.b}, m={cfg.m}, n={cfg.n}, rank {rank})", "",
           "Command (repository root, one MI355X), then the summary:", "", "```", cmd,
           f"python bench.py --trace-summary {prof_dir} --workload {cfg.name} --steps {args.steps} "
           f"--warmup {args.warmup}" + mode.replace(" --no-cpu-baseline --extra-configs ''", ""), "```", "", region, "",
           "| kernel | dispatches | mean, timed region (us) | mean, all (us) | total (ms) | workgroups | "
           "threads | LDS (B) | scratch (B) |",
           "|---|---|---|---|---|---|---|---|---|"]
    total = sum(d[0] for v in by.values() for d in v)
    for nm, v in sorted(by.items(), key=lambda kv: -sum(d[0] for d in kv[1])):
        durs = [d[0] for d in v]
        # kernels launched once per step: the timed region is dispatches [skip, skip + steps)
        per_step = [d for d in durs[skip: skip + args.steps]] if len(durs) >= skip + args.steps else []
        t = f"{np.mean(per_step):.2f}" if per_step else "-"
        d0 = v[0]
        out.append(f"| `{short(nm)}` | {len(v)} | {t} | {np.mean(durs):.2f} | {sum(durs) / 1e3:.3f} | "
                   f"{d0[1]} | {d0[2]} | {d0[5]} | {d0[6]} |")
    out += ["", f"All kernels: {total / 1e3:.3f} ms of GPU time.", ""]
    prefix = "w8a8_" if w8 else ("nvfp4_" if f4 else "")
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{prefix}{cfg.name}.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))
    log(f"wrote {path}")


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, name_pred):
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and name_pred(r["Kernel_Name"]):
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(vals.values())


SQ_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
               "SQ_WAVES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE")
N_XCD, N_SIMD = 8, 1024    # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
PEAK_CLOCK_GHZ = 2.4       # MI355X peak engine clock


def _per_dispatch_duration(rows, name_pred):
    d = {}
    for r in rows:
        if name_pred(r["Kernel_Name"]):
            d[r["Dispatch_Id"]] = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9
    return list(d.values())


def counter_summary(sq_dir, fetch_dir, write_dir, workload, commands):
    """Markdown summary of the two kernels' counters: MFMA and VALU utilisation
    (SQ counters over the dispatch's duration at the peak engine clock) and HBM
    bytes / GB/s (FETCH_SIZE and WRITE_SIZE scaled by the plain copy, as in the
    traffic summary).  Medians over dispatches."""
    sq, fr, wr = _counter_rows(sq_dir), _counter_rows(fetch_dir), _counter_rows(write_dir)
    is_copy = lambda k: "elementwise" in k or "copy" in k.lower()
    f_fac = COPY_BYTES / (max(_per_dispatch(fr, "FETCH_SIZE", is_copy)) * 1024.0)
    w_fac = COPY_BYTES / (max(_per_dispatch(wr, "WRITE_SIZE", is_copy)) * 1024.0)
    kernels = [("GEMM + up-projection", lambda k: GEMM_KERNEL in k),
               # the INT4 activation kernel (split or wide) with the low-rank branch: the
               # rank-0 build (first template argument 0) of the overhead steps is left out
               ("act-quant + down-projection",
                lambda k: ("act_quant_down_kernel<" in k or "act_quant_wide_kernel<" in k) and ", 1>" in k
                and "_kernel<0," not in k)]
    med = lambda v: float(np.median(v)) if v else float("nan")
    out = [f"# Counters: {workload} (one MI355X)", "", "Commands (repository root), then the summary:", "", "```",
           commands, "```", "",
           "Per kernel, medians over its dispatches. Cycles = dispatch duration x 2.4 GHz (the peak engine "
           "clock; GRBM_GUI_ACTIVE / 8 XCDs gives the clock the dispatch ran at, which the short activation "
           "kernel's counter window overstates). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles). "
           "VALU rate = SQ_INSTS_VALU / (1024 x cycles), wave64 VALU instructions per SIMD per cycle. "
           "HBM bytes = FETCH_SIZE and WRITE_SIZE, "
           f"each scaled by what it reads for a plain {COPY_BYTES >> 20} MiB device copy in the same run "
           f"(factors {f_fac:.3f} and {w_fac:.3f}). Durations are the counter runs' dispatch timestamps "
           "(profiling adds overhead).", "",
           "| kernel | dispatches | duration (us) | clock (GHz) | MFMA busy | VALU instr / SIMD / cycle | LDS conflict cycles / LDS instr "
           "| HBM fetch (MB) | HBM write (MB) | HBM GB/s | % of 8 TB/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for label, pred in kernels:
        dur = med(_per_dispatch_duration(sq, pred))
        gui = med(_per_dispatch(sq, "GRBM_GUI_ACTIVE", pred))
        cyc = dur * PEAK_CLOCK_GHZ * 1e9
        mf = med(_per_dispatch(sq, "SQ_VALU_MFMA_BUSY_CYCLES", pred)) / (N_SIMD * cyc)
        va = med(_per_dispatch(sq, "SQ_INSTS_VALU", pred)) / (N_SIMD * cyc)
        lds = med(_per_dispatch(sq, "SQ_LDS_BANK_CONFLICT", pred)) / max(med(_per_dispatch(sq, "SQ_INSTS_LDS", pred)), 1)
        fb = med(_per_dispatch(fr, "FETCH_SIZE", pred)) * 1024.0 * f_fac
        wb = med(_per_dispatch(wr, "WRITE_SIZE", pred)) * 1024.0 * w_fac
        fdur = med(_per_dispatch_duration(fr, pred))
        gbs = (fb + wb) / fdur / 1e9
        out.append(f"| {label} | {len(_per_dispatch(sq, 'GRBM_GUI_ACTIVE', pred))} | {dur * 1e6:.1f} | "
                   f"{gui / N_XCD / dur / 1e9:.2f} | {100 * mf:.1f} % | {va:.3f} | {lds:.2f} | {fb / 1e6:.1f} | "
                   f"{wb / 1e6:.1f} | {gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f} % |")
    out.append("")
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))
    log(f"wrote {path}")


def traffic_summary(fetch_dir, write_dir, workload, commands):
    """Per-launch HBM bytes of the GEMM kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the plain copy of COPY_BYTES."""
    is_copy = lambda k: "elementwise" in k or "copy" in k.lower()
    is_gemm = lambda k: GEMM_KERNEL in k
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    # the copy is the largest elementwise dispatch of the run
    cf = max(_per_dispatch(fr, "FETCH_SIZE", is_copy))
    cw = max(_per_dispatch(wr, "WRITE_SIZE", is_copy))
    f_fac = COPY_BYTES / (cf * 1024.0)
    w_fac = COPY_BYTES / (cw * 1024.0)
    gf = _per_dispatch(fr, "FETCH_SIZE", is_gemm)
    gw = _per_dispatch(wr, "WRITE_SIZE", is_gemm)
    fetch = float(np.median(gf)) * 1024.0 * f_fac
    write = float(np.median(gw)) * 1024.0 * w_fac
    out = {
        "kernel": GEMM_KERNEL, "workload": workload, "source_sha256": gemm_source_hash(),
        "commands": commands,
        "gemm_dispatches": [len(gf), len(gw)],
        "gemm_fetch_kib_median": float(np.median(gf)), "gemm_write_kib_median": float(np.median(gw)),
        "copy_bytes": COPY_BYTES, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_factor": f_fac, "write_factor": w_fac,
        "fetch_bytes": fetch, "write_bytes": write, "traffic_bytes": fetch + write,
    }
    path = traffic_path(workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    log(f"wrote {path}")


def load_traffic(workload):
    """Per-launch HBM bytes of the GEMM kernel, or None when no summary exists or
    the kernel's sources changed since the counters were taken."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != gemm_source_hash():
        return None
    return t


# ---------------------------------------------------------------------------
# oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(inp, cfg, rows, max_threads=0):
    """Time the oracle's linear on the first `rows` rows of the workload (its
    BLAS on at most `max_threads` threads when that is > 0; the oracle's
    preparation, which is not timed, always uses every thread)."""
    import contextlib
    from oracle import svdq_oracle as O
    x = inp["x"]
    log(f"cpu_baseline: oracle preparation (ARPACK SVD) for {cfg.name}")
    lay = O.prepare_weights(inp["w"], O.act_amax(x), cfg.rank, svd="arpack")
    if cfg.lora_rank:
        l1p, l2p = O.append_lora(lay["l1"], lay["l2"], lay["lam32"], inp["lora_a"], inp["lora_b"],
                                 inp["lora_scale"])
        lay = dict(lay, l1=l1p, l2=l2p)
    xs = x[:rows]
    limit = contextlib.nullcontext()
    if max_threads > 0:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=max_threads)
    with limit:
        try:
            from threadpoolctl import threadpool_info
            threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        except Exception:  # pragma: no cover
            threads = len(os.sched_getaffinity(0))
        O.linear(xs[: min(rows, 64)], lay)  # warm-up
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.linear(xs, lay)
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    ops = 2.0 * rows * cfg.m * cfg.n
    log(f"cpu_baseline: {rows} rows, median {dt:.3g} s of 3 runs, {threads} threads")
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle linear (numpy fp64: quantize, Z, dequantized dgemm, up-projection) on "
                      f"{rows} of {x.shape[0]} rows of {cfg.name}; median of 3 runs = {dt:.3g} s; "
                      f"oracle preparation (SVD) excluded"}


# ---------------------------------------------------------------------------
# GPU benchmark
# ---------------------------------------------------------------------------

def prep_refine(names, args):
    """Plain preparation (alpha = 0.5) against the search over migration
    strengths (0.2 .. 1.0) with two factor-refinement steps (Algorithm 1 steps
    6-8), both by the library on the host.  Calibration: the first 256 rows of
    the workload's X (statistics and candidate scores); evaluation: 512 other
    rows, through the fused GPU layer with fp32 output, against X W in fp64."""
    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    dev = torch.device("cuda:0")
    alphas = (0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8, 0.9, 1.0)
    rows = []
    for name in names:
        cfg = workloads.CONFIGS[name]
        inp = workloads.make_inputs(cfg)
        xb, w = inp["x_bits"], inp["w"]
        b = xb.shape[0]
        cal = np.ascontiguousarray(xb[:min(256, b // 2)])
        ev = np.ascontiguousarray(xb[b // 2: b // 2 + min(512, b - b // 2)])
        cal_d = torch.from_numpy(cal.view(np.int16)).to(dev).view(torch.bfloat16)
        amax = S.svdq_calibrate_act_amax(cal_d).cpu().numpy()
        ev_d = torch.from_numpy(ev.view(np.int16)).to(dev).view(torch.bfloat16)
        xe = (ev.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        yref = xe @ w.astype(np.float64)

        def held_out(host):
            y = S.svdq_linear(ev_d, S.DeviceLayer(host, device=dev), torch.float32)
            torch.cuda.synchronize()
            return float(np.linalg.norm(y.cpu().numpy() - yref) / np.linalg.norm(yref))

        t0 = time.perf_counter()
        base = S.svdq_prepare_weights_refined(w, amax, cal, cfg.rank, alphas=(0.5,), iters=0)
        t_base = time.perf_counter() - t0
        t0 = time.perf_counter()
        search = S.svdq_prepare_weights_refined(w, amax, cal, cfg.rank, alphas=alphas, iters=0)
        t_search = time.perf_counter() - t0
        t0 = time.perf_counter()
        refined = S.svdq_prepare_weights_refined(w, amax, cal, cfg.rank, alphas=alphas, iters=2)
        t_ref = time.perf_counter() - t0
        row = {"workload": name, "rank": cfg.rank, "cal_rows": int(cal.shape[0]), "eval_rows": int(ev.shape[0])}
        for key, host, t in (("plain", base, t_base), ("alpha_search", search, t_search),
                             ("alpha_search_refit2", refined, t_ref)):
            row[key] = {"alpha": host["alpha"], "iteration": host["iteration"],
                        "cal_err": round(host["rel_err"], 6), "heldout_err": round(held_out(host), 6),
                        "prep_s": round(t, 2)}
        log(f"prep-refine {name}: " + ", ".join(f"{k} {row[k]['heldout_err']:.5f} (alpha {row[k]['alpha']}, "
                                                f"it {row[k]['iteration']})"
                                                for k in ("plain", "alpha_search", "alpha_search_refit2")))
        rows.append(row)
    print(json.dumps({"prep_refine": rows, "alphas": list(alphas)}), flush=True)


def fusion_ab(cfg, ranks, args):
    """Fused (svdq_linear: 2 kernels) against unfused (svdq_linear_unfused: the
    act quantization, the W4A4 product, a separate down-projection reading X
    again, a separate up-projection writing a second b x n output, an addition)
    at each rank, on layers the library prepares from the workload's X and W
    (LoRA not attached: the rank is the SVD rank).  Warm timing: HIP events
    around each call on the launch stream, median over the steps."""
    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    b, m, n = x.shape[0], cfg.m, cfg.n
    amax = S.svdq_calibrate_act_amax(x).cpu().numpy()
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    y = torch.empty((b, n), dtype=out_dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    ops = 2.0 * b * m * n

    def time_pair(ws_f, ws_u):
        """Fused and unfused calls alternate step by step (same clocks and
        cache state for both), after at least max(50, warmup) pairs and at
        least 0.25 s of them (the host preparation before each rank idles the
        GPU, and its clock needs about 40 ms of work to settle again)."""
        t0, k = time.perf_counter(), 0
        while k < max(50, args.warmup) or (not args.no_settle and time.perf_counter() - t0 < 0.25):
            S.svdq_linear(x, layer, out_dtype, y=y, workspace=ws_f, stream=stream)
            S.svdq_linear_unfused(x, layer, out_dtype, y=y, workspace=ws_u, stream=stream)
            k += 1
        ev = []
        for _ in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            S.svdq_linear(x, layer, out_dtype, y=y, workspace=ws_f, stream=stream)
            e[1].record(stream)
            S.svdq_linear_unfused(x, layer, out_dtype, y=y, workspace=ws_u, stream=stream)
            e[2].record(stream)
            ev.append(e)
        torch.cuda.synchronize()
        return (float(np.median([e[0].elapsed_time(e[1]) for e in ev])),
                float(np.median([e[1].elapsed_time(e[2]) for e in ev])))

    rows = []
    for r in ranks:
        host = S.svdq_prepare_weights(inp["w"], amax, r)
        layer = S.DeviceLayer(host, device=dev)
        wsf = torch.empty(max(S.svdq_linear_workspace_size(b, m, n, r), 1), dtype=torch.uint8, device=dev)
        wsu = torch.empty(max(S.svdq_linear_unfused_workspace_size(b, m, n, r), 1), dtype=torch.uint8,
                          device=dev)
        tf, tu = time_pair(wsf, wsu)
        rows.append({"rank": r, "fused_ms": round(tf, 5), "unfused_ms": round(tu, 5),
                     "fused_TOPs": round(ops / (tf * 1e-3) / 1e12, 1)})
        log(f"fusion A/B {cfg.name} rank {r}: fused {tf * 1e3:.1f} us, unfused {tu * 1e3:.1f} us")
        del layer, wsf, wsu
    base = next((row["fused_ms"] for row in rows if row["rank"] == 0), None)
    for row in rows:
        if base:
            row["fused_overhead"] = round(row["fused_ms"] / base - 1.0, 4)
            row["unfused_overhead"] = round(row["unfused_ms"] / base - 1.0, 4)
    print(json.dumps({"fusion_ab": rows, "workload": cfg.name, "b": b, "m": m, "n": n, "out": args.out,
                      "steps": args.steps,
                      "timing": "warm; fused and unfused calls alternate; median of HIP-event times"}),
          flush=True)


def w8a8_compare(cfg, rank, args):
    """The 8-bit setting (per-token / per-channel INT8 + the rank-r branch)
    against W4A4 at the same rank, on layers the library prepares from the
    workload's X and W.  Warm timing: the four calls (W4A4 activation kernel,
    W4A4 GEMM, 8-bit activation kernels, 8-bit GEMM) alternate step by step,
    HIP events around each on the launch stream, median over the steps.  The
    output error of each against the unquantized product X W (fp64, numpy) is
    measured on sampled rows."""
    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    b, m, n = x.shape[0], cfg.m, cfg.n
    amax = S.svdq_calibrate_act_amax(x).cpu().numpy()
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    stream = torch.cuda.current_stream(dev)
    l4 = S.DeviceLayer(S.svdq_prepare_weights(inp["w"], amax, rank), device=dev)
    l8 = S.DeviceLayer8(S.svdq_w8a8_prepare_weights(inp["w"], amax, rank), device=dev)
    G = m // 64
    y4 = torch.empty((b, n), dtype=out_dtype, device=dev)
    y8 = torch.empty((b, n), dtype=out_dtype, device=dev)
    qx4 = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    as4 = torch.empty((G, b), dtype=torch.float16, device=dev)
    qx8 = torch.empty((G, b, 64), dtype=torch.int8, device=dev)
    as8 = torch.empty(b, dtype=torch.float16, device=dev)
    z = torch.empty((b, max(rank, 1)), dtype=torch.float32, device=dev) if rank else None
    aws = torch.empty(max(S.svdq_act_workspace_size(b, m, rank), 1), dtype=torch.uint8, device=dev)
    gws = torch.empty(max(S.svdq_gemm_workspace_size(b, n, m), 1), dtype=torch.uint8, device=dev)

    def step(ev=None):
        calls = [
            lambda: S.svdq_quantize_act_lowrank_down(x, l4.smooth_inv, l4.l1, rank, qx=qx4, ascale=as4, z=z,
                                                     workspace=aws, stream=stream),
            lambda: S.svdq_gemm_w4a4_lowrank_up(qx4, as4, z, l4, b, out_dtype, y=y4, workspace=gws, stream=stream),
            lambda: S.svdq_w8a8_quantize_act_lowrank_down(x, l8.smooth_inv, l8.l1, rank, qx=qx8, ascale=as8, z=z,
                                                          workspace=aws, stream=stream),
            lambda: S.svdq_w8a8_gemm_lowrank_up(qx8, as8, z, l8, b, out_dtype, y=y8, workspace=gws,
                                                stream=stream),
        ]
        for k, c in enumerate(calls):
            if ev is not None:
                ev[k].record(stream)
            c()
        if ev is not None:
            ev[4].record(stream)

    for _ in range(compare_untimed_steps(b, m, n, args)):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t = [float(np.median([e[k].elapsed_time(e[k + 1]) for e in evs])) for k in range(4)]
    # accuracy on sampled rows against the unquantized product
    rows = np.arange(0, b, max(1, b // 64))
    xr = (inp["x_bits"][rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    yref = xr @ inp["w"].astype(np.float64)

    def err(y):
        yv = y[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
        return float(np.linalg.norm(yv - yref) / np.linalg.norm(yref))

    ops = 2.0 * b * m * n
    res = {"w8a8_vs_w4a4": {
        "workload": cfg.name, "b": b, "m": m, "n": n, "rank": rank, "out": args.out, "steps": args.steps,
        "timing": "warm; the four calls alternate; median of HIP-event times",
        "w4a4": {"act_ms": round(t[0], 5), "gemm_ms": round(t[1], 5), "total_ms": round(t[0] + t[1], 5),
                 "gemm_TOPs": round(ops / (t[1] * 1e-3) / 1e12, 1),
                 "gemm_frac_i8_peak": round(ops / (t[1] * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
                 "rel_err_vs_xw": round(err(y4), 6)},
        "w8a8": {"act_ms": round(t[2], 5), "gemm_ms": round(t[3], 5), "total_ms": round(t[2] + t[3], 5),
                 "gemm_TOPs": round(ops / (t[3] * 1e-3) / 1e12, 1),
                 "gemm_frac_i8_peak": round(ops / (t[3] * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
                 "rel_err_vs_xw": round(err(y8), 6)},
    }}
    log(f"w8a8 {cfg.name} rank {rank}: W4A4 {t[0] * 1e3:.1f} + {t[1] * 1e3:.1f} us, "
        f"W8A8 {t[2] * 1e3:.1f} + {t[3] * 1e3:.1f} us")
    print(json.dumps(res), flush=True)


def fp4_compare(cfg, rank, args):
    """The NVFP4 setting (E2M1 codes, E4M3 scales per 16 channels, f16 MFMA on
    exactly dequantized operands) against INT4 at the same rank, on layers the
    library prepares from the workload's X and W.  Warm timing as in
    ``w8a8_compare``; output error against the unquantized X W on sampled rows."""
    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    inp = workloads.make_inputs(cfg)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    b, m, n = x.shape[0], cfg.m, cfg.n
    amax = S.svdq_calibrate_act_amax(x).cpu().numpy()
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    stream = torch.cuda.current_stream(dev)
    l4 = S.DeviceLayer(S.svdq_prepare_weights(inp["w"], amax, rank), device=dev)
    lf = S.DeviceLayerFp4(S.svdq_fp4_prepare_weights(inp["w"], amax, rank), device=dev)
    G = m // 64
    y4 = torch.empty((b, n), dtype=out_dtype, device=dev)
    yf = torch.empty((b, n), dtype=out_dtype, device=dev)
    qx4 = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    as4 = torch.empty((G, b), dtype=torch.float16, device=dev)
    qxf = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    asf = torch.empty((G, b, 4), dtype=torch.uint8, device=dev)
    z = torch.empty((b, max(rank, 1)), dtype=torch.float32, device=dev) if rank else None
    aws = torch.empty(max(S.svdq_act_workspace_size(b, m, rank), 1), dtype=torch.uint8, device=dev)
    gws = torch.empty(max(S.svdq_gemm_workspace_size(b, n, m), 1), dtype=torch.uint8, device=dev)

    def step(ev=None):
        calls = [
            lambda: S.svdq_quantize_act_lowrank_down(x, l4.smooth_inv, l4.l1, rank, qx=qx4, ascale=as4, z=z,
                                                     workspace=aws, stream=stream),
            lambda: S.svdq_gemm_w4a4_lowrank_up(qx4, as4, z, l4, b, out_dtype, y=y4, workspace=gws, stream=stream),
            lambda: S.svdq_fp4_quantize_act_lowrank_down(x, lf.smooth_inv, lf.l1, rank, lf.t_x, qx=qxf, ascale=asf,
                                                         z=z, workspace=aws, stream=stream),
            lambda: S.svdq_fp4_gemm_lowrank_up(qxf, asf, z, lf, b, out_dtype, y=yf, workspace=gws, stream=stream),
        ]
        for k, c in enumerate(calls):
            if ev is not None:
                ev[k].record(stream)
            c()
        if ev is not None:
            ev[4].record(stream)

    for _ in range(compare_untimed_steps(b, m, n, args)):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t = [float(np.median([e[k].elapsed_time(e[k + 1]) for e in evs])) for k in range(4)]
    rows = np.arange(0, b, max(1, b // 64))
    xr = (inp["x_bits"][rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    yref = xr @ inp["w"].astype(np.float64)

    def err(y):
        yv = y[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
        return float(np.linalg.norm(yv - yref) / np.linalg.norm(yref))

    ops = 2.0 * b * m * n
    res = {"fp4_vs_w4a4": {
        "workload": cfg.name, "b": b, "m": m, "n": n, "rank": rank, "out": args.out, "steps": args.steps,
        "timing": "warm; the four calls alternate; median of HIP-event times",
        "w4a4": {"act_ms": round(t[0], 5), "gemm_ms": round(t[1], 5), "total_ms": round(t[0] + t[1], 5),
                 "gemm_TOPs": round(ops / (t[1] * 1e-3) / 1e12, 1),
                 "gemm_frac_i8_peak": round(ops / (t[1] * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
                 "rel_err_vs_xw": round(err(y4), 6)},
        "nvfp4": {"act_ms": round(t[2], 5), "gemm_ms": round(t[3], 5), "total_ms": round(t[2] + t[3], 5),
                  "gemm_TFLOPs": round(ops / (t[3] * 1e-3) / 1e12, 1),
                  "gemm_frac_f16_peak": round(ops / (t[3] * 1e-3) / 1e12 / F16_PEAK_TFLOPS, 4),
                  "rel_err_vs_xw": round(err(yf), 6), "t_x": lf.t_x, "t_w": lf.t_w},
    }}
    log(f"fp4 {cfg.name} rank {rank}: W4A4 {t[0] * 1e3:.1f} + {t[1] * 1e3:.1f} us, "
        f"NVFP4 {t[2] * 1e3:.1f} + {t[3] * 1e3:.1f} us")
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flux_qkv")
    ap.add_argument("--out", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--rank", type=int, default=None, help="override the SVD rank (0 = bare W4A4)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows for the oracle timing (0 = all)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="BLAS threads for the oracle timing (0 = all the process may use)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-settle", action="store_true",
                    help="time right after the warm-up steps, without the clock-settling steps (from idle)")
    ap.add_argument("--extra-configs", default=EXTRA_CONFIGS,
                    help="further workloads timed by the same method in the same run (comma-separated; "
                         "'' for none)")
    ap.add_argument("--extra-steps", type=int, default=30, help="timed steps of each extra configuration")
    ap.add_argument("--copy-check", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the GEMM traffic summary from two counter runs and exit")
    ap.add_argument("--commands", default="", help="counter-run commands recorded in the summary")
    ap.add_argument("--counter-summary", nargs=3, metavar=("SQ_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the per-kernel counter summary (MFMA / VALU utilisation, HBM GB/s) and exit")
    ap.add_argument("--trace-summary", metavar="PROF_DIR",
                    help="write the kernel-trace summary of a profiled run of this script and exit")
    ap.add_argument("--prep-refine", nargs="?", const="tiny,pixart_fc1,flux_qkv", default=None,
                    metavar="WORKLOADS", help="refined vs plain preparation, output error on held-out rows")
    ap.add_argument("--fusion-ab", nargs="?", const="0,16,32,48,64,128", default=None, metavar="RANKS",
                    help="fused vs unfused timing at these ranks (comma-separated) instead of the metric")
    ap.add_argument("--w8a8", nargs="?", const=16, default=None, type=int, metavar="RANK",
                    help="8-bit setting against W4A4 at this rank (default 16) instead of the metric")
    ap.add_argument("--fp4", nargs="?", const=32, default=None, type=int, metavar="RANK",
                    help="NVFP4 setting against W4A4 at this rank (default 32) instead of the metric")
    args = ap.parse_args()

    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.workload, args.commands)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary, args.workload, args.commands)
        return
    if args.trace_summary:
        import workloads
        cfg = workloads.CONFIGS[args.workload]
        rank = (cfg.rank + cfg.lora_rank) if args.rank is None else args.rank
        if args.w8a8 is not None:
            rank = args.w8a8
        elif args.fp4 is not None:
            rank = args.fp4
        trace_summary(args.trace_summary, cfg, args, rank)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: only the one-GPU path exists (the layer would shard over "
              "token rows with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    if args.prep_refine is not None:
        prep_refine(args.prep_refine.split(","), args)
        return
    cfg = workloads.CONFIGS[args.workload]
    if args.fusion_ab is not None:
        fusion_ab(cfg, [int(v) for v in args.fusion_ab.split(",")], args)
        return
    if args.w8a8 is not None:
        w8a8_compare(cfg, args.w8a8, args)
        return
    if args.fp4 is not None:
        fp4_compare(cfg, args.fp4, args)
        return
    res = measure_layer(cfg, args, distinct_sets=True, steps=args.steps, warmup=args.warmup,
                        copy_check=args.copy_check)
    extra = {}
    if args.extra_configs:
        for name in [w for w in args.extra_configs.split(",") if w and w != cfg.name]:
            log(f"bench: extra configuration {name}")
            extra[name] = summarize_extra(measure_layer(workloads.CONFIGS[name], args, distinct_sets=False,
                                                        steps=args.extra_steps, warmup=args.warmup))
    line = headline(res, cfg, args)
    if extra:
        line["extra_configs"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res["inp"], cfg,
                                            min(args.cpu_rows, res["b"]) if args.cpu_rows else res["b"],
                                            args.cpu_threads)
    print(json.dumps(line), flush=True)


def measure_layer(cfg, args, distinct_sets, steps, warmup, copy_check=False):
    """Time one layer configuration through the C ABI (one step = the act
    kernel + its Z reduction, then the GEMM kernel), after the warm-up and the
    clock-settling steps.

    Cold: the steps rotate over enough input + weight sets to exceed the
    last-level cache.  With distinct_sets every set is drawn and prepared from
    its own seed; otherwise one prepared set is copied to fresh device buffers
    (the same values at other addresses: just as cold, a fraction of the
    preparation time).  Reported: wall time per step between synchronisations
    (mean), and per kernel the mean and median of HIP events recorded on the
    launch stream; the same on one set (warm); the low-rank overhead from
    rank-r and rank-0 steps interleaved on one set (median of HIP-event step
    times each, same codes and scales); and the one-call svdq_linear (warm)."""
    import torch
    import workloads
    import w4a4_rank_corrected_amd as S

    m, n = cfg.m, cfg.n
    rank_svd = cfg.rank if args.rank is None else args.rank
    dev = torch.device("cuda:0")
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32

    def build_set(seed):
        inp = workloads.make_inputs(cfg, seed=seed)
        x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        amax = S.svdq_calibrate_act_amax(x).cpu().numpy()   # calibration statistic on the GPU
        t0 = time.perf_counter()
        host = S.svdq_prepare_weights(inp["w"], amax, rank_svd)  # host preparation in the library
        prep = time.perf_counter() - t0
        if cfg.lora_rank and args.rank is None:
            l1p, l2p = S.svdq_append_lora(host["l1"], host["l2"], m, n, rank_svd, host["lambda"],
                                          inp["lora_a"], inp["lora_b"], inp["lora_scale"])
            host = dict(host, l1=l1p, l2=l2p, rank=rank_svd + cfg.lora_rank)
        layer = S.DeviceLayer(host, device=dev)
        y = torch.empty((x.shape[0], n), dtype=out_dtype, device=dev)
        return {"inp": inp, "x": x, "layer": layer, "y": y, "prep_s": prep}

    def copy_set(st):
        lay = st["layer"]
        c = lambda t: None if t is None else t.clone()
        layer = S.DeviceLayer.from_tensors(m, n, lay.rank, c(lay.qw), c(lay.wscale), c(lay.l1), c(lay.l2),
                                           c(lay.smooth_inv), c(lay.bias))
        return {"x": st["x"].clone(), "layer": layer, "y": torch.empty_like(st["y"]), "prep_s": st["prep_s"]}

    log(f"bench: workload {cfg.name} b={cfg.rows or cfg.b} m={m} n={n}")
    sets = [build_set(0)]
    b = sets[0]["x"].shape[0]
    r = int(sets[0]["layer"].rank)
    per_set, n_sets = set_plan(cfg, r, args.out)
    for s in range(1, n_sets):
        sets.append(build_set(s) if distinct_sets else copy_set(sets[0]))
        sets[-1].pop("inp", None)
    log(f"bench: {n_sets} input+weight sets of {per_set / 2**20:.0f} MiB "
        f"({'each drawn and prepared' if distinct_sets else 'copies of one prepared set'}), rank {r}, "
        f"host preparation {sets[0]['prep_s']:.1f} s per set")

    G = m // 64
    qx = torch.empty((G, b, 32), dtype=torch.uint8, device=dev)
    asc = torch.empty((G, b), dtype=torch.float16, device=dev)
    z = torch.empty((b, max(r, 1)), dtype=torch.float32, device=dev) if r else None
    ws = torch.empty(max(S.svdq_act_workspace_size(b, m, r), 1), dtype=torch.uint8, device=dev)
    gws = torch.empty(max(S.svdq_gemm_workspace_size(b, n, m), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # A step's first call on a (set, layer) pair goes through the binding,
    # which checks every tensor; later calls reuse the C-ABI arguments it was
    # given (the same tensors), so that the host's per-call checks do not pace
    # the short layers' steps.
    from w4a4_rank_corrected_amd import _binding as B
    marshalled = {}

    def marshal(st, layer):
        rr = layer.rank
        lib, P, sp = B.lib(), B._ptr, B._stream(stream)
        zp = P(z) if rr else None
        k1 = functools.partial(lib.svdq_quantize_act_lowrank_down, P(st["x"]), b, m, rr, B.SVDQ_GROUP,
                               P(layer.smooth_inv), P(layer.l1), P(qx), P(asc), zp, P(ws), ws.numel(), sp)
        k2 = functools.partial(lib.svdq_gemm_w4a4_lowrank_up, P(qx), P(asc), zp, ctypes.byref(layer.struct), b,
                               P(st["y"]), B._out_code(out_dtype), P(gws), gws.numel(), sp)
        return k1, k2, st, layer  # the set and layer stay referenced, so their ids are not reused

    def step(st, layer=None, marks=None):
        """One step; marks = (event after the act kernel, event after the
        GEMM), or None.  Two events per step: each record costs the stream
        about 3 us, so the act kernel's time is read from the previous step's
        last event (or the phase's start event) to this step's first."""
        layer = layer or st["layer"]
        rr = layer.rank
        calls = marshalled.get((id(st), id(layer)))
        if calls is None:
            S.svdq_quantize_act_lowrank_down(st["x"], layer.smooth_inv, layer.l1, rr, qx=qx, ascale=asc,
                                             z=z if rr else None, workspace=ws, stream=stream)
        else:
            B._check(calls[0]())
        if marks is not None:
            marks[0].record(stream)
        if calls is None:
            S.svdq_gemm_w4a4_lowrank_up(qx, asc, z if rr else None, layer, b, out_dtype, y=st["y"],
                                        workspace=gws, stream=stream)
            marshalled[(id(st), id(layer))] = marshal(st, layer)
        else:
            B._check(calls[1]())
        if marks is not None:
            marks[1].record(stream)

    l0 = sets[0]["layer"]
    # the same codes and scales without the low-rank branch
    layer0 = S.DeviceLayer.from_tensors(m, n, 0, l0.qw, l0.wscale, None, None, l0.smooth_inv, l0.bias)
    ws_lin = torch.empty(max(S.svdq_linear_workspace_size(b, m, n, r), 1), dtype=torch.uint8, device=dev)
    n_settle = 0 if args.no_settle else settle_steps(b, m, n)
    event = lambda: torch.cuda.Event(enable_timing=True)
    # a phase's events: one at its start, then two per step
    new_chain = lambda k: {"start": event(), "marks": [(event(), event()) for _ in range(k)]}
    # events only around the first and the last settling steps: thousands of
    # live timing events slow every later event record on the host
    n_probe = min(20, n_settle // 2)
    settle_a, settle_b = new_chain(n_probe), new_chain(n_probe)
    cold_ev, warm_ev, pair_ev = new_chain(steps), new_chain(steps), new_chain(2 * steps)

    def run(pick, chain, layer_of=None):
        """The chain's steps, issued without synchronising."""
        chain["start"].record(stream)
        for k, mk in enumerate(chain["marks"]):
            st = pick(k)
            step(st, layer_of(k) if layer_of else None, mk)

    def timed(pick, chain):
        """Steps bracketed by synchronize on both sides (wall ms per step, and
        the host's issue time per step); the events are read after every
        phase has run, so that the GPU does not idle (and lower its clock)
        between phases."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(pick, chain)
        t_issue = time.perf_counter()
        torch.cuda.synchronize()
        k = max(1, len(chain["marks"]))
        return (time.perf_counter() - t0) * 1e3 / k, (t_issue - t0) * 1e3 / k

    def times(chain):
        """Per step: (act kernel + Z reduction, GEMM, whole step) in ms."""
        ends = [chain["start"]] + [mk[1] for mk in chain["marks"]]
        return [(ends[k].elapsed_time(mid), mid.elapsed_time(end), ends[k].elapsed_time(end))
                for k, (mid, end) in enumerate(chain["marks"])]

    def kernel_stats(chain, walls):
        t = times(chain)
        k1, k2 = [v[0] for v in t], [v[1] for v in t]
        return {"wall": walls[0], "host_issue": walls[1],
                "k1_mean": float(np.mean(k1)), "k2_mean": float(np.mean(k2)),
                "k1_median": float(np.median(k1)), "k2_median": float(np.median(k2)),
                "step_median": float(np.median([v[2] for v in t]))}

    # warm-up over every set, the clock-settling steps, then the timed (cold,
    # rotating) region
    rotate = lambda k: sets[k % n_sets]
    for k in range(max(warmup, n_sets)):
        step(rotate(k))
    torch.cuda.synchronize()
    log(f"bench: {n_settle} clock-settling steps, then {steps} timed steps rotating over {n_sets} sets, warm "
        f"steps, rank-r and rank-0 steps interleaved, svdq_linear")
    if n_probe:
        run(rotate, settle_a)
    for k in range(n_probe, n_settle - n_probe):
        step(rotate(k))
    if n_probe:
        run(lambda k: rotate(n_settle - n_probe + k), settle_b)
    cold_wall = timed(rotate, cold_ev)
    warm_wall = timed(lambda k: sets[0], warm_ev)
    # rank-r and rank-0 steps alternate on one set (same clocks and cache state
    # for both)
    for _ in range(3):
        step(sets[0], layer0)
        step(sets[0])
    run(lambda k: sets[0], pair_ev, lambda k: layer0 if k % 2 else None)
    # the one-call entry point (K1 + K2 inside the library), warm
    for _ in range(3):
        S.svdq_linear(sets[0]["x"], l0, out_dtype, y=sets[0]["y"], workspace=ws_lin, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        S.svdq_linear(sets[0]["x"], l0, out_dtype, y=sets[0]["y"], workspace=ws_lin, stream=stream)
    torch.cuda.synchronize()
    linear_ms = (time.perf_counter() - t1) * 1e3 / steps

    cold = kernel_stats(cold_ev, cold_wall)
    warm = kernel_stats(warm_ev, warm_wall)
    tp = times(pair_ev)
    med = lambda i, parity: float(np.median([v[i] for k, v in enumerate(tp) if k % 2 == parity]))
    ov = {"ms_rank_r": med(2, 0), "ms_rank_0": med(2, 1),
          "k1_ms_rank_r": med(0, 0), "k2_ms_rank_r": med(1, 0),
          "k1_ms_rank_0": med(0, 1), "k2_ms_rank_0": med(1, 1)}
    settle = None
    if n_probe:
        first = float(np.median([v[1] for v in times(settle_a)]))
        last = float(np.median([v[1] for v in times(settle_b)]))
        settle = {"steps": n_settle,
                  "ms": round(settle_a["start"].elapsed_time(settle_b["marks"][-1][1]), 2),
                  f"gemm_ms_first_{n_probe}": round(first, 5), f"gemm_ms_last_{n_probe}": round(last, 5)}
        log(f"bench: settling took {settle['ms']:.0f} ms; GEMM median {first * 1e3:.1f} us over its first "
            f"{n_probe} steps, {last * 1e3:.1f} us over its last; timed {cold['k2_mean'] * 1e3:.1f} us")
    del settle_a, settle_b, cold_ev, warm_ev, pair_ev, marshalled

    if copy_check:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copy check of {COPY_BYTES} bytes done")
    return {"cfg": cfg, "b": b, "m": m, "n": n, "r": r, "n_sets": n_sets, "per_set": per_set,
            "cold": cold, "warm": warm, "overhead": ov, "linear_ms": linear_ms, "prep_s": sets[0]["prep_s"],
            "settle": settle,
            "schedule": S.svdq_gemm_schedule(b, n, m), "inp": sets[0].get("inp"),
            "distinct_sets": distinct_sets, "steps": steps}


def kernel_fractions(b, m, n, r, k1_ms, k2_ms):
    """Roofline fractions of the two kernels at the given mean durations: the
    GEMM against the i8 MFMA peak (2 b m n ops), against HBM (its algorithmic
    bytes) and against the fp32 FMA peak for its scale epilogue (2 FMAs per
    output element and channel group, 4 b n (m/64) flops; packed FP32 is not
    used, so the peak is 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz =
    78.6 TFLOP/s); the act kernel against HBM."""
    ops = 2.0 * b * m * n
    k1_bytes, k2_bytes = algorithmic_bytes(b, m, n, r)
    epi = 4.0 * b * n * (m // 64)
    return {"gemm_TOPs": ops / (k2_ms * 1e-3) / 1e12,
            "gemm_frac_i8_peak": ops / (k2_ms * 1e-3) / 1e12 / I8_PEAK_TOPS,
            "gemm_hbm_frac": k2_bytes / (k2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gemm_epilogue_fma_frac": epi / (k2_ms * 1e-3) / 1e12 / FP32_FMA_PEAK_TFLOPS,
            "act_hbm_frac": k1_bytes / (k1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gemm_algorithmic_bytes": k2_bytes, "act_algorithmic_bytes": k1_bytes}


def summarize_extra(res):
    """Compact record of one extra configuration (same method as the headline)."""
    b, m, n, r = res["b"], res["m"], res["n"], res["r"]
    c, ov = res["cold"], res["overhead"]
    f = kernel_fractions(b, m, n, r, c["k1_mean"], c["k2_mean"])
    return {"b": b, "m": m, "n": n, "rank": r,
            "value_TOPs": round(2.0 * b * m * n / (c["wall"] * 1e-3) / 1e12, 2),
            "ms_per_step": round(c["wall"], 5), "host_issue_ms_per_step": round(c["host_issue"], 5),
            "act_quant_down_ms": round(c["k1_mean"], 5), "gemm_w4a4_up_ms": round(c["k2_mean"], 5),
            "gemm_frac_i8_peak": round(f["gemm_frac_i8_peak"], 4), "gemm_hbm_frac": round(f["gemm_hbm_frac"], 4),
            "gemm_epilogue_fma_frac": round(f["gemm_epilogue_fma_frac"], 4),
            "act_hbm_frac": round(f["act_hbm_frac"], 4),
            "lowrank_overhead": round(ov["ms_rank_r"] / ov["ms_rank_0"] - 1.0, 4),
            "schedule": res["schedule"], "clock_settle": res["settle"],
            "timing": f"cold: {res['steps']} steps rotating over {res['n_sets']} copies of one prepared set"}


def headline(res, cfg, args):
    """The benchmark's JSON line for the main configuration."""
    b, m, n, r = res["b"], res["m"], res["n"], res["r"]
    c, w, ov = res["cold"], res["warm"], res["overhead"]
    ops = 2.0 * b * m * n
    value = ops / (c["wall"] * 1e-3) / 1e12
    f = kernel_fractions(b, m, n, r, c["k1_mean"], c["k2_mean"])
    traffic = load_traffic(cfg.name) if args.out == "bf16" and args.rank is None else None
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(c["wall"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "b": b, "m": m, "n": n, "rank": r, "group": 64,
                   "out": args.out, "parallelism": "none (1 GPU)",
                   "timing": f"cold: steps rotate over {res['n_sets']} seeded input+weight sets "
                             f"({res['n_sets'] * res['per_set'] / 2**20:.0f} MiB)"},
        "roofline": {"bound": "mfma", "achieved": round(f["gemm_TOPs"], 2), "peak": I8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(f["gemm_frac_i8_peak"], 4),
                     "traffic": None if traffic is None else round(traffic["traffic_bytes"])},
        "kernels": {"act_quant_down_ms": round(c["k1_mean"], 5), "gemm_w4a4_up_ms": round(c["k2_mean"], 5),
                    "host_issue_ms_per_step": round(c["host_issue"], 5),
                    "act_quant_down_median_ms": round(c["k1_median"], 5),
                    "gemm_w4a4_up_median_ms": round(c["k2_median"], 5),
                    "act_quant_down_GBs": round(f["act_algorithmic_bytes"] / (c["k1_mean"] * 1e-3) / 1e9, 1),
                    "act_quant_down_hbm_frac": round(f["act_hbm_frac"], 4),
                    "gemm_w4a4_up_TOPs": round(f["gemm_TOPs"], 2),
                    "gemm_hbm_frac": round(f["gemm_hbm_frac"], 4),
                    "gemm_epilogue_fma_frac": round(f["gemm_epilogue_fma_frac"], 4),
                    "gemm_algorithmic_bytes": f["gemm_algorithmic_bytes"],
                    "act_algorithmic_bytes": f["act_algorithmic_bytes"],
                    "gemm_hbm_fetch_bytes": None if traffic is None else round(traffic["fetch_bytes"]),
                    "gemm_hbm_write_bytes": None if traffic is None else round(traffic["write_bytes"]),
                    "gemm_schedule": res["schedule"]},
        "warm": {"ms_per_step": round(w["wall"], 5), "value": round(ops / (w["wall"] * 1e-3) / 1e12, 2),
                 "act_quant_down_ms": round(w["k1_median"], 5), "gemm_w4a4_up_ms": round(w["k2_median"], 5),
                 "svdq_linear_ms": round(res["linear_ms"], 5)},
        "lowrank_overhead": {"rank": r, "ms_rank_r": round(ov["ms_rank_r"], 5), "ms_rank_0": round(ov["ms_rank_0"], 5),
                             "overhead": round(ov["ms_rank_r"] / ov["ms_rank_0"] - 1.0, 4),
                             "k1_ms_rank_r": round(ov["k1_ms_rank_r"], 5), "k2_ms_rank_r": round(ov["k2_ms_rank_r"], 5),
                             "k1_ms_rank_0": round(ov["k1_ms_rank_0"], 5), "k2_ms_rank_0": round(ov["k2_ms_rank_0"], 5),
                             "method": "rank-r and rank-0 steps interleaved on one set (warm), "
                                       "median of HIP-event step times"},
        "clock_settle": res["settle"],
        "prep_s": round(res["prep_s"], 2),
    }


if __name__ == "__main__":
    main()
