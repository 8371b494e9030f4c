"""CPU tests of bench.py's host logic: the single-GPU guard, the workload
plan, the algorithmic byte counts, and the profile summarisers on synthetic
rocprofv3 counter files (no GPU, no oracle)."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_source_hash_covers_the_gemm_sources():
    h = bench.gemm_source_hash()
    assert len(h) == 64 and all(os.path.exists(os.path.join(ROOT, r)) for r in bench.GEMM_SOURCES)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cold_plan_rotates_more_than_the_last_level_cache():
    for name in ("flux_qkv", "flux_fc2", "pixart_fc1", "flux_single_fc_b256"):
        cfg = workloads.CONFIGS[name]
        per_set, n_sets = bench.set_plan(cfg, cfg.rank, "bf16")
        assert n_sets >= 3 and per_set * n_sets >= bench.COLD_BYTES


def test_settle_steps_depend_on_the_shape_only():
    # about 0.25 s of work at 1 POP/s, clamped to [50, 5000]
    assert bench.settle_steps(4608, 3072, 9216) == 959
    assert bench.settle_steps(64, 256, 256) == 5000
    assert bench.settle_steps(10**6, 10**4, 10**4) == 50
    for name in ("flux_qkv", "flux_fc2", "pixart_fc1", "flux_single_fc_b256", "flux_single_out_b256"):
        cfg = workloads.CONFIGS[name]
        k = bench.settle_steps(cfg.rows or cfg.b, cfg.m, cfg.n)
        assert k == bench.settle_steps(cfg.rows or cfg.b, cfg.m, cfg.n)
        assert 50 <= k <= 5000
        assert k == 5000 or k * 2.0 * (cfg.rows or cfg.b) * cfg.m * cfg.n >= bench.SETTLE_OPS


def test_algorithmic_bytes_flux_qkv():
    b, m, n, r = 4608, 3072, 9216, 32
    k1, k2 = bench.algorithmic_bytes(b, m, n, r)
    G = m // 64
    # K1: x in, codes and scales out, Z out, L1 and 1/lambda in
    assert k1 == 2 * b * m + b * m // 2 + 2 * b * G + 4 * b * r + 2 * m * r + 4 * m
    # K2: codes and scales of both operands, Z, L2 in; Y (bf16) out
    assert k2 == b * m // 2 + 2 * b * G + 4 * b * r + m * n // 2 + 2 * G * n + 2 * n * r + 2 * b * n
    assert 100e6 < k2 < 120e6


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(disp, kernel, counter, value, t0=0, t1=1000):
    return {"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value,
            "Start_Timestamp": t0, "End_Timestamp": t1}


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_traffic_summary_scales_by_the_copy(fake_root, monkeypatch):
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "sources-hash")
    copy = "__amd_rocclr_copyBuffer"
    gemm = "void svdq::(anonymous namespace)::gemm_w4a4_up_kernel<GemmCfg<128>, true>(...)"
    # the copy of COPY_BYTES reads half its bytes on FETCH_SIZE and all on WRITE_SIZE (KiB)
    half = bench.COPY_BYTES / 2 / 1024
    full = bench.COPY_BYTES / 1024
    fd, wd = str(fake_root / "f"), str(fake_root / "w")
    _write_counters(fd, [_row(1, copy, "FETCH_SIZE", half)] +
                    [_row(2 + k, gemm, "FETCH_SIZE", 1000.0 + k) for k in range(3)])
    _write_counters(wd, [_row(1, copy, "WRITE_SIZE", full)] + [_row(2 + k, gemm, "WRITE_SIZE", 500.0) for k in range(3)])
    bench.traffic_summary(fd, wd, "flux_qkv", "cmd")
    out = json.load(open(fake_root / "profiles" / f"hbm_traffic_{bench.GEMM_KERNEL}_flux_qkv.json"))
    assert out["fetch_factor"] == pytest.approx(2.0) and out["write_factor"] == pytest.approx(1.0)
    assert out["fetch_bytes"] == pytest.approx(1001.0 * 1024 * 2)   # median of 1000, 1001, 1002
    assert out["write_bytes"] == pytest.approx(500.0 * 1024)
    assert out["source_sha256"] == "sources-hash"


def test_counter_summary_utilisation_and_bandwidth(fake_root):
    copy = "__amd_rocclr_copyBuffer"
    gemm = "void svdq::(anonymous namespace)::gemm_w4a4_up_kernel<GemmCfg<128>, true>(...)"
    act = "void svdq::(anonymous namespace)::act_quant_down_kernel<2, true, 1>(...)"
    dur_ns = 100_000                      # 100 us
    cyc = 100e-6 * bench.PEAK_CLOCK_GHZ * 1e9
    sq = []
    for k, name in enumerate((gemm, act)):
        d = 10 + k
        sq += [_row(d, name, "GRBM_GUI_ACTIVE", 8 * cyc, 0, dur_ns),
               _row(d, name, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * cyc, 0, dur_ns),   # 25 % busy
               _row(d, name, "SQ_INSTS_VALU", 0.5 * 1024 * cyc / 4, 0, dur_ns),          # 50 % issue
               _row(d, name, "SQ_INSTS_LDS", 100.0, 0, dur_ns), _row(d, name, "SQ_LDS_BANK_CONFLICT", 50.0, 0, dur_ns)]
    half = bench.COPY_BYTES / 2 / 1024
    fd, wd, sd = str(fake_root / "f"), str(fake_root / "w"), str(fake_root / "s")
    _write_counters(sd, sq)
    _write_counters(fd, [_row(1, copy, "FETCH_SIZE", half)] +
                    [_row(10 + k, nm, "FETCH_SIZE", 400e6 / 2 / 1024, 0, dur_ns) for k, nm in enumerate((gemm, act))])
    _write_counters(wd, [_row(1, copy, "WRITE_SIZE", 2 * half)] +
                    [_row(10 + k, nm, "WRITE_SIZE", 400e6 / 1024, 0, dur_ns) for k, nm in enumerate((gemm, act))])
    bench.counter_summary(sd, fd, wd, "flux_qkv", "cmd")
    text = open(fake_root / "profiles" / "counters_flux_qkv.md").read()
    line = [l for l in text.splitlines() if l.startswith("| GEMM")][0].split("|")
    assert line[4].strip() == "2.40"                      # clock from GRBM_GUI_ACTIVE / 8
    assert line[5].strip() == "25.0 %" and line[6].strip() == "0.125" and line[7].strip() == "0.50"
    # 400 MB fetched + 400 MB written in 100 us = 8000 GB/s = 100 % of peak
    assert line[10].strip() == "8000" and line[11].strip() == "100.0 %"


def _write_trace(d, dispatches):
    """A rocpd-like database with the columns trace_summary reads: one row per
    (name, start, end) dispatch, ns timestamps."""
    import sqlite3
    os.makedirs(d, exist_ok=True)
    c = sqlite3.connect(os.path.join(d, "run_results.db"))
    c.execute("create table kernels (name text, start integer, end integer, grid_x integer, grid_y integer, "
              "workgroup_x integer, workgroup_y integer, vgpr_count integer, accum_vgpr_count integer, "
              "lds_size integer, scratch_size integer)")
    c.executemany("insert into kernels values (?, ?, ?, 256, 1, 256, 1, 128, 0, 0, 0)", dispatches)
    c.commit()
    c.close()


@pytest.mark.parametrize("no_settle", [False, True])
def test_trace_summary_takes_the_timed_steps(fake_root, no_settle):
    # the GEMM's dispatches: warm-up and settling steps (1 us), the timed steps
    # (2 us), then the later phases (5 us); the summary's timed-region mean
    # must be exactly the timed steps'
    cfg = workloads.CONFIGS["flux_qkv"]
    args = type("A", (), dict(steps=7, warmup=10, out="bf16", w8a8=None, fp4=None, no_settle=no_settle,
                              rank=None))()
    _, n_sets = bench.set_plan(cfg, cfg.rank, "bf16")
    skip = max(args.warmup, n_sets) + (0 if no_settle else bench.settle_steps(cfg.b, cfg.m, cfg.n))
    gemm = "void svdq::(anonymous namespace)::gemm_w4a4_up_kernel<GemmCfg<128>, true, false>(...)"
    durs = [1000] * skip + [2000] * args.steps + [5000] * 40
    t, rows = 0, []
    for d in durs:
        rows.append((gemm, t, t + d))
        t += d + 100
    pd = str(fake_root / "prof")
    _write_trace(pd, rows)
    bench.trace_summary(pd, cfg, args, cfg.rank)
    text = open(fake_root / "profiles" / "kernel_trace_flux_qkv.md").read()
    line = [l for l in text.splitlines() if "gemm_w4a4_up_kernel" in l][0].split("|")
    assert line[2].strip() == str(len(durs))
    assert line[3].strip() == "2.00"
    assert f"after {skip} untimed ones" in text
