#!/usr/bin/env python3
"""FP32 SGEMM benchmark on one MI355X: TFLOPS = 2MNK/t at NN 4096^3.

One step is one mi_sgemm call on the headline workload (row-major NN,
M = N = K = 4096, alpha = 1, beta = 0, A and B uniform [-1, 1) from
srand48(4)); inputs are resident in HBM before timing starts. The FLOP
count 2MNK is the convention of the klklkl10086.github.io SGEMM page
(problem definition), where 4096^3 is 137.4 GFLOP.

Before the warm-up steps, back-to-back calls run for --preheat seconds
(default 1): the GPU raises its shader clock over the first ~20 ms of load
and drops it again after about a second idle, so without this the timed
steps would measure the ramp. The preheat is reported in its own field.

Prints one JSON line. Besides the contract fields it carries
  preheat       calls and seconds of the preheat;
  per_call_us   median, min, p90, max, first and last of the timed steps, each
                step bracketed by its own HIP events;
  roofline      the SGEMM kernel against the FP32 matrix-core peak, with the
                average launch time measured by HIP events on the launch stream,
                and HBM traffic from the committed rocprofv3 counter summary
                when that summary was taken on the current kernel source;
  clock         the shader clock sustained under full FP32 matrix load
                (mi_clock_probe, run right after the timed steps), the
                matrix rate the probe reached, and the fraction of the peak
                at that clock;
  check         the headline C at 4,096 seeded positions against the CPU
                oracle (max |GPU - oracle| <= 1e-3; the run fails otherwise);
  configs       every workload family (the ragged, 1024^3, square sweep,
                layer-shaped and skinny products), each preheated, timed
                back to back (and one call at a time from 20 us up), and
                checked at sampled positions against the oracle;
  cpu_baseline  the CPU oracle timed on this host on a bounded sample.

Other modes: --table writes per-workload TFLOPS (and GB/s for the skinny
product) to a JSON-lines file; --mode copy runs a plain device copy of known
size, used to calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import struct
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGEMM TFLOPS (2MNK/t) at 4096^3 and % of MI355X FP32 matrix peak"
PEAK_FP32_MATRIX_TFLOPS = 157.3      # 256 CU x 2.4 GHz x 256 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sgemm_nn_4096.json")
COPY_BYTES = 256 << 20


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def tflops(flops: float, seconds: float) -> float:
    return flops / seconds / 1e12


def kernel_code_hash(symbol):
    """sha256 of one kernel's gfx950 machine code in the built library, or
    None when the library or the kernel is missing."""
    import fp32_gemm_nn_amd as mg
    from fp32_gemm_nn_amd import codeobj

    try:
        return codeobj.kernel_code_sha256(mg.library_path, symbol)
    except (OSError, KeyError, ValueError, struct.error):
        return None


def load_traffic(launch_flops_case):
    """HBM bytes per launch from the committed counter summary, or None if it
    is missing, is for another workload, or was taken on a kernel whose machine
    code differs from the built one (the counters measure that code alone)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != launch_flops_case or not t.get("kernel_symbol"):
        return None
    code = kernel_code_hash(t["kernel_symbol"])
    if code is None or t.get("kernel_code_sha256") != code:
        return None
    return t.get("hbm_bytes_per_launch")


class Problem:
    """Device buffers for one workload, optionally several independent copies."""

    def __init__(self, case, copies=1):
        import torch
        from synthetic import workloads as W

        self.case = case
        inp = W.make_inputs(case)
        self.inp = inp                      # host copy (the oracle's input)
        self.sets = []
        for i in range(copies):
            A = torch.from_numpy(inp.A).cuda()
            B = torch.from_numpy(inp.B).cuda()
            C = torch.from_numpy(inp.C.copy()).cuda()
            self.sets.append((A, B, C))
        torch.cuda.synchronize()

    def call(self, i=0, stream=None, config=None):
        import fp32_gemm_nn_amd as mg

        c = self.case
        A, B, C = self.sets[i % len(self.sets)]
        args = (c.transA, c.transB, c.M, c.N, c.K, c.alpha, A.data_ptr(), c.lda_,
                B.data_ptr(), c.ldb_, c.beta, C.data_ptr(), c.ldc_, stream)
        rc = mg.mi_sgemm(*args) if config is None else mg.mi_sgemm_with_config(config, *args)
        if rc != 0:
            raise RuntimeError(f"mi_sgemm: {mg.mi_sgemm_status_string(rc)}")


def preheat(prob, seconds, config=None):
    """Back-to-back calls for `seconds` of wall time (at least one batch of
    about 10 ms), so that the shader clock has ramped before anything is timed.
    Returns the call count and the time spent."""
    import torch

    handle = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    calls, batch = 0, 4
    while True:
        tb = time.perf_counter()
        for i in range(batch):
            prob.call(calls + i, handle, config)
        torch.cuda.synchronize()
        calls += batch
        dt = time.perf_counter() - tb
        if time.perf_counter() - t0 >= seconds:
            break
        batch = max(1, min(2000, int(batch * 0.01 / max(dt, 1e-6))))
    return {"calls": calls, "seconds": round(time.perf_counter() - t0, 3)}


def time_steps(prob, steps, warmup, config=None):
    """`warmup` untimed calls, then exactly `steps` calls bracketed by
    synchronisations, with a HIP event on the launch stream before the first
    call and after each one. Returns the wall time, the event time from the
    first event to the last (seconds) and each step's event time (us)."""
    import torch

    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    for i in range(warmup):
        prob.call(i, handle, config)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        prob.call(i, handle, config)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]
    return wall, ev[0].elapsed_time(ev[steps]) / 1e3, per


def spread(per_us):
    """Median, min, 90th percentile, max, first and last of per-call times."""
    t = sorted(per_us)
    return {"median": round(t[len(t) // 2], 2), "min": round(t[0], 2), "p90": round(t[(len(t) * 9) // 10], 2),
            "max": round(t[-1], 2), "first": round(per_us[0], 2), "last": round(per_us[-1], 2)}


def time_problem(prob, steps, warmup, config=None):
    """Wall time and HIP-event time of `steps` back-to-back calls on one stream."""
    import torch

    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    for i in range(warmup):
        prob.call(i, handle, config)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        prob.call(i, handle, config)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / 1e3


def per_call_stats(prob, calls, config=None):
    """Median, minimum and 90th percentile of `calls` single-call HIP-event
    timings (microseconds), each call bracketed by its own event pair."""
    import torch

    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        prob.call(i, handle, config)
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    return {"median_us": round(t[len(t) // 2], 3), "min_us": round(t[0], 3), "p90_us": round(t[(len(t) * 9) // 10], 3)}


def cpu_baseline_seconds(case, inp):
    """CPU baseline for one workload: wall time of one product of the CPU
    oracle, as it stands, on the workload's inputs."""
    import oracle

    C = inp.C.copy()
    t0 = time.perf_counter()
    rc = oracle.sgemm(case.transA, case.transB, case.M, case.N, case.K, case.alpha, inp.A, case.lda_,
                      inp.B, case.ldb_, case.beta, C, case.ldc_)
    dt = time.perf_counter() - t0
    if rc != 0:
        raise RuntimeError(f"oracle: status {rc}")
    return dt


def cpu_baseline(case, min_seconds=10.0, max_seconds=30.0):
    """Time the CPU oracle (as it stands) on the headline product.

    The sample is whole products of the headline workload, repeated until at
    least `min_seconds` have passed; if one product would exceed `max_seconds`
    (estimated from a 64-row slice), a leading block of rows is used instead.
    """
    import numpy as np

    import oracle
    from synthetic import workloads as W

    inp = W.make_inputs(case)
    threads = oracle.num_threads()
    # Estimate from a small slice of rows.
    rows = 64
    C = np.zeros((rows, case.N), np.float32)
    t0 = time.perf_counter()
    oracle.sgemm(case.transA, case.transB, rows, case.N, case.K, case.alpha, inp.A, case.lda_, inp.B,
                 case.ldb_, case.beta, C, case.ldc_)
    est_full = (time.perf_counter() - t0) * case.M / rows
    if est_full > max_seconds:
        rows = max(64, int(case.M * max_seconds / est_full / 2))
    else:
        rows = case.M
    C = np.zeros((rows, case.N), np.float32)
    reps, spent = 0, 0.0
    while spent < min_seconds and (reps == 0 or spent + spent / reps <= max_seconds):
        t0 = time.perf_counter()
        rc = oracle.sgemm(case.transA, case.transB, rows, case.N, case.K, case.alpha, inp.A, case.lda_,
                          inp.B, case.ldb_, case.beta, C, case.ldc_)
        spent += time.perf_counter() - t0
        assert rc == 0
        reps += 1
    flops = gemm_flops(rows, case.N, case.K) * reps
    sample = (f"{reps} x full {case.M}x{case.N}x{case.K} {case.transA}{case.transB} product"
              if rows == case.M else
              f"{reps} x first {rows} rows of the {case.M}x{case.N}x{case.K} {case.transA}{case.transB} product")
    return {"value": round(tflops(flops, spent), 6), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds": round(spent, 2)}


CHECK_TOL = 1e-3


def check_sampled(prob, samples, seed, reset=True):
    """The result of one call against the CPU oracle at `samples` seeded
    positions (the four corners among them): max |GPU - oracle|. With `reset`
    C is first restored to C_in and one call is made, so a C that repeated
    timing calls have drifted (beta != 0) is not what is checked."""
    import numpy as np
    import torch

    import oracle

    case, inp = prob.case, prob.inp
    A, B, C = prob.sets[0]
    if reset:
        C.copy_(torch.from_numpy(inp.C))
        torch.cuda.synchronize()
        prob.call(0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got_all = C.cpu().numpy()
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, 0, case.M - 1, case.M - 1], rng.integers(0, case.M, samples - 4)]).astype(np.int32)
    cols = np.concatenate([[0, case.N - 1, 0, case.N - 1], rng.integers(0, case.N, samples - 4)]).astype(np.int32)
    c_in = inp.C[rows, cols] if case.beta != 0.0 else None
    want = oracle.sgemm_entries(case.transA, case.transB, case.M, case.N, case.K, case.alpha, inp.A, case.lda_,
                                inp.B, case.ldb_, case.beta, c_in, rows, cols)
    got = got_all[rows, cols]
    finite = bool(np.all(np.isfinite(got)))
    err = float(np.abs(got.astype(np.float64) - want.astype(np.float64)).max())
    return {"samples": int(samples), "max_abs_err": err, "tol": CHECK_TOL, "pass": finite and err <= CHECK_TOL}


PROBE_ITERS = 100_000     # about 20 ms per launch at 2.4 GHz
PROBE_WORKGROUPS, PROBE_WAVES = 256, 8


def clock_probe():
    """Shader clock under full FP32 matrix load (mi_clock_probe): three
    back-to-back launches, the last one read. Returns the median shader clock
    over the workgroups, the matrix rate the probe reached (FLOPs over the
    longest wall span) and the FP32 matrix peak at the measured clock."""
    import torch

    import fp32_gemm_nn_amd as mg

    stamps = torch.zeros(4 * PROBE_WORKGROUPS, dtype=torch.int64, device="cuda")
    handle = torch.cuda.current_stream().cuda_stream
    khz = 0
    for _ in range(3):
        rc, khz = mg.mi_clock_probe(PROBE_ITERS, stamps.data_ptr(), handle)
        if rc != 0:
            raise RuntimeError(f"mi_clock_probe: {mg.mi_sgemm_status_string(rc)}")
    torch.cuda.synchronize()
    st = stamps.cpu().tolist()
    clk = [st[4 * w + 1] - st[4 * w] for w in range(PROBE_WORKGROUPS)]
    wall = [st[4 * w + 3] - st[4 * w + 2] for w in range(PROBE_WORKGROUPS)]
    mhz = sorted(c / w * khz / 1e3 for c, w in zip(clk, wall) if w > 0)
    sclk = mhz[len(mhz) // 2]
    flops = PROBE_WORKGROUPS * PROBE_WAVES * PROBE_ITERS * 4 * 4096
    probe_tflops = flops / (max(wall) / (khz * 1e3)) / 1e12
    peak_at_sclk = 256 * 256 * sclk * 1e6 / 1e12
    return {"sclk_mhz": round(sclk, 1), "sclk_mhz_min": round(mhz[0], 1), "sclk_mhz_max": round(mhz[-1], 1),
            "wall_clock_khz": khz, "probe_tflops": round(probe_tflops, 2),
            "peak_at_sclk_tflops": round(peak_at_sclk, 2),
            "source": "mi_clock_probe: 256 workgroups x 8 waves of register-only FP32 MFMA, after the timed steps"}


def time_case(case, copies=1, preheat_s=0.1, check_samples=512, seed=0):
    """One workload with its chosen kernel: preheated, then timed as five
    batches of back-to-back calls (each batch at least 2 ms, one HIP event
    pair around it); `us` is the median of the five batch means, the time per
    call at full throughput, as the headline's roofline time is. Calls of 20 us
    or more are also timed one by one (`per_call_us`: an event pair around each
    call, which adds the dispatch gap between calls). Then one call on a fresh
    C is checked against the oracle at sampled positions."""
    import torch

    import fp32_gemm_nn_amd as mg

    prob = Problem(case, copies=copies)
    ph = preheat(prob, preheat_s)
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    est = ph["seconds"] / max(ph["calls"], 1)
    reps = max(5, min(2000, int(2e-3 / max(est, 1e-7))))
    means = []
    for b in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            prob.call(b * reps + i, handle)
        e1.record(stream)
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) * 1e3 / reps)
    us = sorted(means)[2]
    tf = tflops(case.flops, us * 1e-6)
    row = {"workload": case.name, "ops": case.transA + case.transB, "M": case.M, "N": case.N, "K": case.K,
           "alpha": case.alpha, "beta": case.beta,
           "kernel_config": mg.mi_sgemm_config_name(
               mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)),
           "us": round(us, 2), "calls_per_batch": reps, "TFLOPS": round(tf, 2),
           "pct_fp32_matrix_peak": round(100 * tf / PEAK_FP32_MATRIX_TFLOPS, 2)}
    if us >= 20:
        _, _, per = time_steps(prob, max(20, min(200, int(0.05 / (us * 1e-6)))), 2)
        row["per_call_us"] = spread(per)
    if case.M <= 32:
        gbps = case.algorithmic_bytes / (us * 1e-6) / 1e9
        row.update({"GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                    "operand_sets": copies})
    chk = check_sampled(prob, check_samples, seed)
    row["check_max_abs_err"] = chk["max_abs_err"]
    row["check_pass"] = chk["pass"]
    del prob
    return row


def run_configs():
    """Every workload family of the benchmark, in the order C1, C2, the square
    sweep, the layer-shaped products, the skinny product (cold: eight operand
    sets, more than the 256 MB last-level cache; warm: one)."""
    from synthetic import workloads as W

    out = {"C1": time_case(W.C1, seed=1), "C2": time_case(W.C2, seed=2),
           "C3": [time_case(W.c3(n), seed=3) for n in W.C3_SIZES],
           "C5a": [time_case(c, seed=5) for c in W.C5A]}
    cold = time_case(W.C5B, copies=8, seed=6)
    warm = time_case(W.C5B, copies=1, seed=7)
    out["C5b"] = {"cold": cold, "warm": warm}
    return out


def host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0))}


def run_copy(steps, warmup):
    """A plain device copy of COPY_BYTES per launch (counter calibration)."""
    import torch

    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": COPY_BYTES, "bytes_written_per_launch": COPY_BYTES,
                      "steps": steps, "GBps": round(2 * COPY_BYTES * steps / dt / 1e9, 1)}))


def run_table(path, steps, warmup):
    """Every workload with the kernel select_config picks for it, one JSON
    object per line: mean time per call and TFLOP/s; per-call median, minimum
    and 90th percentile for calls of 20 us or more; for the skinny shapes, HBM
    rates cold (eight rotating operand sets) and warm (one set); and the CPU
    baseline (one oracle product) with the GPU's speed-up over it."""
    import fp32_gemm_nn_amd as mg
    from synthetic import workloads as W

    cases = [W.C1, W.C2, *[W.c3(n) for n in W.C3_SIZES], W.C4, *W.C5A, W.C5B, *W.SHARD8]
    with open(path, "w") as out:
        for case in cases:
            skinny = case.M <= 32
            # The skinny product streams 64 MiB of B; rotate 8 independent
            # operand sets (> 512 MiB) so repeated calls do not hit in the
            # 256 MB last-level cache.
            prob = Problem(case, copies=8 if skinny else 1)
            n = max(steps, int(2e-1 / max(case.flops / 100e12, 1e-6))) if not skinny else max(steps, 200)
            n = min(n, 2000)
            _, ev = time_problem(prob, n, warmup)
            per = ev / n
            row = {"workload": case.name, "transA": case.transA, "transB": case.transB, "M": case.M,
                   "N": case.N, "K": case.K, "alpha": case.alpha, "beta": case.beta,
                   "kernel_config": mg.mi_sgemm_config_name(
                       mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)),
                   "us_per_call": round(per * 1e6, 3), "TFLOPS": round(tflops(case.flops, per), 3),
                   "pct_fp32_matrix_peak": round(100 * tflops(case.flops, per) / PEAK_FP32_MATRIX_TFLOPS, 2),
                   "GBps_algorithmic": round(case.algorithmic_bytes / per / 1e9, 1)}
            if skinny:
                row["pct_hbm_peak"] = round(100 * case.algorithmic_bytes / per / 1e9 / PEAK_HBM_GBPS, 2)
                # Warm: one operand set, so B stays in the 256 MB last-level cache.
                warm = Problem(case)
                _, evw = time_problem(warm, n, warmup)
                row["us_per_call_warm"] = round(evw / n * 1e6, 3)
                row["pct_hbm_peak_warm"] = round(100 * case.algorithmic_bytes / (evw / n) / 1e9 / PEAK_HBM_GBPS, 2)
                del warm
            if per >= 20e-6:
                row["per_call"] = per_call_stats(prob, min(n, 200))
            t_cpu = cpu_baseline_seconds(case, prob.inp)
            row["cpu_baseline_s"] = round(t_cpu, 4)
            row["cpu_baseline_gflops"] = round(case.flops / t_cpu / 1e9, 2)
            row["gpu_speedup_vs_cpu_baseline"] = round(t_cpu / per, 1)
            out.write(json.dumps(row) + "\n")
            out.flush()
            print(json.dumps(row), file=sys.stderr, flush=True)
            del prob


def run_workload(name, steps, warmup, configs=None, preheat_s=0.0):
    """One workload with its chosen kernel, or with each of `configs` (names
    or ids) forced: one JSON line of numbers per kernel, each kernel preheated
    for `preheat_s` seconds first."""
    import fp32_gemm_nn_amd as mg
    from synthetic import workloads as W

    cases = {c.name: c for c in [*W.all_cases(), *W.SHARD8]}
    if name not in cases:
        raise SystemExit(f"unknown workload {name!r}; one of: {', '.join(sorted(cases))}")
    case = cases[name]
    skinny = case.M <= 32
    prob = Problem(case, copies=8 if skinny else 1)
    names = mg.config_names()
    chosen = mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)
    ids = [None] if not configs else [int(c) if str(c).isdigit() else names.index(c) for c in configs]
    for cfg in ids:
        if preheat_s > 0:
            preheat(prob, preheat_s, config=cfg)
        _, ev = time_problem(prob, steps, warmup, config=cfg)
        per = ev / steps
        row = {"workload": case.name, "transA": case.transA, "transB": case.transB, "M": case.M, "N": case.N,
               "K": case.K, "kernel_config": names[chosen if cfg is None else cfg],
               "chosen": cfg is None or cfg == chosen,
               "steps": steps, "us_per_call": round(per * 1e6, 3), "TFLOPS": round(tflops(case.flops, per), 3),
               "pct_fp32_matrix_peak": round(100 * tflops(case.flops, per) / PEAK_FP32_MATRIX_TFLOPS, 2),
               "GBps_algorithmic": round(case.algorithmic_bytes / per / 1e9, 1)}
        if skinny:
            row["pct_hbm_peak"] = round(100 * case.algorithmic_bytes / per / 1e9 / PEAK_HBM_GBPS, 2)
        print(json.dumps(row), flush=True)


PEAK_FP32_VECTOR_TFLOPS = 157.3    # FP32 vector FMA: 256 CU x 2.4 GHz x 256 FLOP/clk/CU


def run_ladder(path, sizes=(1024, 4096)):
    """The vector-ALU technique ladder (configs named valu_*), rung by rung,
    beside the matrix-core path mi_sgemm picks, on square NN products with
    alpha = 1, beta = 0: per-call time, TFLOP/s, fraction of the unpacked FP32
    vector peak, and speed relative to the matrix-core path. One JSON object
    per line."""
    import fp32_gemm_nn_amd as mg
    from synthetic import workloads as W

    names = mg.config_names()
    ladder = [i for i, n in enumerate(names) if n.startswith("valu_")]
    with open(path, "w") as out:
        for n in sizes:
            case = W.Case(f"nn_{n}", "N", "N", n, n, n, 1.0, 0.0, seed=2)
            prob = Problem(case)
            rows = []
            for cfg in [None, *ladder]:
                _, first = time_problem(prob, 1, 1, config=cfg)
                calls = max(3, min(2000, int(0.2 / max(first, 1e-6))))
                _, ev = time_problem(prob, calls, 1, config=cfg)
                per = ev / calls
                chosen = mg.mi_sgemm_select_config("N", "N", n, n, n)
                rows.append({"workload": case.name, "M": n, "N": n, "K": n,
                             "kernel_config": names[chosen] if cfg is None else names[cfg],
                             "unit": "matrix cores" if cfg is None else "vector ALUs",
                             "calls": calls, "us_per_call": round(per * 1e6, 3),
                             "TFLOPS": round(tflops(case.flops, per), 3)})
            mfma_us = rows[0]["us_per_call"]
            for row in rows:
                row["pct_fp32_vector_peak"] = round(100 * row["TFLOPS"] / PEAK_FP32_VECTOR_TFLOPS, 2)
                row["pct_fp32_matrix_peak"] = round(100 * row["TFLOPS"] / PEAK_FP32_MATRIX_TFLOPS, 2)
                row["speed_vs_matrix_path"] = round(mfma_us / row["us_per_call"], 4)
                out.write(json.dumps(row) + "\n")
                out.flush()
                print(json.dumps(row), file=sys.stderr, flush=True)
            del prob


def run_config_sweep(path, warmup=3):
    """Every kernel configuration on every workload (one JSON object per line):
    the data the shape-class rule in select_config is chosen from."""
    import fp32_gemm_nn_amd as mg
    from synthetic import workloads as W

    cases = [W.C1, W.C2, *[W.c3(n) for n in W.C3_SIZES], W.C4, *W.C5A, W.C5B]
    names = mg.config_names()
    with open(path, "w") as out:
        for case in cases:
            skinny = case is W.C5B
            prob = Problem(case, copies=8 if skinny else 1)
            chosen = mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)
            for cfg, name in enumerate(names):
                if "skinny" in name and case.M > 64:
                    continue
                n = 200 if skinny else max(10, min(2000, int(2e-1 / max(case.flops / 100e12, 1e-6))))
                _, ev = time_problem(prob, n, warmup, config=cfg)
                per = ev / n
                row = {"workload": case.name, "config": name, "chosen": cfg == chosen,
                       "us_per_call": round(per * 1e6, 3), "TFLOPS": round(tflops(case.flops, per), 3)}
                out.write(json.dumps(row) + "\n")
                out.flush()
            del prob


def run_regret(path, shapes=90, seed=11, warmup=3, ragged=False):
    """Selection check on random shapes: M and N drawn from 768..4096, K from
    256..4096 (with ragged: M, N, K uniform over the multiples of 4 in
    512..4096), op pairs at random (seeded). Every matrix-core tile configuration
    is timed on each shape (best of two runs of back-to-back calls after 25 ms
    of warm-up calls, beta = 0)
    and select_config's pick is scored by its regret against the fastest. One
    JSON object per shape, then a summary line."""
    import random

    import torch

    import fp32_gemm_nn_amd as mg

    names = mg.config_names()
    tile_cfgs = [i for i, n in enumerate(names) if n.startswith("mfma")]
    rng = random.Random(seed)
    dims = [768, 1024, 1152, 1280, 1536, 1792, 2048, 2304, 2560, 3072, 3584, 4096]
    ks = [256, 512, 1024, 2048, 4096]
    todo = []
    while len(todo) < shapes:
        if ragged:
            M, N, K = (4 * rng.randint(128, 1024) for _ in range(3))
        else:
            M, N, K = rng.choice(dims), rng.choice(dims), rng.choice(ks)
        ops = rng.choice(["NN", "NT", "TN", "TT"])
        if (ops, M, N, K) not in todo:
            todo.append((ops, M, N, K))
    torch.manual_seed(seed)
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    regrets = []
    with open(path, "w") as out:
        for ops, M, N, K in todo:
            ta, tb = ops[0], ops[1]
            A = torch.rand((K, M) if ta == "T" else (M, K), device="cuda") * 2 - 1
            B = torch.rand((N, K) if tb == "T" else (K, N), device="cuda") * 2 - 1
            C = torch.zeros(M, N, device="cuda")
            chosen = mg.mi_sgemm_select_config(ta, tb, M, N, K)
            n = max(10, min(500, int(0.04 / max(2.0 * M * N * K / 120e12, 1e-6))))
            best = {}
            for _ in range(2):
                for cfg in tile_cfgs:
                    args = (ta, tb, M, N, K, 1.0, A.data_ptr(), A.shape[1], B.data_ptr(), B.shape[1], 0.0,
                            C.data_ptr(), N, h)
                    # At least `warmup` calls and 25 ms of them: the shader clock
                    # takes about 20 ms to ramp back up after a configuration that
                    # loads only part of the chip.
                    t0, calls = time.perf_counter(), 0
                    while calls < warmup or time.perf_counter() - t0 < 0.025:
                        for _ in range(10):
                            mg.mi_sgemm_with_config(cfg, *args)
                        stream.synchronize()
                        calls += 10
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(n):
                        rc = mg.mi_sgemm_with_config(cfg, *args)
                    e1.record(stream)
                    e1.synchronize()
                    if rc != 0:
                        raise RuntimeError(f"mi_sgemm: {mg.mi_sgemm_status_string(rc)}")
                    best[cfg] = min(best.get(cfg, float("inf")), e0.elapsed_time(e1) * 1e3 / n)
            fastest = min(best, key=best.get)
            regret = best[chosen] / best[fastest] - 1
            regrets.append(regret)
            out.write(json.dumps({"shape": f"{ops} {M}x{N}x{K}", "chosen": names[chosen],
                                  "chosen_us": round(best[chosen], 2), "fastest": names[fastest],
                                  "fastest_us": round(best[fastest], 2), "regret_pct": round(100 * regret, 2),
                                  "all_us": {names[c]: round(t, 2) for c, t in best.items()}}) + "\n")
            out.flush()
            del A, B, C
        summary = {"shapes": len(regrets), "seed": seed, "ragged": ragged, "mean_regret_pct": round(100 * sum(regrets) / len(regrets), 2),
                   "above_3pct": sum(r > 0.03 for r in regrets), "max_regret_pct": round(100 * max(regrets), 2)}
        out.write(json.dumps({"summary": summary}) + "\n")
    print(json.dumps({"regret": summary}), file=sys.stderr)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--mode", choices=["gemm", "copy"], default="gemm")
    ap.add_argument("--table", metavar="PATH", help="also write per-workload numbers to PATH")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--preheat", type=float, default=1.0,
                    help="seconds of back-to-back calls before the warm-up steps (reported as `preheat`; "
                         "with --workload, before each kernel's timing; 0 for none)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workload families (the `configs` field)")
    ap.add_argument("--sweep-configs", metavar="PATH",
                    help="also time every kernel configuration on every workload, to PATH")
    ap.add_argument("--config", action="append", metavar="NAME_OR_ID",
                    help="with --workload: time this kernel configuration instead of the chosen one "
                         "(repeatable)")
    ap.add_argument("--ladder", metavar="PATH",
                    help="time the vector-ALU technique ladder (valu_* configs) beside the matrix-core path at "
                         "1024^3 and 4096^3, to PATH, and exit")
    ap.add_argument("--regret", metavar="PATH",
                    help="time every tile configuration on random shapes and score select_config's picks by "
                         "their regret against the fastest, to PATH, and exit")
    ap.add_argument("--regret-shapes", type=int, default=90, help="with --regret: number of random shapes")
    ap.add_argument("--regret-seed", type=int, default=11, help="with --regret: seed of the shape draw")
    ap.add_argument("--regret-ragged", action="store_true",
                    help="with --regret: draw M, N, K from the multiples of 4 in 512..4096")
    ap.add_argument("--workload", metavar="NAME",
                    help="time only this workload (a name from synthetic/workloads.py) with its chosen "
                         "kernel and print its numbers; for profiling one configuration at a time")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this SGEMM runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp32_gemm_nn_amd as mg
    from synthetic import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mg.load_library()

    if args.mode == "copy":
        run_copy(args.steps, args.warmup)
        return
    if args.workload:
        run_workload(args.workload, args.steps, args.warmup, args.config, args.preheat)
        return
    if args.ladder:
        run_ladder(args.ladder)
        return
    if args.regret:
        run_regret(args.regret, args.regret_shapes, args.regret_seed, ragged=args.regret_ragged)
        return

    case = W.HEADLINE
    prob = Problem(case)
    heat = preheat(prob, args.preheat)
    wall, ev, per = time_steps(prob, args.steps, args.warmup)
    clock = clock_probe()
    flops = case.flops
    value = tflops(flops * args.steps, wall)
    per_launch = ev / args.steps
    achieved = tflops(flops, per_launch)
    clock["pct_of_peak_at_sclk"] = round(100 * achieved / clock["peak_at_sclk_tflops"], 2)
    check = check_sampled(prob, 4096, seed=4, reset=False)
    traffic = load_traffic(case.name)
    cfg_id = mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preheat": heat,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"sgemm_{case.transA}{case.transB}_{case.M}x{case.N}x{case.K}".lower(),
            "M": case.M, "N": case.N, "K": case.K, "transA": case.transA, "transB": case.transB,
            "alpha": case.alpha, "beta": case.beta, "inputs": "uniform [-1,1) from srand48(4)",
            "kernel_config": mg.mi_sgemm_config_name(cfg_id),
            "pct_fp32_matrix_peak": round(100 * value / PEAK_FP32_MATRIX_TFLOPS, 2),
            "gpu": torch.cuda.get_device_name(0),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_MATRIX_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_MATRIX_TFLOPS, 4),
            "traffic": traffic,
            "kernel_us_per_launch": round(per_launch * 1e6, 2),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": case.algorithmic_bytes,
        },
        "per_call_us": spread(per),
        "clock": clock,
        "check": check,
        "configs": None,
        "cpu_baseline": None,
    }
    del prob
    if not args.no_configs:
        result["configs"] = run_configs()
    if args.table:
        run_table(args.table, 20, 5)
    if args.sweep_configs:
        run_config_sweep(args.sweep_configs)
    if not args.no_cpu:
        cb = cpu_baseline(case)
        cb.update(host_info())
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    bad = [] if check["pass"] else ["headline"]
    if result["configs"]:
        c = result["configs"]
        rows = [c["C1"], c["C2"], *c["C3"], *c["C5a"], c["C5b"]["cold"], c["C5b"]["warm"]]
        bad += [r["workload"] for r in rows if not r["check_pass"]]
    if bad:
        print(f"bench.py: result check failed for {', '.join(bad)}", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
