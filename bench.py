"""Throughput of the parallel Newton solver on one MI355X.

A step is one complete quasi-DEER solve of the GRU workload (B=16 sequences,
T=65536 steps, D=64, input 64, weights ~ N(0, 1/D), tol 1e-5, at most 200
iterations): input projection, then per iteration the f / Jacobian-diagonal
evaluation, the device-side convergence test and the diagonal scan, until
every sequence has converged.  Inputs are resident in HBM before timing.

Prints one JSON line: converged trajectory steps per second (B*T / time per
solve), the roofline of the dominant kernel (timed live with HIP events on
the solver's stream), the oracle's sequential CPU rollout of the same
workload as a reported baseline, the standalone diagonal linear scan
(B=32, T=131072, D=256) in GB/s against the HBM peak, the dense-Jacobian DEER
solve of the tanh RNN (B=64, T=16384, D=32) with its chunk-compose rate on the
matrix cores, and the gain sweep of the D=16 tanh RNN (B=32, T=4096) against
the sequential GPU rollout, and the Jacobi / Picard / damped linearisations
of the same solver against it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F32_PEAK_TFLOPS = 157.3   # dense FP32 matrix
VALU_F32_PEAK_TFLOPS = 78.6    # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (no packed FP32)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-scan", action="store_true", help="skip the standalone scan measurement")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-DEER, gain-sweep and linearisation measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the baseline sample")
    ap.add_argument("--only", choices=("dense", "sweep", "scan", "lin", "broyden", "tiny"), default=None,
                    help="run one secondary measurement alone and print its JSON (for profiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 1 GiB device copy (the reference kernel for HBM counter scaling)")
    return ap.parse_args()


def solve_workload(args, dev):
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    w = I.WORKLOADS["gru_d64_t65536"]
    p = I.workload_problem(w.name)
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=dev)
    ws = deer.new_workspace(deer.deer_workspace_size(cell, w.B, w.T, w.mode), device=dev)
    stream = torch.cuda.current_stream()

    def step():
        return deer.deer_solve(cell, x, None, mode=w.mode, tol=w.tol, max_iter=w.max_iter, out=out, workspace=ws,
                               stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps run without per-launch events; a second pass of the same
    # steps with them enabled gives the per-kernel times of the roofline
    iters_seen = []
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        _, iters, _, status, rc = step()
        iters_seen.append(iters.copy())
        assert rc == deer.DEER_OK, (rc, status)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1000.0 / args.steps
    ms_events = start.elapsed_time(stop) / args.steps
    for k in range(5):
        deer.deer_profile_read(k)          # reset counters
    deer.deer_profile_enable(True)
    for _ in range(args.steps):
        _, iters, _, status, rc = step()
        assert rc == deer.DEER_OK, (rc, status)
    torch.cuda.synchronize()
    deer.deer_profile_enable(False)
    prof = {k: deer.deer_profile_read(k) for k in range(5)}
    return w, p, ms_per_step, ms_events, prof, np.array(iters_seen)


def _source_sha(paths):
    """Hash of the kernel's source files, in the given order."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel, sources):
    """HBM bytes per launch from committed rocprofv3 counters, if they were taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != _source_sha(sources):
        return None                       # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def roofline_of(w, prof):
    """Dominant kernel of the solve and its algorithmic rate per launch.

    The quasi-DEER GRU iteration is one fused launch: per position it reads the
    iterate s^(i) (D words) and the input projection (3D words) and writes
    s^(i+1) (D words), and it runs the 3D x D recurrent product on the matrix
    cores (2 * 3D * D flops).  From a zero start with M = D the first launch
    computes the projection itself instead (reads x: D words, writes the
    projection: 3D words and s^(1): D words; the 3D x M input product): the same
    bytes and flops per position, so the average over all launches keeps its
    meaning, and no separate projection launch runs.
    """
    from evaluation_nonlinear_rnns_amd import deer
    BT = w.B * w.T
    step_bytes = BT * w.D * 4 * (1 + 3 + 1)
    step_flops = BT * 2 * 3 * w.D * w.D
    n_e, ms_e = prof[deer.PROFILE_EVAL]
    n_p, ms_p = prof[deer.PROFILE_PROJECTION]
    kernels = {
        "gru_quasi_step": {"launches": n_e, "avg_ms": ms_e / max(n_e, 1), "bytes": step_bytes, "flops": step_flops},
        "input_projection": {"launches": n_p, "avg_ms": ms_p / max(n_p, 1),
                             "bytes": BT * 4 * (w.M + 3 * w.D), "flops": BT * 2 * 3 * w.D * w.M},
    }
    if n_p == 0:
        kernels["input_projection"]["note"] = "computed by the first gru_quasi_step launch of each solve"
    k = kernels["gru_quasi_step"]
    sec = k["avg_ms"] * 1e-3
    achieved = k["bytes"] / sec / 1e9
    tflops = k["flops"] / sec / 1e12
    # the fused kernel's source: its file and the shared device helpers it inlines
    src = [os.path.join(ROOT, "evaluation_nonlinear_rnns_amd", "csrc", f) for f in ("cell_mfma.hip", "internal.h")]
    return "gru_quasi_step", kernels, {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic("gru_quasi_step", src),
        "kernel": "gru_quasi_step", "avg_launch_ms": round(k["avg_ms"], 4),
        "algorithmic_bytes_per_launch": k["bytes"],
        "mfma_tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
    }


def scan_bandwidth(args, dev):
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    w = I.WORKLOADS["diag_scan_d256_t131072"]
    p = I.workload_problem(w.name)
    a = torch.from_numpy(p["a"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    del p
    s = torch.empty_like(a)
    ws = deer.new_workspace(deer.linear_scan_workspace_size(w.B, w.T, w.D), device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(max(args.warmup, 1)):
        deer.linear_scan_diag(a, b, None, out=s, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    reps = max(args.steps, 5)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        deer.linear_scan_diag(a, b, None, out=s, workspace=ws, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    nbytes = 12 * w.B * w.T * w.D
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "avg_launch_ms": round(ms, 4),
            "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "elements_per_s": w.B * w.T * w.D / (ms * 1e-3)}


def stream_ceiling(dev, k, reps=10):
    """Measured HBM ceiling of a plain streaming kernel on this machine for a read /
    write mix of k : 1 (deer_bandwidth_probe: 1 GiB written, k GiB read, 16-byte
    non-temporal accesses), bytes moved over the mean duration (HIP events)."""
    import torch
    from evaluation_nonlinear_rnns_amd import deer
    n = 1 << 28
    src = torch.ones(k * n, dtype=torch.float32, device=dev)
    dst = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        deer.bandwidth_probe(src, dst, stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        deer.bandwidth_probe(src, dst, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    del src, dst
    torch.cuda.empty_cache()
    return round((k + 1) * 4 * n / (ms * 1e-3) / 1e9, 1)


def stream_ceilings(dev):
    """The probe at the read : write mixes of the copy, the diagonal scan (2 : 1)
    and the fused GRU step (4 : 1, algorithmically)."""
    c = {f"read_{k}_write_1_GBs": stream_ceiling(dev, k) for k in (1, 2, 4)}
    c["method"] = ("deer_bandwidth_probe: 1 GiB written, k GiB read (16-byte non-temporal loads and stores), "
                   "bytes moved over the mean of 10 launches after 2 warm-ups")
    return c


def host_info():
    """Host CPU model and the logical CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "nproc": int(avail)}


def _stats(times_s):
    t = np.asarray(times_s, dtype=np.float64)
    return float(np.median(t)), float(np.mean(t))


def gpu_rollout_timer(cell, x, B, T, D, dev, stream):
    """The sequential GPU rollout (deer_rollout) with its buffers allocated once:
    returns (ms per rollout, trajectory tensor)."""
    import torch
    from evaluation_nonlinear_rnns_amd import deer
    seq = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    ws = deer.new_workspace(deer.rollout_workspace_size(cell, B, T), device=dev)
    roll = lambda: deer.deer_rollout(cell, x, None, out=seq, workspace=ws, stream=stream)  # noqa: E731
    ms, _, _ = _time_solves(roll, 10, stream, profile=False)
    return ms, seq


def cpu_rollout_timed(p, threads, runs=5, steps=None):
    """The oracle's float32 sequential rollout on the host: one warm-up run,
    then `runs` timed runs; returns (median s, mean s) per run."""
    from oracle import oracle as O
    cell = O.Cell.from_problem(p)
    xs = p["x"] if steps is None else np.ascontiguousarray(p["x"][:, :steps])
    O.rollout(cell, xs, precision="f32", threads=threads)
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        O.rollout(cell, xs, precision="f32", threads=threads)
        times.append(time.perf_counter() - t0)
    return _stats(times)


def _time_solves(step, reps, stream, profile=True, budget_ms=None):
    """Mean wall time of `reps` calls after one warm-up call.  With `profile`
    the library's per-launch HIP events are on during the timed calls (their
    packets cost a few microseconds per launch, which matters for small
    problems); the per-kernel totals come back in `prof`.  With `budget_ms`
    the count drops (to no fewer than 2) so the timed calls take about that
    long, judged from the warm-up call."""
    import torch
    from evaluation_nonlinear_rnns_amd import deer
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    if budget_ms is not None:
        warm = (time.perf_counter() - t0) * 1000.0
        reps = max(2, min(reps, int(budget_ms / max(warm, 1e-3))))
    for k in range(5):
        deer.deer_profile_read(k)
    deer.deer_profile_enable(profile)
    t0 = time.perf_counter()
    out = None
    for _ in range(reps):
        out = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / reps
    deer.deer_profile_enable(False)
    prof = {k: deer.deer_profile_read(k) for k in range(5)}
    return ms, prof, out


def dense_solve(args, dev):
    """Dense-Jacobian DEER on the tanh RNN (B=64, T=16384, D=32).

    Per iteration the linear solve composes the factored Jacobians
    A_t = diag(1 - s_t^2) W inside chunks: one D x D x D product per position,
    2 D^3 flops, on the matrix cores; that figure over the whole linear-solve
    time (compose, carry and replay launches) is the reported compose rate.
    """
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    w = I.WORKLOADS["tanh_d32_t16384"]
    p = I.workload_problem(w.name)
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=dev)
    ws = deer.new_workspace(deer.deer_workspace_size(cell, w.B, w.T, w.mode), device=dev)
    stream = torch.cuda.current_stream()

    def step():
        return deer.deer_solve(cell, x, None, mode=w.mode, tol=w.tol, max_iter=w.max_iter, out=out, workspace=ws,
                               stream=stream)

    ms, prof, res = _time_solves(step, max(3, args.steps // 2), stream)
    _, iters, _, status, rc = res
    n_s, ms_s = prof[deer.PROFILE_SCAN]
    n_e, ms_e = prof[deer.PROFILE_EVAL]
    n_c, ms_c = prof[deer.PROFILE_COMPOSE]
    scan_ms = ms_s / max(n_s, 1)
    compose_ms = ms_c / max(n_c, 1)
    flops = 2 * w.B * w.T * w.D ** 3
    tflops = flops / (compose_ms * 1e-3) / 1e12
    tflops_scan = flops / (scan_ms * 1e-3) / 1e12
    # the replay of every linear solve also evaluates the cell for the next
    # iteration, so an iteration is one linear solve (plus the first evaluation)
    return {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "rc": int(rc),
            "iterations": sorted(set(int(v) for v in iters)),
            "ms_per_solve": round(ms, 3), "B*T/s": round(w.B * w.T / (ms * 1e-3), 1),
            "linear_solve_with_next_eval_avg_ms": round(scan_ms, 4),
            "eval_in_replay": True,
            "eval_avg_ms": round(ms_e / max(n_e, 1), 4),
            "compose_avg_ms": round(compose_ms, 4),
            "compose_flops_per_launch": flops, "compose_tflops": round(tflops, 2),
            "compose_frac_of_fp32_mfma_peak": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
            "compose_flops_over_linear_solve_tflops": round(tflops_scan, 2)}


def tiny_solve(args, dev):
    """Dense DEER on the tiny tanh RNN (B=1, T=1024, D=4): everything fits in
    cache and the solve is bound by launch and synchronisation latency, so it
    runs as one launch (one workgroup per sequence performs every iteration on
    chip).  Reported as absolute time per solve, next to the multi-launch loop
    on the same problem; no roofline."""
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    w = I.WORKLOADS["tanh_d4_t1024"]
    p = I.workload_problem(w.name)
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=dev)
    ws = deer.new_workspace(deer.deer_workspace_size(cell, w.B, w.T, w.mode), device=dev)
    stream = torch.cuda.current_stream()

    def solver(multi):
        def step():
            return deer.deer_solve(cell, x, None, mode=w.mode, tol=w.tol, max_iter=w.max_iter, out=out,
                                   workspace=ws, stream=stream, multi_launch=multi)
        return step

    # the kernel time from the HIP events of a profiled pass; the solve time
    # from passes without them (their cost is comparable to a launch here)
    _, prof, res = _time_solves(solver(False), 10, stream)
    _, iters, _, status, rc = res
    n_e, ms_e = prof[deer.PROFILE_EVAL]
    reps = max(200, args.steps)
    ms = {}
    for multi in (False, True):
        step = solver(multi)
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        ms[multi] = (time.perf_counter() - t0) * 1000.0 / reps
    return {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "rc": int(rc), "path": "single launch",
            "iterations": sorted(set(int(v) for v in iters)), "solves_timed": reps,
            "ms_per_solve": round(ms[False], 4), "B*T/s": round(w.B * w.T / (ms[False] * 1e-3), 1),
            "solve_kernel_ms": round(ms_e / max(n_e, 1), 4),
            "multi_launch_ms_per_solve": round(ms[True], 4)}


def broyden_solve(args, dev):
    """Parallel Broyden (no Jacobian) on the GRU workload (B=16, T=65536, D=64).

    Per iteration: the value-only GRU evaluation (reads s^(i) and the
    projection, writes f^(i): 5D words per position), then the block update and
    compressed scan in three launches -- fold (reads s^(i) and s^(i-1) at t-1,
    f^(i) and f^(i-1), the block's U, V columns; writes the slot's two columns),
    carry, replay (reads s^(i), f^(i) and the used columns; writes s^(i+1)).
    Algorithmic bytes of the update + scan per position at rank m, rank-one
    variant: fold 4D + 2mD read, 2D written; replay 2D + 2mD read, D written:
    (9 + 4m) D words (the carry's chunk aggregates are O(1/chunk)).  The
    multisecant variant also reads the m stored df columns and rewrites all m
    u columns: + 2m D words.
    """
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    w = I.WORKLOADS["gru_d64_t65536"]
    p = I.workload_problem(w.name)
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    rows = []
    for rank, ms_, chunk in ((2, False, 64), (2, False, 128), (4, False, 128), (4, True, 128), (8, False, 128)):
        sk = torch.from_numpy(I.broyden_sketch(21, w.D, rank)).to(dev)
        ws = deer.new_workspace(deer.deer_broyden_workspace_size(cell, w.B, w.T, rank, ms_, chunk), device=dev)

        def step():
            return deer.deer_solve_broyden(cell, x, sk, rank=rank, multisecant=ms_, alpha=0.5,
                                           gram_reg=1e-6 if ms_ else 0.0, chunk=chunk, tol=w.tol,
                                           max_iter=w.max_iter, out=out, workspace=ws, stream=stream)

        ms, prof, res = _time_solves(step, 2, stream)
        _, iters, _, status, rc = res
        n_s, ms_s = prof[deer.PROFILE_SCAN]
        n_e, ms_e = prof[deer.PROFILE_EVAL]
        step_ms = ms_s / max(n_s, 1)
        nbytes = (9 + 4 * rank + (2 * rank if ms_ else 0)) * w.D * 4 * w.B * w.T
        rows.append({"rank": rank, "multisecant": ms_, "chunk": chunk, "alpha": 0.5, "rc": int(rc),
                     "iterations": sorted(set(int(v) for v in iters)), "ms_per_solve": round(ms, 3),
                     "B*T/s": round(w.B * w.T / (ms * 1e-3), 1), "eval_avg_ms": round(ms_e / max(n_e, 1), 4),
                     "update_scan_avg_ms": round(step_ms, 4), "update_scan_bytes": nbytes,
                     "update_scan_GBs": round(nbytes / (step_ms * 1e-3) / 1e9, 1)})
        del ws
    return {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "tol": w.tol, "runs": rows}


def gain_sweep(args, dev):
    """Dense DEER against the sequential rollout (GPU and the oracle's on the
    host) across the recurrent gain g.

    The gain sets the largest Lyapunov exponent (estimated on the GPU along the
    solved trajectory, deer_lle); the sweep locates the g where the parallel
    solve stops beating the sequential evaluation.  Every gain runs with the
    default options (float32; a stall of the finite-step progress switches the
    linear solve to double accumulation).  At g = 2 the variants are reported
    too: float32 without escalation (the stall), damped Newton k = 0.3 in
    float32, and double accumulation from the start.
    """
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    w = I.WORKLOADS["tanh_d16_t4096_sweep"]
    stream = torch.cuda.current_stream()
    cpu_threads = min(w.B, host_info()["nproc"])
    rows = []
    g2 = None
    for g in w.gains:
        p = I.workload_problem(w.name, gain=g)
        cell = deer.cell_from_problem(p, dev)
        x = torch.from_numpy(p["x"]).to(dev)
        out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=dev)
        ws = deer.new_workspace(deer.deer_workspace_size(cell, w.B, w.T, w.mode), device=dev)

        def solver(**kw):
            def step():
                return deer.deer_solve(cell, x, None, mode=w.mode, tol=w.tol, max_iter=w.max_iter, out=out,
                                       workspace=ws, stream=stream, **kw)
            return step

        # default options: float32, finite-step check, escalation to double accumulation on a stall
        ms, _, res = _time_solves(solver(), 20, stream, profile=False, budget_ms=1500.0)
        _, iters, _, status, rc = res
        if g >= 2.0:
            g2 = {}
            for label, kw in (("float32_no_escalation", {"stall_escalate": False}),
                              ("damped_0.3_float32", {"damping": 0.3, "stall_escalate": False}),
                              ("double_accumulation_from_start", {"scan_f64": True})):
                ms2, _, res2 = _time_solves(solver(**kw), 3, stream, profile=False, budget_ms=1500.0)
                _, it2, _, st2, rc2 = res2
                g2[label] = {"options": kw, "rc": int(rc2), "iterations": [int(v) for v in it2],
                             "status_counts": {str(k): int(v) for k, v in zip(*np.unique(st2, return_counts=True))},
                             "ms_per_solve": round(ms2, 3)}
        ms_seq, _ = gpu_rollout_timer(cell, x, w.B, w.T, w.D, dev, stream)
        v0 = torch.from_numpy(I.lle_probe(50, w.B, w.D)).to(dev)
        lle_out = torch.empty(w.B, dtype=torch.float64, device=dev)
        ms_lle, _, _ = _time_solves(lambda: deer.deer_lle(cell, x, out, v0, out=lle_out, stream=stream), 10, stream,
                                    profile=False)
        row = {"gain": g, "options": "default (float32, stall check, escalation)", "rc": int(rc),
               "status_counts": {str(k): int(v) for k, v in zip(*np.unique(status, return_counts=True))},
               "iterations_max": int(iters.max()),
               "iterations_median": float(np.median(iters)), "deer_ms": round(ms, 3),
               "gpu_rollout_ms": round(ms_seq, 4), "speedup_vs_gpu_rollout": round(ms_seq / ms, 3),
               "lle_mean": round(float(lle_out.mean().item()), 4), "lle_ms": round(ms_lle, 3)}
        if not args.no_cpu:
            med, mean = cpu_rollout_timed(p, cpu_threads)
            row.update({"cpu_rollout_ms_median": round(med * 1e3, 3), "cpu_rollout_ms_mean": round(mean * 1e3, 3),
                        "speedup_vs_cpu_rollout": round(med * 1e3 / ms, 3)})
        rows.append(row)
    out = {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "rows": rows,
           "crossover_vs_gpu_rollout": _crossover(rows, "speedup_vs_gpu_rollout")}
    if g2 is not None:
        out["gain_2_variants"] = g2
    if not args.no_cpu:
        out["crossover_vs_cpu_rollout"] = _crossover(rows, "speedup_vs_cpu_rollout")
        out["cpu"] = dict(host_info(), threads=cpu_threads,
                          timing="oracle float32 rollout of all sequences, median and mean of 5 runs after 1 warm-up")
    return out


def _crossover(rows, key):
    """The gain bracket (largest swept gain where DEER is faster, smallest where it is slower)."""
    faster = [r["gain"] for r in rows if r[key] >= 1.0]
    slower = [r["gain"] for r in rows if r[key] < 1.0]
    return {"faster_up_to": max(faster) if faster else None, "slower_from": min(slower) if slower else None}


def linearizations(args, dev):
    """The same solver with other linearisations of f: iterations, time per solve
    and the ratio to the sequential GPU rollout.  On the contractive tanh
    workload (gain 0.9): Newton, damped Newton (k = 0.5), diagonal quasi-Newton,
    Jacobi (A_t = 0) and Picard (A_t = I, which needs up to T iterations on
    contractive dynamics).  On the GRU workload: quasi-Newton, damped
    quasi-Newton (k = 0.3) and Jacobi."""
    import torch
    from evaluation_nonlinear_rnns_amd import deer, inputs as I

    stream = torch.cuda.current_stream()
    out = {}
    cases = (("tanh_d16_t4096_sweep", 0.9, (("newton", "dense", 0.0), ("newton_damped_0.5", "dense", 0.5),
                                             ("quasi_newton", "diag", 0.0), ("jacobi", "jacobi", 0.0),
                                             ("picard", "picard", 0.0))),
             ("gru_d64_t65536", None, (("quasi_newton", "diag", 0.0), ("quasi_newton_damped_0.3", "diag", 0.3),
                                       ("jacobi", "jacobi", 0.0))))
    for name, gain, runs in cases:
        w = I.WORKLOADS[name]
        p = I.workload_problem(name, gain=gain) if gain is not None else I.workload_problem(name)
        cell = deer.cell_from_problem(p, dev)
        x = torch.from_numpy(p["x"]).to(dev)
        del p
        traj = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=dev)
        ms_seq, seq = gpu_rollout_timer(cell, x, w.B, w.T, w.D, dev, stream)
        rows = {}
        for label, mode, k in runs:
            ws = deer.new_workspace(deer.deer_workspace_size(cell, w.B, w.T, mode), device=dev)
            cap = w.T + 1 if mode == "picard" else w.max_iter

            def step():
                return deer.deer_solve(cell, x, None, mode=mode, tol=w.tol, max_iter=cap, out=traj, workspace=ws,
                                       stream=stream, damping=k)

            ms, _, res = _time_solves(step, 10, stream, profile=False, budget_ms=300.0)
            _, iters, _, status, rc = res
            rows[label] = {"mode": mode, "damping": k, "rc": int(rc), "iterations_max": int(iters.max()),
                           "ms_per_solve": round(ms, 3), "speedup_vs_gpu_rollout": round(ms_seq / ms, 3)}
            del ws
        v0 = torch.from_numpy(I.lle_probe(60, w.B, w.D)).to(dev)
        lle_out = torch.empty(w.B, dtype=torch.float64, device=dev)
        ms_lle, _, _ = _time_solves(lambda: deer.deer_lle(cell, x, seq, v0, out=lle_out, stream=stream), 10, stream,
                                    profile=False)
        out[name] = {"gain": gain, "B": w.B, "T": w.T, "D": w.D, "tol": w.tol, "gpu_rollout_ms": round(ms_seq, 3),
                     "lle_mean_on_rollout": round(float(lle_out.mean().item()), 4), "lle_ms": round(ms_lle, 3),
                     "runs": rows}
        del traj, seq, x
    return out


def cpu_baseline(args, w, p):
    """The oracle's float32 sequential rollout of the headline workload on the
    host cores (one thread per sequence, up to the CPUs available), one warm-up
    run and five timed runs; if a full run would take longer than the budget, a
    prefix of every sequence is timed instead.  Also one sequence on one thread."""
    from oracle import oracle as O

    info = host_info()
    threads = min(w.B, info["nproc"])
    cell = O.Cell.from_problem(p)
    # calibrate on a short prefix: the 6 runs should take about cpu_seconds
    Tc = 2048
    t0 = time.perf_counter()
    O.rollout(cell, p["x"][:, :Tc], precision="f32", threads=threads)
    per_step = (time.perf_counter() - t0) / Tc
    Ts = int(min(w.T, max(Tc, args.cpu_seconds / 6.0 / max(per_step, 1e-9))))
    med, mean = cpu_rollout_timed(p, threads, runs=5, steps=Ts)
    one = dict(p, x=np.ascontiguousarray(p["x"][:1]))
    med1, _ = cpu_rollout_timed(one, 1, runs=3, steps=Ts)
    return {"value": round(w.B * Ts / med, 1), "unit": "B*T/s", "cores": threads, "kind": "oracle",
            "sample": f"float32 sequential rollout of all {w.B} sequences over {Ts} of {w.T} steps, one thread "
                      f"per sequence; median of 5 runs after 1 warm-up ({med:.2f} s per run, mean {mean:.2f} s)",
            "value_mean": round(w.B * Ts / mean, 1), "cpu_model": info["cpu_model"], "nproc": info["nproc"],
            "single_thread_value": round(Ts / med1, 1),
            "single_thread_sample": f"one sequence over {Ts} steps on one thread, median of 3 runs after 1 warm-up"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU runs are not part of it", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from evaluation_nonlinear_rnns_amd import deer

    if not os.path.exists(deer.LIB_PATH):
        from evaluation_nonlinear_rnns_amd import build as hb
        hb.build()
    dev = torch.device("cuda:0")
    deer.load_library()
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only:
        fn = {"dense": dense_solve, "sweep": gain_sweep, "scan": scan_bandwidth, "lin": linearizations,
              "broyden": broyden_solve, "tiny": tiny_solve}[args.only]
        print(json.dumps({args.only: fn(args, dev)}), flush=True)
        return

    w, p, ms_per_step, ms_events, prof, iters = solve_workload(args, dev)
    dom, kernels, roof = roofline_of(w, prof)
    value = w.B * w.T / (ms_per_step * 1e-3)
    line = {
        "metric": "converged trajectory steps/sec (B*T/s)",
        "value": round(value, 1),
        "unit": "B*T/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy draws; random-init GRU weights)",
        "config": {"workload": w.name, "cell": "gru", "mode": "diag (quasi-DEER)", "B": w.B, "T": w.T, "D": w.D,
                   "M": w.M, "tol": w.tol, "max_iter": w.max_iter,
                   "iterations": sorted(set(int(v) for v in iters.reshape(-1)))},
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "ms_per_step_hip_events": round(ms_events, 4),
    }
    ceil = stream_ceilings(dev)
    line["stream_ceiling"] = ceil
    roof["measured_ceiling_GBs"] = ceil["read_4_write_1_GBs"]
    roof["frac_of_measured_ceiling"] = round(roof["achieved"] / ceil["read_4_write_1_GBs"], 4)
    if not args.no_scan:
        line["linear_scan"] = scan_bandwidth(args, dev)
        line["linear_scan"]["measured_ceiling_GBs"] = ceil["read_2_write_1_GBs"]
        line["linear_scan"]["frac_of_measured_ceiling"] = round(
            line["linear_scan"]["achieved_GBs"] / ceil["read_2_write_1_GBs"], 4)
    if not args.no_dense:
        line["dense_deer"] = dense_solve(args, dev)
        line["tiny_dense"] = tiny_solve(args, dev)
        line["gain_sweep"] = gain_sweep(args, dev)
        line["linearizations"] = linearizations(args, dev)
        line["broyden"] = broyden_solve(args, dev)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args, w, p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
