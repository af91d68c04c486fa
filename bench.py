"""Throughput of the parallel Newton solver on one MI355X.

A step is one complete quasi-DEER solve of the GRU workload (B=16 sequences,
T=65536 steps, D=64, input 64, weights ~ N(0, 1/D), tol 1e-5, at most 200
iterations): input projection, then per iteration the f / Jacobian-diagonal
evaluation, the device-side convergence test and the diagonal scan, until
every sequence has converged.  Inputs are resident in HBM before timing.

Prints one JSON line: converged trajectory steps per second (B*T / time per
solve), the roofline of the dominant kernel (timed live with HIP events on
the solver's stream), the oracle's sequential CPU rollout of the same
workload as a reported baseline, and the standalone diagonal linear scan
(B=32, T=131072, D=256) in GB/s against the HBM peak.
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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the baseline sample")
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
    for k in range(4):
        deer.deer_profile_read(k)          # reset counters
    deer.deer_profile_enable(True)
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
    deer.deer_profile_enable(False)
    prof = {k: deer.deer_profile_read(k) for k in range(4)}
    ms_per_step = wall * 1000.0 / args.steps
    return w, p, ms_per_step, start.elapsed_time(stop) / args.steps, prof, np.array(iters_seen)


def roofline_of(w, prof):
    """Dominant kernel of the solve and its algorithmic rate per launch."""
    from evaluation_nonlinear_rnns_amd import deer
    BT = w.B * w.T
    # GRU evaluation: read s (D) and the projection (3D), write a and b (2D) per position
    eval_bytes = BT * w.D * 4 * (1 + 3 + 2)
    eval_flops = BT * 2 * 3 * w.D * w.D
    # diagonal scan: read a, b, write s
    scan_bytes = BT * w.D * 4 * 3
    n_e, ms_e = prof[deer.PROFILE_EVAL]
    n_s, ms_s = prof[deer.PROFILE_SCAN]
    kernels = {
        "gru_eval": {"launches": n_e, "avg_ms": ms_e / max(n_e, 1), "bytes": eval_bytes, "flops": eval_flops},
        "diag_scan": {"launches": n_s, "avg_ms": ms_s / max(n_s, 1), "bytes": scan_bytes, "flops": 2 * BT * w.D},
    }
    # over-enqueued launches after convergence exit at once; time only counts real work
    dom = "gru_eval" if ms_e >= ms_s else "diag_scan"
    k = kernels[dom]
    achieved = k["bytes"] / (k["avg_ms"] * 1e-3) / 1e9
    return dom, kernels, {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
        "kernel": dom, "avg_launch_ms": round(k["avg_ms"], 4),
        "algorithmic_bytes_per_launch": k["bytes"],
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


def cpu_baseline(args, w, p):
    """The oracle's float32 sequential rollout of the same workload on the host cores."""
    from oracle import oracle as O

    cell = O.Cell.from_problem(p)
    threads = min(w.B, O.max_threads())
    # calibrate on a short prefix, then run a bounded sample of about cpu_seconds:
    # the whole workload repeated, or a prefix of it if one pass is longer
    Tc = 2048
    t0 = time.perf_counter()
    O.rollout(cell, p["x"][:, :Tc], precision="f32", threads=threads)
    per_step = (time.perf_counter() - t0) / Tc
    Ts = int(min(w.T, max(Tc, args.cpu_seconds / max(per_step, 1e-9))))
    reps = max(1, int(round(args.cpu_seconds / max(per_step * Ts, 1e-9)))) if Ts == w.T else 1
    xs = p["x"][:, :Ts]
    t0 = time.perf_counter()
    for _ in range(reps):
        O.rollout(cell, xs, precision="f32", threads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(reps * w.B * Ts / dt, 1), "unit": "B*T/s", "cores": threads, "kind": "oracle",
            "sample": f"float32 sequential rollout of all {w.B} sequences over {Ts} of {w.T} steps, "
                      f"{reps} pass(es), {dt:.1f} s, one thread per sequence"}


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
    if not args.no_scan:
        line["linear_scan"] = scan_bandwidth(args, dev)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args, w, p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
