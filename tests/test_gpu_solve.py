"""GPU parity of deer_solve (and the sequential GPU rollout) against the oracle.

Bars: the trajectory matches the oracle's float64 rollout within 1e-4
normwise relative L-infinity per sequence; the iteration count is within one
of the oracle's float32 run of the same algorithm.  Chaotic-at-float32 cases
(float32 and float64 rollouts of the oracle itself part by more than 1e-5)
are certified by their one-step residual in float64 instead, over the whole
trajectory, and by agreement up to the horizon where the oracle's float32
rollout still tracks its float64 one.
"""
import json
import os

import numpy as np
import pytest
import torch

from evaluation_nonlinear_rnns_amd import deer, inputs as I
from gpu_util import device, log, rel_linf

pytestmark = pytest.mark.gpu
TOL = 1e-4
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_full_workloads.json")


def _run(orc, p, mode, tol, max_iter, s0=True, check_iters=True, init=None, scan_f64=False, damping=0.0,
         multi_launch=False):
    dev = device()
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    s0_t = torch.from_numpy(p["s0"]).to(dev) if s0 else None
    init_t = None if init is None else torch.from_numpy(init).to(dev)
    traj, iters, resid, status, rc = deer.deer_solve(cell, x, s0_t, mode=mode, tol=tol, max_iter=max_iter,
                                                     init_guess=init_t, scan_f64=scan_f64, damping=damping,
                                                     multi_launch=multi_launch)
    torch.cuda.synchronize()
    oc = orc.Cell.from_problem(p)
    s0n = p["s0"] if s0 else None
    ref = orc.rollout(oc, p["x"], s0n)
    _, oit, ores, ost = orc.newton(oc, p["x"], s0n, mode=mode, tol=tol, max_iter=max_iter, precision="f32",
                                   init=init, damping=damping)
    got = traj.cpu().numpy()
    if check_iters:
        assert np.all(np.abs(iters - oit) <= 1), (iters, oit)
        assert list(status) == list(ost), (status, ost)
    return got, ref, iters, resid, status, rc, oit


@pytest.mark.parametrize("multi_launch", [False, True])
@pytest.mark.parametrize("mode", ["dense", "diag"])
@pytest.mark.parametrize("B,T,D,M,gain", [(2, 100, 4, 3, 0.5), (3, 777, 8, 8, 0.8), (2, 1000, 16, 16, 0.9),
                                          (2, 500, 32, 32, 0.7), (1, 300, 5, 2, 0.6), (2, 200, 64, 64, 0.6),
                                          (3, 1000, 2, 3, 0.9), (2, 300, 32, 7, 0.7), (3, 31, 32, 32, 0.7)])
def test_tanh_solve_matches_oracle(orc, mode, B, T, D, M, gain, multi_launch):
    p = I.tanh_problem(500 + T + D, B, T, D, M, gain=gain, bias_std=0.3, s0_std=0.5)
    log(f"deer_solve tanh {mode} B={B} T={T} D={D} M={M} multi_launch={multi_launch}")
    got, ref, iters, resid, status, rc, oit = _run(orc, p, mode, 1e-5, T, multi_launch=multi_launch)
    assert rc == deer.DEER_OK and np.all(status == 0)
    assert np.all(rel_linf(got, ref) <= TOL)
    assert np.all(resid <= 1e-5)


@pytest.mark.parametrize("B,T,D,M,gain", [(2, 300, 4, 3, 0.6), (2, 1000, 16, 16, 0.9), (3, 700, 32, 32, 0.7),
                                          (1, 200, 6, 4, 0.8)])
def test_tanh_dense_solve_f64_scan_matches_oracle(orc, B, T, D, M, gain):
    """Dense DEER with the linear solve accumulated in double."""
    p = I.tanh_problem(550 + T + D, B, T, D, M, gain=gain, bias_std=0.3, s0_std=0.5)
    log(f"deer_solve tanh dense f64-scan B={B} T={T} D={D} M={M}")
    got, ref, iters, resid, status, rc, oit = _run(orc, p, "dense", 1e-5, T, scan_f64=True)
    assert rc == deer.DEER_OK and np.all(status == 0)
    assert np.all(rel_linf(got, ref) <= TOL)


@pytest.mark.parametrize("B,T,D,M", [(2, 100, 4, 3), (3, 1000, 16, 16), (2, 777, 32, 8), (2, 2000, 64, 64),
                                     (1, 129, 7, 5), (2, 300, 32, 5), (5, 31, 64, 7), (3, 33, 64, 64)])
def test_gru_solve_matches_oracle(orc, B, T, D, M):
    p = I.gru_problem(600 + T + D, B, T, D, M, bias_std=0.3, s0_std=0.5)
    log(f"deer_solve gru diag B={B} T={T} D={D} M={M}")
    got, ref, iters, resid, status, rc, oit = _run(orc, p, "diag", 1e-5, 200)
    assert rc == deer.DEER_OK and np.all(status == 0)
    assert np.all(rel_linf(got, ref) <= TOL)


@pytest.mark.parametrize("cell,mode,damping,D,T", [
    ("tanh", "jacobi", 0.0, 8, 300), ("tanh", "picard", 0.0, 4, 60), ("tanh", "dense", 0.3, 16, 500),
    ("tanh", "diag", 0.5, 32, 400), ("tanh", "dense", 1.0, 8, 200), ("tanh", "picard", 0.0, 32, 40),
    ("gru", "jacobi", 0.0, 64, 2000), ("gru", "picard", 0.0, 64, 100), ("gru", "diag", 0.3, 64, 3000),
    ("gru", "jacobi", 0.0, 16, 500), ("gru", "diag", 0.4, 32, 1000), ("gru", "picard", 0.0, 8, 50)])
def test_linearisations_match_oracle(orc, cell, mode, damping, D, T):
    """Jacobi (A_t = 0), Picard (A_t = I) and damped Newton / quasi-Newton
    (A_t = (1 - k) J_t): iteration counts within one of the oracle's float32 run
    of the same linearisation, trajectory within 1e-4 of the float64 rollout."""
    B = 2
    if cell == "tanh":
        p = I.tanh_problem(800 + T + D, B, T, D, D, gain=0.7, bias_std=0.3, s0_std=0.5)
    else:
        p = I.gru_problem(900 + T + D, B, T, D, D, bias_std=0.3, s0_std=0.5)
    log(f"deer_solve {cell} {mode} damping={damping} B={B} T={T} D={D}")
    got, ref, iters, resid, status, rc, oit = _run(orc, p, mode, 1e-5, T + 1, damping=damping)
    assert rc == deer.DEER_OK and np.all(status == 0), (iters, status)
    assert np.all(rel_linf(got, ref) <= TOL)
    assert np.all(resid <= 1e-5)


@pytest.mark.parametrize("B,T,D", [(256, 200, 64), (257, 150, 64), (300, 130, 64), (256, 300, 32),
                                   (300, 100, 32)])
def test_gru_fused_step_many_sequences(orc, B, T, D):
    """The fused GRU step keeps per-sequence residual maxima in LDS for up to
    256 sequences and writes per-tile maxima above that.  Both sides of that
    limit, with staggered convergence (per-sequence input scales, so finished
    sequences skip their tiles while others go on) and one sequence whose input
    is not finite (non-finite status, exact prefix before the NaN kept)."""
    p = I.gru_problem(1500 + B + T + D, B, T, D, D, bias_std=0.3, s0_std=0.5)
    x = p["x"] * (0.2 + 1.6 * (np.arange(B) % 9) / 8.0)[:, None, None].astype(np.float32)
    bad, tbad = B // 2 + 1, T // 3
    x[bad, tbad, 1] = np.nan
    p = dict(p, x=np.ascontiguousarray(x, dtype=np.float32))
    log(f"deer_solve gru diag (fused step) B={B} T={T} D={D}, staggered, one NaN sequence")
    got, ref, iters, resid, status, rc, oit = _run(orc, p, "diag", 1e-5, 60)
    assert rc == deer.DEER_NOT_CONVERGED
    ok = np.arange(B) != bad
    assert status[bad] == 2 and np.all(status[ok] == 0), status
    assert len(set(iters[ok].tolist())) >= 3, iters          # convergence is staggered
    assert np.all(rel_linf(got[ok], ref[ok]) <= TOL)
    assert np.abs(got[bad, :tbad] - ref[bad, :tbad]).max() / np.abs(ref[bad, :tbad]).max() <= TOL


def test_damping_one_is_jacobi(orc):
    """k = 1 shrinks the blocks to zero: the damped quasi-Newton solve takes
    Jacobi's steps (same counts, same trajectory)."""
    p = I.gru_problem(951, 2, 1500, 64, 64, bias_std=0.3, s0_std=0.5)
    dev = device()
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    s0 = torch.from_numpy(p["s0"]).to(dev)
    log("deer_solve gru diag damping=1 vs jacobi")
    t1, i1, _, st1, _ = deer.deer_solve(cell, x, s0, mode="diag", tol=1e-5, max_iter=400, damping=1.0)
    t1 = t1.cpu().numpy()
    t2, i2, _, st2, _ = deer.deer_solve(cell, x, s0, mode="jacobi", tol=1e-5, max_iter=400)
    assert list(i1) == list(i2) and list(st1) == list(st2) == [0, 0]
    assert np.array_equal(t1, t2.cpu().numpy())


def test_solve_edge_cases(orc):
    dev = device()
    p = I.tanh_problem(700, 3, 64, 8, 8, gain=0.7, bias_std=0.2)
    oc = orc.Cell.from_problem(p)
    ref32 = orc.rollout(oc, p["x"], precision="f32")
    log("deer_solve warm start at the rollout")
    _, _, iters, _, status, rc, _ = _run(orc, p, "dense", 1e-5, 50, s0=False, init=ref32)
    assert list(iters) == [0, 0, 0] and rc == deer.DEER_OK
    log("deer_solve max_iter=0")
    got, _, iters, _, status, rc, _ = _run(orc, p, "dense", 1e-6, 0, s0=False)
    assert rc == deer.DEER_NOT_CONVERGED and list(status) == [1, 1, 1] and np.all(got == 0)
    log("deer_solve NaN input")
    q = dict(p)
    q["x"] = p["x"].copy()
    q["x"][1, 10, 3] = np.nan
    got, ref, iters, resid, status, rc, _ = _run(orc, q, "diag", 1e-5, 60, s0=False)
    assert rc == deer.DEER_NOT_CONVERGED and status[1] == 2 and status[0] == 0 and status[2] == 0
    assert np.isnan(resid[1])
    # the exact prefix before the NaN is untouched
    assert np.abs(got[1, :10] - ref[1, :10]).max() < 1e-5
    log("deer_solve T=1")
    r = I.tanh_problem(701, 2, 1, 4, 4, gain=0.7)
    got, ref, iters, _, status, rc, _ = _run(orc, r, "dense", 1e-6, 5, s0=False)
    assert list(iters) == [1, 1] and np.all(rel_linf(got, ref) <= TOL)


# ------------------------------------------------ single-launch path (D <= 4, T <= 1024)

@pytest.mark.parametrize("mode,damping", [("dense", 0.0), ("diag", 0.0), ("jacobi", 0.0), ("picard", 0.0),
                                          ("dense", 0.4), ("diag", 0.7)])
@pytest.mark.parametrize("B,T,D,M", [(1, 1, 4, 4), (2, 2, 1, 2), (3, 255, 3, 5), (2, 256, 4, 4), (2, 257, 4, 1),
                                     (1, 512, 2, 2), (2, 513, 4, 3), (1, 1000, 1, 1), (2, 1024, 4, 4)])
def test_single_launch_matches_oracle(orc, mode, damping, B, T, D, M):
    """Thread blocks of 1, 2 and 4 positions, ragged last thread, every
    linearisation: counts within one of the oracle's float32 run, trajectory
    within 1e-4 of the float64 rollout."""
    p = I.tanh_problem(1200 + T + D, B, T, D, M, gain=0.8, bias_std=0.3, s0_std=0.5)
    log(f"deer_solve single launch tanh {mode} damping={damping} B={B} T={T} D={D} M={M}")
    cap = T + 2 if mode in ("jacobi", "picard") else T + 1
    got, ref, iters, resid, status, rc, oit = _run(orc, p, mode, 1e-5, cap, damping=damping)
    assert rc == deer.DEER_OK and np.all(status == 0), (iters, status)
    assert np.all(rel_linf(got, ref) <= TOL)
    assert np.all(resid <= 1e-5)


def test_single_launch_agrees_with_multi_launch(orc):
    """The one-launch solve and the multi-launch loop take the same number of
    iterations and agree to rounding."""
    dev = device()
    p = I.tanh_problem(1301, 4, 1024, 4, 4, gain=0.9, bias_std=0.3, s0_std=0.5)
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    s0 = torch.from_numpy(p["s0"]).to(dev)
    for mode in ("dense", "diag"):
        log(f"deer_solve single vs multi launch {mode}")
        t1, i1, r1, st1, _ = deer.deer_solve(cell, x, s0, mode=mode, tol=1e-6, max_iter=1024)
        t1 = t1.cpu().numpy()
        t2, i2, r2, st2, _ = deer.deer_solve(cell, x, s0, mode=mode, tol=1e-6, max_iter=1024, multi_launch=True)
        assert list(st1) == list(st2) == [0, 0, 0, 0]
        assert np.all(np.abs(i1 - i2) <= 1), (i1, i2)
        assert np.abs(t1 - t2.cpu().numpy()).max() <= 1e-5


def test_single_launch_edge_cases(orc):
    dev = device()
    p = I.tanh_problem(1310, 3, 300, 4, 4, gain=0.7, bias_std=0.2)
    oc = orc.Cell.from_problem(p)
    ref32 = orc.rollout(oc, p["x"], precision="f32")
    log("deer_solve single launch: warm start at the rollout")
    _, _, iters, _, status, rc, _ = _run(orc, p, "dense", 1e-5, 50, s0=False, init=ref32)
    assert list(iters) == [0, 0, 0] and rc == deer.DEER_OK
    log("deer_solve single launch: max_iter=0 and 1")
    got, _, iters, _, status, rc, _ = _run(orc, p, "dense", 1e-6, 0, s0=False)
    assert rc == deer.DEER_NOT_CONVERGED and list(status) == [1, 1, 1] and np.all(got == 0)
    got, _, iters, _, status, rc, _ = _run(orc, p, "diag", 1e-7, 1, s0=False)
    assert rc == deer.DEER_NOT_CONVERGED and list(iters) == [1, 1, 1] and list(status) == [1, 1, 1]
    log("deer_solve single launch: NaN input")
    q = dict(p)
    q["x"] = p["x"].copy()
    q["x"][1, 10, 3] = np.nan
    got, ref, iters, resid, status, rc, _ = _run(orc, q, "diag", 1e-5, 60, s0=False)
    assert rc == deer.DEER_NOT_CONVERGED and status[1] == 2 and status[0] == 0 and status[2] == 0
    assert np.isnan(resid[1])
    assert np.abs(got[1, :10] - ref[1, :10]).max() < 1e-5


@pytest.mark.parametrize("kind,B,T,D,M", [("tanh", 3, 500, 16, 16), ("gru", 3, 500, 64, 64), ("tanh", 2, 1, 4, 4),
                                          ("tanh", 2, 7, 3, 5), ("gru", 1, 9, 5, 2), ("tanh", 2, 333, 8, 100),
                                          ("tanh", 3, 1000, 32, 32), ("gru", 2, 777, 32, 7), ("gru", 2, 300, 16, 16),
                                          ("tanh", 1, 2000, 64, 64), ("gru", 5, 129, 40, 40)])
def test_sequential_rollout_matches_oracle(orc, kind, B, T, D, M):
    """The GPU rollout (projection, then one workgroup per sequence): every
    lane geometry (D up to 4, 8, 16, 32, 64), lengths below, at and past the
    8-step prefetch ring, inputs wider than 64."""
    dev = device()
    if kind == "tanh":
        p = I.tanh_problem(800 + T + D, B, T, D, M, gain=0.9, bias_std=0.2, s0_std=0.3)
    else:
        p = I.gru_problem(801 + T + D, B, T, D, M, bias_std=0.2, s0_std=0.3)
    log(f"deer_rollout {kind} B={B} T={T} D={D} M={M}")
    cell = deer.cell_from_problem(p, dev)
    traj = deer.deer_rollout(cell, torch.from_numpy(p["x"]).to(dev), torch.from_numpy(p["s0"]).to(dev))
    torch.cuda.synchronize()
    ref = orc.rollout(orc.Cell.from_problem(p), p["x"], p["s0"])
    assert np.all(rel_linf(traj.cpu().numpy(), ref) <= TOL)


# ------------------------------------------------------------- full workloads

def _golden(name, gain=None):
    with open(GOLDEN) as f:
        g = json.load(f)[name]
    return g[f"{gain:g}"] if gain is not None else g


def _full(orc, name, gain=None, sample=None, scan_f64=False, multi_launch=False):
    dev = device()
    w = I.WORKLOADS[name]
    gold = _golden(name, gain)
    p = I.workload_problem(name, gain=gain)
    log(f"deer_solve full workload {name} gain={gain} scan_f64={scan_f64}")
    cell = deer.cell_from_problem(p, dev)
    x = torch.from_numpy(p["x"]).to(dev)
    traj, iters, resid, status, rc = deer.deer_solve(cell, x, mode=w.mode, tol=w.tol, max_iter=w.max_iter,
                                                     scan_f64=scan_f64, multi_launch=multi_launch)
    torch.cuda.synchronize()
    seqs = range(w.B) if sample is None else sample
    oc = orc.Cell.from_problem(p)
    ref = orc.rollout(oc, p["x"][list(seqs)])
    got = traj[list(seqs)].cpu().numpy()
    return w, gold, p, got, ref, np.asarray(iters), status, list(seqs)


@pytest.mark.parametrize("multi_launch", [False, True])
def test_full_tanh_d4_t1024(orc, multi_launch):
    w, gold, p, got, ref, iters, status, seqs = _full(orc, "tanh_d4_t1024", multi_launch=multi_launch)
    assert np.all(status == 0)
    assert np.all(np.abs(iters - np.asarray(gold["iters_f32"])) <= 1), (iters, gold["iters_f32"])
    assert np.all(rel_linf(got, ref) <= TOL)


def test_full_gru_d64_t65536(orc):
    w, gold, p, got, ref, iters, status, seqs = _full(orc, "gru_d64_t65536")
    assert np.all(status == 0)
    assert np.all(np.abs(iters - np.asarray(gold["iters_f32"])) <= 1), (iters, gold["iters_f32"])
    assert np.all(rel_linf(got, ref) <= TOL)


def test_full_tanh_d32_t16384(orc):
    w, gold, p, got, ref, iters, status, seqs = _full(orc, "tanh_d32_t16384")
    assert np.all(status == 0)
    assert np.all(np.abs(iters - np.asarray(gold["iters_f32"])) <= 1), (iters, gold["iters_f32"])
    assert np.all(rel_linf(got, ref) <= TOL)


@pytest.mark.parametrize("gain", [0.5, 0.9, 1.2])
def test_full_sweep_predictable(orc, gain):
    w, gold, p, got, ref, iters, status, seqs = _full(orc, "tanh_d16_t4096_sweep", gain=gain)
    assert gold["rollout_gap_f32_f64"] < 1e-5 or min(gold["horizon_1e-5"]) == w.T
    assert np.all(status == 0)
    assert np.all(np.abs(iters - np.asarray(gold["iters_f32"])) <= 1), (iters, gold["iters_f32"])
    assert np.all(rel_linf(got, ref) <= TOL)


def test_full_sweep_gain2_certified(orc):
    """g = 2: float32 and float64 rollouts of the oracle itself part by more than
    1e-4, so no float32 method can meet the literal bound over all of T.  The GPU
    trajectory is certified by its float64 one-step residual and matched up to the
    horizon where the oracle's own float32 rollout still tracks float64.  The
    linear solve accumulates in double here: float32 chunk products are too large
    at this gain for the residual to reach 1e-6."""
    w, gold, p, got, ref, iters, status, seqs = _full(orc, "tanh_d16_t4096_sweep", gain=2.0, scan_f64=True)
    assert np.all(status == 0)
    oc = orc.Cell.from_problem(p)
    # the oracle's float64 residual of the GPU trajectory: max_t |s_t - f(s_{t-1})| <= 10 tol
    _, _, res64, st64 = orc.newton(oc, p["x"][seqs], mode="dense", tol=10 * w.tol, max_iter=0, precision="f64",
                                   init=got)
    assert np.all(st64 == 0), res64
    for k, bi in enumerate(seqs):
        h = gold["horizon_1e-5"][bi]
        if h > 0:
            assert np.abs(got[k, :h] - ref[k, :h]).max() / np.abs(ref[k]).max() <= TOL
    # iteration counts are reported, and stay inside the finite-step bound
    assert np.all(iters <= w.T)


def test_solves_are_bitwise_reproducible(orc):
    """The scans' look-back always yields the left-to-right chain's value, so
    the same solve gives the same bits whatever the workgroup timing."""
    dev = device()
    for cell_kind, mode, D, T in (("gru", "diag", 64, 20000), ("tanh", "diag", 16, 30000), ("tanh", "dense", 32, 5000)):
        if cell_kind == "gru":
            p = I.gru_problem(971, 4, T, D, D, bias_std=0.3, s0_std=0.5)
        else:
            p = I.tanh_problem(972, 4, T, D, D, gain=0.9, bias_std=0.3, s0_std=0.5)
        cell = deer.cell_from_problem(p, dev)
        x = torch.from_numpy(p["x"]).to(dev)
        log(f"deer_solve twice {cell_kind} {mode} T={T}")
        runs = [deer.deer_solve(cell, x, None, mode=mode, tol=1e-6, max_iter=100) for _ in range(3)]
        first = runs[0][0].cpu().numpy()
        for r in runs[1:]:
            assert np.array_equal(first, r[0].cpu().numpy())
            assert list(r[1]) == list(runs[0][1])


def test_picard_long_sequence_matches_oracle(orc):
    """Picard (A_t = I) amplifies any perturbation behind its exact prefix, so it
    reaches tol on a long contractive sequence only if every scan of the solve is
    bit-reproducible: it then needs exactly T iterations, like the oracle."""
    T = 2048
    p = I.workload_problem("tanh_d16_t4096_sweep", gain=0.9)
    p = dict(p, x=np.ascontiguousarray(p["x"][:2, :T]), s0=np.ascontiguousarray(p["s0"][:2]), B=2, T=T)
    log(f"deer_solve tanh picard T={T}")
    got, ref, iters, resid, status, rc, oit = _run(orc, p, "picard", 1e-6, T + 1)
    assert rc == deer.DEER_OK and list(iters) == [T, T] and list(oit) == [T, T]
    assert np.all(rel_linf(got, ref) <= TOL)
