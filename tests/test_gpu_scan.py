"""GPU parity of the linear scans against the oracle's sequential solvers.

Bar (fp32 path against the float64 oracle): per-sequence normwise relative
L-infinity error <= 1e-4.
"""
import numpy as np
import pytest
import torch

from evaluation_nonlinear_rnns_amd import deer, inputs as I
from gpu_util import device, log, rel_linf

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.mark.parametrize("B,T,D", [
    (1, 1, 4), (2, 257, 4), (3, 1000, 64), (2, 777, 5), (1, 4096, 256), (4, 300, 130), (2, 513, 1),
    (1, 70000, 8), (5, 2049, 68),
])
def test_linear_scan_diag_matches_sequential_solve(orc, B, T, D):
    dev = device()
    p = I.diag_scan_problem(100 + T + D, B, T, D, s0_std=1.0)
    log(f"linear_scan_diag B={B} T={T} D={D}")
    a = torch.from_numpy(p["a"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    s0 = torch.from_numpy(p["s0"]).to(dev)
    s = deer.linear_scan_diag(a, b, s0)
    torch.cuda.synchronize()
    ref = orc.solve_diag(p["a"], p["b"], p["s0"])
    err = rel_linf(s.cpu().numpy(), ref)
    assert np.all(err <= TOL), err


def test_linear_scan_diag_reused_workspace(orc):
    """Consecutive calls on one workspace (and shapes that shrink) stay exact."""
    dev = device()
    ws = deer.new_workspace(deer.linear_scan_workspace_size(4, 5000, 64), device=dev)
    for k, (B, T, D) in enumerate([(4, 5000, 64), (4, 5000, 64), (2, 3000, 64), (3, 100, 12), (4, 5000, 64)]):
        p = I.diag_scan_problem(200 + k, B, T, D, a_lo=-1.0, a_hi=1.0, s0_std=1.0)
        log(f"linear_scan_diag reuse #{k} B={B} T={T} D={D}")
        s = deer.linear_scan_diag(torch.from_numpy(p["a"]).to(dev), torch.from_numpy(p["b"]).to(dev),
                                  torch.from_numpy(p["s0"]).to(dev), workspace=ws)
        torch.cuda.synchronize()
        ref = orc.solve_diag(p["a"], p["b"], p["s0"])
        assert np.all(rel_linf(s.cpu().numpy(), ref) <= TOL)


def test_linear_scan_diag_no_s0_is_zero_start(orc):
    dev = device()
    p = I.diag_scan_problem(300, 2, 999, 16)
    log("linear_scan_diag s0=None")
    s = deer.linear_scan_diag(torch.from_numpy(p["a"]).to(dev), torch.from_numpy(p["b"]).to(dev))
    torch.cuda.synchronize()
    ref = orc.solve_diag(p["a"], p["b"], None)
    assert np.all(rel_linf(s.cpu().numpy(), ref) <= TOL)


def test_linear_scan_diag_full_size_sampled(orc):
    """The 32 x 131072 x 256 workload: sampled channels against the oracle over the whole length."""
    dev = device()
    w = I.WORKLOADS["diag_scan_d256_t131072"]
    p = I.workload_problem(w.name)
    log(f"linear_scan_diag full size B={w.B} T={w.T} D={w.D}")
    a = torch.from_numpy(p["a"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    s = deer.linear_scan_diag(a, b)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(s).all())
    rng = np.random.default_rng(7)
    picks = [(int(rng.integers(w.B)), int(rng.integers(w.D))) for _ in range(12)] + [(w.B - 1, w.D - 1), (0, 0)]
    for bi, d in picks:
        got = s[bi, :, d].cpu().numpy()
        ref = orc.solve_diag(p["a"][bi:bi + 1, :, d:d + 1], p["b"][bi:bi + 1, :, d:d + 1])[0, :, 0]
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err <= TOL, (bi, d, err)


@pytest.mark.parametrize("B,T,D", [(1, 1, 4), (2, 100, 3), (2, 300, 16), (1, 257, 32), (2, 70, 64), (3, 1500, 4),
                                   (1, 1000, 32)])
def test_linear_scan_dense_matches_sequential_solve(orc, B, T, D):
    dev = device()
    p = I.dense_scan_problem(400 + T + D, B, T, D, scale=0.9)
    log(f"linear_scan_dense B={B} T={T} D={D}")
    A = torch.from_numpy(p["A"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    s0 = torch.from_numpy(p["s0"]).to(dev)
    s = deer.linear_scan_dense(A, b, s0)
    torch.cuda.synchronize()
    ref = orc.solve_dense(p["A"], p["b"], p["s0"])
    err = rel_linf(s.cpu().numpy(), ref)
    assert np.all(err <= TOL), err


def test_linear_scan_diag_is_bitwise_reproducible(orc):
    """Repeated scans of the same input give the same bits (the look-back's carry
    is always the left-to-right chain's value, whatever the timing)."""
    dev = device()
    p = I.diag_scan_problem(77, 3, 200000, 64)
    a = torch.from_numpy(p["a"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    log("linear_scan_diag x3 B=3 T=200000 D=64")
    outs = [deer.linear_scan_diag(a, b, None).cpu().numpy() for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
