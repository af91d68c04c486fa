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


def test_linear_scan_diag_full_size_every_channel(orc):
    """The 32 x 131072 x 256 workload: every channel against the oracle's
    sequential solve over the whole length (in slices of 32 channels)."""
    dev = device()
    w = I.WORKLOADS["diag_scan_d256_t131072"]
    p = I.workload_problem(w.name)
    log(f"linear_scan_diag full size B={w.B} T={w.T} D={w.D}")
    a = torch.from_numpy(p["a"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    s = deer.linear_scan_diag(a, b)
    torch.cuda.synchronize()
    del a, b
    sl = 32
    for d0 in range(0, w.D, sl):
        got = s[:, :, d0:d0 + sl].cpu().numpy()
        ref = orc.solve_diag(np.ascontiguousarray(p["a"][:, :, d0:d0 + sl]),
                             np.ascontiguousarray(p["b"][:, :, d0:d0 + sl]))
        err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)     # per (sequence, channel)
        assert np.all(err <= TOL), (d0, err.max())


@pytest.mark.parametrize("B,T,D", [(1, 1, 4), (2, 100, 3), (2, 300, 16), (1, 257, 32), (2, 70, 64), (3, 1500, 4),
                                   (1, 1000, 32), (2, 2048, 32), (1, 2113, 32), (1, 5000, 32), (2, 2047, 32)])
def test_linear_scan_dense_matches_sequential_solve(orc, B, T, D):
    """Includes D = 32 with 32 chunks or more (the two-level carry: 16 groups
    of 2, 12 groups of 3 with a last group of one chunk, 16 groups of 5 with a
    last group of 4) and 31 chunks (the one-level walk)."""
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


def test_linear_scan_dense_expanding_products_take_the_one_level_walk(orc):
    """Sequence 1 has expanding blocks (spectral radius about 3), b = 0 and
    s0 = 0: its exact solution is zero, but its group products (128 steps and
    more) overflow float32, where the two-level carry would turn 0 * inf into
    NaN; the kernel sees the out-of-range product and walks that sequence's
    chunks one by one, giving exact zeros.  Sequence 0 (contractive) keeps the
    two-level carry and matches the oracle."""
    dev = device()
    B, T, D = 2, 2048, 32
    p = I.dense_scan_problem(4242, B, T, D, scale=0.9)
    q = I.dense_scan_problem(4243, 1, T, D, scale=3.0)
    p["A"][1] = q["A"][0]
    p["b"][1] = 0.0
    p["s0"][1] = 0.0
    log("linear_scan_dense B=2 T=2048 D=32, sequence 1 expanding with a zero solution")
    A = torch.from_numpy(p["A"]).to(dev)
    b = torch.from_numpy(p["b"]).to(dev)
    s0 = torch.from_numpy(p["s0"]).to(dev)
    s = deer.linear_scan_dense(A, b, s0).cpu().numpy()
    assert np.all(s[1] == 0.0), np.abs(s[1]).max()
    ref = orc.solve_dense(p["A"][[0]], p["b"][[0]], p["s0"][[0]])
    assert rel_linf(s[[0]], ref)[0] <= TOL


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


@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 24) + 16 * 37])
def test_bandwidth_probe_streams(k, nbytes):
    """The bandwidth reference writes the XOR of its k input streams (k = 1: a
    copy), for sizes below, at and past one grid of four vectors per thread."""
    dev = device()
    log(f"deer_bandwidth_probe k={k} {nbytes} bytes out")
    n = nbytes // 16                                   # 16-byte vectors out
    src = torch.randint(-2**31, 2**31 - 1, (k * n, 4), dtype=torch.int32, device=dev)
    dst = torch.zeros((n, 4), dtype=torch.int32, device=dev)
    deer.bandwidth_probe(src, dst)
    torch.cuda.synchronize()
    G, r = n // 64, n % 64
    full = src[:k * 64 * G].reshape(G, k, 64, 4)
    ref = full[:, 0].clone()
    for j in range(1, k):
        ref ^= full[:, j]
    ref = ref.reshape(G * 64, 4)
    if r:
        tail = src[k * 64 * G:].reshape(k, r, 4)
        t = tail[0].clone()
        for j in range(1, k):
            t ^= tail[j]
        ref = torch.cat([ref, t])
    assert torch.equal(dst, ref)
