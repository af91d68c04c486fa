"""Seeded synthetic inputs for the parallel-Newton workloads.

This module only draws random numbers and arranges them in the shapes the
solvers take.  It holds none of the method's arithmetic, and it is the one
piece of code shared by the GPU path and by the CPU oracle: both read the very
same float32 arrays that these functions return.

Recipe (every workload): a ``numpy.random.default_rng(seed)`` (PCG64) stream;
draws are made in float64 and cast to float32; parameters are drawn first,
in the order the C interface lists them, then the inputs.

* tanh RNN ``s_t = tanh(W s_{t-1} + U x_t + b)`` -- the vector form of the scalar
  tanh state space model on the "Predictability Enables Parallelization of
  Nonlinear State Space Models" page (rebuttal, "Application to RNN training
  efficiency"): ``W = gain * W0`` with ``W0 ~ N(0, 1/D)``, ``U ~ N(0, 1/M)``,
  ``b = 0``, ``x ~ N(0, 1)``, ``s0 = 0``.  The same ``W0`` is shared by every
  gain, so a gain sweep varies only the gain.
* GRU cell (gate order r, z, n): ``W_hh ~ N(0, 1/D)`` then ``W_ih ~ N(0, 1/D)``,
  biases 0, ``x ~ N(0, 1)``, ``h0 = 0``.
* diagonal linear recurrence ``s_t = a_t s_{t-1} + b_t``: ``a ~ U(0.9, 0.999)``,
  then ``b ~ N(0, 1)``, ``s0 = 0``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Rows drawn per numpy call when filling large [B, T, ...] arrays; bounds the
# float64 temporaries without changing the stream (draws are sequential).
_CHUNK_ELEMS = 1 << 24


@dataclass(frozen=True)
class Workload:
    """One benchmark configuration: a cell, its sizes and the solver settings."""

    name: str
    cell: str            # "tanh" | "gru" | "diag_scan"
    D: int
    M: int
    T: int
    B: int
    mode: str            # "dense" | "diag" | "scan"
    tol: float
    max_iter: int
    gain: float = 1.0
    seed: int = 0
    gains: tuple = field(default_factory=tuple)


# The five workloads of the benchmark, sizes as specified there.  tol and
# max_iter where a workload leaves them open: tol 1e-6 for the tanh runs,
# max_iter = T (the finite-step bound) unless a cap is given.
WORKLOADS = {
    "tanh_d4_t1024": Workload("tanh_d4_t1024", "tanh", 4, 4, 1024, 1, "dense", 1e-6, 1024, 0.5, 1),
    "gru_d64_t65536": Workload("gru_d64_t65536", "gru", 64, 64, 65536, 16, "diag", 1e-5, 200, 1.0, 2),
    "tanh_d32_t16384": Workload("tanh_d32_t16384", "tanh", 32, 32, 16384, 64, "dense", 1e-6, 16384, 0.7, 3),
    "diag_scan_d256_t131072": Workload("diag_scan_d256_t131072", "diag_scan", 256, 0, 131072, 32, "scan", 0.0, 1, 1.0, 4),
    "tanh_d16_t4096_sweep": Workload("tanh_d16_t4096_sweep", "tanh", 16, 16, 4096, 32, "dense", 1e-6, 4096, 1.0, 5,
                                     (0.5, 0.9, 1.2, 2.0)),
}


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """float64 N(0, std^2) draws cast to float32, filled in bounded pieces."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n = flat.size
    pos = 0
    while pos < n:
        k = min(_CHUNK_ELEMS, n - pos)
        flat[pos:pos + k] = (rng.standard_normal(k) * std).astype(np.float32)
        pos += k
    return out


def _uniform(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n = flat.size
    pos = 0
    while pos < n:
        k = min(_CHUNK_ELEMS, n - pos)
        flat[pos:pos + k] = rng.uniform(lo, hi, k).astype(np.float32)
        pos += k
    return out


def tanh_problem(seed: int, B: int, T: int, D: int, M: int, gain: float = 1.0,
                 bias_std: float = 0.0, s0_std: float = 0.0) -> dict:
    """Parameters and inputs of a random tanh RNN.

    Returns float32 arrays ``W [D,D]``, ``W0 [D,D]`` (unit-gain draw),
    ``U [D,M]``, ``b [D]``, ``x [B,T,M]``, ``s0 [B,D]``.  ``bias_std`` and
    ``s0_std`` (0 in every benchmark workload) give tests non-zero biases and
    initial states.
    """
    rng = np.random.default_rng(seed)
    W0 = _normal(rng, (D, D), 1.0 / np.sqrt(D))
    U = _normal(rng, (D, M), 1.0 / np.sqrt(M)) if M > 0 else np.zeros((D, 0), np.float32)
    b = _normal(rng, (D,), bias_std) if bias_std > 0 else np.zeros(D, np.float32)
    x = _normal(rng, (B, T, M), 1.0)
    s0 = _normal(rng, (B, D), s0_std) if s0_std > 0 else np.zeros((B, D), np.float32)
    W = (np.float64(gain) * W0.astype(np.float64)).astype(np.float32)
    return {"cell": "tanh", "W": W, "W0": W0, "U": U, "b": b, "b2": None, "x": x, "s0": s0,
            "D": D, "M": M, "B": B, "T": T, "gain": gain}


def lowrank_tanh_problem(seed: int, B: int, T: int, D: int, M: int, rank: int = 2, leak: float = 0.5,
                         gain: float = 0.4) -> dict:
    """A tanh RNN whose recurrent matrix is a scaled identity plus a rank-``rank``
    coupling, ``W = leak I + gain P Q^T / D`` with ``P, Q ~ N(0, 1)`` ``[D, rank]``
    -- a stand-in for the low-rank RNNs of the "Parallel Broyden Methods" page
    (appendix F.1), whose Jacobian blocks are diagonal plus low rank.  Then
    ``U ~ N(0, 1/M)``, ``b = 0``, ``x ~ N(0, 1)``, ``s0 = 0``.
    """
    rng = np.random.default_rng(seed)
    P = _normal(rng, (D, rank), 1.0).astype(np.float64)
    Q = _normal(rng, (D, rank), 1.0).astype(np.float64)
    W = (leak * np.eye(D) + gain * (P @ Q.T) / D).astype(np.float32)
    U = _normal(rng, (D, M), 1.0 / np.sqrt(M))
    x = _normal(rng, (B, T, M), 1.0)
    return {"cell": "tanh", "W": W, "U": U, "b": np.zeros(D, np.float32), "b2": None, "x": x,
            "s0": np.zeros((B, D), np.float32), "D": D, "M": M, "B": B, "T": T, "rank": rank,
            "leak": leak, "gain": gain}


def broyden_sketch(seed: int, D: int, rank: int) -> np.ndarray:
    """The random sketch ``Omega [D, rank] ~ N(0, 1)`` of the compressed scan."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (D, rank), 1.0)


def gru_problem(seed: int, B: int, T: int, D: int, M: int, w_std: Optional[float] = None,
                bias_std: float = 0.0, s0_std: float = 0.0) -> dict:
    """Parameters and inputs of a random GRU (gate order r, z, n).

    ``W`` is the recurrent matrix ``W_hh [3D, D]``, ``U`` the input matrix
    ``W_ih [3D, M]``, ``b`` = ``b_ih [3D]``, ``b2`` = ``b_hh [3D]``.
    """
    rng = np.random.default_rng(seed)
    std = (1.0 / np.sqrt(D)) if w_std is None else w_std
    W_hh = _normal(rng, (3 * D, D), std)
    W_ih = _normal(rng, (3 * D, M), std)
    if bias_std > 0:
        b_ih = _normal(rng, (3 * D,), bias_std)
        b_hh = _normal(rng, (3 * D,), bias_std)
    else:
        b_ih = np.zeros(3 * D, np.float32)
        b_hh = np.zeros(3 * D, np.float32)
    x = _normal(rng, (B, T, M), 1.0)
    s0 = _normal(rng, (B, D), s0_std) if s0_std > 0 else np.zeros((B, D), np.float32)
    return {"cell": "gru", "W": W_hh, "U": W_ih, "b": b_ih, "b2": b_hh, "x": x, "s0": s0,
            "D": D, "M": M, "B": B, "T": T}


def diag_scan_problem(seed: int, B: int, T: int, D: int, a_lo: float = 0.9, a_hi: float = 0.999,
                      s0_std: float = 0.0) -> dict:
    """Inputs of a diagonal linear recurrence: ``a [B,T,D]``, ``b [B,T,D]``, ``s0 [B,D]``."""
    rng = np.random.default_rng(seed)
    a = _uniform(rng, (B, T, D), a_lo, a_hi)
    b = _normal(rng, (B, T, D), 1.0)
    s0 = _normal(rng, (B, D), s0_std) if s0_std > 0 else np.zeros((B, D), np.float32)
    return {"a": a, "b": b, "s0": s0, "B": B, "T": T, "D": D}


def dense_scan_problem(seed: int, B: int, T: int, D: int, scale: float = 0.9,
                       s0_std: float = 1.0) -> dict:
    """Inputs of a dense linear recurrence ``s_t = A_t s_{t-1} + b_t``.

    ``A [B,T,D,D] ~ N(0, scale^2 / D)`` (spectral radius about ``scale``),
    ``b [B,T,D] ~ N(0, 1)``, ``s0 [B,D] ~ N(0, s0_std^2)``.
    """
    rng = np.random.default_rng(seed)
    A = _normal(rng, (B, T, D, D), scale / np.sqrt(D))
    b = _normal(rng, (B, T, D), 1.0)
    s0 = _normal(rng, (B, D), s0_std) if s0_std > 0 else np.zeros((B, D), np.float32)
    return {"A": A, "b": b, "s0": s0, "B": B, "T": T, "D": D}


def lle_probe(seed: int, B: int, D: int) -> np.ndarray:
    """Raw Gaussian start vectors ``[B, D]`` for the Lyapunov-exponent estimate."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (B, D), 1.0)


def workload_problem(name: str, gain: Optional[float] = None, B: Optional[int] = None,
                     T: Optional[int] = None) -> dict:
    """The inputs of a named workload, optionally with fewer sequences or steps.

    ``B``/``T`` below the workload's own values take the leading sequences /
    steps of the same draw order only for ``B``; a shorter ``T`` is a fresh draw
    with the same seed (used for bounded CPU samples).
    """
    w = WORKLOADS[name]
    BB = w.B if B is None else B
    TT = w.T if T is None else T
    if w.cell == "tanh":
        g = w.gain if gain is None else gain
        return tanh_problem(w.seed, BB, TT, w.D, w.M, gain=g)
    if w.cell == "gru":
        return gru_problem(w.seed, BB, TT, w.D, w.M)
    if w.cell == "diag_scan":
        return diag_scan_problem(w.seed, BB, TT, w.D)
    raise KeyError(name)
