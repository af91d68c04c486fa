"""Helpers shared by the GPU tests (no arithmetic of the method here)."""
import os
import sys

import numpy as np


def log(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be traced to it."""
    sys.stdout.write(f"[gpu] {msg}\n")
    sys.stdout.flush()


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from evaluation_nonlinear_rnns_amd import deer
    if not os.path.exists(deer.LIB_PATH):
        raise RuntimeError("libdeer.so is not built")
    deer.load_library()
    return torch.device("cuda:0")


def rel_linf(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-sequence normwise relative L-infinity error, arrays [B, ...]."""
    B = ref.shape[0]
    g = got.reshape(B, -1).astype(np.float64)
    r = ref.reshape(B, -1).astype(np.float64)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return np.abs(g - r).max(axis=1) / den
