"""Helpers for the GPU parity tests: moving the seeded inputs to the device,
reading outputs back, and the error measures the tolerances are stated in."""
from __future__ import annotations

import sys

import numpy as np


def say(*args):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray, dtype: str):
    import workloads
    return workloads.to_torch(a, dtype, "cuda")


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else \
        t.detach().cpu().numpy()


def errors(got: np.ndarray, want: np.ndarray) -> dict:
    d = np.abs(got - want)
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0,
            "rel_l2": float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))}


# bf16 tolerances against the fp64 oracle: max/mean abs as stated for the
# throughput workloads, plus a relative L2 bound that a dropped tail tile
# would break even where the absolute bounds would not.
BF16_TOL = {"max_abs": 2e-2, "mean_abs": 1e-3, "rel_l2": 5e-3}
FP32_TOL = {"max_abs": 1e-5}


def assert_close(got, want, dtype: str, what: str = ""):
    e = errors(got, want)
    tol = BF16_TOL if dtype == "bf16" else FP32_TOL
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    bad = {k: (e[k], v) for k, v in tol.items() if not e[k] <= v}
    assert not bad, f"{what}: {bad} (all: {e})"
    return e


def assert_valid(o: np.ndarray, what: str = ""):
    """The validity notion of the pages' Table 1: no NaN/Inf, not all zero."""
    assert np.all(np.isfinite(o)), f"{what}: NaN/Inf in output"
    assert np.any(o != 0), f"{what}: all-zero output"
