"""The timed CPU baseline: the oracle as it stands, never tuned for speed.

One "CPU verify GEMM" = the oracle's W12 decode of a matrix (records +
escapes -> bf16 bits) followed by an FP32 matmul of the decoded weights
against the verify rows. Test infrastructure only; bench.py's cpu_baseline
leg is its one caller outside tests.
"""
from __future__ import annotations

import os
import time

import numpy as np

from . import w12_format


def cpu_verify_gemm(packed: dict, n: int, k: int, x_bits: np.ndarray) -> np.ndarray:
    w = w12_format.decode(packed, n, k)
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    xf = (np.ascontiguousarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return xf @ wf.T


def time_cpu_verify_gemm(packed: dict, n: int, k: int, x_bits: np.ndarray,
                         reps: int = 1) -> dict:
    """Wall time of `reps` CPU verify GEMMs; returns seconds per GEMM and the
    thread count numpy's BLAS was allowed (from the usual env variables)."""
    t0 = time.perf_counter()
    for _ in range(reps):
        cpu_verify_gemm(packed, n, k, x_bits)
    dt = (time.perf_counter() - t0) / reps
    threads = None
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        if os.environ.get(var):
            threads = int(os.environ[var])
            break
    return {"seconds": dt, "threads": threads or os.cpu_count()}
