"""The timed CPU baseline: the oracle as it stands, never tuned for speed.

One "CPU verify GEMM" = the oracle's W12 decode of a matrix (records +
escapes -> bf16 bits) followed by an FP32 matmul of the decoded weights
against the verify rows. Test infrastructure only; bench.py's cpu_baseline
leg is its one caller outside tests.
"""
from __future__ import annotations

import time

import numpy as np

from . import w12_format


def cpu_verify_gemm(packed: dict, n: int, k: int, x_bits: np.ndarray) -> np.ndarray:
    w = w12_format.decode(packed, n, k)
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    xf = (np.ascontiguousarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return xf @ wf.T


def blas_threads() -> int:
    """Threads numpy's BLAS runs its matmul with (read from the loaded BLAS
    library itself); the decode is plain numpy, one thread."""
    try:
        import threadpoolctl
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        if info:
            return int(max(d["num_threads"] for d in info))
    except Exception:  # threadpoolctl missing or unreadable: say so with 0
        pass
    return 0


def time_cpu_verify_gemm(packed: dict, n: int, k: int, x_bits: np.ndarray,
                         reps: int = 1, threads: int | None = None) -> dict:
    """Wall time of `reps` CPU verify GEMMs; returns seconds per GEMM and the
    BLAS thread count used. `threads` limits the BLAS pool for this call
    (None: as loaded)."""
    def run():
        t0 = time.perf_counter()
        for _ in range(reps):
            cpu_verify_gemm(packed, n, k, x_bits)
        return (time.perf_counter() - t0) / reps

    if threads is None:
        np.ones((2, 2), np.float32) @ np.ones((2, 2), np.float32)  # load BLAS before asking
        return {"seconds": run(), "threads": blas_threads()}
    import threadpoolctl
    with threadpoolctl.threadpool_limits(limits=threads, user_api="blas"):
        return {"seconds": run(), "threads": blas_threads()}
