"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Index sets: the band test. For a top-k over scores s >= 0 with tau = the k-th
largest oracle score, every index with s > tau*(1+1e-3) must be selected, none
with s < tau*(1-1e-3) may be, and the GPU list must hold k distinct ascending
indices. Indices inside the band may go either way (several results are correct
there); everything outside it is unique and compared exactly.
Outputs: max |gpu - oracle| <= 2e-2 in bf16 and 1e-4 in fp32, with the oracle run
on the GPU's own selected subset.
"""

from __future__ import annotations

import threading

import numpy as np

BAND = 1e-3
ATOL = {"bf16": 2e-2, "f32": 1e-4}

# worst attention error seen per workload: name -> (max abs error, tolerance, outputs compared);
# printed in the test session's terminal summary so the margin to the tolerance is on record
MARGINS: dict = {}
_MARGINS_LOCK = threading.Lock()  # sequences are checked from a thread pool


def record_margin(name: str, err: float, tol: float, count: int) -> None:
    with _MARGINS_LOCK:
        old = MARGINS.get(name, (0.0, tol, 0))
        MARGINS[name] = (max(old[0], err), tol, old[2] + count)


def band_check(gpu_idx: np.ndarray, score: np.ndarray, k: int, domain: np.ndarray | None = None, what: str = ""):
    """gpu_idx: k picks (values from `domain`, default 0..n-1); score: oracle scores over the domain."""
    gpu_idx = np.asarray(gpu_idx).astype(np.int64)
    n = score.shape[0]
    dom = np.arange(n) if domain is None else np.asarray(domain).astype(np.int64)
    assert gpu_idx.shape == (k,), f"{what}: shape {gpu_idx.shape} != ({k},)"
    assert (np.diff(gpu_idx) > 0).all(), f"{what}: not strictly ascending"
    pos = np.searchsorted(dom, gpu_idx)
    assert (pos < n).all() and (dom[np.minimum(pos, n - 1)] == gpu_idx).all(), f"{what}: index outside the domain"
    tau = np.sort(score)[::-1][k - 1]
    must_in = np.nonzero(score > tau * (1 + BAND))[0]
    must_out = np.nonzero(score < tau * (1 - BAND))[0]
    chosen = np.zeros(n, dtype=bool)
    chosen[pos] = True
    missing = must_in[~chosen[must_in]]
    extra = must_out[chosen[must_out]]
    assert missing.size == 0, f"{what}: {missing.size} indices above the band missing, e.g. {dom[missing[:5]]}"
    assert extra.size == 0, f"{what}: {extra.size} indices below the band selected, e.g. {dom[extra[:5]]}"
    return int(n - must_in.size - must_out.size)  # size of the band (ambiguous zone)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
