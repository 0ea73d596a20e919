"""Comparison rules for HIP-path vs oracle parity (imported by the GPU tests).

Selections: equal to the oracle's, or every index in the symmetric difference scores within
REL_TIE of the oracle's k-th score (score ties within 1e-5 relative are exempt).
Floating-point outputs: per (b, head) row, max |gpu - oracle| <= tol * max |oracle|.
"""
from __future__ import annotations

import numpy as np

from oracle import rocketkv as O

REL_TIE = 1e-5
TOL_OUT = {"bf16": 2e-2, "fp32": 1e-5}


def tie_tolerance(scores: np.ndarray, kth: float) -> float:
    scale = max(abs(kth), 1e-6 * float(np.max(np.abs(scores))) if scores.size else 0.0)
    return REL_TIE * scale


def selection_matches(gpu_sel, oracle_scores, k: int) -> bool:
    """True if gpu_sel equals the oracle's top-k of oracle_scores; raises on a real mismatch;
    returns False when the sets differ only at ties within REL_TIE."""
    oracle_scores = np.asarray(oracle_scores, dtype=np.float64)
    gpu_sel = np.asarray(gpu_sel, dtype=np.int64)
    k = min(k, oracle_scores.shape[0])
    assert gpu_sel.shape[0] == k, (gpu_sel.shape, k)
    assert np.all(np.diff(gpu_sel) > 0), "selection not strictly ascending"
    assert gpu_sel.min(initial=0) >= 0 and gpu_sel.max(initial=0) < oracle_scores.shape[0]
    ref = O.stable_topk(oracle_scores, k)
    if k == 0:
        return True
    sg, sr = set(gpu_sel.tolist()), set(ref.tolist())
    if sg == sr:
        return True
    kth = oracle_scores[ref[-1]]
    tol = tie_tolerance(oracle_scores, kth)
    bad = [j for j in sg ^ sr if abs(oracle_scores[j] - kth) > tol]
    assert not bad, (f"selection differs beyond ties: {len(bad)} indices, e.g. {bad[:5]} "
                     f"scores {[oracle_scores[j] for j in bad[:5]]} kth {kth} tol {tol}")
    return False


def assert_rows_close(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str = "") -> float:
    """Rows over the last axis: max|gpu-ref| <= tol * max|ref| for each row; returns worst ratio."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref).max(axis=-1)
    scale = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    ratio = err / scale
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= tol, f"{what}: worst row error {worst:.3e} > {tol:.1e}"
    return worst
