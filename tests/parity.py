"""Parity protocol between the HIP library and the fp64 oracle.

Assignments: Lloyd's k-means with floating-point distances can legitimately
disagree where two centroids are (nearly) equidistant, and one early flip
changes every later centroid. So each iteration t is checked teacher-forced:
the oracle rebuilds mu^(t-1) in fp64 from the GPU's own c^(t-1) (mu^(0) is the
initial rows; with kept empty clusters the rebuild carries mu^(t-2) along), assigns, and compares with the GPU's c^(t) (obtained by a run
with iters = t, which reproduces the first t iterations of any longer run).
A mismatch is excused only at a near-tie, where the oracle's best-to-second
gap is below NEAR_TIE * ||q_i||^2 and the two centroids are not identical
vectors (identical centroids give identical distances, so the lowest index
must win). Outputs are compared with the oracle's steps after clustering run
on the GPU's final assignment.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

import oracle

NEAR_TIE = 1e-5
TOL = {"f32": 1e-4, "bf16": 2e-2}


@dataclasses.dataclass
class AssignReport:
    iteration: int
    near_ties: int
    excused: int          # GPU != oracle at a near-tie
    bad: int              # GPU != oracle elsewhere (must be 0)
    zero_centroid_tokens: int


def check_assignment_step(Q: np.ndarray, mu: np.ndarray, c_gpu: np.ndarray, t: int) -> AssignReport:
    """Q [..., L, d] fp64, mu [..., K, d] fp64 (the centroids the GPU used)."""
    c_ora, _, gap, qn2 = oracle.assign(Q, mu)
    c_gpu = c_gpu.astype(np.int32)
    K = mu.shape[-2]
    assert c_gpu.min() >= 0 and c_gpu.max() < K, "assignment out of range"
    near = gap < NEAR_TIE * qn2
    diff = c_gpu != c_ora
    # mismatches between identical centroids are never excused
    mu_g = np.take_along_axis(mu, c_gpu[..., None].astype(np.int64), axis=-2)
    mu_o = np.take_along_axis(mu, c_ora[..., None].astype(np.int64), axis=-2)
    identical = np.all(mu_g == mu_o, axis=-1)
    excused = diff & near & ~identical
    bad = diff & ~excused
    zero = np.all(mu_g == 0.0, axis=-1)
    return AssignReport(t, int(near.sum()), int(excused.sum()), int(bad.sum()), int(zero.sum()))


def check_forward(Q, Kt, V, nclust: int, iters: int, W: int, alpha: float, dtype: str,
                  assign_by_iter: List[np.ndarray], out_gpu: np.ndarray,
                  tol: Optional[float] = None, valid: Optional[np.ndarray] = None,
                  flags: int = 0):
    """Full protocol. assign_by_iter[t-1] = GPU c^(t); out_gpu = GPU output
    (as float64 values) of the run with `iters` iterations; valid: the key-
    padding mask of a masked run (the clustering ignores it); flags: the
    listing-compatible variants of the run (oracle.INIT_STEP, ...), which
    the rebuilt centroids follow too."""
    L = Q.shape[-2]
    K = oracle.num_clusters(nclust, L)
    keep = bool(flags & oracle.KEEP_EMPTY)
    reports = []
    mu = oracle.init_centroids(Q, K, step=bool(flags & oracle.INIT_STEP))
    for t in range(1, iters + 1):
        c_gpu = assign_by_iter[t - 1]
        reports.append(check_assignment_step(Q, mu, c_gpu, t))
        mu, _ = oracle.update(Q, c_gpu, K, prev=mu if keep else None)
    ref = oracle.forward_from_assign(Q, Kt, V, assign_by_iter[-1], K, W, alpha, valid=valid,
                                     flags=flags, mu=mu if flags else None)
    err = np.abs(out_gpu - ref["out"])
    tol = TOL[dtype] if tol is None else tol
    return reports, float(err.max()) if err.size else 0.0, tol, ref


def summarize(reports: List[AssignReport]) -> str:
    return "; ".join(f"t={r.iteration}: near={r.near_ties} excused={r.excused} bad={r.bad} "
                     f"zero-centroid={r.zero_centroid_tokens}" for r in reports)
