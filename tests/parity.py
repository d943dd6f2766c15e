"""Parity protocol between the HIP library and the fp64 oracle.

Assignments: Lloyd's k-means with floating-point distances can legitimately
disagree where two centroids are (nearly) equidistant, and one early flip
changes every later centroid. So each iteration t is checked teacher-forced:
the oracle rebuilds mu^(t-1) in fp64 from the GPU's own c^(t-1) (mu^(0) is the
initial rows; with kept empty clusters the rebuild carries mu^(t-2) along),
assigns, and compares with the GPU's c^(t): slot t - 1 of the run's
assignment trace (ca_options_t.assign_hist; tests/test_gpu_trace.py checks on
every path that it equals a separate run with iters = t).
A mismatch is excused only at a near-tie, where the oracle's best-to-second
gap is below NEAR_TIE * ||q_i||^2 and the two centroids are not identical
vectors (identical centroids give identical distances, so the lowest index
must win). Outputs are compared with the oracle's steps after clustering run
on the GPU's final assignment.

Also reported, informational: the free-running mismatch count (the GPU's
final assignment against the oracle's own run from the same inputs, where one
excused flip may move many later assignments), the tokens assigned to a zero
(empty) centroid, and the largest distance error of the GPU's assignment
arithmetic relative to ||q_i||^2 (distance_error).
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Dict, List, Optional

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# where the parity records go (CA_PARITY_RECORDS overrides the default)
RECORD_DIR = os.environ.get("CA_PARITY_RECORDS", os.path.join(ROOT, "gpurun_out", "parity"))

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


def free_running_mismatches(Q, Kt, V, nclust: int, iters: int, W: int, alpha: float,
                            c_gpu: np.ndarray, valid=None, flags: int = 0) -> int:
    """Tokens whose final GPU assignment differs from the oracle's own run
    (informational: a single excused near-tie flip changes later centroids)."""
    ref = oracle.forward(Q, Kt, V, nclust, iters, W, alpha, trace=False, valid=valid,
                         flags=flags)
    return int(np.count_nonzero(ref["assign"] != np.asarray(c_gpu).astype(np.int32)))


def exact_distances(Q: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """||q_i - mu_k||^2 in fp64 for Q [..., L, d], mu [..., K, d] -> [..., L, K],
    as the sum of squared differences, a slice at a time."""
    Q = np.asarray(Q, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    lead = Q.shape[:-2]
    Qs = Q.reshape((-1,) + Q.shape[-2:])
    Ms = mu.reshape((-1,) + mu.shape[-2:])
    out = np.empty((Qs.shape[0], Qs.shape[1], Ms.shape[1]))
    for s in range(Qs.shape[0]):
        for k in range(Ms.shape[1]):
            diff = Qs[s] - Ms[s, k][None, :]
            out[s, :, k] = np.einsum("ld,ld->l", diff, diff)
    return out.reshape(lead + out.shape[1:])


def distance_error(Q: np.ndarray, mu_ref: np.ndarray, scores_gpu: np.ndarray) -> float:
    """max over tokens and clusters of |D_gpu - D_ref| / ||q_i||^2, where
    D_gpu = ||q_i||^2 - 2 score_gpu (the GPU's score is mu.q - ||mu||^2/2) and
    D_ref = ||q_i - mu_ref_k||^2 in fp64. A flip between two clusters can only
    happen where their true gap is below twice this error, so the near-tie
    window NEAR_TIE * ||q||^2 covers every flip when 2 * error < NEAR_TIE."""
    Q = np.asarray(Q, dtype=np.float64)
    qn2 = np.einsum("...d,...d->...", Q, Q)
    d_ref = exact_distances(Q, mu_ref)
    d_gpu = qn2[..., None] - 2.0 * np.asarray(scores_gpu, dtype=np.float64)
    ok = qn2 > 0
    if not np.any(ok):
        return 0.0
    rel = np.abs(d_gpu - d_ref) / np.where(ok, qn2, 1.0)[..., None]
    return float(rel[ok].max())


def report_dict(case: str, plan: Optional[str], reports: List[AssignReport], out_err: float,
                tol: float, free_running: Optional[int], dist_err: Optional[List[float]],
                extra: Optional[Dict] = None) -> Dict:
    rec = {
        "case": case, "plan": plan,
        "iterations": [dataclasses.asdict(r) for r in reports],
        "near_ties": sum(r.near_ties for r in reports),
        "excused": sum(r.excused for r in reports),
        "bad": sum(r.bad for r in reports),
        "zero_centroid_tokens_last": reports[-1].zero_centroid_tokens if reports else 0,
        "free_running_mismatches": free_running,
        "max_out_err": out_err, "tol": tol,
        "max_dist_err_rel": max(dist_err) if dist_err else None,
        "dist_err_rel_by_iter": dist_err,
        "near_tie_window": NEAR_TIE,
    }
    if extra:
        rec.update(extra)
    return rec


def write_record(name: str, rec: Dict) -> None:
    """Keep one JSON record per case under RECORD_DIR, so that the counts
    outlive pytest's captured output."""
    os.makedirs(RECORD_DIR, exist_ok=True)
    safe = "".join(ch if ch.isalnum() or ch in "-_." else "_" for ch in name)
    with open(os.path.join(RECORD_DIR, safe + ".json"), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
