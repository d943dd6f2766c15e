"""Exact brute force for tiny cluster-attention inputs (pins the C oracle).

TEST INFRASTRUCTURE ONLY. Pure Python, no numpy arithmetic: Lloyd's k-means
runs in exact rationals (``fractions.Fraction``; float inputs convert
exactly), so every distance, tie and mean is exact; the two softmax branches
run in 50-digit ``decimal`` arithmetic. Written independently of
``oracle.c`` from the same passages:
  * model card "Hooshaai/distilbert-sst2-cluster-attention", Mathematical
    Formulation section 1 (strided init, assignment, max(1, n) update) and
    the Architecture Overview figure (centroid cross-attention with scale
    1/8 = 1/sqrt(64), gather, local window, convex fusion);
  * "ClusterFormer" specification (svd-sst2-roberta-cluster page), sections
    2.1 and 3.
Readings shared with the oracle: window |i - j| <= floor(W/2) clipped to the
sequence; lowest index wins a tie; an empty cluster's centroid is zero.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction
from typing import List, Sequence, Tuple

PREC = 50

Vec = List[Fraction]


def to_frac_rows(rows) -> List[Vec]:
    return [[Fraction(float(x)) if not isinstance(x, (int, Fraction)) else Fraction(x)
             for x in r] for r in rows]


def sqdist(a: Sequence[Fraction], b: Sequence[Fraction]) -> Fraction:
    total = Fraction(0)
    for x, y in zip(a, b):
        total += (x - y) * (x - y)
    return total


def lloyd(Q: List[Vec], nclust: int, iters: int):
    """Exact Lloyd's k-means on one slice.

    Returns (K, init_rows, c_hist, mu_hist, gap_hist) where c_hist[t] is the
    assignment of iteration t+1, mu_hist[t] the centroids mu^(t) and
    gap_hist[t] the exact best-to-second gap per token at iteration t+1.
    """
    L = len(Q)
    d = len(Q[0])
    K = nclust if nclust < L else L
    init_rows = []
    for k in range(K):
        # floor(k L / K) by integer division of non-negative integers
        init_rows.append((k * L) // K)
    mu = [list(Q[r]) for r in init_rows]
    c_hist, mu_hist, gap_hist = [], [mu], []
    for _ in range(iters):
        c, gaps = [], []
        for q in Q:
            dists = [sqdist(q, m) for m in mu]
            best_k = 0
            for k in range(1, K):
                if dists[k] < dists[best_k]:
                    best_k = k
            rest = [dists[k] for k in range(K) if k != best_k]
            gaps.append(min(rest) - dists[best_k] if rest else None)
            c.append(best_k)
        new_mu = []
        for k in range(K):
            members = [q for q, ck in zip(Q, c) if ck == k]
            sums = [Fraction(0)] * d
            for q in members:
                sums = [s + x for s, x in zip(sums, q)]
            n = max(1, len(members))
            new_mu.append([s / n for s in sums])
        mu = new_mu
        c_hist.append(c)
        mu_hist.append(mu)
        gap_hist.append(gaps)
    return K, init_rows, c_hist, mu_hist, gap_hist


def _dec(x) -> Decimal:
    if isinstance(x, Fraction):
        return Decimal(x.numerator) / Decimal(x.denominator)
    return Decimal(float(x)) if not isinstance(x, Decimal) else x


def softmax_attend(q: Sequence, keys: List[Sequence], values: List[Sequence]) -> List[Decimal]:
    """sum_j softmax_j(q . k_j / sqrt(d)) v_j in 50-digit decimal."""
    with localcontext() as ctx:
        ctx.prec = PREC
        d = len(q)
        scale = Decimal(1) / Decimal(d).sqrt()
        qd = [_dec(x) for x in q]
        scores = []
        for kr in keys:
            s = Decimal(0)
            for a, b in zip(qd, kr):
                s += a * _dec(b)
            scores.append(s * scale)
        m = max(scores)
        e = [(s - m).exp() for s in scores]
        z = sum(e, Decimal(0))
        out = [Decimal(0)] * len(values[0])
        for w, vr in zip(e, values):
            p = w / z
            out = [o + p * _dec(x) for o, x in zip(out, vr)]
        return out


def forward_slice(Q, Kt, V, nclust: int, iters: int, W: int, alpha) -> Tuple[list, list]:
    """One slice, exact: returns (out rows as floats, final assignment)."""
    Qf = to_frac_rows(Q)
    L = len(Qf)
    K, _, c_hist, mu_hist, _ = lloyd(Qf, nclust, iters)
    c = c_hist[-1]
    mu = mu_hist[-1]
    Kd = [[_dec(x) for x in r] for r in to_frac_rows(Kt)]
    Vd = [[_dec(x) for x in r] for r in to_frac_rows(V)]
    vcent = [softmax_attend(m, Kd, Vd) for m in mu]
    r = W // 2
    out = []
    with localcontext() as ctx:
        ctx.prec = PREC
        a = _dec(Fraction(alpha) if not isinstance(alpha, Fraction) else alpha)
        for i in range(L):
            lo = max(0, i - r)
            hi = min(L - 1, i + r)
            loc = softmax_attend(Qf[i], Kd[lo:hi + 1], Vd[lo:hi + 1])
            g = vcent[c[i]]
            out.append([float((1 - a) * gx + a * lx) for gx, lx in zip(g, loc)])
    return out, c
