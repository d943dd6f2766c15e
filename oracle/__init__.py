"""Python face of the fp64 CPU oracle for cluster attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library and its binding never
do. The arithmetic lives in ``oracle.c`` (plain C, float64, one loop nest per
formula of the pages); this module compiles it with gcc, marshals numpy arrays
and composes the full-layer variant from the C steps. ``exact.py`` holds the
independent exact-rational / 50-digit brute force that pins it.

Sources are cited per function in ``oracle.c``: the model card "Hooshaai/
distilbert-sst2-cluster-attention" (Architecture Overview, Mathematical
Formulation 1-2) and the "ClusterFormer" specification on the "Hooshaai/svd-
sst2-roberta-cluster" page (sections 2.1-4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        L = ctypes.c_long
        i = ctypes.c_int
        d = ctypes.c_double
        sig = {
            "ora_num_threads": (i, []),
            "ora_set_num_threads": (None, [i]),
            "ora_num_clusters": (i, [i, i]),
            "ora_radius": (i, [i]),
            "ora_init_centroids": (None, [_dp, L, i, i, i, _dp]),
            "ora_init_centroids_step": (None, [_dp, L, i, i, i, _dp]),
            "ora_soft_gather": (None, [_dp, _dp, _dp, L, i, i, i, _dp]),
            "ora_assign": (None, [_dp, _dp, L, i, i, i, _ip, _dp, _dp, _dp]),
            "ora_update": (None, [_dp, _ip, L, i, i, i, _dp, _dp, _ip]),
            "ora_objective": (None, [_dp, _dp, _ip, L, i, i, i, _dp]),
            "ora_centroid_xattn": (None, [_dp, _dp, _dp, L, i, i, i, _ip, _dp, _dp]),
            "ora_local_attn": (None, [_dp, _dp, _dp, L, i, i, i, _ip, _dp, _dp]),
            "ora_fuse": (None, [_dp, _ip, _dp, L, i, i, i, d, _ip, _dp, _dp]),
            "ora_forward": (i, [_dp, _dp, _dp, i, i, i, i, i, i, i, d, _ip, i, _dp, _ip,
                                _dp, _ip, _dp, _dp, _dp, _dp, _dp, _dp]),
            "ora_forward_from_assign": (None, [_dp, _dp, _dp, L, i, i, i, _ip, i, d, _ip, i,
                                               _dp, _dp, _dp, _dp, _dp]),
            "ora_backward": (None, [_dp, _dp, _dp, _dp, L, i, i, i, _ip, i, d, _ip,
                                    _dp, _dp, _dp, _dp]),
            "ora_exact_attention": (None, [_dp, _dp, _dp, L, i, i, i, i, _ip, _ip, _dp]),
            "ora_matmul": (None, [_dp, _dp, L, L, L, _dp]),
            "ora_round_bf16": (d, [d]),
            "ora_round_bf16_array": (None, [_dp, L]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    if a.dtype == np.float64:
        return a.ctypes.data_as(_dp)
    if a.dtype == np.int32:
        return a.ctypes.data_as(_ip)
    raise TypeError(a.dtype)


def num_threads() -> int:
    return _load().ora_num_threads()


def set_num_threads(n: int) -> None:
    _load().ora_set_num_threads(int(n))


def num_clusters(nclust: int, L: int) -> int:
    return _load().ora_num_clusters(nclust, L)


def radius(W: int) -> int:
    return _load().ora_radius(W)


def _mask(valid, lead: tuple, L: int) -> Optional[np.ndarray]:
    """Key-padding mask as int32 [*lead, L] (one row per slice), or None.

    valid is either per slice ([*lead, L]) or per batch row ([B, L] for
    tensors [B, H, L, d], shared by the H heads); nonzero = real token.
    """
    if valid is None:
        return None
    v = np.asarray(valid)
    if v.shape == tuple(lead) + (L,):
        out = v
    elif len(lead) == 2 and v.shape == (lead[0], L):
        out = np.broadcast_to(v[:, None, :], tuple(lead) + (L,))
    else:
        raise ValueError("mask shape %s does not fit slices %s x %d" % (v.shape, lead, L))
    return np.ascontiguousarray(out != 0, dtype=np.int32)


def _slices(x: np.ndarray):
    """View [..., L, d] as S slices; returns (array, S, L, d)."""
    x = _f64(x)
    L, d = x.shape[-2], x.shape[-1]
    S = int(np.prod(x.shape[:-2])) if x.ndim > 2 else 1
    return x, S, L, d


# listing-compatible variants (flags of forward), see oracle.c
INIT_STEP, KEEP_EMPTY, SOFT_GATHER, BAND, ALPHA_LOGIT = 1, 2, 4, 8, 16
LISTING = INIT_STEP | KEEP_EMPTY | SOFT_GATHER | BAND | ALPHA_LOGIT


def init_centroids(Q, K: int, step: bool = False) -> np.ndarray:
    """mu^(0) = Q[floor(k L / K)], or Q[k * max(1, L // K)] with step=True."""
    Q, S, L, d = _slices(Q)
    mu = np.empty(Q.shape[:-2] + (K, d))
    fn = _load().ora_init_centroids_step if step else _load().ora_init_centroids
    fn(_p(Q), S, L, d, K, _p(mu))
    return mu


def assign(Q, mu):
    """Returns (c, dbest, gap, qn2) for one assignment step against mu."""
    Q, S, L, d = _slices(Q)
    mu = _f64(mu)
    K = mu.shape[-2]
    c = np.empty(Q.shape[:-1], np.int32)
    dbest = np.empty(Q.shape[:-1])
    gap = np.empty(Q.shape[:-1])
    qn2 = np.empty(Q.shape[:-1])
    _load().ora_assign(_p(Q), _p(mu), S, L, d, K, _p(c), _p(dbest), _p(gap), _p(qn2))
    return c, dbest, gap, qn2


def update(Q, c, K: int, prev=None):
    """Returns (mu, counts) for one update step from assignment c; with prev
    (the previous centroids) an empty cluster keeps its previous centroid."""
    Q, S, L, d = _slices(Q)
    c = _i32(c)
    pv = _f64(prev) if prev is not None else None
    mu = np.empty(Q.shape[:-2] + (K, d))
    counts = np.empty(Q.shape[:-2] + (K,), np.int32)
    _load().ora_update(_p(Q), _p(c), S, L, d, K, _p(pv), _p(mu), _p(counts))
    return mu, counts


def soft_gather(Q, mu, vcent) -> np.ndarray:
    """G_i = sum_k softmax_k(q_i . mu_k / sqrt(d)) vcent_k."""
    Q, S, L, d = _slices(Q)
    mu, vcent = _f64(mu), _f64(vcent)
    G = np.empty(Q.shape)
    _load().ora_soft_gather(_p(Q), _p(mu), _p(vcent), S, L, d, mu.shape[-2], _p(G))
    return G


def objective(Q, mu, c) -> np.ndarray:
    Q, S, L, d = _slices(Q)
    mu = _f64(mu)
    c = _i32(c)
    J = np.empty(Q.shape[:-2] if Q.ndim > 2 else (1,))
    _load().ora_objective(_p(Q), _p(mu), _p(c), S, L, d, mu.shape[-2], _p(J))
    return J


def centroid_xattn(mu, Kt, V, valid=None):
    """Returns (V^cent, probability row sums); valid: optional key-padding mask."""
    Kt, S, L, d = _slices(Kt)
    mu = _f64(mu)
    V = _f64(V)
    K = mu.shape[-2]
    vm = _mask(valid, Kt.shape[:-2], L)
    vc = np.empty(mu.shape)
    ps = np.empty(mu.shape[:-1])
    _load().ora_centroid_xattn(_p(mu), _p(Kt), _p(V), S, L, d, K, _p(vm), _p(vc), _p(ps))
    return vc, ps


def local_attn(Q, Kt, V, W: int, valid=None):
    """Returns (O^loc, probability row sums); valid: optional key-padding mask."""
    Q, S, L, d = _slices(Q)
    Kt = _f64(Kt)
    V = _f64(V)
    vm = _mask(valid, Q.shape[:-2], L)
    o = np.empty(Q.shape)
    ps = np.empty(Q.shape[:-1])
    _load().ora_local_attn(_p(Q), _p(Kt), _p(V), S, L, d, W, _p(vm), _p(o), _p(ps))
    return o, ps


def fuse(vcent, c, oloc, alpha: float, valid=None) -> np.ndarray:
    oloc, S, L, d = _slices(oloc)
    vcent = _f64(vcent)
    c = _i32(c)
    vm = _mask(valid, oloc.shape[:-2], L)
    out = np.empty(oloc.shape)
    _load().ora_fuse(_p(vcent), _p(c), _p(oloc), S, L, d, vcent.shape[-2],
                     float(alpha), _p(vm), None, _p(out))
    return out


def forward(Q, Kt, V, nclust: int, iters: int, W: int, alpha: float,
            trace: bool = True, valid=None, flags: int = 0) -> Dict[str, np.ndarray]:
    """Whole forward pass; Q, K, V are float64 [B, H, L, d]; valid: optional
    key-padding mask [B, L] or [B, H, L] (nonzero = real token); flags:
    listing-compatible variants (INIT_STEP, KEEP_EMPTY, SOFT_GATHER, BAND,
    ALPHA_LOGIT)."""
    Q, Kt, V = _f64(Q), _f64(Kt), _f64(V)
    B, H, L, d = Q.shape
    S = B * H
    vm = _mask(valid, (B, H), L)
    K = num_clusters(nclust, L)
    out = np.empty(Q.shape)
    c = np.empty((B, H, L), np.int32)
    res = {"out": out, "assign": c, "K": K}
    if trace:
        res.update(
            mu_hist=np.empty((iters + 1, B, H, K, d)),
            c_hist=np.empty((iters, B, H, L), np.int32),
            gap_hist=np.empty((iters, B, H, L)),
            J=np.empty((iters, B, H)),
            Jp=np.empty((iters, B, H)),
            qn2=np.empty((B, H, L)),
            vcent=np.empty((B, H, K, d)),
            oloc=np.empty((B, H, L, d)),
        )
    g = res.get
    rc = _load().ora_forward(
        _p(Q), _p(Kt), _p(V), B, H, L, d, nclust, iters, W, float(alpha), _p(vm), int(flags),
        _p(out), _p(c), _p(g("mu_hist")), _p(g("c_hist")), _p(g("gap_hist")),
        _p(g("J")), _p(g("Jp")), _p(g("qn2")), _p(g("vcent")), _p(g("oloc")))
    if rc < 0:
        raise ValueError("oracle: invalid arguments")
    if trace:
        res["mu"] = res["mu_hist"][-1]
    return res


def backward(Q, Kt, V, dO, c, K: int, W: int, alpha: float, valid=None):
    """Gradients of sum(dO * O) for the forward with the final assignment c
    held fixed (equations' rules): returns dQ, dK, dV (shapes of Q, K, V) and
    dalpha (a float, summed over every slice)."""
    Q, S, L, d = _slices(Q)
    vm = _mask(valid, Q.shape[:-2], L)
    Kt, V, dO, c = _f64(Kt), _f64(V), _f64(dO), _i32(c)
    if c.size and (c.min() < 0 or c.max() >= K):
        raise ValueError("assignment out of range")
    dQ, dK, dV = np.empty(Q.shape), np.empty(Q.shape), np.empty(Q.shape)
    da = ctypes.c_double(0.0)
    _load().ora_backward(_p(Q), _p(Kt), _p(V), _p(dO), S, L, d, K, _p(c), W, float(alpha),
                         _p(vm), _p(dQ), _p(dK), _p(dV), ctypes.byref(da))
    return dQ, dK, dV, da.value


def exact_attention(Q, Kt, V, causal: bool, qvalid=None, kvalid=None) -> np.ndarray:
    """Decoder / cross-attention branch: exact attention over all keys with the
    -10000 fill for padded keys and (causal) future keys; padded queries give
    zero rows. Q [B, H, L, d]; K, V [B, H, Nk, d]; qvalid [B, L] and kvalid
    [B, Nk] (or per slice), nonzero = real token."""
    Q, S, L, d = _slices(Q)
    Kt, V = _f64(Kt), _f64(V)
    Nk = Kt.shape[-2]
    qm = _mask(qvalid, Q.shape[:-2], L)
    km = _mask(kvalid, Q.shape[:-2], Nk)
    out = np.empty(Q.shape)
    _load().ora_exact_attention(_p(Q), _p(Kt), _p(V), S, L, Nk, d, int(bool(causal)), _p(qm),
                                _p(km), _p(out))
    return out


def forward_from_assign(Q, Kt, V, c, K: int, W: int, alpha: float, valid=None,
                        flags: int = 0, mu=None):
    """Steps after clustering from a given final assignment c (e.g. the GPU's);
    mu: the final centroids (default: the update of c)."""
    Q, S, L, d = _slices(Q)
    vm = _mask(valid, Q.shape[:-2], L)
    mu_in = _f64(mu) if mu is not None else None
    Kt, V, c = _f64(Kt), _f64(V), _i32(c)
    if c.size and (c.min() < 0 or c.max() >= K):
        raise ValueError("assignment out of range")
    out = np.empty(Q.shape)
    mu = np.empty(Q.shape[:-2] + (K, d))
    vc = np.empty(Q.shape[:-2] + (K, d))
    ol = np.empty(Q.shape)
    _load().ora_forward_from_assign(_p(Q), _p(Kt), _p(V), S, L, d, K, _p(c), W,
                                    float(alpha), _p(vm), int(flags), _p(mu_in), _p(out),
                                    _p(mu), _p(vc), _p(ol))
    return {"out": out, "mu": mu, "vcent": vc, "oloc": ol}


def matmul(A, Bm) -> np.ndarray:
    A, Bm = _f64(A), _f64(Bm)
    M, P = A.shape
    P2, N = Bm.shape
    assert P == P2
    C = np.empty((M, N))
    _load().ora_matmul(_p(A), _p(Bm), M, P, N, _p(C))
    return C


def round_bf16(x) -> np.ndarray:
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    _load().ora_round_bf16_array(_p(x), x.size)
    return x


def repeat_kv(x, G: int) -> np.ndarray:
    """Grouped K/V heads: [B, Hkv, L, d] -> [B, Hkv*G, L, d], query head h
    reading K/V head h // G (the repeat_kv step of the ClusterAttention
    listing on the "Hooshaai/svd-sst2-roberta-cluster" page, read as the
    usual consecutive grouping)."""
    x = _f64(x)
    return np.ascontiguousarray(np.repeat(x, int(G), axis=1))


def fold_kv(x, G: int) -> np.ndarray:
    """Adjoint of repeat_kv: [B, Hkv*G, L, d] -> [B, Hkv, L, d], summing the
    G query heads that share a K/V head (their K/V gradients add up)."""
    x = _f64(x)
    B, H = x.shape[:2]
    return np.ascontiguousarray(x.reshape(B, H // int(G), int(G), *x.shape[2:]).sum(axis=2))


def split_heads(x2d: np.ndarray, B: int, L: int, H: int, d: int) -> np.ndarray:
    """[B*L, H*d] -> [B, H, L, d]; head h is columns h*d .. h*d+d-1."""
    return np.ascontiguousarray(x2d.reshape(B, L, H, d).transpose(0, 2, 1, 3))


def merge_heads(x: np.ndarray) -> np.ndarray:
    """[B, H, L, d] -> [B*L, H*d]."""
    B, H, L, d = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B * L, H * d))


def project_qkv(X, Wq, Wk, Wv, H: int):
    """Q, K, V = X W (fp64), rounded to bf16 storage, split into heads.

    X is [B, L, Dm]; each W is [Dm, H*d] (Y = X W, no bias), following the
    model card's pipeline figure (multi-head projections of X, Y = O W_O).
    """
    X = _f64(X)
    B, L, Dm = X.shape
    X2 = X.reshape(B * L, Dm)
    outs = []
    for Wm in (Wq, Wk, Wv):
        Wm = _f64(Wm)
        d = Wm.shape[1] // H
        outs.append(split_heads(round_bf16(matmul(X2, Wm)), B, L, H, d))
    return outs


def output_projection(O_bhld, Wo) -> np.ndarray:
    """Y = round_bf16(O) merged over heads times W_O: [B, L, Dm] in fp64."""
    B, H, L, d = O_bhld.shape
    Om = merge_heads(round_bf16(O_bhld))
    Y = matmul(Om, _f64(Wo))
    return Y.reshape(B, L, -1)


def layer_forward(X, Wq, Wk, Wv, Wo, H: int, nclust: int, iters: int, W: int,
                  alpha: float) -> Dict[str, np.ndarray]:
    """Full layer: projections, cluster attention, output projection."""
    q, k, v = project_qkv(X, Wq, Wk, Wv, H)
    att = forward(q, k, v, nclust, iters, W, alpha, trace=True)
    att["Y"] = output_projection(att["out"], Wo)
    att["q"], att["k"], att["v"] = q, k, v
    return att
