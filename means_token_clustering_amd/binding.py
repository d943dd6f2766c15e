"""ctypes binding of libclusterattn.so (the C ABI in include/clusterattn.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing, every call raises.
The Python names match the C entry points.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libclusterattn.so")

CA_OK, CA_ERR_INVALID_ARG, CA_ERR_UNSUPPORTED, CA_ERR_HIP = 0, 1, 2, 3
CA_ERR_SCRATCH_TOO_SMALL = 4
CA_NOALLOC_SCRATCH_BYTES = 64 << 20
CA_F32, CA_BF16 = 0, 1
CA_PATH_AUTO, CA_PATH_FUSED, CA_PATH_STAGED, CA_PATH_SEGMENTED = 0, 1, 2, 3
# listing-compatible variants (ca_options_t.flags)
CA_FLAG_INIT_STEP, CA_FLAG_KEEP_EMPTY, CA_FLAG_SOFT_GATHER, CA_FLAG_BAND = 1, 2, 4, 8
CA_FLAG_ALPHA_LOGIT = 16
CA_FLAG_LISTING = 31

_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "ca_status_string": (ctypes.c_char_p, [_i]),
    "ca_version": (_i, []),
    "cluster_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "cluster_attn_plan": (ctypes.c_char_p, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "cluster_attn_plan_dt": (ctypes.c_char_p, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "cluster_attn_workspace_size_ex": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "cluster_attn_forward": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i,
                                  _vp, _sz, _vp]),
    "cluster_attn_forward_ex": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                     _i, _vp, _sz, _i, _vp]),
    "cluster_attn_forward_masked": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                                         _vp, _i, _vp, _sz, _i, _vp]),
    "cluster_attn_forward_opts": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                       _vp, _i, _vp, _sz, _i, _vp]),
    "cluster_attn_forward_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                                          _vp, _vp, _i, _i, _vp]),
    "ca_kmeans_assign": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "ca_kmeans_scores": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "ca_centroid_update": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "ca_centroid_update_workspace_size": (_sz, [_i, _i, _i, _i]),
    "ca_centroid_xattn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "ca_centroid_xattn_workspace_size": (_sz, [_i, _i, _i, _i]),
    "ca_local_window_attn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "ca_gather_fuse": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "cluster_attn_layer_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "cluster_attn_layer_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                        _f, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ca_gemm_bf16": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp]),
    "ca_gemm_bf16_kn": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp]),
    "cluster_attn_exact_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp,
                                        _i, _vp]),
    "cluster_attn_backward_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "cluster_attn_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                   _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
}


class CaOptions(ctypes.Structure):
    """ca_options_t of the C ABI."""
    _fields_ = [("valid", _vp), ("kv_heads", _i), ("flags", _i), ("assign_hist", _vp)]


class CaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib():
    """Load libclusterattn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it first "
                    "(python -m means_token_clustering_amd.build)")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
        return _lib


def status_string(status: int) -> str:
    return lib().ca_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != CA_OK:
        raise CaError(status, where)


# ------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return CA_F32
    if t.dtype == torch.bfloat16:
        return CA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        return workspace
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _aligned_ptr(ws) -> Optional[int]:
    if ws is None:
        return None
    p = ws.data_ptr()
    return (p + 255) // 256 * 256


def _ws_bytes(ws) -> int:
    if ws is None:
        return 0
    p = ws.data_ptr()
    return ws.numel() * ws.element_size() - ((p + 255) // 256 * 256 - p)


def cluster_attn_plan(B, H, L, nclust, W, flags=0, masked=False, path=CA_PATH_AUTO,
                      dtype=CA_F32):
    """Name of the launch sequence the forward takes for these arguments and
    storage type (None when the call would be rejected)."""
    r = lib().cluster_attn_plan_dt(B, H, L, nclust, W, int(flags), int(bool(masked)), int(path),
                                   int(dtype))
    return r.decode() if r is not None else None


def cluster_attn_workspace_size(B, H, L, d, nclust, dtype=CA_F32, path=CA_PATH_AUTO) -> int:
    return lib().cluster_attn_workspace_size_ex(B, H, L, d, nclust, dtype, path)


def cluster_attn_forward(Q, K, V, nclust: int, iters: int, W: int, alpha: float, out=None,
                         assign_out=None, path: int = CA_PATH_AUTO, workspace=None,
                         stream=None, want_assign: bool = True, valid=None, flags: int = 0,
                         assign_hist=None):
    """Q: contiguous [B, H, L, d] float32 or bfloat16 GPU tensor; K, V:
    [B, Hkv, L, d] of the same dtype, Hkv dividing H (Hkv < H: grouped K/V
    heads, cluster_attn_forward_opts).

    valid: optional key-padding mask, a contiguous [B, L] uint8 (or bool) GPU
    tensor, nonzero = real token (cluster_attn_forward_masked). flags: OR of
    CA_FLAG_* (listing-compatible variants, cluster_attn_forward_opts).
    assign_hist: optional int32 GPU tensor [iters, B, H, L] receiving every
    iteration's assignment (ca_options_t.assign_hist).
    Returns (out, assign_out); allocates out/assign_out/workspace with torch
    when not given.
    """
    torch = _torch()
    B, H, L, d = Q.shape
    dt = _dtype_code(Q)
    if out is None:
        out = torch.empty_like(Q)
    if assign_out is None and want_assign:
        assign_out = torch.empty((B, H, L), dtype=torch.int32, device=Q.device)
    need = cluster_attn_workspace_size(B, H, L, d, nclust, dt, path)
    ws = _workspace(need, Q.device, workspace)
    hkv = K.shape[1]
    if tuple(V.shape) != tuple(K.shape) or K.shape[0] != B or K.shape[2:] != Q.shape[2:]:
        raise ValueError("K and V must be [B, Hkv, L, d] with Q's B, L and d")
    if valid is not None and (tuple(valid.shape) != (B, L) or valid.element_size() != 1):
        raise ValueError("valid must be a [B, L] tensor of one-byte elements")
    if assign_hist is not None and (tuple(assign_hist.shape) != (iters, B, H, L)
                                    or assign_hist.dtype != torch.int32):
        raise ValueError("assign_hist must be an int32 [iters, B, H, L] tensor")
    if hkv != H or flags or assign_hist is not None:
        opts = CaOptions(_ptr(valid), hkv, int(flags), _ptr(assign_hist))
        st = lib().cluster_attn_forward_opts(
            _ptr(Q), _ptr(K), _ptr(V), B, H, L, d, nclust, iters, W, float(alpha),
            ctypes.byref(opts), _ptr(out), _ptr(assign_out), dt, _aligned_ptr(ws), _ws_bytes(ws),
            path, _stream(stream))
        _check(st, "cluster_attn_forward_opts")
        return out, assign_out
    if valid is not None:
        st = lib().cluster_attn_forward_masked(
            _ptr(Q), _ptr(K), _ptr(V), _ptr(valid), B, H, L, d, nclust, iters, W, float(alpha),
            _ptr(out), _ptr(assign_out), dt, _aligned_ptr(ws), _ws_bytes(ws), path,
            _stream(stream))
        _check(st, "cluster_attn_forward_masked")
        return out, assign_out
    st = lib().cluster_attn_forward_ex(
        _ptr(Q), _ptr(K), _ptr(V), B, H, L, d, nclust, iters, W, float(alpha), _ptr(out),
        _ptr(assign_out), dt, _aligned_ptr(ws), _ws_bytes(ws), path, _stream(stream))
    _check(st, "cluster_attn_forward")
    return out, assign_out


def cluster_attn_backward(Q, K, V, dO, assign, nclust: int, W: int, alpha: float, valid=None,
                          dQ=None, dK=None, dV=None, workspace=None, stream=None,
                          want_dalpha: bool = True):
    """Gradients of sum(dO * O) of the forward with its final assignment
    `assign` held fixed. Q, dO: [B, H, L, d]; K, V: [B, Hkv, L, d]; valid:
    the forward's key-padding mask or None. Returns (dQ, dK, dV, dalpha), with
    dalpha a one-element float32 GPU tensor (None unless want_dalpha)."""
    torch = _torch()
    B, H, L, d = Q.shape
    hkv = K.shape[1]
    dt = _dtype_code(Q)
    if tuple(V.shape) != tuple(K.shape) or tuple(dO.shape) != tuple(Q.shape):
        raise ValueError("K, V must share a shape and dO must match Q")
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.empty_like(K) if dK is None else dK
    dV = torch.empty_like(V) if dV is None else dV
    da = torch.empty(1, dtype=torch.float32, device=Q.device) if want_dalpha else None
    need = lib().cluster_attn_backward_workspace_size(B, H, hkv, L, d, nclust, dt)
    ws = _workspace(need, Q.device, workspace)
    st = lib().cluster_attn_backward(
        _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(assign), _ptr(valid), B, H, hkv, L, d, nclust,
        W, float(alpha), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(da), dt, _aligned_ptr(ws),
        _ws_bytes(ws), _stream(stream))
    _check(st, "cluster_attn_backward")
    return dQ, dK, dV, da


def cluster_attn_exact_forward(Q, K, V, causal: bool, q_valid=None, k_valid=None, out=None,
                               stream=None):
    """Exact attention of the decoder / cross-attention branch. Q: [B, H, L, d];
    K, V: [B, Hkv, Nk, d]; q_valid [B, L] and k_valid [B, Nk] one-byte masks or
    None. Returns out [B, H, L, d]."""
    torch = _torch()
    B, H, L, d = Q.shape
    hkv, Nk = K.shape[1], K.shape[2]
    if tuple(V.shape) != tuple(K.shape):
        raise ValueError("K and V must share a shape")
    out = torch.empty_like(Q) if out is None else out
    st = lib().cluster_attn_exact_forward(_ptr(Q), _ptr(K), _ptr(V), _ptr(q_valid), _ptr(k_valid),
                                          B, H, hkv, L, Nk, d, int(bool(causal)), _ptr(out),
                                          _dtype_code(Q), _stream(stream))
    _check(st, "cluster_attn_exact_forward")
    return out


def ca_kmeans_assign(Q, mu, Kc: int, assign=None, stream=None):
    torch = _torch()
    B, H, L, d = Q.shape
    if assign is None:
        assign = torch.empty((B, H, L), dtype=torch.int32, device=Q.device)
    st = lib().ca_kmeans_assign(_ptr(Q), _ptr(mu), B * H, L, d, Kc, _dtype_code(Q), _ptr(assign),
                                _stream(stream))
    _check(st, "ca_kmeans_assign")
    return assign


def ca_kmeans_scores(Q, mu, scores=None, stream=None):
    """Scores mu_k . q_i - ||mu_k||^2 / 2 of the matrix-core assignment step:
    Q [B, H, L, d], mu fp32 [B, H, Kc, d]; returns fp32 [B, H, L, Kc]."""
    torch = _torch()
    B, H, L, d = Q.shape
    Kc = mu.shape[2]
    if scores is None:
        scores = torch.empty((B, H, L, Kc), dtype=torch.float32, device=Q.device)
    st = lib().ca_kmeans_scores(_ptr(Q), _ptr(mu), B * H, L, d, Kc, _dtype_code(Q), _ptr(scores),
                                _stream(stream))
    _check(st, "ca_kmeans_scores")
    return scores


def ca_centroid_update(Q, assign, Kc: int, stream=None):
    torch = _torch()
    B, H, L, d = Q.shape
    mu = torch.empty((B, H, Kc, d), dtype=torch.float32, device=Q.device)
    counts = torch.empty((B, H, Kc), dtype=torch.int32, device=Q.device)
    need = lib().ca_centroid_update_workspace_size(B * H, L, d, Kc)
    ws = _workspace(need, Q.device, None)
    st = lib().ca_centroid_update(_ptr(Q), _ptr(assign), B * H, L, d, Kc, _dtype_code(Q),
                                  _ptr(mu), _ptr(counts), _aligned_ptr(ws), _ws_bytes(ws),
                                  _stream(stream))
    _check(st, "ca_centroid_update")
    return mu, counts


def ca_centroid_xattn(mu, K, V, stream=None):
    torch = _torch()
    B, H, L, d = K.shape
    Kc = mu.shape[-2]
    vcent = torch.empty((B, H, Kc, d), dtype=torch.float32, device=K.device)
    need = lib().ca_centroid_xattn_workspace_size(B * H, L, d, Kc)
    ws = _workspace(need, K.device, None)
    st = lib().ca_centroid_xattn(_ptr(mu), _ptr(K), _ptr(V), B * H, L, d, Kc, _dtype_code(K),
                                 _ptr(vcent), _aligned_ptr(ws), _ws_bytes(ws), _stream(stream))
    _check(st, "ca_centroid_xattn")
    return vcent


def ca_local_window_attn(Q, K, V, W: int, stream=None):
    torch = _torch()
    B, H, L, d = Q.shape
    oloc = torch.empty((B, H, L, d), dtype=torch.float32, device=Q.device)
    st = lib().ca_local_window_attn(_ptr(Q), _ptr(K), _ptr(V), B * H, L, d, W, _dtype_code(Q),
                                    _ptr(oloc), _stream(stream))
    _check(st, "ca_local_window_attn")
    return oloc


def ca_gather_fuse(vcent, assign, oloc, alpha: float, dtype, stream=None):
    torch = _torch()
    B, H, L, d = oloc.shape
    Kc = vcent.shape[-2]
    out = torch.empty((B, H, L, d), dtype=dtype, device=oloc.device)
    st = lib().ca_gather_fuse(_ptr(vcent), _ptr(assign), _ptr(oloc), B * H, L, d, Kc,
                              float(alpha), _dtype_code(out), _ptr(out), _stream(stream))
    _check(st, "ca_gather_fuse")
    return out


def cluster_attn_layer_forward(X, Wq, Wk, Wv, Wo, H: int, nclust: int, iters: int, W: int,
                               alpha: float, want_qkv: bool = False, stream=None):
    """X [B, L, Dm] and W* [Dm, Dm] bfloat16 GPU tensors; returns (Y, assign, qkv)."""
    torch = _torch()
    B, L, Dm = X.shape
    d = Dm // H
    Y = torch.empty((B, L, Dm), dtype=torch.bfloat16, device=X.device)
    assign = torch.empty((B, H, L), dtype=torch.int32, device=X.device)
    qkv = torch.empty((3, B, H, L, d), dtype=torch.bfloat16, device=X.device) if want_qkv else None
    need = lib().cluster_attn_layer_workspace_size(B, L, Dm, H, d, nclust)
    ws = _workspace(need, X.device, None)
    st = lib().cluster_attn_layer_forward(
        _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo), B, L, Dm, H, d, nclust, iters, W,
        float(alpha), _ptr(Y), _ptr(assign), _ptr(qkv), _aligned_ptr(ws), _ws_bytes(ws),
        _stream(stream))
    _check(st, "cluster_attn_layer_forward")
    return Y, assign, qkv


def ca_gemm_bf16(A, Bt, stream=None):
    """C = A Bt^T for bfloat16 GPU tensors A [M, Kd] and Bt [N, Kd]; returns C [M, N]."""
    torch = _torch()
    M, Kd = A.shape
    N, Kb = Bt.shape
    if Kb != Kd:
        raise ValueError("A and Bt disagree on the contraction length")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    st = lib().ca_gemm_bf16(_ptr(A), _ptr(Bt), M, N, Kd, _ptr(C), _stream(stream))
    _check(st, "ca_gemm_bf16")
    return C


def ca_gemm_bf16_kn(A, W, stream=None):
    """C = A W for bfloat16 GPU tensors A [M, Kd] and W [Kd, N] ([in, out]); returns C [M, N]."""
    torch = _torch()
    M, Kd = A.shape
    Kw, N = W.shape
    if Kw != Kd:
        raise ValueError("A and W disagree on the contraction length")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    st = lib().ca_gemm_bf16_kn(_ptr(A), _ptr(W), M, N, Kd, _ptr(C), _stream(stream))
    _check(st, "ca_gemm_bf16_kn")
    return C
