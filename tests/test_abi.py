"""C ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments on the host (before any
launch), with the documented status codes. Pointers here are fake, aligned
addresses: every call below must fail validation and never touch them."""
import ctypes
import os
import re

import pytest

from means_token_clustering_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clusterattn.h")

INV, UNS = b.CA_ERR_INVALID_ARG, b.CA_ERR_UNSUPPORTED

# distinct, non-overlapping, 256-aligned fake device addresses
Q, K, V, OUT, ASG, WS = (0x10000000 * (i + 1) for i in range(6))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:ca|cluster_attn)_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = b.lib()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
        assert name in b.SIGNATURES, name


def test_flag_values_match_header():
    text = open(HEADER).read()
    defs = {m[0]: int(m[1]) for m in re.findall(r"#define (CA_FLAG_\w+) (\d+)", text)}
    assert defs == {"CA_FLAG_INIT_STEP": 1, "CA_FLAG_KEEP_EMPTY": 2, "CA_FLAG_SOFT_GATHER": 4,
                    "CA_FLAG_BAND": 8, "CA_FLAG_ALPHA_LOGIT": 16, "CA_FLAG_LISTING": 31}
    for name, value in defs.items():
        assert getattr(b, name) == value, name


def test_status_strings():
    assert b.status_string(b.CA_OK) == "ok"
    assert b.status_string(INV) == "invalid argument"
    assert b.status_string(UNS).startswith("unsupported")
    assert b.status_string(b.CA_ERR_HIP).startswith("HIP")
    assert b.lib().ca_version() >= 100


def fwd(**kw):
    a = dict(Q=Q, K=K, V=V, B=2, H=3, L=128, d=64, nclust=16, iters=3, W=32, alpha=0.5,
             out=OUT, assign=ASG, dt=b.CA_F32, ws=WS, wsb=1 << 30, path=b.CA_PATH_STAGED)
    a.update(kw)
    return b.lib().cluster_attn_forward_ex(a["Q"], a["K"], a["V"], a["B"], a["H"], a["L"], a["d"],
                                           a["nclust"], a["iters"], a["W"], a["alpha"], a["out"],
                                           a["assign"], a["dt"], a["ws"], a["wsb"], a["path"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(K=None), INV), (dict(V=None), INV), (dict(out=None), INV),
    (dict(B=0), INV), (dict(H=-1), INV), (dict(L=0), INV), (dict(d=0), INV),
    (dict(nclust=0), INV), (dict(iters=0), INV), (dict(W=-1), INV),
    (dict(alpha=-0.1), INV), (dict(alpha=1.5), INV), (dict(alpha=float("nan")), INV),
    (dict(dt=7), INV), (dict(path=9), INV),
    (dict(Q=Q + 4), INV), (dict(out=OUT + 8), INV), (dict(assign=ASG + 2), INV),
    (dict(out=Q), INV), (dict(out=K + 1024), INV), (dict(assign=OUT + 4096), INV),
    (dict(ws=None), INV), (dict(wsb=16), INV), (dict(ws=WS + 16), INV), (dict(ws=OUT), INV),
    (dict(d=32), UNS), (dict(d=128), UNS), (dict(nclust=300, L=400), UNS),
    (dict(B=1 << 12, H=1 << 8, L=4096), UNS), (dict(B=1 << 16, H=1 << 10, L=4096), INV),
])
def test_forward_rejects(kw, code):
    assert fwd(**kw) == code


def test_fused_path_unsupported_shapes():
    # the single-launch paths take L <= 512 with at most 16 clusters, and
    # beyond 128 tokens a window radius <= 16
    assert fwd(path=b.CA_PATH_FUSED, L=5000) == UNS
    assert fwd(path=b.CA_PATH_FUSED, L=300, nclust=17) == UNS
    assert fwd(path=b.CA_PATH_FUSED, L=513) == UNS
    assert fwd(path=b.CA_PATH_FUSED, L=300, W=34) == UNS
    assert fwd(path=b.CA_PATH_FUSED, L=128, nclust=17) == UNS


def test_workspace_sizes():
    lib = b.lib()
    staged = b.cluster_attn_workspace_size(32, 12, 128, 64, 16, b.CA_F32, b.CA_PATH_STAGED)
    assert staged > 0 and staged % 256 == 0
    assert b.cluster_attn_workspace_size(1, 12, 8192, 64, 64, b.CA_F32, b.CA_PATH_STAGED) > 0
    assert b.cluster_attn_workspace_size(1, 1, 128, 32, 16) == 0          # unsupported d
    assert lib.ca_centroid_update_workspace_size(4, 100, 64, 8) > 0
    assert lib.ca_centroid_xattn_workspace_size(4, 64, 64, 8) == 0         # one key range
    assert lib.ca_centroid_xattn_workspace_size(1024, 128, 64, 8) == 0     # enough slices
    assert lib.ca_centroid_xattn_workspace_size(4, 8192, 64, 8) > 0


def test_step_entry_points_reject():
    lib = b.lib()
    assert lib.ca_kmeans_assign(None, None, 1, 8, 64, 2, 0, ASG, None) == INV
    assert lib.ca_kmeans_assign(Q, None, 1, 8, 64, 9, 0, ASG, None) == INV   # init needs Kc <= L
    assert lib.ca_kmeans_assign(Q, None, 1, 8, 64, 300, 0, ASG, None) == UNS
    assert lib.ca_kmeans_assign(Q, None, 1, 8, 48, 2, 0, ASG, None) == UNS
    assert lib.ca_centroid_update(Q, ASG, 1, 8, 64, 2, 0, OUT, None, None, 0, None) == INV
    assert lib.ca_centroid_update(Q, ASG, 1, 8, 64, 2, 0, OUT, None, WS, 1, None) == INV
    assert lib.ca_centroid_xattn(None, K, V, 1, 8, 64, 2, 0, OUT, None, 0, None) == INV
    assert lib.ca_local_window_attn(Q, K, V, 1, 8, 64, -2, 0, OUT, None) == INV
    assert lib.ca_gather_fuse(Q, ASG, V, 1, 8, 64, 2, 2.0, 0, OUT, None) == INV
    assert lib.ca_gather_fuse(Q, ASG, V, 1, 8, 64, 2, 0.5, 5, OUT, None) == INV


def test_scores_entry_point_rejects():
    lib = b.lib()
    assert lib.ca_kmeans_scores(None, K, 1, 8, 64, 2, 0, OUT, None) == INV
    assert lib.ca_kmeans_scores(Q, None, 1, 8, 64, 2, 0, OUT, None) == INV
    assert lib.ca_kmeans_scores(Q, K, 1, 8, 64, 65, 0, OUT, None) == UNS   # matrix-core step only
    assert lib.ca_kmeans_scores(Q, K, 1, 8, 48, 2, 0, OUT, None) == UNS
    assert lib.ca_kmeans_scores(Q, K, 1, 8, 64, 2, 0, Q + 64, None) == INV  # scores over Q
    assert lib.ca_kmeans_scores(Q, K, 1, 8, 64, 2, 0, OUT + 2, None) == INV


def test_noalloc_rejects_before_any_launch():
    """The allocation-free forward checks its workspace need against the
    device array before touching the GPU (fake pointers here)."""
    lib = b.lib()
    need = b.cluster_attn_workspace_size(1, 12, 16384, 64, 64, b.CA_F32, b.CA_PATH_STAGED)
    assert need > b.CA_NOALLOC_SCRATCH_BYTES
    assert lib.cluster_attn_forward_noalloc(Q, K, V, 1, 12, 16384, 64, 64, 1, 32, 0.5, None, OUT,
                                            ASG, b.CA_F32, b.CA_PATH_STAGED, None) == 4
    assert b.status_string(4).startswith("the call needs more workspace")
    # single-launch shapes need no workspace: argument errors come first
    assert lib.cluster_attn_forward_noalloc(None, K, V, 2, 12, 128, 64, 16, 3, 32, 0.5, None, OUT,
                                            ASG, b.CA_F32, b.CA_PATH_AUTO, None) == INV
    assert lib.cluster_attn_forward_noalloc(Q, K, V, 2, 12, 128, 64, 16, 3, 32, 1.5, None, OUT,
                                            ASG, b.CA_F32, b.CA_PATH_AUTO, None) == INV


def test_plan_names():
    """The launch-sequence query follows the forward's own decision; without a
    GPU the CU count is unknown, so only the shape-decided plans are checked."""
    assert b.cluster_attn_plan(32, 12, 128, 16, 32) == "fused"
    assert b.cluster_attn_plan(1, 2, 300, 16, 32, path=b.CA_PATH_FUSED) == "fused512"
    assert b.cluster_attn_plan(1, 2, 300, 16, 32, masked=True, path=b.CA_PATH_FUSED) is None
    assert b.cluster_attn_plan(1, 2, 300, 16, 32, flags=b.CA_FLAG_KEEP_EMPTY).startswith(
        "staged: kmeans_mfma steps + reduce")
    assert b.cluster_attn_plan(1, 1, 600, 32, 32).startswith("staged: kmeans_mfma steps (chained)")
    assert b.cluster_attn_plan(1, 1, 300, 80, 32).startswith("staged: scalar kmeans steps")
    assert b.cluster_attn_plan(1, 1, 300, 16, 64).endswith("local_scalar")   # radius 32
    assert b.cluster_attn_plan(0, 1, 300, 16, 32) is None
    assert b.cluster_attn_plan(1, 1, 300, 16, -1) is None
    assert b.cluster_attn_plan(1, 1, 300, 16, 32, flags=64) is None


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        b.cluster_attn_forward(x, x, x, 2, 1, 4, 0.5, path=b.CA_PATH_STAGED,
                               out=torch.zeros(1, 1, 8, 64), assign_out=None, want_assign=False,
                               workspace=None)


def layer(**kw):
    X, WQ, WK, WV, WO, Y, LWS = (0x10000000 * (i + 10) for i in range(7))
    a = dict(X=X, Wq=WQ, Wk=WK, Wv=WV, Wo=WO, B=2, L=160, Dm=256, H=4, d=64, nclust=16,
             iters=3, W=32, alpha=0.5, Y=Y, assign=None, qkv=None, ws=LWS, wsb=1 << 28)
    a.update(kw)
    return b.lib().cluster_attn_layer_forward(
        a["X"], a["Wq"], a["Wk"], a["Wv"], a["Wo"], a["B"], a["L"], a["Dm"], a["H"], a["d"],
        a["nclust"], a["iters"], a["W"], a["alpha"], a["Y"], a["assign"], a["qkv"], a["ws"],
        a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), INV), (dict(Wo=None), INV), (dict(Y=None), INV), (dict(ws=None), INV),
    (dict(B=0), INV), (dict(Dm=0), INV), (dict(iters=0), INV), (dict(alpha=2.0), INV),
    (dict(X=0x100000a8), INV), (dict(ws=0x10000000 * 16 + 64), INV), (dict(wsb=4096), INV),
    (dict(Y=0x10000000 * 10 + 512), INV),                  # Y inside X
    (dict(qkv=0x10000000 * 16 + 4096), INV),               # qkv_out inside the workspace
    (dict(d=32, Dm=128), UNS), (dict(Dm=320), UNS),        # d != 64; Dm != H d
])
def test_layer_rejects(kw, code):
    assert layer(**kw) == code


def test_layer_workspace_size():
    lib = b.lib()
    n = lib.cluster_attn_layer_workspace_size(16, 512, 768, 12, 64, 16)
    # Q/K/V + O + staged attention workspace (no copy of the weights)
    assert n >= 4 * 16 * 512 * 768 * 2 and n % 256 == 0
    assert n < 4 * 768 * 768 * 2 + 4 * 16 * 512 * 768 * 2 + (64 << 20)
    assert lib.cluster_attn_layer_workspace_size(16, 512, 768, 12, 32, 16) == 0
    assert lib.cluster_attn_layer_workspace_size(16, 512, 700, 12, 64, 16) == 0


def test_gemm_rejects():
    lib = b.lib()
    A_, B_, C_ = Q, K, V
    assert lib.ca_gemm_bf16(None, B_, 64, 64, 64, C_, None) == INV
    assert lib.ca_gemm_bf16(A_, B_, 0, 64, 64, C_, None) == INV
    assert lib.ca_gemm_bf16(A_, B_, 64, 64, 64, A_ + 1024, None) == INV   # C overlaps A
    assert lib.ca_gemm_bf16(A_ + 8, B_, 64, 64, 64, C_, None) == INV
    assert lib.ca_gemm_bf16(A_, B_, 64, 100, 64, C_, None) == UNS
    assert lib.ca_gemm_bf16(A_, B_, 64, 64, 96, C_, None) == UNS
    for fn in (lib.ca_gemm_bf16, lib.ca_gemm_bf16_kn):
        assert fn(A_, None, 64, 64, 64, C_, None) == INV
        assert fn(A_, B_, 64, 64, 64, B_ + 2048, None) == INV   # C overlaps the weight
        assert fn(A_, B_, 64, 64, 64, C_ + 4, None) == INV
        assert fn(A_, B_, 64, 64, 0, C_, None) == INV
        assert fn(A_, B_, 64, 192, 32, C_, None) == UNS
        far = [1 << 44, 2 << 44, 3 << 44]   # distinct, 16-byte aligned, never touched
        assert fn(far[0], far[1], 64, 1 << 16, 1 << 15, far[2], None) == UNS   # N * Kd >= 2^31


MASK = 0x10000000 * 8


def fwd_masked(**kw):
    a = dict(Q=Q, K=K, V=V, valid=MASK, B=2, H=3, L=128, d=64, nclust=16, iters=3, W=32,
             alpha=0.5, out=OUT, assign=ASG, dt=b.CA_F32, ws=WS, wsb=1 << 30,
             path=b.CA_PATH_STAGED)
    a.update(kw)
    return b.lib().cluster_attn_forward_masked(
        a["Q"], a["K"], a["V"], a["valid"], a["B"], a["H"], a["L"], a["d"], a["nclust"],
        a["iters"], a["W"], a["alpha"], a["out"], a["assign"], a["dt"], a["ws"], a["wsb"],
        a["path"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(valid=None), INV), (dict(valid=OUT + 64), INV), (dict(valid=ASG), INV),
    (dict(valid=WS + 1024), INV), (dict(Q=None), INV), (dict(alpha=2.0), INV),
    (dict(iters=0), INV), (dict(ws=None), INV), (dict(d=32), UNS),
    (dict(path=b.CA_PATH_FUSED, L=5000), UNS),
    (dict(path=b.CA_PATH_FUSED, L=300), UNS),   # no single launch with a mask beyond 128
])
def test_masked_forward_rejects(kw, code):
    """The masked entry point runs the same host checks, plus: a mask is
    required and must not overlap the outputs or the workspace."""
    assert fwd_masked(**kw) == code


def _Opts(valid, kv_heads, flags, hist=None):
    return b.CaOptions(valid, kv_heads, flags, hist)


def test_options_layout_matches_header():
    """ca_options_t: valid, kv_heads, flags, assign_hist (the binding's mirror)."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} ca_options_t;", text, flags=re.S).group(1)
    fields = re.findall(r"(\w+);", body)
    assert fields == [f for f, _ in b.CaOptions._fields_]
    assert ctypes.sizeof(b.CaOptions) == 24


def fwd_opts(opts, **kw):
    a = dict(Q=Q, K=K, V=V, B=2, H=12, L=128, d=64, nclust=16, iters=3, W=32, alpha=0.5,
             out=OUT, assign=ASG, dt=b.CA_F32, ws=WS, wsb=1 << 30, path=b.CA_PATH_STAGED)
    a.update(kw)
    return b.lib().cluster_attn_forward_opts(
        a["Q"], a["K"], a["V"], a["B"], a["H"], a["L"], a["d"], a["nclust"], a["iters"], a["W"],
        a["alpha"], ctypes.byref(opts) if opts is not None else None, a["out"], a["assign"],
        a["dt"], a["ws"], a["wsb"], a["path"], None)


@pytest.mark.parametrize("opts,kw,code", [
    (_Opts(None, 5, 0), {}, INV),          # 12 heads do not split into 5 groups
    (_Opts(None, 24, 0), {}, INV),         # more K/V heads than query heads
    (_Opts(None, -1, 0), {}, INV),
    (_Opts(None, 4, 32), {}, INV),         # no such flag
    (_Opts(None, 4, -1), {}, INV),
    (_Opts(None, 4, 31), dict(W=-1), INV),  # the listing's flags keep the other checks
    (_Opts(None, 4, 16), dict(alpha=float("nan")), INV),
    (_Opts(None, 4, 16), dict(alpha=7.5, Q=None), INV),   # any finite parameter passes the alpha check
    (_Opts(None, 4, 0), dict(Q=None), INV),
    (_Opts(None, 4, 0), dict(out=K + 4096), INV),   # out overlaps the smaller K
    (_Opts(MASK, 3, 0), dict(alpha=-1.0), INV),
    (None, dict(ws=None), INV),
    (_Opts(None, 0, 0, WS + (1 << 29) + 2), {}, INV),      # trace not 4-byte aligned
    (_Opts(None, 0, 0, OUT + 64), {}, INV),                # trace over the output
    (_Opts(None, 0, 0, ASG - 4096), {}, INV),              # trace runs into assign_out
    (_Opts(None, 0, 0, WS + 4096), {}, INV),               # trace over the workspace
    (_Opts(MASK - 256, 0, 0, MASK - 512), {}, INV),        # trace over the mask
])
def test_opts_forward_rejects(opts, kw, code):
    assert fwd_opts(opts, **kw) == code


def bwd(**kw):
    a = dict(Q=Q, K=K, V=V, dO=OUT, assign=ASG, valid=None, B=2, H=4, Hkv=0, L=128, d=64,
             nclust=16, W=32, alpha=0.5, dQ=WS + (1 << 28), dK=WS + (2 << 28), dV=WS + (3 << 28),
             da=None, dt=b.CA_F32, ws=WS, wsb=1 << 27)
    a.update(kw)
    return b.lib().cluster_attn_backward(
        a["Q"], a["K"], a["V"], a["dO"], a["assign"], a["valid"], a["B"], a["H"], a["Hkv"], a["L"],
        a["d"], a["nclust"], a["W"], a["alpha"], a["dQ"], a["dK"], a["dV"], a["da"], a["dt"],
        a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(dO=None), INV), (dict(assign=None), INV), (dict(dK=None), INV),
    (dict(ws=None), INV), (dict(wsb=1024), INV), (dict(Hkv=3), INV), (dict(Hkv=8), INV),
    (dict(Hkv=-1), INV), (dict(W=-1), INV), (dict(alpha=float("nan")), INV),
    (dict(alpha=1.5), INV), (dict(dt=5), INV), (dict(B=0), INV),
    (dict(Q=Q + 4), INV), (dict(assign=ASG + 2), INV), (dict(da=WS + (4 << 28) + 2), INV),
    (dict(ws=WS + 64), INV),
    (dict(dQ=Q), INV),                  # an output over an input
    (dict(dK=WS + (1 << 28)), INV),     # two outputs over each other
    (dict(d=32), UNS), (dict(nclust=300, L=300), UNS),
])
def test_backward_rejects(kw, code):
    assert bwd(**kw) == code


def test_backward_workspace_size():
    lib = b.lib()
    n = lib.cluster_attn_backward_workspace_size(32, 12, 0, 128, 64, 16, b.CA_F32)
    assert n > 0 and n % 256 == 0
    assert lib.cluster_attn_backward_workspace_size(32, 12, 5, 128, 64, 16, b.CA_F32) == 0
    assert lib.cluster_attn_backward_workspace_size(32, 12, 4, 128, 32, 16, b.CA_F32) == 0


def exact(**kw):
    a = dict(Q=Q, K=K, V=V, qv=None, kv=None, B=2, H=4, Hkv=0, L=128, Nk=128, d=64, causal=1,
             out=OUT, dt=b.CA_F32)
    a.update(kw)
    return b.lib().cluster_attn_exact_forward(a["Q"], a["K"], a["V"], a["qv"], a["kv"], a["B"],
                                              a["H"], a["Hkv"], a["L"], a["Nk"], a["d"],
                                              a["causal"], a["out"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(out=None), INV), (dict(causal=2), INV), (dict(Nk=0), INV),
    (dict(L=0), INV), (dict(Hkv=3), INV), (dict(dt=9), INV), (dict(Q=Q + 8), INV),
    (dict(out=Q), INV), (dict(qv=OUT + 64), INV), (dict(d=128), UNS),
])
def test_exact_rejects(kw, code):
    assert exact(**kw) == code
