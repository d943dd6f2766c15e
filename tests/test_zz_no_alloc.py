"""cluster_attn_forward_noalloc (the allocation-free entry point) against
cluster_attn_forward_opts with a caller-owned workspace: same kernels, so the
outputs and assignments must agree bit for bit. Two staged calls in a row, the
second on a smaller input (the shared device array keeps the first call's
contents), a single-launch call that needs no workspace, and a call that needs
more workspace than the array holds."""
import ctypes

import numpy as np
import pytest

from means_token_clustering_amd import inputs as gen

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _b():
    from means_token_clustering_amd import binding
    return binding


def _dev(a: np.ndarray, dtype: str):
    if dtype == gen.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _args(x, path, valid=None):
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    dt = b.CA_BF16 if x.dtype == gen.BF16 else b.CA_F32
    opts = b.CaOptions(valid.data_ptr() if valid is not None else None, 0, 0, None)
    return q, k, v, dt, opts


def _noalloc(x, q, k, v, dt, opts, path, out, c):
    b = _b()
    return b.lib().cluster_attn_forward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), x.B, x.H, x.L, x.d, x.nclust, x.iters, x.W,
        float(x.alpha), ctypes.byref(opts), out.data_ptr(), c.data_ptr(), dt, path,
        torch.cuda.current_stream().cuda_stream)


def _with_workspace(x, q, k, v, dt, opts, path):
    b = _b()
    out = torch.empty_like(q)
    c = torch.empty((x.B, x.H, x.L), dtype=torch.int32, device="cuda")
    need = b.cluster_attn_workspace_size(x.B, x.H, x.L, x.d, x.nclust, dt, path)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    st = b.lib().cluster_attn_forward_opts(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), x.B, x.H, x.L, x.d, x.nclust, x.iters, x.W,
        float(x.alpha), ctypes.byref(opts), out.data_ptr(), c.data_ptr(), dt, b._aligned_ptr(ws),
        b._ws_bytes(ws), path, torch.cuda.current_stream().cuda_stream)
    assert st == b.CA_OK
    return out, c


def _check_case(x, path, valid=None):
    b = _b()
    print(f"[noalloc] B={x.B} H={x.H} L={x.L} K={x.nclust} I={x.iters} {x.dtype} path={path} "
          f"workspace={b.cluster_attn_workspace_size(x.B, x.H, x.L, x.d, x.nclust, 0, path)}",
          flush=True)
    q, k, v, dt, opts = _args(x, path, valid)
    out = torch.full_like(q, float("nan"))
    c = torch.full((x.B, x.H, x.L), -1, dtype=torch.int32, device="cuda")
    assert _noalloc(x, q, k, v, dt, opts, path, out, c) == b.CA_OK
    ref_out, ref_c = _with_workspace(x, q, k, v, dt, opts, path)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(c, ref_c)


def test_noalloc_two_calls_then_single_launch():
    b = _b()
    # 1: the long-sequence workload (37.5 MiB of staged workspace)
    _check_case(gen.workload("long_l8192"), b.CA_PATH_AUTO)
    # 2: a smaller staged call with a key-padding mask, after the first
    x = gen.make_inputs(2, 3, 300, 64, nclust=16, iters=3, W=32, alpha=0.5, seed=91, blobs=8)
    valid = torch.from_numpy(gen.make_mask(2, 300, seed=91)).cuda()
    _check_case(x, b.CA_PATH_STAGED, valid)
    # 3: the single launch needs no workspace
    _check_case(gen.make_inputs(2, 3, 128, 64, nclust=16, iters=3, seed=92, blobs=8),
                b.CA_PATH_AUTO)


def test_noalloc_rejects_a_call_beyond_the_array():
    b = _b()
    x = gen.make_inputs(1, 12, 16384, 64, nclust=64, iters=1, seed=93)
    need = b.cluster_attn_workspace_size(x.B, x.H, x.L, x.d, x.nclust, 0, b.CA_PATH_STAGED)
    assert need > b.CA_NOALLOC_SCRATCH_BYTES
    q, k, v, dt, opts = _args(x, b.CA_PATH_STAGED)
    out = torch.full_like(q, 7.0)
    c = torch.full((x.B, x.H, x.L), -1, dtype=torch.int32, device="cuda")
    st = _noalloc(x, q, k, v, dt, opts, b.CA_PATH_STAGED, out, c)
    torch.cuda.synchronize()
    assert st == b.CA_ERR_SCRATCH_TOO_SMALL
    assert bool((out == 7.0).all()) and bool((c == -1).all())
