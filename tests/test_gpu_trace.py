"""Per-iteration assignment trace (ca_options_t.assign_hist) and prefix
determinism, on every clustering path of the library.

Lloyd's iterations t = 1..I (model card "Hooshaai/distilbert-sst2-cluster-
attention", Mathematical Formulation 1; the ClusterFormer spec on the
"Hooshaai/svd-sst2-roberta-cluster" page, section 2.1): a run with iters = t
must reproduce the first t iterations of any longer run, bit for bit. For each
path, slot t - 1 of the trace of an iters = I run must equal assign_out of a
separate iters = t run, and asking for the trace must change no other output.
The parity protocol (tests/parity.py) rests on this: it takes c^(t) from the
trace.
"""
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


# name, path, B, H, L, nclust, iters, W, dtype, blobs, flags, masked
PATHS = [
    ("fused", 0, 2, 3, 128, 16, 4, 32, "f32", 16, 0, False),
    ("fused ragged bf16", 0, 1, 2, 77, 16, 3, 10, "bf16", 8, 0, False),
    ("fused masked", 0, 2, 2, 100, 12, 3, 32, "f32", 8, 0, True),
    ("fused kept centroids", 0, 1, 3, 128, 16, 3, 32, "f32", 6, 2, False),
    ("fused512", 1, 2, 3, 300, 16, 3, 32, "f32", 12, 0, False),
    ("fused512 bf16", 1, 1, 2, 512, 16, 4, 33, "bf16", 16, 0, False),
    ("fused512 split (auto, 96 slices)", 0, 8, 12, 512, 16, 3, 32, "bf16", 16, 0, False),
    ("fused512 split, ragged (auto)", 0, 1, 3, 300, 12, 4, 20, "bf16", 10, 0, False),
    ("kmeans_slice + key ranges (96 slices)", 2, 8, 12, 512, 16, 3, 32, "bf16", 16, 0, False),
    ("kmeans_slice + key ranges, ragged", 2, 8, 12, 400, 12, 3, 32, "f32", 12, 0, False),
    ("kmeans_slice (132 slices)", 2, 11, 12, 512, 16, 3, 32, "bf16", 16, 0, False),
    ("kmeans_window (window beside)", 2, 1, 4, 300, 16, 3, 32, "f32", 10, 0, False),
    ("chained matrix-core steps", 2, 1, 2, 600, 32, 4, 32, "f32", 20, 0, False),
    ("steps with reduce launches", 2, 1, 2, 1100, 20, 3, 32, "f32", 20, 0, False),
    ("steps over runs of blocks", 2, 1, 8, 8269, 64, 3, 32, "f32", 64, 0, False),
    ("scalar steps (K > 64)", 2, 1, 1, 300, 80, 3, 32, "f32", 40, 0, False),
    ("staged kept centroids", 2, 1, 2, 200, 16, 3, 32, "f32", 6, 2, False),
    ("staged masked", 2, 2, 2, 257, 24, 3, 20, "bf16", 10, 0, True),
    ("segmented, owner exchange", 3, 1, 2, 1100, 40, 4, 32, "f32", 20, 0, False),
    ("segmented, every workgroup adds", 3, 8, 12, 512, 16, 3, 32, "bf16", 16, 0, False),
]


@pytest.mark.parametrize("case", PATHS, ids=[c[0] for c in PATHS])
def test_trace_equals_prefix_runs(case):
    name, path, B, H, L, nclust, iters, W, dtype, blobs, flags, masked = case
    print(f"[trace] {name}: B={B} H={H} L={L} K={nclust} I={iters} W={W} {dtype} "
          f"path={path} flags={flags} masked={masked}", flush=True)
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=0.5, dtype=dtype,
                        seed=7000 + L + nclust, blobs=blobs, name="trace")
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    valid = None
    if masked:
        valid = torch.from_numpy(gen.make_mask(B, L, seed=L)).cuda()
    hist = torch.full((iters, B, H, L), -1, dtype=torch.int32, device="cuda")
    out_h, c_h = b.cluster_attn_forward(q, k, v, nclust, iters, W, 0.5, path=path, valid=valid,
                                        flags=flags, assign_hist=hist)
    out_n, c_n = b.cluster_attn_forward(q, k, v, nclust, iters, W, 0.5, path=path, valid=valid,
                                        flags=flags)
    torch.cuda.synchronize()
    # the trace changes no other output
    assert torch.equal(out_h, out_n) and torch.equal(c_h, c_n)
    assert torch.equal(hist[iters - 1], c_n)
    for t in range(1, iters + 1):
        _, c_t = b.cluster_attn_forward(q, k, v, nclust, t, W, 0.5, path=path, valid=valid,
                                        flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(hist[t - 1], c_t), f"iteration {t} of the trace != the iters={t} run"
    Kc = min(nclust, L)
    assert int(hist.min()) >= 0 and int(hist.max()) < Kc


def test_trace_rejects_wrong_shape():
    b = _b()
    x = gen.make_inputs(1, 2, 64, 64, nclust=8, iters=3, seed=3)
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    bad = torch.empty((2, 1, 2, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        b.cluster_attn_forward(q, k, v, 8, 3, 32, 0.5, assign_hist=bad)
