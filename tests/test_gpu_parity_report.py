"""Parity report of the five benchmark configurations (P0 protocol at full size).

For each configuration the forward runs once on the path the benchmark takes
(CA_PATH_AUTO) with the assignment trace, and the record kept as
report_<workload>.json in the records folder of tests/parity.py holds, per
Lloyd iteration:

- near-ties (the oracle's best-to-second gap below 1e-5 ||q_i||^2),
- GPU != oracle at a near-tie (excused) and elsewhere (must be 0),
- tokens assigned to a zero (empty) centroid;

and for the run: the free-running mismatch count against the oracle's own
run, the largest |out - oracle| on the GPU's final assignment, and the
largest distance error of the GPU's assignment arithmetic relative to
||q_i||^2: the GPU's update (ca_centroid_update) of c^(t-1) and its scores
(ca_kmeans_scores, the matrix-core chain every clustering kernel uses)
against ||q_i - mu_k||^2 from the oracle's fp64 update of the same c^(t-1).

The full-layer configuration runs the attention P0 on the layer's own bf16
projections (qkv_out). python -m tests.parity_report turns the records into
a markdown table.
"""
import numpy as np
import pytest

import oracle
from means_token_clustering_amd import inputs as gen
from tests import parity

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _b():
    from means_token_clustering_amd import binding
    return binding


def _dev(a: np.ndarray, dtype: str):
    if dtype == gen.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def distance_errors(q_dev, Q64, hist: np.ndarray, K: int):
    """Largest |D_gpu - D_ref| / ||q||^2 of each iteration t, at the centroids
    mu^(t-1) both sides form from the GPU's c^(t-1) (mu^(0): the initial rows)."""
    b = _b()
    errs = []
    for t in range(1, hist.shape[0] + 1):
        if t == 1:
            mu_ref = oracle.init_centroids(Q64, K)
            mu_gpu = torch.from_numpy(mu_ref.astype(np.float32)).cuda()   # exact rows of Q
        else:
            c_prev = hist[t - 2]
            mu_ref, _ = oracle.update(Q64, c_prev, K)
            mu_gpu, _ = b.ca_centroid_update(q_dev, torch.from_numpy(c_prev).cuda(), K)
        scores = b.ca_kmeans_scores(q_dev, mu_gpu)
        torch.cuda.synchronize()
        errs.append(parity.distance_error(Q64, mu_ref, scores.cpu().numpy()))
    return errs


def p0_record(name, q_dev, k_dev, v_dev, Q64, K64, V64, nclust, iters, W, alpha, dtype, extra):
    b = _b()
    B, H, L, _ = Q64.shape
    plan = b.cluster_attn_plan(B, H, L, nclust, W,
                               dtype=b.CA_BF16 if dtype == gen.BF16 else b.CA_F32)
    print(f"[report] {name}: B={B} H={H} L={L} K={nclust} I={iters} W={W} {dtype} plan={plan}",
          flush=True)
    hist = torch.empty((iters, B, H, L), dtype=torch.int32, device="cuda")
    out, c = b.cluster_attn_forward(q_dev, k_dev, v_dev, nclust, iters, W, alpha,
                                    assign_hist=hist)
    torch.cuda.synchronize()
    h = hist.cpu().numpy()
    assert np.array_equal(h[-1], c.cpu().numpy())
    reports, err, tol, _ = parity.check_forward(Q64, K64, V64, nclust, iters, W, alpha, dtype,
                                                [h[t] for t in range(iters)], _host(out))
    free = parity.free_running_mismatches(Q64, K64, V64, nclust, iters, W, alpha, h[-1])
    K = min(nclust, L)
    derr = distance_errors(q_dev, Q64, h, K)
    rec = parity.report_dict("report_" + name, plan, reports, err, tol, free, derr, extra)
    parity.write_record("report_" + name, rec)
    print(f"  {parity.summarize(reports)}; free-running={free}; max|out-ref|={err:.3e} "
          f"(tol {tol}); max dist err/|q|^2 = {max(derr):.3e}", flush=True)
    for r in reports:
        assert r.bad == 0, parity.summarize(reports)
    assert err <= tol
    return rec


@pytest.mark.parametrize("name", ["tiny", "distilbert", "bf16_l512", "long_l8192"])
def test_report_attention_workload(name):
    x = gen.workload(name)
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    extra = {"workload": name, "B": x.B, "H": x.H, "L": x.L, "K": x.nclust, "iters": x.iters,
             "W": x.W, "alpha": x.alpha, "dtype": x.dtype, "seed": x.seed}
    p0_record(name, q, k, v, x.values("q"), x.values("k"), x.values("v"), x.nclust, x.iters,
              x.W, x.alpha, x.dtype, extra)


def test_report_layer_workload():
    x = gen.workload("layer_bf16")
    b = _b()
    X, Wq, Wk, Wv, Wo = (_dev(getattr(x, n), gen.BF16) for n in ("x", "wq", "wk", "wv", "wo"))
    _, c_layer, qkv = b.cluster_attn_layer_forward(X, Wq, Wk, Wv, Wo, x.H, x.nclust, x.iters,
                                                   x.W, x.alpha, want_qkv=True)
    torch.cuda.synchronize()
    q, k, v = (qkv[i].contiguous() for i in range(3))
    Q64, K64, V64 = (_host(t) for t in (q, k, v))
    extra = {"workload": "layer_bf16", "B": x.B, "H": x.H, "L": x.L, "K": x.nclust,
             "iters": x.iters, "W": x.W, "alpha": x.alpha, "dtype": gen.BF16, "seed": x.seed,
             "inputs": "the layer's own bf16 Q, K, V projections (qkv_out)"}
    rec = p0_record("layer_bf16", q, k, v, Q64, K64, V64, x.nclust, x.iters, x.W, x.alpha,
                    gen.BF16, extra)
    # the layer's assignment is the attention's own
    c_attn = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha)[1]
    assert torch.equal(c_attn, c_layer)
    assert rec["bad"] == 0
