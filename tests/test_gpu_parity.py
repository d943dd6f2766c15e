"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Every test here needs an MI355X and the built library; run with -m gpu.
"""
import sys

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


def _say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_iters(x: gen.AttnInputs, path: int):
    """GPU assignment of every iteration (the run's trace, slot t - 1 = c^(t))
    and the output of the run."""
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    hist = torch.empty((x.iters, x.B, x.H, x.L), dtype=torch.int32, device="cuda")
    out, c = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, path=path,
                                    assign_hist=hist)
    torch.cuda.synchronize()
    h = hist.cpu().numpy()
    assert np.array_equal(h[-1], c.cpu().numpy())
    return [h[t] for t in range(x.iters)], _host(out), (q, k, v)


def check(x: gen.AttnInputs, path: int, tol=None, record: str = None):
    b = _b()
    plan = b.cluster_attn_plan(x.B, x.H, x.L, x.nclust, x.W, path=path,
                               dtype=b.CA_BF16 if x.dtype == gen.BF16 else b.CA_F32)
    _say(f"[parity] {x.name or 'case'} B={x.B} H={x.H} L={x.L} K={x.nclust} I={x.iters} "
         f"W={x.W} a={x.alpha} {x.dtype} seed={x.seed} path={path} plan={plan}")
    assigns, out, _ = run_iters(x, path)
    q64, k64, v64 = x.values("q"), x.values("k"), x.values("v")
    reports, err, tol, ref = parity.check_forward(
        q64, k64, v64, x.nclust, x.iters, x.W, x.alpha, x.dtype, assigns, out, tol)
    free = parity.free_running_mismatches(q64, k64, v64, x.nclust, x.iters, x.W, x.alpha,
                                          assigns[-1])
    _say(f"  {parity.summarize(reports)}; free-running mismatches={free}; "
         f"max|out-ref|={err:.3e} (tol {tol})")
    name = record or (f"{x.name or 'case'}_B{x.B}_H{x.H}_L{x.L}_K{x.nclust}_I{x.iters}_W{x.W}"
                      f"_a{x.alpha}_{x.dtype}_s{x.seed}_p{path}")
    parity.write_record(name, parity.report_dict(name, plan, reports, err, tol, free, None))
    for r in reports:
        assert r.bad == 0, parity.summarize(reports)
    assert err <= tol
    return assigns, out, ref


PATHS = [0, 2]   # auto, staged


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", ["tiny", "distilbert", "bf16_l512", "long_l8192"])
def test_workloads(name, path):
    check(gen.workload(name), path)


@pytest.mark.parametrize("seed", range(101, 117))
def test_tiny_seed_sweep(seed):
    check(gen.workload("tiny", seed=seed), 0)


EDGE = [  # B, H, L, nclust, iters, W, alpha, dtype, blobs
    (1, 1, 1, 16, 2, 32, 0.5, "f32", None),       # single token
    (2, 3, 65, 16, 3, 32, 0.5, "f32", 4),          # one full tile + ragged
    (1, 2, 200, 16, 3, 32, 0.5, "bf16", 8),        # several tiles, ragged tail
    (2, 2, 130, 7, 4, 17, 0.3, "f32", 5),          # odd W, K not dividing L
    (1, 2, 40, 64, 2, 10, 0.5, "f32", None),       # nclust > L: K = L
    (1, 3, 96, 1, 3, 8, 0.5, "f32", 3),            # single cluster
    (1, 2, 150, 16, 3, 0, 0.5, "f32", 6),          # W = 0: self only
    (1, 2, 150, 16, 3, 1, 0.5, "bf16", 6),         # W = 1: radius 0
    (1, 2, 150, 16, 3, 400, 0.5, "f32", 6),        # W >= 2L: dense local branch
    (1, 2, 128, 16, 3, 32, 0.0, "f32", 6),         # pure centroid branch
    (1, 2, 128, 16, 3, 32, 1.0, "f32", 6),         # pure local branch
    (1, 1, 300, 256, 2, 32, 0.5, "f32", 40),       # maximum cluster count
    (3, 5, 128, 16, 3, 32, 0.5, "bf16", 16),       # more slices
    (1, 1, 1100, 32, 3, 64, 0.5, "f32", 32),       # split-key centroid attention
    (1, 2, 128, 16, 3, 100, 0.5, "f32", 6),        # wide window, single launch
    (2, 2, 100, 16, 3, 60, 0.4, "bf16", 6),        # wide window, ragged, bf16
    (1, 2, 128, 16, 3, 400, 0.5, "f32", 6),        # dense local branch, single launch
    (1, 2, 37, 5, 2, 33, 0.5, "f32", 3),           # radius 16 on a short ragged slice
    (1, 2, 257, 48, 3, 32, 0.5, "f32", 12),        # one-token last block, three full groups
    (2, 2, 129, 17, 2, 32, 0.5, "f32", 9),         # 17 clusters: a one-row last group
    (1, 1, 640, 64, 2, 24, 0.5, "bf16", 20),       # most clusters of the matrix-core step
    (1, 2, 120, 64, 2, 32, 0.5, "f32", 20),        # all four groups, one key range
    (2, 3, 300, 60, 3, 20, 0.5, "bf16", 24),       # 60 clusters, three ragged key ranges
    (1, 2, 200, 65, 2, 32, 0.5, "f32", 20),        # first count above it (scalar step)
    (2, 2, 512, 16, 3, 33, 0.5, "f32", 16),        # longest single-launch slice, radius 16
    (1, 3, 385, 9, 2, 12, 0.7, "bf16", 9),         # three key chunks and a one-token fourth
    # staged: window blocks in the clustering launch (S x blocks even), gather after
    (1, 3, 160, 16, 3, 32, 0.5, "f32", 8),         # six window blocks, two key ranges
    (1, 2, 384, 12, 3, 20, 0.6, "bf16", 10),       # three ranges, ragged clusters
    # staged: S x blocks odd, the launches in sequence
    (1, 1, 300, 16, 3, 32, 0.5, "bf16", 10),       # three blocks
    # staged: the clustering launch forms the four key ranges (86-128 slices)
    (8, 12, 400, 16, 3, 32, 0.5, "f32", 16),       # ragged last range
    (9, 12, 512, 12, 2, 20, 0.5, "bf16", 12),      # 108 slices, 12 clusters
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", EDGE)
def test_edge_cases(case, path):
    B, H, L, nclust, iters, W, alpha, dtype, blobs = case
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha,
                        dtype=dtype, seed=1000 + L + W, blobs=blobs, name="edge")
    check(x, path)


# the 16-wave single launch for 128 < L <= 512, forced with CA_PATH_FUSED
# (the auto path takes it only when the slices fill half to all of the CUs)
SINGLE512 = [  # B, H, L, nclust, iters, W, alpha, dtype, blobs
    (1, 2, 129, 16, 3, 32, 0.5, "f32", 8),         # two key chunks, the second of one key
    (1, 2, 300, 16, 3, 32, 0.5, "f32", 12),        # ragged last chunk and pass
    (2, 3, 512, 16, 3, 33, 0.5, "f32", 16),        # four full chunks, radius 16
    (1, 3, 385, 9, 2, 12, 0.7, "bf16", 9),         # a one-token fourth chunk
    (1, 2, 272, 4, 4, 0, 0.3, "f32", 4),           # W = 0, first pass ends on its halo
    (2, 2, 200, 16, 1, 20, 1.0, "bf16", 6),        # one iteration, pure local branch
    (1, 2, 450, 16, 3, 32, 0.0, "f32", 16),        # pure centroid branch
]


@pytest.mark.parametrize("case", SINGLE512)
def test_single_launch_long(case):
    B, H, L, nclust, iters, W, alpha, dtype, blobs = case
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha,
                        dtype=dtype, seed=3000 + L + W, blobs=blobs, name="single512")
    check(x, 1)


def test_single_launch_long_full_batch():
    check(gen.workload("bf16_l512"), 1)


# the split form of that launch (bf16 storage, at most half the CUs' worth of
# slices): a window workgroup per slice beside its clustering workgroup, taken
# by the auto path
SPLIT512 = [  # B, H, L, nclust, iters, W, alpha, blobs
    (1, 1, 129, 16, 3, 32, 0.5, 8),               # one slice, one pass, a one-key second chunk
    (1, 2, 256, 16, 3, 32, 0.5, 8),               # exactly one pass
    (1, 3, 257, 16, 3, 32, 0.5, 8),               # a second pass of one query
    (2, 3, 300, 7, 4, 17, 0.3, 6),                # odd W, K not dividing L, ragged pass
    (1, 2, 512, 16, 3, 33, 0.5, 16),              # radius 16, two full passes
    (1, 2, 272, 4, 4, 0, 0.3, 4),                 # W = 0
    (2, 2, 200, 16, 1, 20, 1.0, 6),               # one iteration, pure local branch
    (1, 2, 450, 16, 3, 32, 0.0, 16),              # pure centroid branch
    (8, 16, 512, 16, 3, 32, 0.5, 16),             # 128 slices: every CU of the grid busy
]


@pytest.mark.parametrize("case", SPLIT512)
def test_single_launch_split(case):
    B, H, L, nclust, iters, W, alpha, blobs = case
    b = _b()
    plan = b.cluster_attn_plan(B, H, L, nclust, W, dtype=b.CA_BF16)
    if not plan.startswith("fused512 split"):
        pytest.skip(f"this device's CU count gives the plan {plan!r}")
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha,
                        dtype=gen.BF16, seed=3500 + L + W, blobs=blobs, name="split512")
    check(x, 0)


def test_single_launch_split_full_batch_and_repeats():
    """The bf16 L = 512 workload through the split form, three calls in a row
    on the same workspace: identical outputs (the flags are cleared per call)."""
    x = gen.workload("bf16_l512")
    b = _b()
    plan = b.cluster_attn_plan(x.B, x.H, x.L, x.nclust, x.W, dtype=b.CA_BF16)
    if not plan.startswith("fused512 split"):
        pytest.skip(f"this device's CU count gives the plan {plan!r}")
    check(x, 0)
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    ws = torch.empty(b.cluster_attn_workspace_size(x.B, x.H, x.L, 64, x.nclust, b.CA_BF16) + 256,
                     dtype=torch.uint8, device="cuda")
    runs = [b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, workspace=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    for o, c in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(c, runs[0][1])


# the segmented single launch (each slice over several co-resident
# workgroups), forced with CA_PATH_SEGMENTED; with few slices the launch
# takes many short segments (exchange through owner workgroups), with more
# slices a few long ones (every workgroup adds the segment sums itself)
SEGMENTED = [  # B, H, L, nclust, iters, W, alpha, dtype, blobs
    (1, 2, 300, 16, 3, 32, 0.5, "f32", 12),        # many 16-token segments, one group
    (8, 12, 512, 16, 3, 32, 0.5, "bf16", 16),      # two 256-token segments per slice
    (2, 12, 1100, 32, 3, 32, 0.5, "f32", 24),      # ten segments, two groups, ragged
    (1, 12, 2000, 48, 4, 24, 0.4, "f32", 40),      # three groups, owners of 3-4 rows
    (2, 12, 1500, 64, 2, 33, 0.6, "bf16", 48),     # four groups, radius 16
    (4, 16, 1000, 20, 3, 0, 0.5, "f32", 16),       # W = 0, one-level, 3 segments of 336
    (2, 8, 960, 16, 1, 32, 1.0, "f32", 16),        # one iteration, pure local branch
    (1, 12, 777, 64, 3, 32, 0.0, "f32", 30),       # pure centroid branch, ragged
    (3, 12, 481, 16, 3, 32, 0.5, "bf16", 16),      # 7 segments of 80 on 256 CUs: the last holds one token
]


@pytest.mark.parametrize("case", SEGMENTED)
def test_segmented_launch(case):
    B, H, L, nclust, iters, W, alpha, dtype, blobs = case
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha,
                        dtype=dtype, seed=5000 + L + W, blobs=blobs, name="segmented")
    check(x, 3)


def test_segmented_long_workload():
    check(gen.workload("long_l8192"), 3)


# staged Lloyd steps whose workgroups take runs of three 128-token blocks
# (more blocks than two per compute unit); the slices' last runs are shorter
# and launch after the full ones
LLOYD_RUNS = [  # B, H, L, nclust, iters, W, alpha, dtype, blobs
    (1, 8, 8498, 64, 2, 32, 0.5, "f32", 64),       # 67 blocks: a last run of one 50-token block
    (1, 6, 11000, 48, 3, 24, 0.5, "bf16", 48),     # 86 blocks: a last run of two, ragged
    (1, 6, 11000, 56, 3, 24, 0.5, "bf16", 56),     # four cluster groups, the last one half empty
    (1, 2, 1300, 50, 3, 32, 0.5, "f32", 50),       # four groups, single blocks with the reduce
    (1, 6, 11008, 48, 3, 24, 0.5, "bf16", 48),     # whole blocks only (86 of them)
    (1, 5, 13312, 32, 2, 32, 0.5, "f32", 32),      # whole blocks only (104), two groups
]


@pytest.mark.parametrize("case", LLOYD_RUNS)
def test_lloyd_block_runs(case):
    B, H, L, nclust, iters, W, alpha, dtype, blobs = case
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha,
                        dtype=dtype, seed=7000 + L, blobs=blobs, name="lloyd_runs")
    check(x, 0)


def test_empty_cluster_and_exact_ties():
    """L=8, K=2, Q[4] = Q[0]: identical initial centroids tie exactly, so all
    tokens take cluster 0; cluster 1 becomes the zero vector; at iteration 2
    token i joins cluster 1 iff q_i . m < ||m||^2 / 2 (m = mean query)."""
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((1, 1, 8, 64)).astype(np.float32) + 0.5
    Q[0, 0, 4] = Q[0, 0, 0]
    Kt = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    V = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    b = _b()
    q, k, v = _dev(Q, "f32"), _dev(Kt, "f32"), _dev(V, "f32")
    for path in PATHS:
        _, c1 = b.cluster_attn_forward(q, k, v, 2, 1, 4, 0.5, path=path)
        out, c2 = b.cluster_attn_forward(q, k, v, 2, 2, 4, 0.5, path=path)
        assert c1.cpu().numpy().ravel().tolist() == [0] * 8
        Qd = Q[0, 0].astype(np.float64)
        m = Qd.mean(axis=0)
        want = [1 if float(qq @ m) < float(m @ m) / 2 else 0 for qq in Qd]
        assert c2.cpu().numpy().ravel().tolist() == want
        ref = oracle.forward_from_assign(Q.astype(np.float64), Kt.astype(np.float64),
                                         V.astype(np.float64), c2.cpu().numpy(), 2, 4, 0.5)
        assert np.abs(_host(out) - ref["out"]).max() <= 1e-4


@pytest.mark.parametrize("path", PATHS + [1, 3])   # 1: the 16-wave single launch, 3: segmented
def test_determinism_and_slice_independence(path):
    x = gen.make_inputs(2, 3, 160, 64, nclust=16, iters=3, W=32, alpha=0.5, seed=21, blobs=8)
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    o1, c1 = b.cluster_attn_forward(q, k, v, 16, 3, 32, 0.5, path=path)
    o2, c2 = b.cluster_attn_forward(q, k, v, 16, 3, 32, 0.5, path=path)
    assert torch.equal(o1, o2) and torch.equal(c1, c2)
    # duplicate heads in a permuted order: outputs follow bitwise
    perm = [2, 0, 1]
    qq, kk, vv = (torch.cat([t, t[:, perm]], dim=1).contiguous() for t in (q, k, v))
    o3, c3 = b.cluster_attn_forward(qq, kk, vv, 16, 3, 32, 0.5, path=path)
    assert torch.equal(o3[:, :3], o1) and torch.equal(o3[:, 3:], o1[:, perm])
    assert torch.equal(c3[:, 3:], c1[:, perm])


def test_alpha_is_convex_weight():
    x = gen.make_inputs(1, 4, 128, 64, nclust=16, iters=3, W=32, seed=22, blobs=16)
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    outs = {a: _host(b.cluster_attn_forward(q, k, v, 16, 3, 32, a)[0]) for a in (0.0, 0.5, 1.0)}
    assert np.abs(outs[0.5] - 0.5 * (outs[0.0] + outs[1.0])).max() <= 1e-6


# ------------------------------------------------------------ single steps
def test_step_assign_and_update():
    x = gen.make_inputs(2, 3, 200, 64, nclust=12, seed=31, blobs=10, dtype="bf16")
    b = _b()
    q = _dev(x.q, x.dtype)
    Qd = x.values("q")
    # strided init (mu = NULL)
    c0 = b.ca_kmeans_assign(q, None, 12).cpu().numpy()
    mu0 = oracle.init_centroids(Qd, 12)
    r = parity.check_assignment_step(Qd, mu0, c0, 1)
    assert r.bad == 0, r
    # update from that assignment, then assign against the GPU centroids
    mu_g, cnt_g = b.ca_centroid_update(q, torch.from_numpy(c0).cuda(), 12)
    mu_o, cnt_o = oracle.update(Qd, c0, 12)
    assert np.array_equal(cnt_g.cpu().numpy(), cnt_o)
    assert np.abs(mu_g.cpu().numpy() - mu_o).max() <= 1e-5
    c1 = b.ca_kmeans_assign(q, mu_g, 12).cpu().numpy()
    r = parity.check_assignment_step(Qd, mu_g.cpu().numpy().astype(np.float64), c1, 2)
    assert r.bad == 0, r


@pytest.mark.parametrize("L", [128, 1100])
def test_step_xattn_local_fuse(L):
    x = gen.make_inputs(1, 3, L, 64, nclust=16, seed=32 + L, blobs=8)
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    Qd, Kd, Vd = x.values("q"), x.values("k"), x.values("v")
    mu = oracle.init_centroids(Qd, 16).astype(np.float32)
    vc = b.ca_centroid_xattn(torch.from_numpy(mu).cuda(), k, v).cpu().numpy()
    vc_o, _ = oracle.centroid_xattn(mu.astype(np.float64), Kd, Vd)
    assert np.abs(vc - vc_o).max() <= 1e-5
    for W in (0, 5, 32, 3 * L):
        ol = b.ca_local_window_attn(q, k, v, W).cpu().numpy()
        ol_o, _ = oracle.local_attn(Qd, Kd, Vd, W)
        assert np.abs(ol - ol_o).max() <= 1e-5, W
    c = np.random.default_rng(0).integers(0, 16, size=(1, 3, L)).astype(np.int32)
    ol = b.ca_local_window_attn(q, k, v, 32)
    out = b.ca_gather_fuse(torch.from_numpy(vc).cuda(), torch.from_numpy(c).cuda(), ol, 0.25,
                           torch.float32)
    want = oracle.fuse(vc.astype(np.float64), c, ol.cpu().numpy().astype(np.float64), 0.25)
    assert np.abs(_host(out) - want).max() <= 1e-6


# the centroid attention with all four 16-centroid groups in one pass (49 to
# 64 centroids): one key range, several, and a ragged last range
@pytest.mark.parametrize("L,K", [(128, 64), (1100, 56), (300, 49)])
def test_step_xattn_all_groups(L, K):
    x = gen.make_inputs(1, 3, L, 64, nclust=K, seed=52 + L, blobs=8)
    b = _b()
    k, v = (_dev(getattr(x, n), x.dtype) for n in ("k", "v"))
    Qd, Kd, Vd = x.values("q"), x.values("k"), x.values("v")
    mu = oracle.init_centroids(Qd, K).astype(np.float32)
    vc = b.ca_centroid_xattn(torch.from_numpy(mu).cuda(), k, v).cpu().numpy()
    vc_o, _ = oracle.centroid_xattn(mu.astype(np.float64), Kd, Vd)
    assert np.abs(vc - vc_o).max() <= 1e-5


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("scales", [(1e3, 1e5, 1e5), (1e-3, 1e-6, 1e-7), (64.0, 1.0, 0.01),
                                    (1e-4, 1e4, 1.0)])
def test_extreme_magnitudes(scales, path):
    """Inputs far from unit scale (the single-launch path rescales them by
    powers of two before its fp16 split): same protocol, output tolerance
    relative to the scale of V. The products of the Q and K scales are either
    about 1 or so large that the softmax is a hard maximum (1e8): in between
    (logits of order 1e3) any fp32 evaluation of the logits is already off by
    more than the tolerance, so such cases pin nothing."""
    sq, sk, sv = scales
    x = gen.make_inputs(1, 3, 128, 64, nclust=16, iters=3, W=32, alpha=0.5, seed=77, blobs=8)
    q = (x.q.astype(np.float64) * sq).astype(np.float32)
    k = (x.k.astype(np.float64) * sk).astype(np.float32)
    v = (x.v.astype(np.float64) * sv).astype(np.float32)
    _say(f"[parity] magnitudes q*{sq} k*{sk} v*{sv} path={path}")
    b = _b()
    qd, kd, vd = _dev(q, "f32"), _dev(k, "f32"), _dev(v, "f32")
    assigns = []
    for t in range(1, 4):
        out, c = b.cluster_attn_forward(qd, kd, vd, 16, t, 32, 0.5, path=path)
        assigns.append(c.cpu().numpy())
    reports, err, _, _ = parity.check_forward(
        q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 16, 3, 32, 0.5, "f32",
        assigns, _host(out))
    _say(f"  {parity.summarize(reports)}; max|out-ref|/{sv}={err / sv:.3e}")
    for r in reports:
        assert r.bad == 0, parity.summarize(reports)
    assert err <= 1e-4 * sv


@pytest.mark.parametrize("case", [(128, 0), (512, 1), (512, 2), (300, 2)])
def test_bf16_tiny_elements(case):
    """bf16 Q, K, V where a tenth of the elements are 2^-20 times smaller
    than the rest: after the power-of-two scaling into fp16's range those fall
    below fp16's smallest normal, the one place where the bf16 kernels'
    omission of the m planes (zero for every other bf16 value) drops anything
    (m parts under 2^-24 in scaled units). Same protocol and tolerances."""
    L, path = case
    x = gen.make_inputs(1, 3, L, 64, nclust=16, iters=3, W=32, alpha=0.5, dtype=gen.BF16,
                        seed=91 + L, blobs=8, name="bf16_tiny")
    rng = np.random.default_rng(5 + L)
    for name in ("q", "k", "v"):
        vals = gen.bf16_bits_to_f32(getattr(x, name)).astype(np.float64)
        tiny = rng.random(vals.shape) < 0.1
        vals = np.where(tiny, vals * 2.0 ** -20, vals).astype(np.float32)
        setattr(x, name, gen.f32_to_bf16_bits(vals))
    check(x, path)


# ---------------------------------------------------------------- key-padding mask
def check_masked(x: gen.AttnInputs, mask: np.ndarray, path: int, tol=None):
    """Masked forward: per-iteration assignments equal the unmasked run's (the
    clustering ignores the mask), outputs match the oracle's masked steps on
    the GPU's assignment, padded query rows are exactly zero."""
    b = _b()
    _say(f"[masked] {x.name or 'case'} B={x.B} H={x.H} L={x.L} K={x.nclust} I={x.iters} "
         f"W={x.W} {x.dtype} seed={x.seed} path={path} real={int(mask.sum())}/{mask.size}")
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    vd = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    assigns, out = [], None
    for t in range(1, x.iters + 1):
        o, c = b.cluster_attn_forward(q, k, v, x.nclust, t, x.W, x.alpha, path=path, valid=vd)
        o0, c0 = b.cluster_attn_forward(q, k, v, x.nclust, t, x.W, x.alpha, path=path)
        assert torch.equal(c, c0), "the mask changed the clustering"
        assigns.append(c.cpu().numpy())
        out = o
    torch.cuda.synchronize()
    outh = _host(out)
    pad = np.broadcast_to((mask == 0)[:, None, :], (x.B, x.H, x.L))
    assert np.all(outh[pad] == 0.0), "padded query rows must be zero"
    reports, err, tol, _ = parity.check_forward(
        x.values("q"), x.values("k"), x.values("v"), x.nclust, x.iters, x.W, x.alpha, x.dtype,
        assigns, outh, tol, valid=mask)
    _say(f"  {parity.summarize(reports)}; max|out-ref|={err:.3e} (tol {tol})")
    for r in reports:
        assert r.bad == 0, parity.summarize(reports)
    assert err <= tol


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", ["tiny", "distilbert", "bf16_l512"])
def test_masked_workloads(name, path):
    x = gen.workload(name)
    check_masked(x, gen.make_mask(x.B, x.L, seed=x.seed + 500), path)


MASK_EDGE = [  # B, H, L, nclust, iters, W, alpha, dtype, mask kind
    (2, 3, 128, 16, 3, 32, 0.5, gen.F32, "holes"),
    (3, 2, 100, 16, 3, 32, 0.3, gen.F32, "prefix"),   # L < 128: partial tiles
    (2, 2, 128, 16, 3, 100, 0.5, gen.F32, "holes"),   # wide window
    (2, 2, 90, 8, 2, 70, 0.6, gen.BF16, "holes"),
    (1, 2, 300, 16, 3, 32, 0.5, gen.F32, "prefix"),   # staged only (L > 128)
    (2, 2, 260, 40, 3, 20, 0.5, gen.F32, "holes"),    # staged, ragged last block
    (2, 2, 128, 16, 3, 32, 0.5, gen.F32, "zeros"),    # everything padded
    (2, 4, 8300, 64, 2, 32, 0.5, gen.F32, "prefix"),  # Lloyd steps over runs of blocks
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", MASK_EDGE)
def test_masked_edge_cases(case, path):
    B, H, L, nclust, iters, W, alpha, dtype, kind = case
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha, dtype=dtype,
                        seed=700 + L + W, blobs=8)
    check_masked(x, gen.make_mask(B, L, seed=L + W, kind=kind), path)


@pytest.mark.parametrize("path", PATHS)
def test_masked_all_real_equals_unmasked(path):
    """An all-ones mask gives bit-identical outputs to the unmasked call."""
    b = _b()
    x = gen.workload("distilbert")
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    vd = torch.ones((x.B, x.L), dtype=torch.uint8, device="cuda")
    o1, c1 = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, path=path, valid=vd)
    o0, c0 = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, path=path)
    torch.cuda.synchronize()
    assert torch.equal(c1, c0)
    assert torch.equal(o1, o0)


# ---------------------------------------------------------------- grouped K/V heads
GQA = [  # B, H, Hkv, L, W, dtype, mask kind (None: no mask)
    (2, 12, 4, 128, 32, gen.F32, None),
    (2, 12, 1, 128, 32, gen.F32, "prefix"),
    (2, 6, 3, 100, 70, gen.BF16, None),
    (1, 4, 2, 300, 32, gen.F32, "holes"),
    (2, 8, 2, 400, 24, gen.BF16, None),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", GQA)
def test_grouped_kv_heads(case, path):
    """K and V with Hkv < H heads: query head h reads K/V head h // (H / Hkv);
    the oracle runs on K and V repeated to H heads."""
    b = _b()
    B, H, Hkv, L, W, dtype, kind = case
    G = H // Hkv
    x = gen.make_inputs(B, H, L, 64, nclust=16, iters=3, W=W, alpha=0.4, dtype=dtype,
                        seed=900 + H + Hkv + L, blobs=8)
    kv = gen.make_inputs(B, Hkv, L, 64, dtype=dtype, seed=901 + L)
    mask = gen.make_mask(B, L, seed=L, kind=kind) if kind else None
    _say(f"[gqa] B={B} H={H} Hkv={Hkv} L={L} W={W} {dtype} mask={kind} path={path}")
    q = _dev(x.q, dtype)
    k, v = _dev(kv.k, dtype), _dev(kv.v, dtype)
    vd = torch.from_numpy(mask).cuda() if mask is not None else None
    assigns, out = [], None
    for t in range(1, 4):
        o, c = b.cluster_attn_forward(q, k, v, 16, t, W, 0.4, path=path, valid=vd)
        assigns.append(c.cpu().numpy())
        out = o
    torch.cuda.synchronize()
    kr, vr = oracle.repeat_kv(kv.values("k"), G), oracle.repeat_kv(kv.values("v"), G)
    reports, err, tol, _ = parity.check_forward(x.values("q"), kr, vr, 16, 3, W, 0.4, dtype,
                                                assigns, _host(out), valid=mask)
    _say(f"  {parity.summarize(reports)}; max|out-ref|={err:.3e} (tol {tol})")
    for r in reports:
        assert r.bad == 0, parity.summarize(reports)
    assert err <= tol


@pytest.mark.parametrize("case", [(2, 8, 2, 400, 24, gen.BF16, None),
                                  (1, 12, 4, 300, 32, gen.F32, None)])
def test_grouped_kv_heads_single_launch_long(case):
    """The 16-wave single launch (forced) on grouped K/V heads."""
    test_grouped_kv_heads(case, 1)


# ---------------------------------------------------------------- listing-compatible variants
LF = oracle.LISTING
LISTING = [  # B, H, L, nclust, iters, W, alpha, dtype, flags, mask kind (None: no mask)
    (32, 12, 128, 16, 3, 32, 0.5, gen.F32, LF, "prefix"),      # the distilbert batch, padded
    (8, 12, 512, 16, 3, 32, 0.5, gen.BF16, LF, None),          # the bf16 L = 512 batch
    (2, 12, 128, 16, 3, 16, 0.5, gen.F32, LF, None),           # band radius 16, single launch
    (2, 4, 120, 16, 3, 40, 0.5, gen.F32, LF, None),            # step rows differ from floor(kL/K)
    (2, 4, 100, 16, 3, 8, 0.3, gen.BF16, LF, "holes"),
    (2, 3, 128, 16, 3, 0, 0.5, gen.F32, LF, None),             # W = 0: soft gather only
    (2, 3, 128, 16, 3, 128, 0.5, gen.F32, oracle.BAND, None),  # W >= L: hard gather only
    (1, 2, 300, 16, 3, 32, 0.5, gen.F32, LF, "prefix"),        # staged only (L > 128)
    (1, 2, 130, 7, 4, 17, 0.4, gen.F32, LF, None),             # K not dividing L, odd W
    (2, 3, 128, 16, 3, 32, 0.5, gen.F32, oracle.INIT_STEP, None),
    (2, 3, 128, 16, 3, 32, 0.5, gen.F32, oracle.SOFT_GATHER, None),
    (2, 3, 90, 5, 3, 20, 0.6, gen.BF16, oracle.SOFT_GATHER | oracle.BAND, None),
    (1, 1, 300, 256, 2, 32, 0.5, gen.F32, LF, None),           # soft gather over 256 centroids
]


def check_listing(x: gen.AttnInputs, flags: int, mask, path: int):
    b = _b()
    _say(f"[listing] B={x.B} H={x.H} L={x.L} K={x.nclust} I={x.iters} W={x.W} a={x.alpha} "
         f"{x.dtype} flags={flags} mask={mask is not None} seed={x.seed} path={path}")
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    vd = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda() if mask is not None else None
    assigns, out = [], None
    for t in range(1, x.iters + 1):
        o, c = b.cluster_attn_forward(q, k, v, x.nclust, t, x.W, x.alpha, path=path, valid=vd,
                                      flags=flags)
        assigns.append(c.cpu().numpy())
        out = o
    torch.cuda.synchronize()
    outh = _host(out)
    reports, err, tol, ref = parity.check_forward(
        x.values("q"), x.values("k"), x.values("v"), x.nclust, x.iters, x.W, x.alpha, x.dtype,
        assigns, outh, valid=mask, flags=flags)
    _say(f"  {parity.summarize(reports)}; max|out-ref|={err:.3e} (tol {tol})")
    for r in reports:
        assert r.bad == 0, parity.summarize(reports)
    assert err <= tol
    if mask is not None:
        pad = np.broadcast_to((mask == 0)[:, None, :], (x.B, x.H, x.L))
        assert np.all(outh[pad] == 0.0), "padded query rows must be zero"
    return outh, ref


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", LISTING)
def test_listing_variants(case, path):
    B, H, L, nclust, iters, W, alpha, dtype, flags, kind = case
    x = gen.make_inputs(B, H, L, 64, nclust=nclust, iters=iters, W=W, alpha=alpha, dtype=dtype,
                        seed=1300 + L + W + flags, blobs=8)
    mask = gen.make_mask(B, L, seed=L + 3, kind=kind) if kind else None
    check_listing(x, flags, mask, path)


@pytest.mark.parametrize("flags,W", [
    (oracle.INIT_STEP | oracle.BAND | oracle.ALPHA_LOGIT, 16),   # band radius 16
    (oracle.BAND, 0),                                              # the listing's skip
    (oracle.INIT_STEP, 32),
])
def test_listing_variants_single_launch_long(flags, W):
    """The listing variants that the 16-wave single launch takes (initial
    rows, band radius, alpha logit), forced on a 300-token batch."""
    x = gen.make_inputs(2, 3, 300, 64, nclust=16, iters=3, W=W, alpha=0.5, dtype=gen.F32,
                        seed=1700 + W + flags, blobs=8)
    check_listing(x, flags, None, 1)


@pytest.mark.parametrize("path", PATHS)
def test_listing_kept_empty_clusters(path):
    """Queries repeating with period 4 (rows r0..r3, r3 close to -(r0+r1+r2))
    and step-initial rows 8k: every initial centroid is r0, so the first
    assignment puts every token in cluster 0 (exact ties, lowest index) and
    clusters 1..15 are empty. Cluster 0 becomes the small mean m. The
    listing's rule keeps r0 in clusters 1..15, so at the second assignment
    the r0 tokens tie exactly among them and take cluster 1; the default
    rule's zero centroids take the r3 tokens (q . m < ||m||^2 / 2) instead.
    At the third, cluster 1 is the mean of 32 copies of r0: the rows carry
    bf16 precision so that this mean is r0 exactly in fp32 too, and its tie
    with the kept copies of r0 is exact on the GPU as in the oracle."""
    rng = np.random.default_rng(31)
    base = rng.standard_normal((2, 3, 4, 64))
    base[:, :, 3] = -(base[:, :, 0] + base[:, :, 1] + base[:, :, 2]) + 0.1 * base[:, :, 0]
    base = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(base.astype(np.float32)))
    Q = np.tile(base, (1, 1, 32, 1))   # L = 128, token i = base[i % 4]
    x = gen.make_inputs(2, 3, 128, 64, nclust=16, iters=3, W=32, alpha=0.5, seed=32)
    x.q = Q
    b = _b()
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    keep = oracle.INIT_STEP | oracle.KEEP_EMPTY
    phase = np.arange(128) % 4
    for flags in (keep, oracle.INIT_STEP):
        _, c1 = b.cluster_attn_forward(q, k, v, 16, 1, 32, 0.5, path=path, flags=flags)
        assert int(c1.max()) == 0
    _, c2 = b.cluster_attn_forward(q, k, v, 16, 2, 32, 0.5, path=path, flags=keep)
    c2 = c2.cpu().numpy()
    assert np.all(c2[..., phase == 0] == 1), "kept centroids: r0 tokens take cluster 1"
    _, c2d = b.cluster_attn_forward(q, k, v, 16, 2, 32, 0.5, path=path, flags=oracle.INIT_STEP)
    c2d = c2d.cpu().numpy()
    assert np.all(c2d[..., phase == 0] == 0) and np.all(c2d[..., phase == 3] == 1)
    check_listing(x, keep, None, path)
    check_listing(x, oracle.LISTING, None, path)


@pytest.mark.parametrize("path", PATHS)
def test_listing_skip_is_gather_exactly(path):
    """With the band flag and W = 0 or W >= L the output is the gathered
    context alone: alpha does not change it, bit for bit."""
    b = _b()
    x = gen.make_inputs(2, 3, 128, 64, nclust=16, iters=3, seed=33, blobs=8)
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    for W in (0, 128, 500):
        o1, _ = b.cluster_attn_forward(q, k, v, 16, 3, W, 0.0, path=path, flags=oracle.LISTING)
        o2, _ = b.cluster_attn_forward(q, k, v, 16, 3, W, 0.9, path=path, flags=oracle.LISTING)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), W


def test_listing_flags_zero_is_default():
    b = _b()
    x = gen.workload("distilbert")
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    kk = k[:, :4].contiguous()
    vv = v[:, :4].contiguous()
    o0, c0 = b.cluster_attn_forward(q, kk.repeat_interleave(3, dim=1), vv.repeat_interleave(3, dim=1),
                                    16, 3, 32, 0.5)
    o1, c1 = b.cluster_attn_forward(q, kk, vv, 16, 3, 32, 0.5, flags=0)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(o0, o1)


def test_single_launch_split_graph_replays():
    """The split form captured in a HIP graph (its flag-clearing launch is
    recorded ahead of it, as replays repeat the launch number): three replays,
    with eager forwards on other inputs between them, each bitwise equal to
    the eager result."""
    x = gen.workload("bf16_l512")
    b = _b()
    plan = b.cluster_attn_plan(x.B, x.H, x.L, x.nclust, x.W, dtype=b.CA_BF16)
    if not plan.startswith("fused512 split"):
        pytest.skip(f"this device's CU count gives the plan {plan!r}")
    q, k, v = (_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v"))
    ws = torch.empty(b.cluster_attn_workspace_size(x.B, x.H, x.L, 64, x.nclust, b.CA_BF16) + 256,
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    c = torch.empty((x.B, x.H, x.L), dtype=torch.int32, device="cuda")
    o_ref, c_ref = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the side stream before capture
        b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, out=out, assign_out=c,
                               workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, out=out, assign_out=c,
                               workspace=ws)
    ws2 = torch.empty_like(ws)
    for r in range(3):
        out.zero_()
        c.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(c, c_ref), f"replay {r}"
        # eager work between replays: other inputs, another workspace
        b.cluster_attn_forward(k, v, q, x.nclust, x.iters, x.W, x.alpha, workspace=ws2)
        torch.cuda.synchronize()


def test_single_launch_split_concurrent_streams():
    """Split-form forwards in flight on two streams at once (each launch takes
    its own ring of flags): every output equals the same call made alone."""
    b = _b()
    xs = [gen.make_inputs(4, 12, 512, 64, nclust=16, iters=3, W=32, alpha=0.5, dtype=gen.BF16,
                          seed=3900 + i, blobs=16, name="split512") for i in range(2)]
    plan = b.cluster_attn_plan(4, 12, 512, 16, 32, dtype=b.CA_BF16)
    if not plan.startswith("fused512 split"):
        pytest.skip(f"this device's CU count gives the plan {plan!r}")
    ins = [tuple(_dev(getattr(x, n), x.dtype) for n in ("q", "k", "v")) for x in xs]
    refs = []
    for (q, k, v), x in zip(ins, xs):
        refs.append(b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    torch.cuda.synchronize()
    for r in range(4):
        for i, ((q, k, v), x) in enumerate(zip(ins, xs)):
            with torch.cuda.stream(streams[i]):
                outs[i].append(b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha))
    torch.cuda.synchronize()
    for i in range(2):
        for o, c in outs[i]:
            assert torch.equal(o, refs[i][0]) and torch.equal(c, refs[i][1])
