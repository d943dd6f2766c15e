"""GPU parity of the full attention layer (projections, cluster attention,
output projection) and of its bf16 GEMM, through the C ABI, against the fp64
oracle. Run with -m gpu."""
import sys

import numpy as np
import pytest

import oracle
from means_token_clustering_amd import inputs as gen
from tests import parity

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ACC = 64.0 * 2.0 ** -24   # fp32 accumulation allowance per unit of sum |a_k b_k|


def _b():
    from means_token_clustering_amd import binding
    return binding


def _say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def check_rounded_product(got, A, Bm, what: str):
    """got = bf16(A Bm) from fp32 accumulation: within half an ulp of the exact
    product plus the accumulation allowance; report how often it differs from
    the correctly rounded value."""
    exact = oracle.matmul(A, Bm)
    bound = half_ulp(exact) + ACC * oracle.matmul(np.abs(A), np.abs(Bm))
    err = np.abs(got - exact)
    flips = int((got != oracle.round_bf16(exact)).sum())
    _say(f"  {what}: max err/bound={float((err / bound).max()):.3f}, "
         f"{flips} of {got.size} differ from the correctly rounded value")
    assert np.all(err <= bound), what
    assert flips <= max(1, got.size // 1000), what


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("M,N,Kd", [(300, 192, 256), (64, 64, 64), (1, 128, 768), (513, 768, 768)])
def test_gemm_bf16(M, N, Kd):
    _say(f"[gemm] M={M} N={N} Kd={Kd}")
    rng = np.random.default_rng(M * 7 + N)
    A = gen.f32_to_bf16_bits(rng.standard_normal((M, Kd)).astype(np.float32))
    Bt = gen.f32_to_bf16_bits((0.05 * rng.standard_normal((N, Kd))).astype(np.float32))
    C = _b().ca_gemm_bf16(_dev_bf16(A), _dev_bf16(Bt))
    torch.cuda.synchronize()
    A64 = gen.bf16_bits_to_f32(A).astype(np.float64)
    B64 = gen.bf16_bits_to_f32(Bt).astype(np.float64)
    check_rounded_product(_host(C), A64, np.ascontiguousarray(B64.T), "C")


@pytest.mark.parametrize("M,N,Kd", [(300, 192, 256), (64, 64, 64), (1, 128, 768), (513, 768, 768),
                                    (257, 320, 128), (129, 2304, 768), (8192, 2304, 64),
                                    (8100, 2304, 128)])
def test_gemm_bf16_kn(M, N, Kd):
    """Weights in the [in, out] layout: partial 192-column tiles (N = 64, 128,
    320), ragged M, one k step, the stand-alone projection shape's width; with
    at least as many 256 x 288 tiles as CUs (the last two) the large-tile
    launch runs, here with two and four k steps and a ragged last row tile."""
    _say(f"[gemm kn] M={M} N={N} Kd={Kd}")
    rng = np.random.default_rng(M * 11 + N)
    A = gen.f32_to_bf16_bits(rng.standard_normal((M, Kd)).astype(np.float32))
    W = gen.f32_to_bf16_bits((0.05 * rng.standard_normal((Kd, N))).astype(np.float32))
    C = _b().ca_gemm_bf16_kn(_dev_bf16(A), _dev_bf16(W))
    torch.cuda.synchronize()
    A64 = gen.bf16_bits_to_f32(A).astype(np.float64)
    W64 = gen.bf16_bits_to_f32(W).astype(np.float64)
    check_rounded_product(_host(C), A64, W64, "C")


# ------------------------------------------------------------------ layer
def run_layer(x: gen.LayerInputs):
    """Layer runs with iters = 1..I; returns per-iteration assignments, the
    final Y and Q/K/V (as device tensors)."""
    b = _b()
    X, Wq, Wk, Wv, Wo = (_dev_bf16(getattr(x, n)) for n in ("x", "wq", "wk", "wv", "wo"))
    assigns, Y, qkv = [], None, None
    for t in range(1, x.iters + 1):
        Y, c, qkv = b.cluster_attn_layer_forward(X, Wq, Wk, Wv, Wo, x.H, x.nclust, t, x.W,
                                                 x.alpha, want_qkv=True)
        assigns.append(c.cpu().numpy())
    torch.cuda.synchronize()
    return assigns, Y, qkv


def check_projections(x: gen.LayerInputs, qkv: np.ndarray, rows=None):
    """qkv [3, B, H, L, d] from the GPU against X W per (sampled) token row."""
    X = x.values("x").reshape(x.B * x.L, x.Dm)
    idx = np.arange(x.B * x.L) if rows is None else rows
    for n, name in enumerate(("wq", "wk", "wv")):
        got = oracle.merge_heads(qkv[n]).reshape(x.B * x.L, x.Dm)[idx]
        check_rounded_product(got, np.ascontiguousarray(X[idx]), x.values(name), name)


def check_attention(x: gen.LayerInputs, assigns, qkv_dev, slices):
    """P0 on the GPU's own Q, K, V for the given (b, h) slices."""
    b = _b()
    q, k, v = qkv_dev[0], qkv_dev[1], qkv_dev[2]
    out, c = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha)
    assert torch.equal(c.cpu(), torch.from_numpy(assigns[-1])), "layer and attention disagree"
    qn, kn, vn, on = (_host(t) for t in (q, k, v, out))
    refs = {}
    for (bb, hh) in slices:
        sl = (slice(bb, bb + 1), slice(hh, hh + 1))
        reports, err, tol, ref = parity.check_forward(
            qn[sl], kn[sl], vn[sl], x.nclust, x.iters, x.W, x.alpha, gen.BF16,
            [a[sl] for a in assigns], on[sl])
        _say(f"  slice b={bb} h={hh}: {parity.summarize(reports)}; max|O-ref|={err:.3e}")
        for r in reports:
            assert r.bad == 0, parity.summarize(reports)
        assert err <= tol
        refs[(bb, hh)] = ref["out"][0, 0]
    return qn, kn, vn, refs


def check_output_projection(x: gen.LayerInputs, Y: np.ndarray, O_ref_b: dict, rows):
    """Y rows (b, l) against round_bf16(O_ref) merged times W_O (fp64)."""
    Wo = x.values("wo")
    worst = 0.0
    for bb, ls in rows.items():
        Om = O_ref_b[bb]                          # [H, L, d] fp64 of batch bb
        Yref = oracle.output_projection(Om[None], Wo)[0]   # [L, Dm]
        err = np.abs(Y[bb, ls] - Yref[ls])
        worst = max(worst, float(err.max()))
    _say(f"  Y: max|Y-ref|={worst:.3e} (tol {parity.TOL['bf16']})")
    assert worst <= parity.TOL["bf16"]


def test_layer_small_full_check():
    x = gen.make_layer_inputs(2, 160, 256, 4, seed=51, name="layer-small")
    _say(f"[layer] B={x.B} L={x.L} Dm={x.Dm} H={x.H} K={x.nclust} I={x.iters} W={x.W}")
    assigns, Y, qkv = run_layer(x)
    check_projections(x, _host(qkv))
    slices = [(bb, hh) for bb in range(x.B) for hh in range(x.H)]
    _, _, _, refs = check_attention(x, assigns, qkv, slices)
    O_ref_b = {bb: np.stack([refs[(bb, hh)] for hh in range(x.H)]) for bb in range(x.B)}
    check_output_projection(x, _host(Y), O_ref_b, {bb: np.arange(x.L) for bb in range(x.B)})


def test_layer_config_full_size():
    """X [16, 512, 768], W 768 x 768 (std 0.02), H = 12: the attention P0 on
    all 192 slices and Y on every row of four batch rows (every row of every
    batch row would only repeat the same product); the projections on 1,024
    sampled rows (the fp64 reference product is the costly part)."""
    x = gen.workload("layer_bf16")
    _say(f"[layer] B={x.B} L={x.L} Dm={x.Dm} H={x.H} K={x.nclust} I={x.iters} W={x.W}")
    assigns, Y, qkv = run_layer(x)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(x.B * x.L, size=1024, replace=False))
    check_projections(x, _host(qkv), rows)
    slices = [(bb, hh) for bb in range(x.B) for hh in range(x.H)]
    _, _, _, refs = check_attention(x, assigns, qkv, slices)
    bsel = [0, 3, 11, 15]
    O_ref_b = {bb: np.stack([refs[(bb, hh)] for hh in range(x.H)]) for bb in bsel}
    check_output_projection(x, _host(Y), O_ref_b, {bb: np.arange(x.L) for bb in bsel})
