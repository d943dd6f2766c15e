"""Benchmark: cluster-attention forward throughput on one MI355X.

A step is one whole forward pass (k-means, centroid cross-attention, local
window branch, gather + fusion) over one batch of the DistilBERT-shaped
workload: B=32, H=12, L=128, d=64, K=16 clusters, 3 Lloyd iterations,
W=32, alpha=0.5, fp32 (queries from a 16-blob Gaussian mixture, keys and
values N(0,1)). Inputs are resident in HBM before timing starts; input/output
sets rotate so the working set exceeds the 256 MB Infinity Cache.

Prints one JSON line with throughput (tokens/s = B*L per second, all heads),
the roofline record of the dominant kernel and the CPU-oracle baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "cluster-attention fwd tokens/s (B·L per s, all heads) + % HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 matrix (v_mfma_f32_*_f16)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix
MALL_BYTES = 256 << 20         # Infinity Cache
SPLIT_PRODUCTS = 3             # fp32-accurate contraction = 3 fp16 products of an h/m split
REPEATS = 5                    # timed groups inside the K steps (their median is reported)
PARITY_REPORT = os.path.join(ROOT, "profiles", "parity_report.md")


# HBM traffic of the fused kernel on the distilbert workload, measured with
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch), each
# scaled by what the same counter reads for the 12 MiB copy kernel that clones
# the input sets below (FETCH 12288 / 6156.6 = 1.996, WRITE 12288 / 12288 = 1).
# It is reported only while the kernel source (comments aside) is the one the
# counters were taken on.
TRAFFIC = {"workload": "distilbert", "bytes": 50681041,
           "read_kib": 37013.2, "write_kib": 12_480.0,
           "digest": "03cf8b21d36fbcb038a15bc92643e667bb5402c0779dc89e410ca09f07b20f4f"}
KERNEL_SOURCES = ("means_token_clustering_amd/csrc/fused.hip",   # device code only
                  "means_token_clustering_amd/csrc/mfma_split.h",
                  "means_token_clustering_amd/csrc/common.h")


def code_digest() -> str:
    """sha256 of the fused kernel's sources with comments and blank space removed."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        text = open(os.path.join(ROOT, rel)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()


def algorithmic_bytes(B, H, L, d, elem) -> int:
    """Read Q, K, V once; write the output and the int32 assignment."""
    return 4 * B * H * L * d * elem + 4 * B * H * L


def algorithmic_flops(B, H, L, d, K, iters, W) -> int:
    """FLOPs of one forward (an FMA is 2): distances 2ILKd, centroid sums ILd,
    centroid attention 4KLd, local window 4Pd (P in-window pairs), fusion 3Ld,
    per slice."""
    r = W // 2
    P = sum(min(L - 1, i + r) - max(0, i - r) + 1 for i in range(L))
    per = 2 * iters * L * K * d + iters * L * d + 4 * K * L * d + 4 * P * d + 3 * L * d
    return B * H * per


def contraction_flops(B, H, L, d, K, iters, W) -> int:
    """The algorithmic FLOPs of the contractions alone (distances 2ILKd,
    centroid attention 4KLd, local window 4Pd, per slice): the work the fp16
    matrix cores carry, SPLIT_PRODUCTS times over."""
    r = W // 2
    P = sum(min(L - 1, i + r) - max(0, i - r) + 1 for i in range(L))
    return B * H * (2 * iters * L * K * d + 4 * K * L * d + 4 * P * d)


def compute_record(x, ms) -> dict:
    """Rates of one step: all algorithmic FLOPs, and the fp16 matrix-core work
    (every fp32-accurate contraction runs as SPLIT_PRODUCTS fp16 products of an
    h/m split) against the dense fp16 peak. The path is not bound by it."""
    kc = min(x.nclust, x.L)
    flops = algorithmic_flops(x.B, x.H, x.L, x.d, kc, x.iters, x.W)
    cf = contraction_flops(x.B, x.H, x.L, x.d, kc, x.iters, x.W)
    mfma = SPLIT_PRODUCTS * cf / (ms / 1e3) / 1e12
    return {"flops_per_launch": flops, "achieved_TFLOPs": round(flops / (ms / 1e3) / 1e12, 2),
            "contraction_flops": cf, "fp16_products_per_contraction": SPLIT_PRODUCTS,
            "achieved_fp16_mfma_TFLOPs": round(mfma, 2), "peak_fp16_mfma_TFLOPs": FP16_PEAK_TFLOPS,
            "frac": round(mfma / FP16_PEAK_TFLOPS, 4)}


def parity_summary(workload: str):
    """The parity record of this workload from profiles/parity_report.md (made
    by tests/test_gpu_parity_report.py on the GPU); None if absent."""
    try:
        text = open(PARITY_REPORT).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(workload)
    if rec is None:
        return None
    keys = ("plan", "near_ties", "excused", "bad", "zero_centroid_tokens_last",
            "free_running_mismatches", "max_dist_err_rel", "near_tie_window", "max_out_err", "tol")
    out = {k: rec.get(k) for k in keys}
    out["near_ties_by_iter"] = [i["near_ties"] for i in rec.get("iterations", [])]
    out["source"] = ("profiles/parity_report.md (python -m pytest tests/test_gpu_parity_report.py "
                     "-m gpu; P0 protocol of tests/parity.py)")
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_steps(torch, stream, step, steps: int, warmup: int):
    """W untimed steps, then exactly K timed steps between two synchronisations,
    with HIP events on the launch stream at the ends and at REPEATS - 1 group
    boundaries inside. Returns (ms per step over all K, the groups' ms per step)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    groups = max(1, min(REPEATS, steps))
    bounds = [round(steps * g / groups) for g in range(groups + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    ev[0].record(stream)
    for g in range(groups):
        for i in range(bounds[g], bounds[g + 1]):
            step(i)
        ev[g + 1].record(stream)
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[-1]) / steps
    per = [ev[g].elapsed_time(ev[g + 1]) / max(1, bounds[g + 1] - bounds[g]) for g in range(groups)]
    return total, per


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="distilbert",
                   choices=["tiny", "distilbert", "bf16_l512", "long_l8192", "layer_bf16"])
    p.add_argument("--path", default="auto", choices=["auto", "fused", "staged", "segmented"])
    p.add_argument("--batch", type=int, default=0,
                   help="batch size B of the attention workload (0 = the workload's own)")
    p.add_argument("--sets", type=int, default=0, help="input sets to rotate (0 = auto)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="time budget of the CPU-oracle baseline (0 disables it)")
    p.add_argument("--masked", action="store_true",
                   help="padded batch: key-padding mask with right padding, row lengths "
                        "~ U{L/4..L} (cluster_attn_forward_masked)")
    p.add_argument("--flags", type=int, default=0,
                   help="listing-compatible variants, OR of CA_FLAG_* (15 = all four; "
                        "cluster_attn_forward_opts)")
    p.add_argument("--decoder", action="store_true",
                   help="time the decoder branch (cluster_attn_exact_forward, causal exact "
                        "attention) instead of the clustering forward")
    p.add_argument("--no-probe", action="store_true",
                   help="skip the HBM copy probe (achievable copy rates reported beside the "
                        "nominal peak)")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (cluster_attn_backward) on the forward's "
                        "assignment instead of the forward")
    return p.parse_args()


def hbm_probe(torch, set_bytes: int) -> dict:
    """Achievable HBM rates from plain device-to-device copies (torch copy_, one
    kernel per copy, timed with events on the current stream): a 1 GiB copy,
    and copies whose read + write bytes equal one forward launch's algorithmic
    bytes, rotating through enough buffer pairs to miss the Infinity Cache."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def rate(pairs, reps):
        for i in range(3):
            pairs[i % len(pairs)][1].copy_(pairs[i % len(pairs)][0])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(reps):
            src, dst = pairs[i % len(pairs)]
            dst.copy_(src)
        t1.record(stream)
        torch.cuda.synchronize()
        s = t0.elapsed_time(t1) / 1e3 / reps
        return 2 * pairs[0][0].numel() * pairs[0][0].element_size() / s / 1e9, s

    big = [(torch.empty(1 << 28, dtype=torch.float32, device=dev),
            torch.empty(1 << 28, dtype=torch.float32, device=dev))]
    big[0][0].fill_(1.0)
    big_rate, _ = rate(big, 10)
    del big
    n = set_bytes // 2 // 4
    npairs = max(2, MALL_BYTES // (2 * 4 * n) + 2)
    small = [(torch.ones(n, dtype=torch.float32, device=dev),
              torch.empty(n, dtype=torch.float32, device=dev)) for _ in range(npairs)]
    small_rate, small_s = rate(small, 200)
    return {"copy_1GiB_GBps": round(big_rate, 1), "copy_same_bytes_GBps": round(small_rate, 1),
            "copy_same_bytes_us": round(small_s * 1e6, 3), "same_bytes": 2 * 4 * n,
            "note": "device-to-device copies; same_bytes = one launch's algorithmic bytes, "
                    "half read and half written"}


def cpu_baseline(x, seconds: float, mask=None, flags: int = 0):
    """The oracle on the same batch: three runs on all host threads (value: their
    median) and three on one thread, each run repeating the whole batch until its
    share of the time budget has passed."""
    import oracle
    q, k, v = x.values("q"), x.values("k"), x.values("v")

    def once():
        oracle.forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, trace=False, valid=mask,
                       flags=flags)

    return _cpu_legs(once, x.B * x.L, seconds,
                     f"the whole {x.name} batch (B={x.B}, H={x.H}, L={x.L}), fp64 C oracle with "
                     f"OpenMP over slices")


def _cpu_legs(once, tokens: int, seconds: float, what: str):
    import oracle
    cores = oracle.num_threads()

    def leg(budget):
        rates, reps_all = [], []
        once()   # warm
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                once()
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget / 3:
                    break
            rates.append(tokens * reps / el)
            reps_all.append(reps)
        return median(rates), reps_all

    value, reps = leg(0.75 * seconds)
    oracle.set_num_threads(1)
    try:
        one, reps1 = leg(0.25 * seconds)
    finally:
        oracle.set_num_threads(cores)
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}; median of 3 runs of {reps} batch repeats on {cores} threads",
            "cpu_model": cpu_model(),
            "single_thread": {"value": one, "cores": 1,
                              "sample": f"median of 3 runs of {reps1} batch repeats"}}


def cpu_baseline_backward(x, seconds: float, mask=None):
    import numpy as np
    import oracle
    q, k, v = x.values("q"), x.values("k"), x.values("v")
    dO = np.random.default_rng(x.seed + 600).standard_normal(q.shape)
    c = oracle.forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, trace=False, valid=mask)["assign"]
    K = oracle.num_clusters(x.nclust, x.L)
    return _cpu_legs(lambda: oracle.backward(q, k, v, dO, c, K, x.W, x.alpha, valid=mask),
                     x.B * x.L, seconds,
                     f"the backward pass of the whole {x.name} batch (B={x.B}, H={x.H}, L={x.L}) "
                     f"on the oracle's own assignment, fp64 C oracle with OpenMP over slices")


def bench_backward(args, x, mask, b, gen, torch, np):
    """A step is one backward pass (cluster_attn_backward) over the batch,
    on the assignment of a forward run made before timing."""
    elem = 2 if x.dtype == gen.BF16 else 4
    dt = b.CA_BF16 if elem == 2 else b.CA_F32
    dev = torch.device("cuda:0")

    def to_dev(a):
        if x.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    n = x.B * x.H * x.L * x.d
    set_bytes = 7 * n * elem + 4 * x.B * x.H * x.L + (mask.size if mask is not None else 0)
    nsets = args.sets or max(2, MALL_BYTES // set_bytes + 2)
    vdev = torch.from_numpy(mask).to(dev) if mask is not None else None
    base = [to_dev(getattr(x, nm)) for nm in ("q", "k", "v")]
    dO = torch.randn(base[0].shape, generator=torch.Generator().manual_seed(x.seed + 600))
    dO = dO.to(base[0].dtype).to(dev)
    sets = []
    for _ in range(nsets):
        q, k, v, g = (t.clone() for t in (*base, dO))
        _, c = b.cluster_attn_forward(q, k, v, x.nclust, x.iters, x.W, x.alpha, valid=vdev)
        sets.append((q, k, v, g, c, torch.empty_like(q), torch.empty_like(k),
                     torch.empty_like(v), torch.empty(1, dtype=torch.float32, device=dev)))
    need = b.lib().cluster_attn_backward_workspace_size(x.B, x.H, 0, x.L, x.d, x.nclust, dt)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wsp, wsn = b._aligned_ptr(ws), b._ws_bytes(ws)
    lib = b.lib()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    vptr = vdev.data_ptr() if vdev is not None else None

    def step(i):
        q, k, v, g, c, dq, dk, dv, da = sets[i % nsets]
        st = lib.cluster_attn_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                       c.data_ptr(), vptr, x.B, x.H, 0, x.L, x.d, x.nclust, x.W,
                                       float(x.alpha), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), da.data_ptr(), dt, wsp, wsn, sptr)
        if st != b.CA_OK:
            raise b.CaError(st, "cluster_attn_backward")

    ms, groups = timed_steps(torch, stream, step, args.steps, args.warmup)
    achieved = set_bytes / (ms / 1e3) / 1e9
    rec = {"metric": "cluster-attention bwd tokens/s (B·L per s, all heads) + % HBM roofline",
           "value": round(x.B * x.L / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if elem == 2 else "f32", "data": "synthetic",
           "config": {"workload": x.name, "B": x.B, "H": x.H, "L": x.L, "d": x.d, "K": x.nclust,
                      "iters": x.iters, "W": x.W, "alpha": x.alpha, "storage": x.dtype,
                      "pass": "backward", "input_sets": nsets},
           "timing": {"groups": len(groups), "median_ms_per_step": round(median(groups), 6)},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": None, "kernel": "backward launch sequence",
                        "bytes_per_launch": set_bytes}}
    if mask is not None:
        rec["config"]["mask"] = (f"right padding, row lengths ~ U{{{max(1, x.L // 4)}..{x.L}}}, "
                                 f"{int(mask.sum())} of {mask.size} tokens real")
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_backward(x, args.cpu_seconds, mask)
    print(json.dumps(rec), flush=True)


def bench_layer(args, x, b, gen, torch, np):
    """A step is one whole attention layer (cluster_attn_layer_forward: the
    Q/K/V projections, cluster attention, the output projection) over the
    batch X [B, L, 768] in bf16. The roofline record covers the dominant
    kernel, the Q/K/V projection GEMM, timed on its own with the same
    shape ([B*L, 768] x [768, 3*768])."""
    dev = torch.device("cuda:0")

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    B, L, Dm, H, d = x.B, x.L, x.Dm, x.H, x.d
    Xb = to_dev(x.x)
    Wq, Wk, Wv, Wo = (to_dev(getattr(x, nm)) for nm in ("wq", "wk", "wv", "wo"))
    set_bytes = 2 * 2 * B * L * Dm   # X read, Y written
    nsets = args.sets or max(2, MALL_BYTES // set_bytes + 2)
    sets = [(Xb.clone(), torch.empty_like(Xb),
             torch.empty((B, H, L), dtype=torch.int32, device=dev)) for _ in range(nsets)]
    lib = b.lib()
    need = lib.cluster_attn_layer_workspace_size(B, L, Dm, H, d, x.nclust)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wsp, wsn = b._aligned_ptr(ws), b._ws_bytes(ws)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i):
        X, Y, c = sets[i % nsets]
        st = lib.cluster_attn_layer_forward(X.data_ptr(), Wq.data_ptr(), Wk.data_ptr(),
                                            Wv.data_ptr(), Wo.data_ptr(), B, L, Dm, H, d,
                                            x.nclust, x.iters, x.W, float(x.alpha), Y.data_ptr(),
                                            c.data_ptr(), None, wsp, wsn, sptr)
        if st != b.CA_OK:
            raise b.CaError(st, "cluster_attn_layer_forward")

    def timed(fn, steps, warmup):
        return timed_steps(torch, stream, fn, steps, warmup)[0]

    ms, groups = timed_steps(torch, stream, step, args.steps, args.warmup)
    # the projection GEMM alone: C [B*L, 3*768] = X [B*L, 768] . Wqkv with
    # Wqkv = [Wq | Wk | Wv] in the [in, out] layout the layer reads (the same
    # 128 x 192 tiles as the layer's Q/K/V launch)
    Wqkv = torch.cat([Wq, Wk, Wv], dim=1).contiguous()
    C = torch.empty((B * L, 3 * Dm), dtype=torch.bfloat16, device=dev)
    gsets = [X.view(B * L, Dm) for X, _, _ in sets]

    def gstep(i):
        A = gsets[i % nsets]
        st = lib.ca_gemm_bf16_kn(A.data_ptr(), Wqkv.data_ptr(), B * L, 3 * Dm, Dm, C.data_ptr(),
                                 sptr)
        if st != b.CA_OK:
            raise b.CaError(st, "ca_gemm_bf16_kn")

    gms = timed(gstep, 100, 10)
    gflops = 2.0 * B * L * Dm * 3 * Dm
    g_tflops = gflops / (gms / 1e3) / 1e12
    proj = 2.0 * B * L * Dm * Dm * 4
    att = algorithmic_flops(B, H, L, d, min(x.nclust, L), x.iters, x.W)
    rec = {"metric": "cluster-attention layer tokens/s (B·L per s) + % MFMA roofline of the "
                     "projection GEMM",
           "value": round(B * L / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": x.name, "B": B, "L": L, "Dm": Dm, "H": H, "d": d,
                      "K": x.nclust, "iters": x.iters, "W": x.W, "alpha": x.alpha,
                      "input_sets": nsets},
           "timing": {"groups": len(groups), "median_ms_per_step": round(median(groups), 6)},
           "roofline": {"bound": "mfma", "achieved": round(g_tflops, 1),
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(g_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "gemm_bf16_kernel, [%d x %d] x [%d x %d]" % (B * L, Dm, Dm, 3 * Dm),
                        "kernel_us": round(gms * 1e3, 3), "flops_per_launch": int(gflops)},
           "compute": {"flops_per_step": int(proj + att),
                       "achieved_TFLOPs": round((proj + att) / (ms / 1e3) / 1e12, 2),
                       "projection_flops": int(proj), "attention_flops": int(att)}}
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_layer(x, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def cpu_baseline_layer(x, seconds: float):
    """The oracle's layer on a sample of the batch: the first batch row (the
    fp64 projections dominate; one row is 1/B of the work)."""
    import oracle
    X1 = x.values("x")[:1]
    args = (x.values("wq"), x.values("wk"), x.values("wv"), x.values("wo"))
    return _cpu_legs(lambda: oracle.layer_forward(X1, *args, x.H, x.nclust, x.iters, x.W,
                                                  x.alpha),
                     x.L, seconds,
                     f"batch row 0 of {x.name} (1 x {x.L} tokens, all {x.H} heads), fp64 "
                     f"projections and the C oracle")


def bench_decoder(args, x, mask, b, gen, torch, np):
    """A step is one causal exact attention (the decoder branch) over the batch."""
    elem = 2 if x.dtype == gen.BF16 else 4
    dt = b.CA_BF16 if elem == 2 else b.CA_F32
    dev = torch.device("cuda:0")

    def to_dev(a):
        if x.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    n = x.B * x.H * x.L * x.d
    set_bytes = 4 * n * elem + (2 * mask.size if mask is not None else 0)
    nsets = args.sets or max(2, MALL_BYTES // set_bytes + 2)
    vdev = torch.from_numpy(mask).to(dev) if mask is not None else None
    vptr = vdev.data_ptr() if vdev is not None else None
    base = [to_dev(getattr(x, nm)) for nm in ("q", "k", "v")]
    sets = [(*(t.clone() for t in base), torch.empty_like(base[0])) for _ in range(nsets)]
    lib = b.lib()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i):
        q, k, v, o = sets[i % nsets]
        st = lib.cluster_attn_exact_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), vptr, vptr,
                                            x.B, x.H, 0, x.L, x.L, x.d, 1, o.data_ptr(), dt, sptr)
        if st != b.CA_OK:
            raise b.CaError(st, "cluster_attn_exact_forward")

    ms, groups = timed_steps(torch, stream, step, args.steps, args.warmup)
    achieved = set_bytes / (ms / 1e3) / 1e9
    rec = {"metric": "causal exact attention (decoder branch) tokens/s + % HBM roofline",
           "value": round(x.B * x.L / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if elem == 2 else "f32", "data": "synthetic",
           "config": {"workload": x.name, "B": x.B, "H": x.H, "L": x.L, "d": x.d,
                      "storage": x.dtype, "pass": "decoder", "input_sets": nsets},
           "timing": {"groups": len(groups), "median_ms_per_step": round(median(groups), 6)},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": None,
                        "kernel": "exact_fused_kernel" if x.L <= 128 else "exact_attn_kernel",
                        "bytes_per_launch": set_bytes}}
    if args.cpu_seconds > 0:
        import oracle
        q, k, v = x.values("q"), x.values("k"), x.values("v")
        rec["cpu_baseline"] = _cpu_legs(
            lambda: oracle.exact_attention(q, k, v, True, qvalid=mask, kvalid=mask), x.B * x.L,
            args.cpu_seconds, f"causal exact attention of the whole {x.name} batch, fp64 C oracle")
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the slices are "
              "independent, so more GPUs would each run their own batch share.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from means_token_clustering_amd import binding as b
    from means_token_clustering_amd import inputs as gen

    x = gen.workload(args.workload, B=args.batch or None)
    if args.workload == "layer_bf16":
        bench_layer(args, x, b, gen, torch, np)
        return
    if args.backward or args.decoder:
        mask = gen.make_mask(x.B, x.L, seed=x.seed + 500) if args.masked else None
        (bench_backward if args.backward else bench_decoder)(args, x, mask, b, gen, torch, np)
        return
    elem = 2 if x.dtype == gen.BF16 else 4
    path = {"auto": b.CA_PATH_AUTO, "fused": b.CA_PATH_FUSED, "staged": b.CA_PATH_STAGED,
            "segmented": b.CA_PATH_SEGMENTED}[args.path]
    dev = torch.device("cuda:0")

    def to_dev(a):
        if x.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    set_bytes = algorithmic_bytes(x.B, x.H, x.L, x.d, elem)
    mask = gen.make_mask(x.B, x.L, seed=x.seed + 500) if args.masked else None
    if mask is not None:
        set_bytes += mask.size   # one byte per token, read once per launch
    vdev = torch.from_numpy(mask).to(dev) if mask is not None else None
    nsets = args.sets or max(2, MALL_BYTES // set_bytes + 2)
    base = [to_dev(getattr(x, n)) for n in ("q", "k", "v")]
    sets = []
    for _ in range(nsets):
        q, k, v = (t.clone() for t in base)
        sets.append((q, k, v, torch.empty_like(q),
                     torch.empty((x.B, x.H, x.L), dtype=torch.int32, device=dev)))
    ws_bytes = b.cluster_attn_workspace_size(x.B, x.H, x.L, x.d, x.nclust,
                                             b.CA_BF16 if elem == 2 else b.CA_F32, path)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev) if ws_bytes else None
    lib = b.lib()
    dt = b.CA_BF16 if elem == 2 else b.CA_F32
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    wsp = b._aligned_ptr(ws)
    wsn = b._ws_bytes(ws)

    opts = b.CaOptions(vdev.data_ptr() if vdev is not None else None, 0, args.flags)

    def step(i):
        q, k, v, o, c = sets[i % nsets]
        if args.flags:
            st = lib.cluster_attn_forward_opts(q.data_ptr(), k.data_ptr(), v.data_ptr(), x.B, x.H,
                                               x.L, x.d, x.nclust, x.iters, x.W, float(x.alpha),
                                               ctypes.byref(opts), o.data_ptr(), c.data_ptr(), dt,
                                               wsp, wsn, path, sptr)
        elif vdev is not None:
            st = lib.cluster_attn_forward_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 vdev.data_ptr(), x.B, x.H, x.L, x.d, x.nclust,
                                                 x.iters, x.W, float(x.alpha), o.data_ptr(),
                                                 c.data_ptr(), dt, wsp, wsn, path, sptr)
        else:
            st = lib.cluster_attn_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), x.B, x.H,
                                             x.L, x.d, x.nclust, x.iters, x.W, float(x.alpha),
                                             o.data_ptr(), c.data_ptr(), dt, wsp, wsn, path, sptr)
        if st != b.CA_OK:
            raise b.CaError(st, "cluster_attn_forward")

    ms, groups = timed_steps(torch, stream, step, args.steps, args.warmup)
    tokens = x.B * x.L
    value = tokens / (ms / 1e3)

    # the launch sequence the library takes (its own dispatch decision)
    plan = b.cluster_attn_plan(x.B, x.H, x.L, x.nclust, x.W, flags=args.flags,
                               masked=mask is not None, path=path, dtype=dt)
    fused = plan == "fused"
    achieved = set_bytes / (ms / 1e3) / 1e9
    traffic = None
    if (fused and mask is None and not args.flags and not args.batch
            and x.name == TRAFFIC["workload"]
            and code_digest() == TRAFFIC["digest"]):
        traffic = TRAFFIC["bytes"]
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": ("cluster_attn_fused_kernel" if fused else
                       "cluster_attn_fused512_kernel" if plan == "fused512" else
                       "cluster_attn_fused512_kernel, split form"
                       if plan.startswith("fused512 split") else
                       "launch sequence " + plan),
            "bytes_per_launch": set_bytes}
    rec = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if elem == 2 else "f32", "data": "synthetic",
           "config": {"workload": x.name, "B": x.B, "H": x.H, "L": x.L, "d": x.d, "K": x.nclust,
                      "iters": x.iters, "W": x.W, "alpha": x.alpha, "storage": x.dtype,
                      "path": plan, "input_sets": nsets},
           "roofline": roof,
           "timing": {"groups": len(groups), "ms_per_step_by_group": [round(g, 6) for g in groups],
                      "median_ms_per_step": round(median(groups), 6),
                      "note": "the K timed steps split into equal groups between HIP events "
                              "on the launch stream; value uses all K steps"}}
    if mask is not None:
        rec["config"]["mask"] = (f"right padding, row lengths ~ U{{{max(1, x.L // 4)}..{x.L}}}, "
                                 f"{int(mask.sum())} of {mask.size} tokens real")
    if args.flags:
        rec["config"]["flags"] = args.flags
    rec["compute"] = compute_record(x, ms)
    # the same launches on one input set (reads served partly from the
    # Infinity Cache): labelled, never the value
    one = sets[0]
    cms, _ = timed_steps(torch, stream, lambda i: step(0), max(1, args.steps // 2), 3)
    rec["cache_resident"] = {"ms_per_step": round(cms, 6), "input_sets": 1,
                             "note": "one input set reused, so reads may hit the 256 MB "
                                     "Infinity Cache; not the headline value"}
    del one
    if not args.no_probe:
        rec["hbm_probe"] = hbm_probe(torch, set_bytes)
        roof["frac_of_copy"] = round(achieved / rec["hbm_probe"]["copy_same_bytes_GBps"], 4)
    if mask is None and not args.flags and not args.batch:
        rec["parity"] = parity_summary(x.name)
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds, mask, args.flags)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
