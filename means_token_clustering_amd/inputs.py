"""Seeded synthetic inputs for cluster attention.

This module only draws random numbers and stores them in the layouts the
library expects. It holds none of the method's arithmetic, so both the GPU
path (through the Python binding) and the CPU oracle can be fed from it.

Stand-ins for the pages' workload: the model card "distilbert-sst2-cluster-
attention" measures on GLUE SST-2 with DistilBERT (6 layers, 12 heads, hidden
768, L=128, B=32; section "Empirical Benchmark Table"). That data and the
trained weights are not available, so queries are drawn from a Gaussian
mixture (tokens of one sentence share a few semantic groups) and keys/values
from N(0, 1).

Recipe (fixed; tests and the benchmark rely on it):
  * generator: numpy.random.default_rng(seed) (PCG64);
  * draw order: Q, then K, then V (full-layer workload: X, W_Q, W_K, W_V, W_O);
  * mixture Q: centres C ~ N(0, I_d) of shape [B,H,M,d]; labels z ~ U{0..M-1}
    of shape [B,H,L]; noise E ~ N(0, I_d) of shape [B,H,L,d];
    Q = C[z] + sigma * E (tokens stay in draw order along the sequence);
  * every value is drawn in float64 and rounded to float32; bf16 storage
    rounds that float32 to the nearest bf16 (ties to even).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the float32 values they encode."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class AttnInputs:
    """One batch of attention inputs, contiguous [B, H, L, d].

    ``q``, ``k``, ``v`` hold the *stored* values: float32 arrays for f32, or
    uint16 bf16 bit patterns for bf16. ``values(name)`` returns the exact
    values as float64 for the oracle.
    """
    B: int
    H: int
    L: int
    d: int
    nclust: int
    iters: int
    W: int
    alpha: float
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seed: int
    name: str = ""

    def values(self, which: str) -> np.ndarray:
        a = getattr(self, which)
        if self.dtype == BF16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    @property
    def S(self) -> int:
        return self.B * self.H


@dataclasses.dataclass
class LayerInputs:
    """Full attention layer inputs: X [B, L, Dm] and W_{Q,K,V,O} [Dm, Dm], bf16 bits."""
    B: int
    L: int
    Dm: int
    H: int
    d: int
    nclust: int
    iters: int
    W: int
    alpha: float
    x: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    seed: int
    name: str = ""

    def values(self, which: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, which)).astype(np.float64)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32)


def mixture_queries(rng: np.random.Generator, B: int, H: int, L: int, d: int,
                    blobs: int, sigma: float) -> np.ndarray:
    """Q = C[z] + sigma * E in float64 (draws C, then z, then E)."""
    centres = _normal(rng, (B, H, blobs, d))
    labels = rng.integers(0, blobs, size=(B, H, L))
    noise = _normal(rng, (B, H, L, d))
    gathered = np.take_along_axis(centres, labels[..., None], axis=2)
    return gathered + sigma * noise


def make_inputs(B: int, H: int, L: int, d: int = 64, *, nclust: int = 16,
                iters: int = 3, W: int = 32, alpha: float = 0.5,
                dtype: str = F32, seed: int = 0, blobs: Optional[int] = None,
                sigma: float = 0.3, name: str = "") -> AttnInputs:
    """Draw Q, K, V. ``blobs=None`` gives iid N(0,1) queries, else a mixture."""
    rng = np.random.default_rng(seed)
    if blobs is None:
        q = _normal(rng, (B, H, L, d))
    else:
        q = mixture_queries(rng, B, H, L, d, blobs, sigma)
    k = _normal(rng, (B, H, L, d))
    v = _normal(rng, (B, H, L, d))
    return AttnInputs(B, H, L, d, nclust, iters, W, alpha, dtype,
                      _store(q, dtype), _store(k, dtype), _store(v, dtype),
                      seed, name)


def make_layer_inputs(B: int = 16, L: int = 512, Dm: int = 768, H: int = 12,
                      *, nclust: int = 16, iters: int = 3, W: int = 32,
                      alpha: float = 0.5, wstd: float = 0.02, seed: int = 5,
                      name: str = "") -> LayerInputs:
    """Draw X ~ N(0,1) [B,L,Dm] and four Dm x Dm weights ~ N(0, wstd^2), bf16."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (B, L, Dm))
    ws = [wstd * _normal(rng, (Dm, Dm)) for _ in range(4)]
    d = Dm // H
    return LayerInputs(B, L, Dm, H, d, nclust, iters, W, alpha,
                       _store(x, BF16), *(_store(w, BF16) for w in ws),
                       seed, name)


# The five workloads: name -> constructor. Sizes follow the model card's
# DistilBERT shape (12 heads of 64, L=128, B=32) and three variations of it.
def workload(name: str, seed: Optional[int] = None, B: Optional[int] = None):
    """The named workload; B overrides the batch size of the attention ones."""
    if name == "tiny":
        return make_inputs(B or 1, 2, 128, 64, nclust=16, iters=3, W=32, alpha=0.5,
                           dtype=F32, seed=1 if seed is None else seed,
                           blobs=None, name=name)
    if name == "distilbert":
        return make_inputs(B or 32, 12, 128, 64, nclust=16, iters=3, W=32, alpha=0.5,
                           dtype=F32, seed=2 if seed is None else seed,
                           blobs=16, name=name)
    if name == "bf16_l512":
        return make_inputs(B or 8, 12, 512, 64, nclust=16, iters=3, W=32, alpha=0.5,
                           dtype=BF16, seed=3 if seed is None else seed,
                           blobs=16, name=name)
    if name == "long_l8192":
        return make_inputs(B or 1, 12, 8192, 64, nclust=64, iters=5, W=32, alpha=0.5,
                           dtype=F32, seed=4 if seed is None else seed,
                           blobs=64, name=name)
    if name == "layer_bf16":
        return make_layer_inputs(16, 512, 768, 12, nclust=16, iters=3, W=32,
                                 alpha=0.5, seed=5 if seed is None else seed,
                                 name=name)
    raise KeyError(name)


WORKLOADS = ("tiny", "distilbert", "bf16_l512", "long_l8192", "layer_bf16")


def make_mask(B: int, L: int, *, seed: int = 0, kind: str = "prefix",
              min_len: Optional[int] = None) -> np.ndarray:
    """Key-padding mask [B, L] uint8 (1 = real token, 0 = padding).

    kind "prefix": right padding as in a padded batch of sentences; row b keeps
    its first n_b tokens, n_b ~ U{min_len .. L} (min_len defaults to L // 4,
    at least 1), drawn with numpy.random.default_rng(seed). kind "holes":
    every token is real with probability 0.7, independently (rows may lose
    any token, including all of them). kind "ones" / "zeros": all real / all
    padding.
    """
    rng = np.random.default_rng(seed)
    if kind == "ones":
        return np.ones((B, L), np.uint8)
    if kind == "zeros":
        return np.zeros((B, L), np.uint8)
    if kind == "holes":
        return (rng.random((B, L)) < 0.7).astype(np.uint8)
    if kind != "prefix":
        raise ValueError(kind)
    lo = max(1, L // 4 if min_len is None else min_len)
    n = rng.integers(lo, L + 1, size=B)
    return (np.arange(L)[None, :] < n[:, None]).astype(np.uint8)
