"""Seeded synthetic workloads for the SLA2 forward pass.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It holds ONLY input generation (random draws, a Gaussian blur that
builds spatially smooth fields, bf16 rounding of the generated values) and the
table of workload shapes.  It holds none of the method's arithmetic: no
pooling, projection, scoring, top-k, softmax, feature map or combine.

Workloads (shapes follow the Wan2.1 latent grids of the SLA2 pages: the
Wan2.1-1.3B-480P and Wan2.1-14B-720P models named in the experiments section
of "SLA2 深度解读", section 09; block sizes b_q=128, b_kv=64 from section 05):

* ``tiny``   B=1,H=2,N=1024,d=64, fp32, b_q=b_kv=64, top-k 25 %.
             K_base rows are 8 Gaussian centroids (N(0,1)*1.5) picked by
             token index // 128; Q = K_base + N(0,0.3), K = K_base + N(0,0.3).
* ``wan13b`` B=1,H=12,N=32760 (21x30x52 latent grid), d=128, bf16, top-k 3 %.
* ``wan14b`` B=1,H=40,N=75600 (21x45x80 latent grid), d=128, bf16, top-k 3 %.
  Q/K for both Wan shapes: a per-head smooth field F (white N(0,1) blurred
  with sigma=2 cells along frame/row/column, re-standardised per channel),
  Q = s(F + N(0,0.5)), K = s(F + N(0,0.5)), with one scale s chosen so that
  q.k/sqrt(d) over 65,536 random token pairs of head 0 has std 3.
  V ~ N(0,1).  Everything is rounded to bf16 (RNE) last.
* Router projections Wq, Wk are d x d with entries N(0, 1/d) (variance 1/d),
  shared by all heads.  alpha: tiny -> (0.7, 0.4); Wan shapes -> U(0.5,0.95)
  per head.

Draw order.  ``tiny`` draws sequentially from one PCG64(seed) stream:
per (b,h): centroids (8,d), eps_Q (N,d), eps_K (N,d), V (N,d); then Wq, Wk.
Wan shapes use SeedSequence(seed).spawn(B*H + 2): child b*H+h draws that
head's field (f,y,x,d), eps_Q, eps_K and V in that order; child B*H draws
Wq, Wk, alpha; child B*H+1 draws the 65,536 (t,u) pairs for the scale.
Heads are generated in parallel threads; each head has its own stream, so the
result does not depend on the thread count.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np


# --------------------------------------------------------------------------
# workload table
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    bq: int
    bkv: int
    topk_frac: float
    dtype: str                      # "f32" or "bf16" (dtype of Q, K, V)
    gen: str                        # "centroids" or "smooth"
    grid: tuple = ()                # (frames, rows, cols) for "smooth"
    alpha: tuple = ()               # fixed per-head alpha, else drawn
    seed: int = 0
    k_noise: float = 0.3            # centroid workload: std of the K noise
    note: str = ""

    @property
    def Tq(self) -> int:
        return -(-self.N // self.bq)

    @property
    def Tkv(self) -> int:
        return -(-self.N // self.bkv)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny", 1, 2, 1024, 64, 64, 64, 0.25, "f32", "centroids",
                alpha=(0.7, 0.4), note="B=1 H=2 N=1024 d=64 fp32, 16x16 blocks, top-4")
WAN13B = Workload("wan13b", 1, 12, 32760, 128, 128, 64, 0.03, "bf16", "smooth",
                  grid=(21, 30, 52), note="Wan2.1-1.3B-480P attention shape, 3% of KV blocks")
WAN14B = Workload("wan14b", 1, 40, 75600, 128, 128, 64, 0.03, "bf16", "smooth",
                  grid=(21, 45, 80), note="Wan2.1-14B-720P attention shape, 3% of KV blocks")
SWEEP_FRACS = (0.10, 0.05, 0.03, 0.01)

WORKLOADS = {w.name: w for w in (TINY, WAN13B, WAN14B)}


# --------------------------------------------------------------------------
# helpers (input preparation only)
# --------------------------------------------------------------------------
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    Used only to store generated inputs in bf16; finite inputs assumed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class Inputs:
    """Host-side inputs of one workload.

    q, k, v: [B,H,N,d]; float32 arrays for dtype f32, uint16 bf16 bit
    patterns for dtype bf16.  wq, wk: [1,d,d] float32 (proj(x) = x @ W).
    alpha: [H] float32."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    alpha: np.ndarray
    meta: dict = field(default_factory=dict)


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def _centroid_inputs(wl: Workload) -> Inputs:
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    q = np.empty((B, H, N, d), np.float32)
    k = np.empty((B, H, N, d), np.float32)
    v = np.empty((B, H, N, d), np.float32)
    group = (np.arange(N) // 128) % 8
    for b in range(B):
        for h in range(H):
            cent = rng.standard_normal((8, d)) * 1.5
            eq = rng.standard_normal((N, d)) * 0.3
            ek = rng.standard_normal((N, d)) * wl.k_noise
            vv = rng.standard_normal((N, d))
            base = cent[group]
            q[b, h] = base + eq
            k[b, h] = base + ek
            v[b, h] = vv
    wq = (rng.standard_normal((1, d, d)) / math.sqrt(d)).astype(np.float32)
    wk = (rng.standard_normal((1, d, d)) / math.sqrt(d)).astype(np.float32)
    if wl.alpha:
        alpha = np.asarray(wl.alpha, np.float32)
        if alpha.shape[0] != H:
            alpha = np.resize(alpha, H).astype(np.float32)
    else:
        alpha = rng.uniform(0.5, 0.95, H).astype(np.float32)
    if wl.dtype == "bf16":
        q, k, v = (round_to_bf16_bits(a) for a in (q, k, v))
    return Inputs(wl, q, k, v, wq, wk, alpha)


def _smooth_field(rng: np.random.Generator, grid, d: int) -> np.ndarray:
    import scipy.ndimage as ndi
    f = rng.standard_normal(tuple(grid) + (d,), dtype=np.float32)
    for ax in range(3):
        f = ndi.gaussian_filter1d(f, 2.0, axis=ax, mode="reflect", truncate=4.0)
    f = f.reshape(-1, d)
    mu = f.mean(axis=0, dtype=np.float64)
    sd = f.std(axis=0, dtype=np.float64)
    sd = np.where(sd > 0, sd, 1.0)  # a single-token field has no spread
    return ((f - mu) / sd).astype(np.float32)


def _grid_for(wl: Workload):
    if wl.grid and int(np.prod(wl.grid)) == wl.N:
        return wl.grid
    # other N (property tests): a 1 x 1 x N strip
    return (1, 1, wl.N)


def _smooth_inputs(wl: Workload, threads: int | None = None) -> Inputs:
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    grid = _grid_for(wl)
    children = np.random.SeedSequence(wl.seed).spawn(B * H + 2)

    def raw(bh):
        rng = np.random.Generator(np.random.PCG64(children[bh]))
        f = _smooth_field(rng, grid, d)
        eq = rng.standard_normal((N, d), dtype=np.float32) * np.float32(0.5)
        ek = rng.standard_normal((N, d), dtype=np.float32) * np.float32(0.5)
        vv = rng.standard_normal((N, d), dtype=np.float32)
        return f + eq, f + ek, vv

    # scale from head 0: std(q_t . k_u / sqrt(d)) over 65,536 random pairs = 3
    q0, k0, _ = raw(0)
    rs = np.random.Generator(np.random.PCG64(children[B * H + 1]))
    t = rs.integers(0, N, 65536)
    u = rs.integers(0, N, 65536)
    x = np.einsum("ij,ij->i", q0[t].astype(np.float64), k0[u].astype(np.float64)) / math.sqrt(d)
    sx = float(x.std())
    # a one-token field gives identical pairs (std ~ 0): keep the unit scale
    s = math.sqrt(3.0 / sx) if sx > 1e-6 else 1.0
    del q0, k0

    store_bf16 = wl.dtype == "bf16"
    dt = np.uint16 if store_bf16 else np.float32
    q = np.empty((B, H, N, d), dt)
    k = np.empty((B, H, N, d), dt)
    v = np.empty((B, H, N, d), dt)

    def fill(bh):
        qr, kr, vr = raw(bh)
        qr *= np.float32(s)
        kr *= np.float32(s)
        b, h = divmod(bh, H)
        if store_bf16:
            q[b, h] = round_to_bf16_bits(qr)
            k[b, h] = round_to_bf16_bits(kr)
            v[b, h] = round_to_bf16_bits(vr)
        else:
            q[b, h], k[b, h], v[b, h] = qr, kr, vr

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(fill, range(B * H)))

    rw = np.random.Generator(np.random.PCG64(children[B * H]))
    wq = (rw.standard_normal((1, d, d)) / math.sqrt(d)).astype(np.float32)
    wk = (rw.standard_normal((1, d, d)) / math.sqrt(d)).astype(np.float32)
    alpha = rw.uniform(0.5, 0.95, H).astype(np.float32)
    if wl.alpha:
        alpha = np.resize(np.asarray(wl.alpha, np.float32), H).astype(np.float32)
    return Inputs(wl, q, k, v, wq, wk, alpha, meta={"scale": s, "grid": grid})


def make_inputs(wl: Workload, threads: int | None = None) -> Inputs:
    if wl.gen == "centroids":
        return _centroid_inputs(wl)
    if wl.gen == "smooth":
        return _smooth_inputs(wl, threads)
    raise ValueError(f"unknown generator {wl.gen!r}")

