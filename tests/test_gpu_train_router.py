"""GPU parity of the training-time router (SoftTop-k, its gradient, the
gradient of the router projections) against the CPU oracle, through the C
ABI.

Bars: M within 2e-7 (fp32 storage of fp64 values; the bisection's sign
decisions may differ only where the row sum sits within rounding of the
budget).  lambda is unique only up to the flat stretch where a row's
sigmoids are saturated (well separated scores at tau = 0.1 leave the row sum
at k over a wide range of lambda), so it is checked through what defines
it: with the oracle's scores, the GPU's lambda must give a row sum within
1e-6 of k.  The gradients, computed in fp64 and stored in fp32, within
5e-7 of the largest entry of the oracle's.
"""
import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S
from tests.test_gpu_parity import dev, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu

SHAPES = [  # name, N, H, d, bq, dtype, frac, w_heads
    ("ragged-f32", 700, 2, 64, 64, "f32", 0.25, 1),
    ("bf16", 4100, 3, 128, 128, "bf16", 0.05, 3),
    ("k0", 900, 2, 128, 128, "bf16", 0.0, 1),
    ("all", 640, 2, 128, 128, "bf16", 1.0, 1),
]


def inputs(name, N, H, d, bq, dtype, frac, wh):
    gen = "centroids" if dtype == "f32" else "smooth"
    w = I.Workload(name, 1, H, N, d, bq, 64, frac, dtype, gen, seed=8)
    x = I.make_inputs(w)
    rng = np.random.default_rng(12)
    wq = rng.normal(0, d ** -0.5, (wh, d, d)).astype(np.float32)
    wk = rng.normal(0, d ** -0.5, (wh, d, d)).astype(np.float32)
    return w, x, wq, wk


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_soft_topk_and_grad(orc, dev, shape):
    name, N, H, d, bq, dtype, frac, wh = shape
    say(f"case soft top-k {name}: N={N} H={H} d={d} frac={frac}")
    w, x, wq, wk = inputs(*shape)
    q, k, _, _, _, _ = to_dev(x, dev)
    p = S.problem(1, H, N, d, bq, 64, frac, wh, dtype)
    tau = float(np.float32(0.1))  # the ABI takes tau as fp32: use that exact value
    M, lam = S.soft_topk(p, q, k, torch.from_numpy(wq).to(dev), torch.from_numpy(wk).to(dev),
                         tau)
    torch.cuda.synchronize()
    op = orc.problem(1, H, N, d, bq, 64, frac, wh, dtype)
    _, _, _, sc = orc.route(op, x.q, x.k, wq, wk, want_scores=True)
    oM, olam = orc.soft_topk(sc, orc.topk(op), tau)
    Mg, lg = M.cpu().numpy(), lam.cpu().numpy()
    err = np.abs(Mg.astype(np.float64) - oM).max()
    fin = np.isfinite(olam)
    kk = orc.topk(op)
    if fin.any():
        z = sc / tau + lg[..., None]
        rows = (1.0 / (1.0 + np.exp(-z))).sum(-1)
        berr = np.abs(rows[fin] - kk).max()
    else:
        berr = 0.0
    say(f"  M max-abs {err:.2e}, budget error at the GPU's lambda {berr:.2e}")
    assert err <= 2e-7 and berr <= 1e-6
    assert np.array_equal(np.isfinite(lg), fin) and np.array_equal(np.sign(lg[~fin]),
                                                                   np.sign(olam[~fin]))
    # gradient through SoftTop-k, from the GPU's own fp32 mask
    dM = np.random.default_rng(2).normal(0, 1, Mg.shape).astype(np.float32)
    dS = S.soft_topk_grad(p, M, torch.from_numpy(dM).to(dev), tau)
    torch.cuda.synchronize()
    odS = orc.soft_topk_grad(Mg, dM, tau)
    g = dS.cpu().numpy().astype(np.float64)
    scale = max(np.abs(odS).max(), 1e-30)
    say(f"  dS max-abs {np.abs(g - odS).max():.2e} (scale {scale:.2e})")
    assert np.abs(g - odS).max() <= 5e-7 * scale


@pytest.mark.parametrize("shape", SHAPES[:2], ids=[s[0] for s in SHAPES[:2]])
def test_route_grad(orc, dev, shape):
    name, N, H, d, bq, dtype, frac, wh = shape
    say(f"case route grad {name}: N={N} H={H} d={d} w_heads={wh}")
    w, x, wq, wk = inputs(*shape)
    q, k, _, _, _, _ = to_dev(x, dev)
    p = S.problem(1, H, N, d, bq, 64, frac, wh, dtype)
    dS = np.random.default_rng(5).normal(0, 1, (1, H, w.Tq, w.Tkv)).astype(np.float32)
    gq, gk = S.route_grad(p, q, k, torch.from_numpy(wq).to(dev), torch.from_numpy(wk).to(dev),
                          torch.from_numpy(dS).to(dev))
    torch.cuda.synchronize()
    op = orc.problem(1, H, N, d, bq, 64, frac, wh, dtype)
    oq, ok = orc.route_grad(op, x.q, x.k, wq, wk, dS.astype(np.float64))
    for got, want in ((gq, oq), (gk, ok)):
        g = got.cpu().numpy().astype(np.float64)
        scale = np.abs(want).max()
        say(f"  max-abs {np.abs(g - want).max():.2e} (scale {scale:.2e})")
        assert np.abs(g - want).max() <= 5e-7 * scale


def test_soft_topk_wan14b_budget(dev):
    """At the 14B shape every row of the GPU mask sums to k = 36 (fp64 sum of
    the fp32 mask, within the fp32 storage rounding of 1182 entries)."""
    w = I.WAN14B
    x = I.make_inputs(w)
    q, k, _, wq, wk, _ = to_dev(x, dev)
    p = S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    M, lam = S.soft_topk(p, q, k, wq, wk, 0.1)
    torch.cuda.synchronize()
    rows = M.double().sum(-1)
    say(f"  row sums: min {rows.min().item():.9f} max {rows.max().item():.9f}")
    assert (rows - 36).abs().max().item() < 1182 * 6e-8
    assert torch.isfinite(lam).all()
