"""GPU parity of sla2_backward against the CPU oracle's backward, through the
C ABI.

Both sides differentiate the same forward (same inputs, same selection); the
oracle works in fp64.  The GPU takes one of two paths: bf16 inputs with
d = b_q = 128 run on the matrix cores (every fp32 operand split into two
bf16 parts, 16 significant bits, fp32 accumulation), every other problem on
the vector-ALU kernels (fp32).  The bar is relative to each tensor's scale:
max-abs error <= 2e-4 x max |oracle| for dQ, dK, dV and dalpha (sums over up
to a few thousand terms of products carried to about 2^-16 relative).
"""
import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S
from tests.test_gpu_parity import dev, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu

REL = 2e-4

CASES = [  # name, dtype, N, H, d, bq, frac, alpha_mode, layout
    ("f32-d64-bq64", "f32", 700, 2, 64, 64, 0.25, S.ALPHA_PER_HEAD, S.LAYOUT_BHND),
    ("bf16-d128", "bf16", 1500, 2, 128, 128, 0.1, S.ALPHA_PER_HEAD, S.LAYOUT_BHND),
    ("bf16-ragged-qblock-alpha", "bf16", 1000, 3, 128, 128, 0.2, S.ALPHA_PER_QBLOCK,
     S.LAYOUT_BHND),
    ("bf16-bnhd", "bf16", 900, 2, 128, 64, 0.3, S.ALPHA_PER_HEAD, S.LAYOUT_BNHD),
    ("bf16-bnhd-bq128", "bf16", 1300, 2, 128, 128, 0.25, S.ALPHA_PER_QBLOCK, S.LAYOUT_BNHD),
    ("bf16-all-selected", "bf16", 700, 2, 128, 128, 1.0, S.ALPHA_PER_HEAD, S.LAYOUT_BHND),
    ("k0", "bf16", 640, 2, 128, 128, 0.0, S.ALPHA_PER_HEAD, S.LAYOUT_BHND),
    ("all-selected", "f32", 500, 2, 64, 64, 1.0, S.ALPHA_PER_HEAD, S.LAYOUT_BHND),
    ("one-token", "bf16", 1, 2, 128, 128, 1.0, S.ALPHA_PER_HEAD, S.LAYOUT_BHND),
]


def _check(name, got, ref, floor=0.0):
    ref = np.asarray(ref, np.float64)
    g = np.asarray(got, np.float64)
    scale = max(np.abs(ref).max(), floor, 1e-30)
    err = np.abs(g - ref).max()
    say(f"  {name}: max-abs {err:.2e} (scale {scale:.2e})")
    assert np.isfinite(g).all()
    assert err <= REL * scale, (name, err, scale)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(orc, dev, case):
    name, dtype, N, H, d, bq, frac, amode, layout = case
    say(f"case backward {name}: N={N} H={H} d={d} bq={bq} frac={frac}")
    gen = "centroids" if dtype == "f32" else "smooth"
    w = I.Workload(name, 1, H, N, d, bq, 64, frac, dtype, gen, seed=13)
    x = I.make_inputs(w)
    rng = np.random.default_rng(3)
    alpha = (rng.uniform(0.2, 0.9, (H, w.Tq)).astype(np.float32) if amode else x.alpha)
    dO = rng.normal(0, 1, (1, H, N, d)).astype(np.float32)
    q, k, v, wq, wk, _ = to_dev(x, dev)
    p = S.problem(1, H, N, d, bq, 64, frac, 1, dtype, layout=layout, alpha_mode=amode)
    idx, _ = S.route(S.problem(1, H, N, d, bq, 64, frac, 1, dtype), q, k, wq, wk,
                     want_mask=False)
    t = ((lambda a: a.permute(0, 2, 1, 3).contiguous()) if layout == S.LAYOUT_BNHD
         else (lambda a: a))
    dOd = t(torch.from_numpy(dO).to(dev))
    dQ, dK, dV, da = S.backward(p, t(q), t(k), t(v), idx, torch.from_numpy(alpha).to(dev), dOd)
    torch.cuda.synchronize()
    back = (lambda a: a.permute(0, 2, 1, 3).contiguous()) if layout == S.LAYOUT_BNHD else t
    op = orc.problem(1, H, N, d, bq, 64, frac, 1, dtype, alpha_mode=amode)
    oidx = idx.cpu().numpy()
    rQ, rK, rV, ra = orc.backward(op, x.q, x.k, x.v, oidx, alpha, dO.astype(np.float64))
    fq = fk = 0.0
    if N == 1:
        # a single token attends to itself only: P = 1 and dP = D, so dQ and dK
        # are exactly 0 by cancellation; the bar is relative to the cancelling
        # terms, |D| = |alpha dO . v| times |k| (or |q|) / sqrt(d)
        qf, kf, vf = (np.asarray(I.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a,
                                 np.float64) for a in (x.q, x.k, x.v))
        Dm = np.abs(np.reshape(alpha, (H, -1))[:, :1] * (dO[0] * vf[0]).sum(-1)).max()
        fq = Dm * np.abs(kf).max() / np.sqrt(d)
        fk = Dm * np.abs(qf).max() / np.sqrt(d)
    _check("dQ", back(dQ).cpu().numpy(), rQ, fq)
    _check("dK", back(dK).cpu().numpy(), rK, fk)
    _check("dV", back(dV).cpu().numpy(), rV)
    _check("dalpha", da.cpu().numpy(), ra)


@pytest.mark.parametrize("dtype,bq", [("bf16", 128), ("f32", 64)], ids=["matrix-core", "valu"])
def test_backward_two_batches(orc, dev, dtype, bq):
    """B = 2 with per-query-block alpha: the batch stride and the head of each
    (batch, head) pair on both paths."""
    B, H, N, d = 2, 2, 700, 128 if dtype == "bf16" else 64
    say(f"case backward B=2 {dtype}: N={N} H={H} d={d} bq={bq}")
    gen = "centroids" if dtype == "f32" else "smooth"
    w = I.Workload("b2", B, H, N, d, bq, 64, 0.2, dtype, gen, seed=21)
    x = I.make_inputs(w)
    rng = np.random.default_rng(6)
    alpha = rng.uniform(0.2, 0.9, (H, w.Tq)).astype(np.float32)
    dO = rng.normal(0, 1, (B, H, N, d)).astype(np.float32)
    q, k, v, wq, wk, _ = to_dev(x, dev)
    p = S.problem(B, H, N, d, bq, 64, 0.2, 1, dtype, alpha_mode=S.ALPHA_PER_QBLOCK)
    idx, _ = S.route(S.problem(B, H, N, d, bq, 64, 0.2, 1, dtype), q, k, wq, wk, want_mask=False)
    dQ, dK, dV, da = S.backward(p, q, k, v, idx, torch.from_numpy(alpha).to(dev),
                                torch.from_numpy(dO).to(dev))
    torch.cuda.synchronize()
    op = orc.problem(B, H, N, d, bq, 64, 0.2, 1, dtype, alpha_mode=S.ALPHA_PER_QBLOCK)
    rQ, rK, rV, ra = orc.backward(op, x.q, x.k, x.v, idx.cpu().numpy(), alpha,
                                  dO.astype(np.float64))
    _check("dQ", dQ.cpu().numpy(), rQ)
    _check("dK", dK.cpu().numpy(), rK)
    _check("dV", dV.cpu().numpy(), rV)
    _check("dalpha", da.cpu().numpy(), ra)


def test_backward_wan13b_one_head(orc, dev):
    """One head of the 1.3B shape (N = 32760, k = 16 of 512): every gradient
    entry against the oracle."""
    w = I.WAN13B.with_(H=1)
    x = I.make_inputs(w)
    q, k, v, wq, wk, al = to_dev(x, dev)
    p = S.problem(1, 1, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    idx, _ = S.route(p, q, k, wq, wk, want_mask=False)
    dO = np.random.default_rng(4).normal(0, 1, (1, 1, w.N, w.d)).astype(np.float32)
    dQ, dK, dV, da = S.backward(p, q, k, v, idx, al, torch.from_numpy(dO).to(dev))
    torch.cuda.synchronize()
    op = orc.problem(1, 1, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    rQ, rK, rV, ra = orc.backward(op, x.q, x.k, x.v, idx.cpu().numpy(), x.alpha,
                                  dO.astype(np.float64))
    _check("dQ", dQ.cpu().numpy(), rQ)
    _check("dK", dK.cpu().numpy(), rK)
    _check("dV", dV.cpu().numpy(), rV)
    _check("dalpha", da.cpu().numpy(), ra)


def test_backward_ragged_product_tiles(orc, dev):
    """One head with N = 41003 (k = 20 of 641 KV blocks): the selected
    summaries are summed by 0/1 products of 320-row tiles, here two row tiles
    over the 321 query blocks (the second holding one) and three over the
    641 KV blocks (the last holding one), and the last KV block is ragged.
    Every gradient entry against the oracle."""
    w = I.WAN13B.with_(H=1, N=41003)
    say("case backward ragged product tiles: N=41003 H=1")
    x = I.make_inputs(w)
    q, k, v, wq, wk, al = to_dev(x, dev)
    p = S.problem(1, 1, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    assert (S.num_q_blocks(p), S.num_kv_blocks(p)) == (321, 641)
    idx, _ = S.route(p, q, k, wq, wk, want_mask=False)
    dO = np.random.default_rng(5).normal(0, 1, (1, 1, w.N, w.d)).astype(np.float32)
    dQ, dK, dV, da = S.backward(p, q, k, v, idx, al, torch.from_numpy(dO).to(dev))
    torch.cuda.synchronize()
    op = orc.problem(1, 1, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    rQ, rK, rV, ra = orc.backward(op, x.q, x.k, x.v, idx.cpu().numpy(), x.alpha,
                                  dO.astype(np.float64))
    _check("dQ", dQ.cpu().numpy(), rQ)
    _check("dK", dK.cpu().numpy(), rK)
    _check("dV", dV.cpu().numpy(), rV)
    _check("dalpha", da.cpu().numpy(), ra)


@pytest.mark.parametrize("dtype,bq,frac", [("bf16", 128, 0.2), ("bf16", 128, 1.0), ("f32", 64, 0.25)],
                         ids=["matrix-core", "matrix-core-all-selected", "valu"])
def test_backward_ignores_workspace_contents(dev, dtype, bq, frac):
    """A workspace filled with NaN bit patterns gives the same gradients, bit
    for bit, as a zeroed one: no pass reads workspace memory it has not
    written in the same call."""
    N, H, d = 1100, 2, 128 if dtype == "bf16" else 64
    gen = "centroids" if dtype == "f32" else "smooth"
    w = I.Workload("ws", 1, H, N, d, bq, 64, frac, dtype, gen, seed=41)
    x = I.make_inputs(w)
    q, k, v, wq, wk, al = to_dev(x, dev)
    p = S.problem(1, H, N, d, bq, 64, frac, 1, dtype)
    idx, _ = S.route(p, q, k, wq, wk, want_mask=False)
    dO = torch.from_numpy(np.random.default_rng(8).normal(0, 1, (1, H, N, d)).astype(np.float32)).to(dev)
    outs = []
    for fill in (0x00, 0xFF):
        ws = S.workspace(p, S.OP_BACKWARD, dev)
        ws.fill_(fill)
        outs.append(S.backward(p, q, k, v, idx, al, dO, ws=ws))
        torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


SOFTMAX_CASES = [  # name, dtype, N, H, d, bq, frac
    ("bf16-d128-bq128", "bf16", 1300, 2, 128, 128, 0.15),
    ("bf16-d128-bq64", "bf16", 900, 2, 128, 64, 0.25),
    ("f32-d64-bq64", "f32", 700, 2, 64, 64, 0.2),
    ("bf16-k0", "bf16", 640, 2, 128, 128, 0.0),
    ("f32-all-selected", "f32", 500, 2, 64, 64, 1.0),
]


@pytest.mark.parametrize("case", SOFTMAX_CASES, ids=[c[0] for c in SOFTMAX_CASES])
def test_backward_softmax_phi(orc, dev, case):
    """phi = the softmax of each row (the SLA notes' training choice): the
    gradients run through the row softmax's Jacobian, dx = p (dphi - p .
    dphi), on the vector-ALU kernels; against the oracle's backward, whose
    softmax-phi derivative is pinned to torch autograd on the CPU."""
    name, dtype, N, H, d, bq, frac = case
    say(f"case backward softmax phi {name}: N={N} H={H} d={d} bq={bq} frac={frac}")
    gen = "centroids" if dtype == "f32" else "smooth"
    w = I.Workload(name, 1, H, N, d, bq, 64, frac, dtype, gen, seed=17)
    x = I.make_inputs(w)
    rng = np.random.default_rng(12)
    dO = rng.normal(0, 1, (1, H, N, d)).astype(np.float32)
    q, k, v, wq, wk, al = to_dev(x, dev)
    p = S.problem(1, H, N, d, bq, 64, frac, 1, dtype, phi=S.PHI_SOFTMAX)
    idx, _ = S.route(p, q, k, wq, wk, want_mask=False)
    dQ, dK, dV, da = S.backward(p, q, k, v, idx, al, torch.from_numpy(dO).to(dev))
    torch.cuda.synchronize()
    op = orc.problem(1, H, N, d, bq, 64, frac, 1, dtype, phi=1)
    rQ, rK, rV, ra = orc.backward(op, x.q, x.k, x.v, idx.cpu().numpy(), x.alpha,
                                  dO.astype(np.float64))
    _check("dQ", dQ.cpu().numpy(), rQ)
    _check("dK", dK.cpu().numpy(), rK)
    _check("dV", dV.cpu().numpy(), rV)
    _check("dalpha", da.cpu().numpy(), ra)
