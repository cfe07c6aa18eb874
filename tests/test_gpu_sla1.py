"""GPU parity of the softmax feature map and the SLA (v1) mode against the
CPU oracle, through the C ABI.

Bar as for the other forward tests: critical / negligible indices and the
ternary mask bit-exact (the oracle's margin report guards both cuts), outputs
within 2e-3 max-abs for bf16 inputs and 1e-5 for fp32.  Shapes the matrix-core
kernels do not take (b_q = 64 as in the SLA notes' setting, d = 64, fp32)
run on the vector-ALU kernels.
"""
import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S
from tests.test_gpu_parity import TOL, compare_blocks, dev, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu


def problem(w, phi=S.PHI_ELU1, w_heads=1, **kw):
    return S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, w_heads, w.dtype, phi=phi,
                     **kw)


def oracle_problem(orc, w, phi, w_heads=1, low=0.0, mode=1):
    return orc.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, w_heads, w.dtype, phi=phi,
                       mode=mode, low_frac=low)


def route_both(orc, x, q, k, low, heads=None):
    """GPU and oracle v1 routing; indices and masks must agree bit for bit."""
    w = x.wl
    p = problem(w)
    crit, negl, mask = S.route_v1(p, q, k, low)
    torch.cuda.synchronize()
    op = oracle_problem(orc, w, 0, low=low)
    oc, on, om, gap, _ = orc.route_v1(op, x.q, x.k, heads=heads)
    sel = slice(None) if heads is None else np.asarray(heads)
    nbh = w.B * w.H
    g = gap.reshape(nbh, -1)[sel]
    assert not ((g > 0) & (g < 1e-12)).any(), "workload has a near-tie at a routing cut"
    for got, want in ((crit, oc), (negl, on), (mask, om)):
        got = got.cpu().numpy().reshape(nbh, *got.shape[2:])[sel]
        assert np.array_equal(got, want.reshape(nbh, *want.shape[2:])[sel])
    return crit, negl, oc, on


def compare_v1(orc, x, O, oc, on, wp, phi, low, blocks, w_heads=1):
    w = x.wl
    tol = TOL[w.dtype]
    op = oracle_problem(orc, w, phi, w_heads, low)
    ref = orc.forward_v1(op, x.q, x.k, x.v, oc, on, wp, blocks)
    Oc = O.float().cpu().numpy().reshape(w.B * w.H, w.N, w.d)
    worst = 0.0
    for n, (bh, i) in enumerate(blocks):
        t0 = i * w.bq
        nv = min(w.bq, w.N - t0)
        err = np.abs(Oc[bh, t0:t0 + nv] - ref[n, :nv])
        assert np.isfinite(err).all()
        worst = max(worst, float(err.max()))
    say(f"  max-abs error over {len(blocks)} blocks: {worst:.3e} (tol {tol})")
    assert worst <= tol


CASES = [  # name, N, H, k_h frac, k_l frac, phi, w_heads
    ("ragged", 700, 2, 0.2, 0.3, S.PHI_SOFTMAX, 1),
    ("tiles", 4100, 3, 0.05, 0.10, S.PHI_SOFTMAX, 3),
    ("elu", 2000, 2, 0.1, 0.2, S.PHI_ELU1, 1),
    ("no-critical", 1500, 2, 0.0, 0.25, S.PHI_SOFTMAX, 1),
    ("no-negligible", 1500, 2, 0.2, 0.0, S.PHI_SOFTMAX, 2),
    ("all-marginal", 900, 2, 0.0, 0.0, S.PHI_SOFTMAX, 1),
    ("no-marginal", 1200, 2, 0.4, 0.6, S.PHI_SOFTMAX, 1),
    ("one-token", 1, 2, 1.0, 0.0, S.PHI_SOFTMAX, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sla1_parity(orc, dev, case):
    name, N, H, kh, low, phi, wh = case
    say(f"case sla1 {name}: N={N} H={H} k_h={kh} k_l={low} phi={phi} w_heads={wh}")
    w = I.Workload(name, 1, H, N, 128, 128, 64, kh, "bf16", "smooth", seed=5)
    x = I.make_inputs(w)
    q, k, v, _, _, _ = to_dev(x, dev)
    crit, negl, oc, on = route_both(orc, x, q, k, low)
    wp = np.random.default_rng(9).normal(0, 0.15, (wh, 128, 128)).astype(np.float32)
    p = problem(w, phi, wh)
    O = S.forward_v1(p, q, k, v, crit, negl, low, torch.from_numpy(wp).to(dev))
    torch.cuda.synchronize()
    compare_v1(orc, x, O, oc, on, wp, phi, low, orc.all_blocks(oracle_problem(orc, w, phi)), wh)


def test_sla1_route_all_scores_equal(orc, dev):
    """Every key block the same, so every score of a row ties: the critical
    blocks are the k_h lowest indices (ties to the lower index) and the
    negligible ones the k_l highest (the order's last blocks)."""
    w = I.Workload("v1-ties", 1, 2, 3000, 128, 128, 64, 0.1, "bf16", "smooth", seed=5)
    x = I.make_inputs(w)
    x.k = np.ascontiguousarray(np.broadcast_to(x.k[:, :, :1, :], x.k.shape))
    q, k, v, _, _, _ = to_dev(x, dev)
    low = 0.2
    crit, negl, oc, on = route_both(orc, x, q, k, low)
    kh, kl, T = crit.shape[-1], negl.shape[-1], w.Tkv
    assert (crit.cpu().numpy() == np.arange(kh)).all()
    assert (negl.cpu().numpy() == np.arange(T - kl, T)).all()


@pytest.mark.parametrize("N", [1200 * 64, 1200 * 64 + 1])
def test_sla1_route_at_the_one_pass_limit(orc, dev, N):
    """Critical and negligible indices and the ternary mask exact at 1200 KV
    blocks (scores and both selections in one pass) and at 1201 (scores
    through memory, two top-k passes)."""
    say(f"case sla1 route at T_kv limit: N={N}")
    w = I.Workload("v1-limit", 1, 2, N, 128, 128, 64, 0.05, "bf16", "smooth", seed=7)
    x = I.make_inputs(w)
    q, k, v, _, _, _ = to_dev(x, dev)
    route_both(orc, x, q, k, 0.1)


# the vector-ALU kernels: b_q = 64 (the SLA notes' b_q = b_kv = 64), d = 64, fp32
VALU_CASES = [  # name, N, H, d, b_q, dtype, k_h frac, k_l frac, phi, w_heads
    ("b64-ragged", 700, 2, 128, 64, "bf16", 0.2, 0.3, S.PHI_SOFTMAX, 1),
    ("b64-tiles", 4100, 2, 128, 64, "bf16", 0.05, 0.10, S.PHI_SOFTMAX, 2),
    ("b64-d64-f32", 1500, 2, 64, 64, "f32", 0.1, 0.2, S.PHI_SOFTMAX, 1),
    ("b64-elu", 2000, 2, 128, 64, "bf16", 0.1, 0.2, S.PHI_ELU1, 1),
    ("b64-no-marginal", 1200, 2, 128, 64, "bf16", 0.4, 0.6, S.PHI_SOFTMAX, 1),
    ("b64-no-critical", 1500, 2, 128, 64, "bf16", 0.0, 0.25, S.PHI_SOFTMAX, 1),
    ("b64-all-marginal", 900, 2, 128, 64, "bf16", 0.0, 0.0, S.PHI_SOFTMAX, 1),
    ("b128-d64", 1300, 2, 64, 128, "bf16", 0.1, 0.2, S.PHI_SOFTMAX, 1),
    ("b128-f32", 900, 2, 128, 128, "f32", 0.15, 0.1, S.PHI_SOFTMAX, 2),
]


@pytest.mark.parametrize("case", VALU_CASES, ids=[c[0] for c in VALU_CASES])
def test_sla1_parity_valu_shapes(orc, dev, case):
    name, N, H, d, bq, dt, kh, low, phi, wh = case
    say(f"case sla1 {name}: N={N} H={H} d={d} b_q={bq} {dt} k_h={kh} k_l={low} phi={phi}")
    w = I.Workload(name, 1, H, N, d, bq, 64, kh, dt, "smooth", seed=8)
    x = I.make_inputs(w)
    q, k, v, _, _, _ = to_dev(x, dev)
    crit, negl, oc, on = route_both(orc, x, q, k, low)
    wp = np.random.default_rng(10).normal(0, 0.15, (wh, d, d)).astype(np.float32)
    p = problem(w, phi, wh)
    O = S.forward_v1(p, q, k, v, crit, negl, low, torch.from_numpy(wp).to(dev))
    torch.cuda.synchronize()
    compare_v1(orc, x, O, oc, on, wp, phi, low, orc.all_blocks(oracle_problem(orc, w, phi)), wh)


def test_sla1_wan13b_notes_blocks(orc, dev):
    """The SLA notes' own setting at the 1.3B shape: b_q = b_kv = 64, k_h =
    5 %, k_l = 10 %, softmax phi; routing of two heads bit-exact, sampled
    query blocks (first, last, random) to 2e-3."""
    w = I.WAN13B.with_(bq=64, topk_frac=0.05)
    x = I.make_inputs(w)
    low = 0.10
    q, k, v, _, _, _ = to_dev(x, dev)
    heads = [3, 10]
    crit, negl, oc, on = route_both(orc, x, q, k, low, heads=heads)
    assert S.topk(problem(w)) == 26 and S.num_negligible(problem(w), low) == 52
    wp = np.random.default_rng(2).normal(0, 0.1, (1, 128, 128)).astype(np.float32)
    say("sla1 wan13b b_q = 64: forward")
    O = S.forward_v1(problem(w, S.PHI_SOFTMAX), q, k, v, crit, negl, low,
                     torch.from_numpy(wp).to(dev))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    blocks = [(h, int(i)) for h in heads for i in {0, w.Tq - 1, *rng.choice(w.Tq, 4).tolist()}]
    compare_v1(orc, x, O, oc, on, wp, S.PHI_SOFTMAX, low, blocks)


def test_sla1_bf16_output_and_token_major_layout(orc, dev):
    """[B,N,H,d] inputs and a bf16 output: the same values, the output the
    fp32 result rounded once."""
    w = I.Workload("layout", 1, 3, 2000, 128, 128, 64, 0.1, "bf16", "smooth", seed=6)
    x = I.make_inputs(w)
    low = 0.15
    q, k, v, _, _, _ = to_dev(x, dev)
    crit, negl, oc, on = route_both(orc, x, q, k, low)
    wp = np.random.default_rng(3).normal(0, 0.15, (1, 128, 128)).astype(np.float32)
    wpd = torch.from_numpy(wp).to(dev)
    t = lambda a: a.permute(0, 2, 1, 3).contiguous()
    outs = {}
    for od in (S.F32, S.BF16):
        p = problem(w, S.PHI_SOFTMAX, layout=S.LAYOUT_BNHD, out_dtype=od)
        outs[od] = S.forward_v1(p, t(q), t(k), t(v), crit, negl, low, wpd)
    torch.cuda.synchronize()
    assert torch.equal(outs[S.BF16], outs[S.F32].to(torch.bfloat16))
    O = outs[S.F32].permute(0, 2, 1, 3).contiguous()
    compare_v1(orc, x, O, oc, on, wp, S.PHI_SOFTMAX, low,
               orc.all_blocks(oracle_problem(orc, w, S.PHI_SOFTMAX)))


def test_sla1_wan13b_sampled(orc, dev):
    """The 1.3B shape (N = 32760, 12 heads) with the notes' k_h = 5 %, k_l =
    10 %: routing of two heads bit-exact, sampled query blocks to 2e-3."""
    w = I.WAN13B.with_(topk_frac=0.05)
    x = I.make_inputs(w)
    low = 0.10
    q, k, v, _, _, _ = to_dev(x, dev)
    heads = [2, 9]
    crit, negl, oc, on = route_both(orc, x, q, k, low, heads=heads)
    assert S.topk(problem(w)) == 26 and S.num_negligible(problem(w), low) == 52
    wp = np.random.default_rng(1).normal(0, 0.1, (1, 128, 128)).astype(np.float32)
    O = S.forward_v1(problem(w, S.PHI_SOFTMAX), q, k, v, crit, negl, low,
                     torch.from_numpy(wp).to(dev))
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    blocks = [(h, int(i)) for h in heads for i in {0, w.Tq - 1, *rng.choice(w.Tq, 3).tolist()}]
    compare_v1(orc, x, O, oc, on, wp, S.PHI_SOFTMAX, low, blocks)


SMPHI_VALU = [  # N, d, b_q, dtype, frac
    (700, 128, 64, "bf16", 0.25), (2100, 64, 128, "bf16", 0.1), (1500, 128, 128, "f32", 0.1),
    (900, 64, 64, "f32", 0.0), (640, 128, 64, "bf16", 1.0)]


@pytest.mark.parametrize("N,d,bq,dt,frac", SMPHI_VALU,
                         ids=[f"N{c[0]}-d{c[1]}-bq{c[2]}-{c[3]}-k{c[4]}" for c in SMPHI_VALU])
def test_sla2_softmax_phi_valu_shapes(orc, dev, N, d, bq, dt, frac):
    """The SLA2 forward with the softmax feature map on the vector-ALU
    kernels (b_q = 64, d = 64, fp32), one call and route + forward."""
    w = I.Workload("smphi-valu", 1, 2, N, d, bq, 64, frac, dt, "smooth", seed=9)
    x = I.make_inputs(w)
    say(f"case sla2 softmax phi (vector ALU): N={N} d={d} b_q={bq} {dt} frac={frac}")
    q, k, v, wq, wk, al = to_dev(x, dev)
    p = problem(w, S.PHI_SOFTMAX)
    idx, O = S.attention(p, q, k, v, wq, wk, al)
    O0 = S.forward(p, q, k, v, idx, al)
    torch.cuda.synchronize()
    assert torch.equal(O, O0)
    op = orc.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, frac, 1, dt, phi=1)
    oidx, _, _, _ = orc.route(op, x.q, x.k, x.wq, x.wk)
    if S.topk(p) > 0:
        assert np.array_equal(idx.cpu().numpy(), oidx)
    compare_blocks(orc, x, oidx, O, orc.all_blocks(op), TOL[dt], op=op)


@pytest.mark.parametrize("N,frac", [(700, 0.25), (4100, 0.05), (900, 0.0), (640, 1.0)])
def test_sla2_with_softmax_phi(orc, dev, N, frac):
    """The SLA2 forward with the softmax feature map (alpha mix unchanged)."""
    w = I.Workload("smphi", 1, 2, N, 128, 128, 64, frac, "bf16", "smooth", seed=7)
    x = I.make_inputs(w)
    say(f"case sla2 softmax phi: N={N} frac={frac}")
    q, k, v, wq, wk, al = to_dev(x, dev)
    p = problem(w, S.PHI_SOFTMAX)
    idx, _ = S.route(p, q, k, wq, wk, want_mask=False)
    O = S.forward(p, q, k, v, idx, al)
    torch.cuda.synchronize()
    op = orc.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, frac, 1, "bf16", phi=1)
    oidx, _, _, _ = orc.route(op, x.q, x.k, x.wq, x.wk)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    compare_blocks(orc, x, oidx, O, orc.all_blocks(op), TOL["bf16"], op=op)
