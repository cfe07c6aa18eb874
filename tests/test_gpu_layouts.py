"""GPU parity of the problem options: the token-major [B,N,H,d] layout of Q,
K, V and O, alpha per (head, query block) -- the granularity of the pages'
algorithm ("SLA2 深度解读" 08) -- and a bf16 output.

Every kernel path is covered: fp32 (vector ALU), bf16 with b_q = 64 (vector
ALU), bf16 d = 64 (matrix cores), bf16 d = 128 (fused d = 128 kernel) and the
low-bit sparse branch.  The oracle takes the same inputs transposed to
[B,H,N,d]; its router must match bit for bit, its output within the path's
tolerance.  A bf16 output must equal, bit for bit, the round-to-nearest-even
of the fp32 output of the same call.
"""
import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S
from tests.test_gpu_parity import TOL, compare_blocks, check_route, dev, say  # noqa: F401

pytestmark = pytest.mark.gpu

PATHS = [  # name, dtype, N, d, bq, frac, fp8, lowbit
    ("f32", "f32", 700, 128, 128, 0.3, False, S.LOWBIT_QK),
    ("bf16-bq64", "bf16", 513, 128, 64, 0.2, False, S.LOWBIT_QK),
    ("bf16-d64", "bf16", 1000, 64, 128, 0.3, False, S.LOWBIT_QK),
    ("bf16-d128", "bf16", 4100, 128, 128, 0.05, False, S.LOWBIT_QK),
    ("fp8", "bf16", 2000, 128, 128, 0.1, True, S.LOWBIT_QK),
    ("fp8-v", "bf16", 2000, 128, 128, 0.1, True, S.LOWBIT_QKV),
    ("i8-v", "bf16", 2000, 128, 128, 0.1, True, S.LOWBIT_I8QKV),
]
OPTS = [  # layout, alpha mode
    (S.LAYOUT_BNHD, S.ALPHA_PER_HEAD),
    (S.LAYOUT_BHND, S.ALPHA_PER_QBLOCK),
    (S.LAYOUT_BNHD, S.ALPHA_PER_QBLOCK),
]


def upload(a, dev, layout):
    if layout == S.LAYOUT_BNHD:
        a = np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


@pytest.mark.parametrize("opt", OPTS, ids=["bnhd", "alpha-qblock", "bnhd-alpha-qblock"])
@pytest.mark.parametrize("path", PATHS, ids=[c[0] for c in PATHS])
def test_layout_alpha_and_bf16_output(orc, dev, path, opt):
    name, dtype, N, d, bq, frac, fp8, lowbit = path
    layout, amode = opt
    H = 3
    gen = "centroids" if dtype == "f32" else "smooth"
    x = I.make_inputs(I.Workload(name, 1, H, N, d, bq, 64, frac, dtype, gen, seed=11))
    w = x.wl
    say(f"case {name}: layout {layout} alpha mode {amode} N={N} d={d} bq={bq}")
    Tq = w.Tq
    alpha = (np.random.default_rng(7).uniform(0.2, 0.95, (H, Tq)).astype(np.float32)
             if amode == S.ALPHA_PER_QBLOCK else x.alpha)
    q, k, v = (upload(a, dev, layout) for a in (x.q, x.k, x.v))
    wq, wk = (torch.from_numpy(a).to(dev) for a in (x.wq, x.wk))
    al = torch.from_numpy(alpha).to(dev)
    outs = {}
    for od in (S.F32, S.BF16):
        p = S.problem(1, H, N, d, bq, 64, frac, 1, dtype, layout=layout, alpha_mode=amode,
                      out_dtype=od, lowbit=lowbit)
        idx, mask = S.route(p, q, k, wq, wk)
        outs[od] = S.forward(p, q, k, v, idx, al, fp8=fp8)
        torch.cuda.synchronize()
    oidx = check_route(orc, x, idx, mask)
    # bf16 output: the fp32 result rounded once, to nearest even
    assert torch.equal(outs[S.BF16], outs[S.F32].to(torch.bfloat16))
    O = outs[S.F32]
    if layout == S.LAYOUT_BNHD:
        O = O.permute(0, 2, 1, 3).contiguous()
    op = orc.problem(1, H, N, d, bq, 64, frac, 1, dtype, alpha_mode=amode,
                     lowbit_v=lowbit & 1, int8_qk=(lowbit >> 1) & 1)
    tol = TOL["fp8"] if fp8 else TOL[dtype]
    compare_blocks(orc, x, oidx, O, orc.all_blocks(op), tol,
                   variant="fp8" if fp8 else "exact", op=op, alpha=alpha)


@pytest.mark.parametrize("path", PATHS[:4], ids=[c[0] for c in PATHS[:4]])
def test_attention_call_equals_route_then_forward(orc, dev, path):
    """sla2_attention (router and block summaries overlapped on the bf16 bq =
    128 path) gives the same selection and the same output bits as
    sla2_route followed by sla2_forward."""
    name, dtype, N, d, bq, frac, fp8, lowbit = path
    gen = "centroids" if dtype == "f32" else "smooth"
    x = I.make_inputs(I.Workload(name, 1, 3, N, d, bq, 64, frac, dtype, gen, seed=17))
    say(f"case attention call {name}: N={N} d={d} bq={bq}")
    q, k, v = (upload(a, dev, S.LAYOUT_BHND) for a in (x.q, x.k, x.v))
    wq, wk, al = (torch.from_numpy(a).to(dev) for a in (x.wq, x.wk, x.alpha))
    p = S.problem(1, 3, N, d, bq, 64, frac, 1, dtype)
    idx0, _ = S.route(p, q, k, wq, wk, want_mask=False)
    O0 = S.forward(p, q, k, v, idx0, al)
    for _ in range(2):  # the helper stream and its events are reused
        idx1, O1 = S.attention(p, q, k, v, wq, wk, al)
        torch.cuda.synchronize()
        assert torch.equal(idx0, idx1)
        assert torch.equal(O0, O1)


ATTN_CASES = [  # B, H, layout, alpha mode, w_heads, out dtype, frac
    (2, 8, S.LAYOUT_BHND, S.ALPHA_PER_HEAD, 8, S.F32, 0.1),
    (1, 12, S.LAYOUT_BNHD, S.ALPHA_PER_QBLOCK, 1, S.BF16, 0.2),
    (2, 9, S.LAYOUT_BNHD, S.ALPHA_PER_QBLOCK, 9, S.F32, 0.0),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=["b2-h8-whead", "h12-bnhd-bf16out", "b2-h9-k0"])
def test_attention_batches_and_options(dev, case):
    """sla2_attention with two batch entries, per-head projections, the
    token-major layout, bf16 output and k = 0: the selection and the output
    bits equal sla2_route followed by sla2_forward."""
    B, H, lay, amode, wh, odt, frac = case
    N, d = 1300, 128
    say(f"case attention call: B={B} H={H} layout={lay} alpha={amode} w_heads={wh}")
    x = I.make_inputs(I.Workload("attn", B, H, N, d, 128, 64, frac, "bf16", "smooth", seed=23))
    rng = np.random.default_rng(9)
    q, k, v = (upload(a, dev, lay) for a in (x.q, x.k, x.v))
    wq = torch.from_numpy(rng.normal(0, d ** -0.5, (wh, d, d)).astype(np.float32)).to(dev)
    wk = torch.from_numpy(rng.normal(0, d ** -0.5, (wh, d, d)).astype(np.float32)).to(dev)
    p = S.problem(B, H, N, d, 128, 64, frac, wh, "bf16", layout=lay, alpha_mode=amode,
                  out_dtype=odt)
    shape = (H, S.num_q_blocks(p)) if amode == S.ALPHA_PER_QBLOCK else (H,)
    al = torch.from_numpy(rng.uniform(0.2, 0.9, shape).astype(np.float32)).to(dev)
    if frac > 0:
        idx0, _ = S.route(p, q, k, wq, wk, want_mask=False)
    else:
        idx0 = None
    O0 = S.forward(p, q, k, v, idx0, al)
    for _ in range(2):
        idx1, O1 = S.attention(p, q, k, v, wq, wk, al)
        torch.cuda.synchronize()
        if frac > 0:
            assert torch.equal(idx0, idx1)
        assert torch.equal(O0, O1)


@pytest.mark.parametrize("lowbit", [S.LOWBIT_QK, S.LOWBIT_QKV, S.LOWBIT_I8QK, S.LOWBIT_I8QKV],
                         ids=["fp8", "fp8-v", "i8", "i8-v"])
def test_attention_fp8_equals_route_then_forward_fp8(dev, lowbit):
    """sla2_attention_fp8 (query codes and K block sums from the router's
    pooling pass, block summaries and key codes on the helper stream) gives
    the same selection and the same output bits as sla2_route followed by
    sla2_forward_fp8; two batch entries, token-major layout, per-query-block
    alpha."""
    B, H, N, d = 2, 3, 2000, 128
    say(f"case attention fp8 lowbit={lowbit}: B={B} H={H} N={N}")
    x = I.make_inputs(I.Workload("a8", B, H, N, d, 128, 64, 0.1, "bf16", "smooth", seed=29))
    lay = S.LAYOUT_BNHD
    q, k, v = (upload(a, dev, lay) for a in (x.q, x.k, x.v))
    wq, wk = (torch.from_numpy(a).to(dev) for a in (x.wq, x.wk))
    p = S.problem(B, H, N, d, 128, 64, 0.1, 1, "bf16", layout=lay,
                  alpha_mode=S.ALPHA_PER_QBLOCK, lowbit=lowbit)
    rng = np.random.default_rng(31)
    al = torch.from_numpy(rng.uniform(0.2, 0.9, (H, S.num_q_blocks(p))).astype(np.float32)).to(dev)
    idx0, _ = S.route(p, q, k, wq, wk, want_mask=False)
    O0 = S.forward(p, q, k, v, idx0, al, fp8=True)
    for _ in range(2):
        idx1, O1 = S.attention(p, q, k, v, wq, wk, al, fp8=True)
        torch.cuda.synchronize()
        assert torch.equal(idx0, idx1)
        assert torch.equal(O0, O1)


@pytest.mark.parametrize("frac", [0.0, 1.0], ids=["k0", "all-selected"])
@pytest.mark.parametrize("lowbit", [S.LOWBIT_QK, S.LOWBIT_I8QKV], ids=["fp8", "i8-v"])
def test_attention_fp8_edge_selections(dev, lowbit, frac):
    """sla2_attention_fp8 with nothing selected (k = 0: only the linear
    branch) and with every block selected (k = T_kv): the same output bits as
    sla2_route + sla2_forward_fp8; ragged last blocks (N = 1500)."""
    B, H, N, d = 1, 2, 1500, 128
    say(f"case attention fp8 lowbit={lowbit} frac={frac}: N={N}")
    x = I.make_inputs(I.Workload("a8e", B, H, N, d, 128, 64, frac, "bf16", "smooth", seed=37))
    q, k, v = (upload(a, dev, S.LAYOUT_BHND) for a in (x.q, x.k, x.v))
    wq, wk, al = (torch.from_numpy(a).to(dev) for a in (x.wq, x.wk, x.alpha))
    p = S.problem(B, H, N, d, 128, 64, frac, 1, "bf16", lowbit=lowbit)
    idx0 = S.route(p, q, k, wq, wk, want_mask=False)[0] if frac > 0 else None
    O0 = S.forward(p, q, k, v, idx0, al, fp8=True)
    idx1, O1 = S.attention(p, q, k, v, wq, wk, al, fp8=True)
    torch.cuda.synchronize()
    if frac > 0:
        assert torch.equal(idx0, idx1)
    assert torch.equal(O0, O1)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_attention_ignores_workspace_contents(dev, fp8):
    """A workspace filled with NaN bit patterns gives the same selection and
    output bits as a zeroed one."""
    B, H, N, d = 1, 2, 1500, 128
    x = I.make_inputs(I.Workload("ws", B, H, N, d, 128, 64, 0.15, "bf16", "smooth", seed=43))
    q, k, v = (upload(a, dev, S.LAYOUT_BHND) for a in (x.q, x.k, x.v))
    wq, wk, al = (torch.from_numpy(a).to(dev) for a in (x.wq, x.wk, x.alpha))
    p = S.problem(B, H, N, d, 128, 64, 0.15, 1, "bf16")
    outs = []
    for fill in (0x00, 0xFF):
        ws = S.workspace(p, S.OP_ATTENTION_FP8 if fp8 else S.OP_ATTENTION, dev)
        ws.fill_(fill)
        outs.append(S.attention(p, q, k, v, wq, wk, al, ws=ws, fp8=fp8))
        torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
