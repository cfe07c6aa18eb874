"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: block masks and top-k indices bit-exact; outputs within 1e-5 max-abs
for fp32 inputs, 2e-3 for bf16 inputs, 3e-2 for the fp8 sparse branch.
The oracle's margin report guards the mask comparison: a seed whose k-th and
(k+1)-th router scores sit within 1e-12 (relative) would make the selection
depend on rounding order and is reported as a failure of the workload, not
of either side.
"""
import os

import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 3e-2}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    S.lib()
    return torch.device("cuda:0")


def to_dev(x, dev):
    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)
    return t(x.q), t(x.k), t(x.v), t(x.wq), t(x.wk), t(x.alpha)


def problem_of(x, lowbit=S.LOWBIT_QK):
    w = x.wl
    return S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, x.wq.shape[0], w.dtype,
                     lowbit=lowbit)


def oracle_problem(orc, x, lowbit=S.LOWBIT_QK):
    w = x.wl
    return orc.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, x.wq.shape[0], w.dtype,
                       lowbit_v=lowbit & 1, int8_qk=(lowbit >> 1) & 1)


def run_gpu(x, dev, fp8=False, want_mask=True, lowbit=S.LOWBIT_QK):
    p = problem_of(x, lowbit)
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, mask = S.route(p, q, k, wq, wk, want_mask=want_mask)
    o = S.forward(p, q, k, v, idx, al, fp8=fp8)
    torch.cuda.synchronize()
    return p, idx, mask, o


def check_route(orc, x, idx, mask, heads=None):
    op = orc.problem_of(x)
    oidx, omask, gap, _ = orc.route(op, x.q, x.k, x.wq, x.wk, heads=heads)
    sel = slice(None) if heads is None else np.asarray(heads)
    g = gap.reshape(-1, gap.shape[-1])[sel]
    assert not ((g > 0) & (g < 1e-12)).any(), "workload has a near-tie at the top-k boundary"
    nbh = x.wl.B * x.wl.H
    gi = idx.cpu().numpy().reshape(nbh, *idx.shape[2:])[sel]
    assert np.array_equal(gi, oidx.reshape(nbh, *oidx.shape[2:])[sel])
    if mask is not None:
        gm = mask.cpu().numpy().reshape(nbh, *mask.shape[2:])[sel]
        assert np.array_equal(gm, omask.reshape(nbh, *omask.shape[2:])[sel])
    return oidx


# Relative accumulation error of the e4m3 matrix-core dot products of the
# low-bit logits, |computed - exact| <= FP8_ACC_EPS * sum |q^_c k^_c|.  The
# gfx950 fp8 MFMA does not sum its 64 products exactly; over 2^22 dot
# products of length 128 of absmax-scaled Gaussian codes (independent and
# correlated rows) the error stays near 2^-15 of sum|ab|, measured and
# asserted by test_fp8_matrix_core_accumulation_error below through
# sla2_fp8_dot_tiles (the same instruction and operand layout).
FP8_ACC_EPS = 2.0 ** -14
# Rows the low-bit gate lets past 3e-2 (each only through a recorded flip):
# at most this share of the compared rows (and at least 2).
FP8_OVER_SHARE = 1e-3
# Low-bit bulk agreement: 90 % of the rows within 3e-4, 99 % within 5e-3.
FP8_BULK = (3e-4, 5e-3)


def compare_blocks(orc, x, oidx, O, blocks, tol, variant="exact", op=None, alpha=None):
    """Element-wise comparison on whole query blocks.  For the low-bit
    variant a row may also move by the oracle's per-row bound: a P value
    whose 256 P~ lies closer to an e4m3 rounding midpoint than the logit
    error of the matrix-core accumulation (FP8_ACC_EPS) can reach may be
    rounded to either neighbouring code, and both are correct results; the
    bound is the largest effect of such flips on the row (0 for rows without
    such a decision).  On top of that the bulk of the rows must agree to
    FP8_BULK, which no flip-free difference comes near."""
    op = orc.problem_of(x) if op is None else op
    alpha = x.alpha if alpha is None else alpha
    if variant == "fp8":
        ref, bound = orc.forward(op, x.q, x.k, x.v, oidx, alpha, blocks, variant=variant,
                                 acc_eps=FP8_ACC_EPS)
    else:
        ref, bound = orc.forward(op, x.q, x.k, x.v, oidx, alpha, blocks), None
    w = x.wl
    Oc = O.cpu().numpy().reshape(w.B * w.H, w.N, w.d)
    errs, bnds = [], []
    for n, (bh, i) in enumerate(blocks):
        t0 = i * w.bq
        nv = min(w.bq, w.N - t0)
        err = np.abs(Oc[bh, t0:t0 + nv] - ref[n, :nv]).max(axis=1)
        assert np.isfinite(err).all()
        errs.append(err)
        bnds.append(bound[n, :nv] if bound is not None else np.zeros(nv))
    err, bnd = np.concatenate(errs), np.concatenate(bnds)
    worst = float(err.max()) if err.size else 0.0
    extra = ""
    if bound is not None and err.size:
        q = np.quantile(err, [0.5, 0.9, 0.99])
        extra = (f"; rows {err.size}, with a flippable decision {int((bnd > 0).sum())}, "
                 f"err quantiles 50/90/99% {q[0]:.1e}/{q[1]:.1e}/{q[2]:.1e}, "
                 f"rows over 1e-4 {int((err > 1e-4).sum())}, over 1e-3 {int((err > 1e-3).sum())}, "
                 f"over tol {int((err > tol).sum())}")
    say(f"  max-abs error over {len(blocks)} blocks: {worst:.3e} (tol {tol}{extra})")
    bad = np.flatnonzero(err > tol + bnd)
    assert bad.size == 0, (int(bad[0]), float(err[bad[0]]), float(bnd[bad[0]]))
    if bound is not None:
        # every row past tol is there through a recorded flip (bnd > 0 by the
        # check above), and such rows stay rare
        over = err > tol
        n_over = int(over.sum())
        cap = max(2, int(np.ceil(FP8_OVER_SHARE * err.size)))
        used = float((err - tol)[over].max()) if n_over else 0.0
        say(f"  rows over {tol}: {n_over} of {err.size} (cap {cap}); largest allowance "
            f"used {used:.2e}; plain max-abs {worst:.3e}")
        assert n_over <= cap, (n_over, cap)
    if bound is not None and err.size >= 100:
        # Flips are rare and every other difference is fp32 rounding, so the
        # bulk of the rows must agree far more tightly than tol: a wrong max,
        # scale or tile order moves most rows by 1e-3 or more.
        assert np.quantile(err, 0.9) <= FP8_BULK[0], np.quantile(err, 0.9)
        assert np.quantile(err, 0.99) <= FP8_BULK[1], np.quantile(err, 0.99)
    return worst


def wl(name, dtype, N, d, bq, frac, H=2, seed=0, gen=None, alpha=()):
    gen = gen or ("centroids" if dtype == "f32" else "smooth")
    return I.Workload(name, 1, H, N, d, bq, 64, frac, dtype, gen, seed=seed, alpha=alpha)


# --------------------------------------------------------------------------
# small workloads: the whole output against the oracle
# --------------------------------------------------------------------------
SMALL = [
    wl("tiny", "f32", 1024, 64, 64, 0.25, alpha=(0.7, 0.4)),
    wl("f32-ragged", "f32", 700, 128, 128, 0.3),
    wl("f32-bq64", "f32", 333, 64, 64, 0.4),
    wl("bf16-ragged", "bf16", 700, 128, 128, 0.25),
    wl("bf16-d64", "bf16", 1000, 64, 128, 0.3),
    wl("bf16-bq64", "bf16", 513, 128, 64, 0.2),
    wl("bf16-tiles", "bf16", 4100, 128, 128, 0.05, H=3),
    wl("bf16-k0", "bf16", 900, 128, 128, 0.0),
    wl("bf16-dense", "bf16", 640, 128, 128, 1.0, alpha=(1.0, 1.0)),
    wl("bf16-all-sel", "bf16", 600, 64, 128, 1.0, alpha=(0.3, 0.9)),
    wl("bf16-one-token", "bf16", 1, 128, 128, 1.0),
    wl("bf16-alpha0", "bf16", 1500, 128, 128, 0.1, alpha=(0.0, 0.0)),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_parity(orc, dev, w):
    say(f"case {w.name}: N={w.N} d={w.d} bq={w.bq} frac={w.topk_frac} {w.dtype}")
    x = I.make_inputs(w)
    p, idx, mask, O = run_gpu(x, dev)
    oidx = check_route(orc, x, idx, mask)
    op = orc.problem_of(x)
    blocks = orc.all_blocks(op)
    compare_blocks(orc, x, oidx, O, blocks, TOL[w.dtype])


def test_tiny_workload_full_output(orc, dev):
    """The tiny fp32 workload, whole tensor, 1e-5."""
    x = I.make_inputs(I.TINY)
    p, idx, mask, O = run_gpu(x, dev)
    oidx = check_route(orc, x, idx, mask)
    op = orc.problem_of(x)
    ref = orc.forward_full(op, x.q, x.k, x.v, oidx, x.alpha)
    err = np.abs(O.cpu().numpy() - ref).max()
    say(f"tiny: max-abs {err:.3e}")
    assert err <= 1e-5


def test_tie_breaking_on_duplicated_blocks(orc, dev):
    x = I.make_inputs(I.TINY.with_(k_noise=0.0, topk_frac=5 / 16))
    p, idx, mask, O = run_gpu(x, dev)
    op = orc.problem_of(x)
    oidx, omask, gap, _ = orc.route(op, x.q, x.k, x.wq, x.wk)
    assert (gap == 0).all()
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(mask.cpu().numpy(), omask)


def test_selection_paths_with_equal_keys(orc, dev):
    """The one-pass top-k first keeps the keys at or above the k-th largest of
    the 64 lane maxima (at most 128, sorted two per lane) and falls back to
    the radix select when more pass.  Head 0: every key row of the head the
    same, so all T_kv scores of a row tie (the fallback; the first k blocks).
    Head 1: two groups of 100 blocks, equal within the group (100 candidates
    in two slots, ties at the k-th place).  Head 2: the usual keys.  Indices
    and masks bit-exact against the oracle (ties to the lower index)."""
    w = wl("equal-keys", "bf16", 200 * 64, 128, 128, 0.17, H=3)
    say("case selection paths: N=12800 k=34 of 200, equal key groups")
    x = I.make_inputs(w)
    nb = w.N // 64
    x.k[0, 0] = x.k[0, 0, :1]
    hot = np.random.default_rng(7).choice(nb, 100, replace=False)
    rows = np.repeat(np.isin(np.arange(nb), hot), 64)
    ka, kb = x.k[0, 1, 0].copy(), x.k[0, 1, 64 * 100 + 5].copy()
    x.k[0, 1, rows] = ka
    x.k[0, 1, ~rows] = kb
    p, idx, mask, O = run_gpu(x, dev)
    oidx = check_route(orc, x, idx, mask)
    k = oidx.shape[-1]
    assert k <= 48  # the filtered selection is tried
    assert (oidx[0, 0] == np.arange(k)).all()
    grp = np.isin(np.arange(nb), hot)
    # head 1: the first k blocks of one group
    for r in oidx[0, 1]:
        assert len(set(grp[r])) == 1


@pytest.mark.parametrize("N", [1200 * 64, 1200 * 64 + 1])
def test_route_at_the_one_pass_limit(orc, dev, N):
    """Selection and mask exact at T_kv = 1200, the most KV blocks whose 16
    score rows the one-pass score + top-k kernel keeps in LDS, and at 1201,
    where the scores go through memory to the separate top-k kernel."""
    w = wl("tkv-limit", "bf16", N, 128, 128, 0.03, H=2)
    say(f"case route at T_kv limit: N={N}")
    x = I.make_inputs(w)
    p = problem_of(x)
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, mask = S.route(p, q, k, wq, wk)
    torch.cuda.synchronize()
    check_route(orc, x, idx, mask)


@pytest.mark.parametrize("d", [64, 128])
def test_route_batches_per_head_projections(orc, dev, d):
    """Two batch entries, per-head projections, a ragged last block and a row
    block count that is not a multiple of 16 (the one-pass score + top-k
    kernel takes 16 query blocks per work-group): selection and mask exact."""
    B, H, N = 2, 3, 2500  # T_q = 20, T_kv = 40
    w = I.Workload("route-b2", B, H, N, d, 128, 64, 0.15, "bf16", "smooth", seed=5)
    x = I.make_inputs(w)
    rng = np.random.default_rng(12)
    x.wq = (rng.standard_normal((H, d, d)) / np.sqrt(d)).astype(np.float32)
    x.wk = (rng.standard_normal((H, d, d)) / np.sqrt(d)).astype(np.float32)
    say(f"case route B={B} H={H} N={N} d={d} per-head W")
    p = problem_of(x)
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, mask = S.route(p, q, k, wq, wk)
    torch.cuda.synchronize()
    check_route(orc, x, idx, mask)


def test_route_all_scores_equal(orc, dev):
    """Every key block the same: all scores of a row tie, and the selection
    is the k lowest block indices (ties to the lower index)."""
    w = wl("all-equal", "bf16", 3000, 128, 128, 0.1, H=2)
    x = I.make_inputs(w)
    x.k = np.ascontiguousarray(np.broadcast_to(x.k[:, :, :1, :], x.k.shape))
    p = problem_of(x)
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, mask = S.route(p, q, k, wq, wk)
    torch.cuda.synchronize()
    kk = S.topk(p)
    gi = idx.cpu().numpy()
    assert (gi == np.arange(kk, dtype=np.int32)).all()
    check_route(orc, x, idx, mask)


def test_per_head_projections(orc, dev):
    w = wl("per-head", "bf16", 900, 128, 128, 0.2, H=3)
    x = I.make_inputs(w)
    rng = np.random.default_rng(4)
    x.wq = (rng.standard_normal((3, 128, 128)) / np.sqrt(128)).astype(np.float32)
    x.wk = (rng.standard_normal((3, 128, 128)) / np.sqrt(128)).astype(np.float32)
    p, idx, mask, O = run_gpu(x, dev)
    oidx = check_route(orc, x, idx, mask)
    compare_blocks(orc, x, oidx, O, orc.all_blocks(orc.problem_of(x)), TOL["bf16"])


def test_deterministic_and_no_stray_writes(dev):
    """Two runs are bitwise equal; guard bands around every output stay intact."""
    w = wl("det", "bf16", 2000, 128, 128, 0.1, H=2)
    x = I.make_inputs(w)
    p = problem_of(x)
    q, k, v, wq, wk, al = to_dev(x, dev)
    Tq, Tkv, kk = S.num_q_blocks(p), S.num_kv_blocks(p), S.topk(p)
    G = 4096
    outs = []
    for rep in range(2):
        idx_buf = torch.full((G + 2 * Tq * kk + G,), -7, dtype=torch.int32, device=dev)
        mask_buf = torch.full((G + 2 * Tq * Tkv + G,), 0xAB, dtype=torch.uint8, device=dev)
        o_buf = torch.full((G + 2 * w.N * w.d + G,), 12345.0, dtype=torch.float32, device=dev)
        idx = idx_buf[G:G + 2 * Tq * kk]
        mask = mask_buf[G:G + 2 * Tq * Tkv]
        O = o_buf[G:G + 2 * w.N * w.d]
        S.sla2_route(p, q, k, wq, wk, idx, mask, S.workspace(p, S.OP_ROUTE))
        S.sla2_forward(p, q, k, v, idx, al, O, S.workspace(p, S.OP_FORWARD))
        torch.cuda.synchronize()
        for buf, fill, n in ((idx_buf, -7, 2 * Tq * kk), (mask_buf, 0xAB, 2 * Tq * Tkv),
                             (o_buf, 12345.0, 2 * w.N * w.d)):
            assert (buf[:G] == fill).all() and (buf[G + n:] == fill).all()
        outs.append((idx.clone(), mask.clone(), O.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


# --------------------------------------------------------------------------
# full-size Wan workloads: every mask row exact, sampled blocks element-wise
# --------------------------------------------------------------------------
def sample_blocks(x, n_heads, per_head, seed=0):
    w = x.wl
    rng = np.random.default_rng(seed)
    heads = sorted(rng.choice(w.B * w.H, size=min(n_heads, w.B * w.H), replace=False))
    blocks = []
    for bh in heads:
        ii = set(rng.choice(w.Tq, size=per_head, replace=False).tolist())
        ii |= {0, w.Tq - 1}  # first block and the ragged last block
        blocks += [(int(bh), int(i)) for i in sorted(ii)]
    return blocks


@pytest.mark.parametrize("name", ["wan13b", "wan14b"])
def test_wan_shapes(orc, dev, name):
    w = I.WORKLOADS[name]
    say(f"case {name}: generating inputs")
    x = I.make_inputs(w)
    say(f"case {name}: GPU route + forward")
    p, idx, mask, O = run_gpu(x, dev)
    assert torch.isfinite(O).all()
    say(f"case {name}: oracle route (all heads)")
    oidx = check_route(orc, x, idx, mask)
    blocks = sample_blocks(x, n_heads=3, per_head=6)
    say(f"case {name}: oracle forward on {len(blocks)} blocks")
    compare_blocks(orc, x, oidx, O, blocks, TOL["bf16"])


@pytest.mark.parametrize("frac", I.SWEEP_FRACS)
def test_sparsity_sweep(orc, dev, frac):
    w = I.WAN13B.with_(topk_frac=frac)
    x = I.make_inputs(w)
    p, idx, mask, O = run_gpu(x, dev)
    heads = [0, 7]
    oidx = check_route(orc, x, idx, mask, heads=heads)
    full = np.zeros((w.B, w.H) + oidx.shape[2:], np.int32)
    full[0, heads] = oidx[0, heads]
    rng = np.random.default_rng(1)
    blocks = [(h, int(i)) for h in heads for i in {0, w.Tq - 1, *rng.choice(w.Tq, 3).tolist()}]
    compare_blocks(orc, x, full, O, blocks, TOL["bf16"])


# --------------------------------------------------------------------------
# low-bit sparse branch
# --------------------------------------------------------------------------
def quantize_gpu(x, dev, lowbit=S.LOWBIT_QK):
    p = problem_of(x, lowbit)
    q, k, _, _, _, _ = to_dev(x, dev)
    w = x.wl
    BH = w.B * w.H
    qh = torch.empty((BH, w.Tq * w.bq, w.d), dtype=torch.uint8, device=dev)
    kh = torch.empty((BH, w.Tkv * 64, w.d), dtype=torch.uint8, device=dev)
    sq = torch.empty((BH, w.Tq), dtype=torch.float32, device=dev)
    sk = torch.empty((BH, w.Tkv), dtype=torch.float32, device=dev)
    mu = torch.empty((BH, w.d), dtype=torch.float32, device=dev)
    S.sla2_quantize_fp8(p, q, k, qh, kh, sq, sk, mu, S.workspace(p, S.OP_FORWARD_FP8))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (qh, kh, sq, sk, mu)]


@pytest.mark.parametrize("lowbit", [S.LOWBIT_QK, S.LOWBIT_I8QK], ids=["e4m3", "int8"])
@pytest.mark.parametrize("N,H", [(700, 2), (4100, 3), (75600, 1)])
def test_quantized_inputs_match_oracle(orc, dev, N, H, lowbit):
    """Q/K codes, per-block scales and the K channel mean are bit-exact."""
    w = wl(f"q{N}", "bf16", N, 128, 128, 0.03, H=H)
    if N == 75600:
        w = w.with_(grid=(21, 45, 80))
    x = I.make_inputs(w)
    say(f"case quantize N={N} H={H} lowbit {lowbit}")
    qh, kh, sq, sk, mu = quantize_gpu(x, dev, lowbit)
    op = oracle_problem(orc, x, lowbit)
    for bh in range(w.B * w.H):
        oqh, okh, osq, osk, omu = orc.quant_fp8(op, x.q, x.k, bh)
        assert np.array_equal(mu[bh], omu)
        assert np.array_equal(sq[bh], osq) and np.array_equal(sk[bh], osk)
        assert np.array_equal(qh[bh, :N], oqh), int((qh[bh, :N] != oqh).sum())
        assert np.array_equal(kh[bh, :N], okh), int((kh[bh, :N] != okh).sum())
        assert not qh[bh, N:].any() and not kh[bh, N:].any()


FP8_SMALL = [
    wl("fp8-ragged", "bf16", 700, 128, 128, 0.25),
    wl("fp8-tiles", "bf16", 4100, 128, 128, 0.05, H=3),
    wl("fp8-dense", "bf16", 640, 128, 128, 1.0, alpha=(1.0, 1.0)),
    wl("fp8-k0", "bf16", 900, 128, 128, 0.0),
    wl("fp8-one-token", "bf16", 1, 128, 128, 1.0),
    wl("fp8-alpha1", "bf16", 2000, 128, 128, 0.1, alpha=(1.0, 1.0)),
]


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float -> OCP e4m3 codes (torch's float8_e4m3fn conversion; |x| <= 448)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values(c: np.ndarray) -> np.ndarray:
    return torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("kind", ["gaussian", "correlated"])
def test_fp8_matrix_core_accumulation_error(dev, kind):
    """The constant FP8_ACC_EPS of the low-bit gate, measured on the GPU: the
    e4m3 matrix-core dot products of sla2_fp8_dot_tiles (the instruction and
    operand layout of the low-bit Q K^T) against exact float64 sums, for rows
    scaled to absmax 448 as the per-block scales do; 2^22 dot products."""
    rng = np.random.default_rng(7 if kind == "gaussian" else 8)
    nt = 4096
    a = rng.standard_normal((nt, 32, 128))
    if kind == "gaussian":
        b = rng.standard_normal((nt, 32, 128))
    else:  # each row of B close to a row of A: large positive dot products
        b = a[:, rng.permutation(32)] + 0.3 * rng.standard_normal((nt, 32, 128))
    a = a / np.abs(a).max(axis=2, keepdims=True) * 448.0
    b = b / np.abs(b).max(axis=2, keepdims=True) * 448.0
    ca, cb = e4m3_codes(a), e4m3_codes(b)
    A = torch.from_numpy(ca).to(dev)
    B = torch.from_numpy(cb).to(dev)
    Cd = torch.empty((nt, 32, 32), dtype=torch.float32, device=dev)
    S.sla2_fp8_dot_tiles(A, B, Cd, nt)
    torch.cuda.synchronize()
    va, vb = e4m3_values(ca), e4m3_values(cb)
    exact = np.matmul(va, vb.transpose(0, 2, 1))      # exact in float64
    absum = np.matmul(np.abs(va), np.abs(vb).transpose(0, 2, 1))
    got = Cd.cpu().numpy().astype(np.float64)
    rel = np.abs(got - exact) / np.maximum(absum, 1e-300)
    worst = float(rel.max())
    say(f"fp8 dot products ({kind}): largest |computed - exact| / sum|ab| = {worst:.3e} "
        f"= 2^{np.log2(max(worst, 1e-300)):.2f}; exact results {float((rel == 0).mean()):.1%}; "
        f"gate constant 2^{np.log2(FP8_ACC_EPS):.0f}")
    assert worst <= FP8_ACC_EPS


LOWBITS = [S.LOWBIT_QK, S.LOWBIT_QKV, S.LOWBIT_I8QK, S.LOWBIT_I8QKV]
LOWBIT_IDS = ["qk", "qkv", "i8qk", "i8qkv"]


@pytest.mark.parametrize("lowbit", LOWBITS, ids=LOWBIT_IDS)
@pytest.mark.parametrize("w", FP8_SMALL, ids=[w.name for w in FP8_SMALL])
def test_fp8_forward_parity(orc, dev, w, lowbit):
    say(f"case {w.name}: N={w.N} frac={w.topk_frac} lowbit {lowbit}")
    x = I.make_inputs(w)
    p, idx, mask, O = run_gpu(x, dev, fp8=True, lowbit=lowbit)
    oidx = check_route(orc, x, idx, mask)
    op = oracle_problem(orc, x, lowbit)
    compare_blocks(orc, x, oidx, O, orc.all_blocks(op), TOL["fp8"], variant="fp8", op=op)


@pytest.mark.parametrize("N,H", [(700, 2), (4100, 3), (75600, 1)])
def test_quantized_v_matches_oracle(orc, dev, N, H):
    """Per-channel V scales and codes of the fully low-bit branch, bit-exact."""
    w = wl(f"v{N}", "bf16", N, 128, 128, 0.03, H=H)
    if N == 75600:
        w = w.with_(grid=(21, 45, 80))
    x = I.make_inputs(w)
    p = problem_of(x, S.LOWBIT_QKV)
    _, _, v, _, _, _ = to_dev(x, dev)
    BH = w.B * w.H
    vh = torch.empty((BH, w.Tkv * 64, w.d), dtype=torch.uint8, device=dev)
    sv = torch.empty((BH, w.d), dtype=torch.float32, device=dev)
    S.sla2_quantize_v_fp8(p, v, vh, sv, S.workspace(p, S.OP_FORWARD_FP8))
    torch.cuda.synchronize()
    vh, sv = vh.cpu().numpy(), sv.cpu().numpy()
    op = oracle_problem(orc, x, S.LOWBIT_QKV)
    for bh in range(BH):
        ovh, osv = orc.quant_v_fp8(op, x.v, bh)
        assert np.array_equal(sv[bh], osv)
        assert np.array_equal(vh[bh, :N], ovh), int((vh[bh, :N] != ovh).sum())
        assert not vh[bh, N:].any()


def test_attention_fp8_wan14b_equals_route_then_forward_fp8(dev):
    """At the full 14B shape, in the configuration the bench times, the
    one-call low-bit attention (query codes and K block sums from the
    router's pooling pass) gives the same selection and output bits as
    sla2_route followed by sla2_forward_fp8 (whose codes the quantisation
    tests pin to the oracle)."""
    x = I.make_inputs(I.WAN14B)
    p = problem_of(x, S.LOWBIT_QK)
    q, k, v, wq, wk, al = to_dev(x, dev)
    say("case attention fp8 at the 14B shape")
    idx0, _ = S.route(p, q, k, wq, wk, want_mask=False)
    O0 = S.forward(p, q, k, v, idx0, al, fp8=True)
    idx1, O1 = S.attention(p, q, k, v, wq, wk, al, fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(idx0, idx1)
    assert torch.equal(O0, O1)


@pytest.mark.parametrize("lowbit", LOWBITS, ids=LOWBIT_IDS)
def test_fp8_wan14b_sampled(orc, dev, lowbit):
    w = I.WAN14B
    x = I.make_inputs(w)
    p, idx, mask, O = run_gpu(x, dev, fp8=True, want_mask=False, lowbit=lowbit)
    assert torch.isfinite(O).all()
    heads = [5, 31]
    op = orc.problem_of(x)
    oidx, _, _, _ = orc.route(op, x.q, x.k, x.wq, x.wk, heads=heads)
    gi = idx.cpu().numpy().reshape(w.B * w.H, w.Tq, -1)
    assert np.array_equal(gi[heads], oidx.reshape(w.B * w.H, w.Tq, -1)[heads])
    rng = np.random.default_rng(3)
    blocks = [(h, int(i)) for h in heads for i in {0, w.Tq - 1, *rng.choice(w.Tq, 4).tolist()}]
    compare_blocks(orc, x, oidx, O, blocks, TOL["fp8"], variant="fp8",
                   op=oracle_problem(orc, x, lowbit))
