"""GPU parity of the one-call path and of the edge cases, through the C ABI.

* The call the bench times (sla2_attention) against the oracle on every
  query block of whole heads at the Wan-14B shape, and bit-identical to
  sla2_route + sla2_forward there.
* The stage switches (SLA2_FLAG_SKIP_LINEAR / SKIP_SPARSE) against the
  oracle with alpha = 1 and alpha = 0, and the dense baseline they give.
* Inputs that stress the linear branch: V with a large common mean (large
  |H_i|, past the fp16 range), and k = T_kv - 1, T_kv - 2 at
  N = 32760 (only one or two blocks left to the linear branch).
* Seeded random edge shapes: N < 64, N = 1 mod 64, k in {0, 1, T_kv - 1,
  T_kv}, d in {64, 128}, b_q in {64, 128}, fp32 and bf16, whole outputs.
Tolerances are those of the parity tests: 2e-3 max-abs for bf16 inputs,
1e-5 for fp32.
"""
import itertools

import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S
from tests.test_gpu_parity import TOL, check_route, compare_blocks, say, to_dev, wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    S.lib()
    return torch.device("cuda:0")


def prob(x, **kw):
    w = x.wl
    return S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, x.wq.shape[0], w.dtype, **kw)


def with_alpha(x, value):
    x.alpha = np.full_like(x.alpha, value)
    return x


# --------------------------------------------------------------------------
# the one-call path at the full 14B shape
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def wan14b_run(dev):
    x = I.make_inputs(I.WAN14B)
    p = prob(x)
    q, k, v, wq, wk, al = to_dev(x, dev)
    say("wan14b: sla2_attention")
    idx1, O1 = S.attention(p, q, k, v, wq, wk, al)
    torch.cuda.synchronize()
    return x, p, (q, k, v, wq, wk, al), idx1, O1


def test_attention_wan14b_whole_heads(orc, wan14b_run):
    """sla2_attention at the 14B shape against the oracle on every query block
    (591, the last with 80 valid rows) of four whole heads."""
    x, p, _, idx, O = wan14b_run
    assert torch.isfinite(O).all()
    heads = [0, 13, 26, 39]
    oidx = check_route(orc, x, idx, None, heads=heads)
    blocks = [(h, i) for h in heads for i in range(x.wl.Tq)]
    say(f"wan14b: oracle forward on {len(blocks)} blocks (4 whole heads)")
    compare_blocks(orc, x, oidx, O, blocks, TOL["bf16"])


def test_attention_wan14b_equals_route_then_forward(wan14b_run):
    """At the 14B shape the one-call attention (block summaries on the helper
    stream beside the router) gives the selection and output bits of
    sla2_route followed by sla2_forward."""
    x, p, (q, k, v, wq, wk, al), idx1, O1 = wan14b_run
    idx0, _ = S.route(p, q, k, wq, wk, want_mask=False)
    O0 = S.forward(p, q, k, v, idx0, al)
    torch.cuda.synchronize()
    assert torch.equal(idx0, idx1)
    assert torch.equal(O0, O1)


# --------------------------------------------------------------------------
# stage switches
# --------------------------------------------------------------------------
FLAG_CASES = [wl("flags-ragged", "bf16", 700, 128, 128, 0.25),
              wl("flags-tiles", "bf16", 4100, 128, 128, 0.05, H=3)]


@pytest.mark.parametrize("one_call", [False, True], ids=["forward", "attention"])
@pytest.mark.parametrize("w", FLAG_CASES, ids=[w.name for w in FLAG_CASES])
def test_stage_flags(orc, dev, w, one_call):
    """SKIP_LINEAR with alpha = 1 and SKIP_SPARSE with alpha = 0 are the full
    method with that alpha (oracle); the other alpha gives O = 0 exactly."""
    for flag, a_match, name in ((S.FLAG_SKIP_LINEAR, 1.0, "skip-linear"),
                                (S.FLAG_SKIP_SPARSE, 0.0, "skip-sparse")):
        x = with_alpha(I.make_inputs(w), a_match)
        p = prob(x, flags=flag)
        q, k, v, wq, wk, al = to_dev(x, dev)
        if one_call:
            idx, O = S.attention(p, q, k, v, wq, wk, al)
        else:
            idx, _ = S.route(p, q, k, wq, wk, want_mask=False)
            O = S.forward(p, q, k, v, idx, al)
        torch.cuda.synchronize()
        say(f"case {w.name} {name}")
        oidx = check_route(orc, x, idx, None)
        compare_blocks(orc, x, oidx, O, orc.all_blocks(orc.problem_of(x)), TOL["bf16"])
        al0 = torch.full_like(al, 1.0 - a_match)
        O0 = S.forward(p, q, k, v, idx, al0)
        torch.cuda.synchronize()
        assert (O0 == 0).all(), name


def test_dense_baseline_is_dense_attention(orc, dev):
    """k = T_kv, alpha = 1 and SKIP_LINEAR: plain softmax attention (the
    bench's dense reference point), against the oracle."""
    w = wl("dense-flag", "bf16", 1100, 128, 128, 1.0)
    x = with_alpha(I.make_inputs(w), 1.0)
    p = prob(x, flags=S.FLAG_SKIP_LINEAR)
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, O = S.attention(p, q, k, v, wq, wk, al)
    torch.cuda.synchronize()
    oidx = check_route(orc, x, idx, None)
    compare_blocks(orc, x, oidx, O, orc.all_blocks(orc.problem_of(x)), TOL["bf16"])


# --------------------------------------------------------------------------
# large |H|: V with a common mean of 2
# --------------------------------------------------------------------------
def shift_v(x, mean):
    v = I.bf16_bits_to_f32(x.v) + np.float32(mean)
    x.v = I.round_to_bf16_bits(v)
    return x


LARGE_V = {"wan13b": I.WAN13B, "wan14b": I.WAN14B,
           "wan13b-d64": I.WAN13B.with_(d=64, H=3)}


@pytest.mark.parametrize("name", list(LARGE_V))
def test_large_v_mean(orc, dev, name):
    """V ~ N(2, 1): every entry of H_i is about (tokens left out) x 2 x
    mean phi(K), far past the fp16 range at these shapes.  d = 128 carries
    H_i in bf16; d = 64 scales it by a power of two before narrowing to
    fp16; either way the output stays within the bf16 tolerance."""
    x = shift_v(I.make_inputs(LARGE_V[name]), 2.0)
    p = prob(x)
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, O = S.attention(p, q, k, v, wq, wk, al)
    torch.cuda.synchronize()
    assert torch.isfinite(O).all()
    heads = [1, x.wl.H - 1]
    oidx = check_route(orc, x, idx, None, heads=heads)
    rng = np.random.default_rng(11)
    blocks = [(h, int(i)) for h in heads
              for i in sorted({0, x.wl.Tq - 1, *rng.choice(x.wl.Tq, 6).tolist()})]
    compare_blocks(orc, x, oidx, O, blocks, TOL["bf16"])


# --------------------------------------------------------------------------
# one or two blocks left to the linear branch at N = 32760
# --------------------------------------------------------------------------
@pytest.mark.parametrize("left", [1, 2])
def test_few_blocks_left_to_linear(orc, dev, left):
    """k = T_kv - 1 and T_kv - 2 at the 1.3B shape (T_kv = 512, last block 56
    tokens), alpha < 1: H_i sums one or two blocks, directly."""
    base = I.WAN13B.with_(H=2)
    tkv = base.Tkv
    w = base.with_(topk_frac=(tkv - left - 0.5) / tkv)
    x = I.make_inputs(w)
    p = prob(x)
    assert S.topk(p) == tkv - left
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, O = S.attention(p, q, k, v, wq, wk, al)
    torch.cuda.synchronize()
    oidx = check_route(orc, x, idx, None)
    assert (x.alpha < 1).all()
    blocks = [(h, i) for h in range(2) for i in (0, 77, w.Tq - 1)]
    compare_blocks(orc, x, oidx, O, blocks, TOL["bf16"])


# --------------------------------------------------------------------------
# seeded random edge shapes
# --------------------------------------------------------------------------
def _edge_cases():
    rng = np.random.default_rng(2025)
    cases = []
    for n_kind, d, bq, k_kind in itertools.product(("short", "one-over"), (64, 128), (64, 128),
                                                   ("0", "1", "tkv-1", "tkv")):
        n = int(rng.integers(1, 64)) if n_kind == "short" else 64 * int(rng.integers(2, 20)) + 1
        tkv = -(-n // 64)
        kk = {"0": 0, "1": 1, "tkv-1": tkv - 1, "tkv": tkv}[k_kind]
        frac = 0.0 if kk == 0 else (kk - 0.5) / tkv
        dtype = "bf16" if (len(cases) % 2 == 0) else "f32"
        name = f"{n_kind}-N{n}-d{d}-bq{bq}-k{k_kind}-{dtype}"
        cases.append((name, wl(name, dtype, n, d, bq, frac, seed=len(cases)), kk))
    return cases


EDGE = _edge_cases()


@pytest.mark.parametrize("name,w,kk", EDGE, ids=[c[0] for c in EDGE])
def test_random_edge_shapes(orc, dev, name, w, kk):
    x = I.make_inputs(w)
    p = prob(x)
    assert S.topk(p) == kk
    q, k, v, wq, wk, al = to_dev(x, dev)
    idx, O = S.attention(p, q, k, v, wq, wk, al)
    idx0, _ = S.route(p, q, k, wq, wk, want_mask=False)
    O0 = S.forward(p, q, k, v, idx0, al)
    torch.cuda.synchronize()
    if kk > 0:
        assert torch.equal(idx, idx0)
    assert torch.equal(O, O0)
    oidx = check_route(orc, x, idx, None)
    compare_blocks(orc, x, oidx, O, orc.all_blocks(orc.problem_of(x)), TOL[w.dtype])


# --------------------------------------------------------------------------
# several host threads
# --------------------------------------------------------------------------
def test_attention_from_two_host_threads(dev):
    """Two host threads, each with its own stream and workspace, call
    sla2_attention concurrently (the library's helper stream and its events
    are shared); every result equals that of a lone call."""
    import threading
    cases = [wl("thr-a", "bf16", 4100, 128, 128, 0.05, H=3, seed=1),
             wl("thr-b", "bf16", 3000, 128, 128, 0.1, H=2, seed=2)]
    xs = [I.make_inputs(w) for w in cases]
    ref = []
    for x in xs:
        idx, O = S.attention(prob(x), *to_dev(x, dev))
        torch.cuda.synchronize()
        ref.append((idx.cpu(), O.cpu()))
    errors, ok = [], [0, 0]
    start = threading.Barrier(2)

    def run(i):
        try:
            x = xs[i]
            p = prob(x)
            st = torch.cuda.Stream()  # default priority
            with torch.cuda.stream(st):
                args = to_dev(x, dev)
                ws = S.workspace(p, S.OP_ATTENTION, dev)
                st.synchronize()
                start.wait()
                for _ in range(10):
                    idx, O = S.attention(p, *args, ws=ws, stream=st)
                    st.synchronize()
                    if torch.equal(idx.cpu(), ref[i][0]) and torch.equal(O.cpu(), ref[i][1]):
                        ok[i] += 1
        except Exception as e:  # reported below
            errors.append(repr(e))

    th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(120)
    assert not errors, errors
    say(f"two host threads: {ok} of 10 calls each equal to the lone call")
    assert ok == [10, 10]
