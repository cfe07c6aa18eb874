"""Every entry point of the CPU oracle on small seeded problems (both
dtypes, ragged blocks, k = 0 / some / all, SLA (v1), low bit, backward,
SoftTop-k, router gradient).  Started by tests/test_sanitizers.py in a child
process with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (SLA2_ORACLE_LIB) and the sanitizer runtime
preloaded; any report aborts that process.  Prints "ok" at the end."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle import oracle as orc  # noqa: E402
from sparse_linear_attention_amd import inputs as I  # noqa: E402


def finite(*arrs):
    for a in arrs:
        assert np.isfinite(np.asarray(a, np.float64)).all()


rng = np.random.default_rng(0)
for dtype, N, d, bq, frac in (("f32", 300, 16, 64, 0.4), ("bf16", 700, 64, 128, 0.25),
                              ("bf16", 130, 32, 64, 0.0), ("f32", 200, 16, 64, 1.0)):
    w = I.Workload(f"asan-{dtype}-{N}", 1, 2, N, d, bq, 64, frac, dtype, "smooth", seed=3)
    x = I.make_inputs(w)
    p = orc.problem_of(x)
    idx, mask, gap, sc = orc.route(p, x.q, x.k, x.wq, x.wk, want_scores=True)
    O = orc.forward_full(p, x.q, x.k, x.v, idx, x.alpha)
    finite(O)
    dO = rng.normal(0, 1, (1, 2, N, d))
    finite(*orc.backward(p, x.q, x.k, x.v, idx, x.alpha, dO))
    Tq, Tkv = orc.num_blocks(N, bq), orc.num_blocks(N, 64)
    finite(*orc.route_grad(p, x.q, x.k, x.wq, x.wk, rng.normal(0, 1, (1, 2, Tq, Tkv))))
    M, lam = orc.soft_topk(sc, orc.topk(p))
    finite(M, orc.soft_topk_grad(M, rng.normal(0, 1, M.shape)))
    for lowbit_v, int8_qk in ((0, 0), (1, 0), (0, 1), (1, 1)):
        pl = orc.problem(1, 2, N, d, bq, 64, frac, 1, dtype, lowbit_v=lowbit_v, int8_qk=int8_qk)
        out, bnd = orc.forward(pl, x.q, x.k, x.v, idx, x.alpha, orc.all_blocks(pl),
                               variant="lowbit", acc_eps=2.0 ** -14)
        finite(out, bnd)
        finite(*orc.quant_fp8(pl, x.q, x.k, 1)[2:], orc.quant_v_fp8(pl, x.v, 0)[1])
    for phi in (0, 1):
        p1 = orc.problem(1, 2, N, d, bq, 64, frac * 0.5, 1, dtype, phi=phi, mode=1,
                         low_frac=0.2)
        crit, negl, m1, _, _ = orc.route_v1(p1, x.q, x.k)
        wp = rng.normal(0, 0.2, (1, d, d)).astype(np.float32)
        finite(orc.forward_v1_full(p1, x.q, x.k, x.v, crit, negl, wp))
for c in range(256):
    orc.e4m3_decode(c)
for v in (0.0, -1.5, 448.0, 1e9, 3e-3):
    orc.e4m3_encode(v), orc.i8_encode(v), orc.bf16_encode(v)
print("ok")
