"""The bench's work accounting against the cost figures the pages print
(tests/golden/flop_ratios.json).  No GPU: only the host functions of bench.py
that turn a selection into FLOP counts."""
import json
import os

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "flop_ratios.json")))


def test_linear_branch_over_dense():
    """SLA notes, key design 3: the linear branch costs O(N d^2), 0.004 of the
    O(N^2 d) dense attention at N = 32K, d = 128."""
    g = GOLD["linear_over_dense"]
    N, d = g["N"], g["d"]
    lin = bench.linear_summary_flop(1, N, d) + bench.linear_apply_flop(1, N, d)
    ratio = lin / bench.dense_equivalent_flop(1, 1, N, d)
    assert abs(ratio - g["ratio"]) <= g["rel_tol"] * g["ratio"], ratio


def selection(N, frac, rng):
    """k of the T_kv KV blocks per query block (k from the pages' k %), drawn
    without replacement; [1, T_q, k]."""
    tkv, tq = -(-N // 64), -(-N // 128)
    k = int(np.ceil(frac * tkv - 1e-6))
    return np.stack([np.sort(rng.choice(tkv, k, replace=False)) for _ in range(tq)])[None]


@pytest.mark.parametrize("case", GOLD["sparse_fraction_97"]["cases"],
                         ids=lambda c: f"N{c['N']}")
def test_sparse_fraction_at_97_percent(case):
    """"SLA2 深度解读" 02 prints the attention FLOPs at 97 % sparsity as 3.45 %
    (1.3B-480P) and 3.16 % (14B-720P) of dense: the sparse branch (3 % of the
    KV blocks) plus the linear branch (d / N)."""
    N, d = case["N"], case["d"]
    rng = np.random.default_rng(0)
    idx = selection(N, 0.03, rng)
    dense = bench.dense_equivalent_flop(1, 1, N, d)
    sparse = bench.sparse_flop(idx, N, d, 128, 64)
    lin = bench.linear_summary_flop(1, N, d) + bench.linear_apply_flop(1, N, d)
    frac = (sparse + lin) / dense
    assert abs(frac - case["printed"]) <= case["abs_tol"], frac


def test_sparse_flop_counts_valid_tokens_only():
    """A ragged last KV block counts its valid tokens only, and so does a
    ragged last query block: N = 200, b_q = 128, b_kv = 64 (query blocks of
    128 and 72 rows, KV blocks of 64, 64, 64, 8)."""
    idx = np.array([[[0, 3], [1, 3]]])  # [1, T_q = 2, k = 2]
    got = bench.sparse_flop(idx, 200, 128, 128, 64)
    want = 4 * 128 * (128 * (64 + 8) + 72 * (64 + 8))
    assert got == want
    assert bench.sparse_flop(np.zeros((1, 2, 0), np.int64), 200, 128, 128, 64) == 0.0
