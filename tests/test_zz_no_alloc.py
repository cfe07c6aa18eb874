"""sla2_attention_noalloc (the entry point for callers that cannot allocate)
against sla2_attention, through the C ABI: two calls in a row on one stream,
the second with a smaller problem, each bit-identical to sla2_attention on the
same inputs (same kernels, same order of every sum)."""
import numpy as np
import pytest
import torch

from sparse_linear_attention_amd import inputs as I
from sparse_linear_attention_amd import sla2 as S
from tests.test_gpu_parity import to_dev, wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    S.lib()
    return torch.device("cuda:0")


def run_both(x, dev):
    w = x.wl
    p = S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    assert S.workspace_bytes(p, S.OP_ATTENTION) <= S.noalloc_scratch_bytes()
    q, k, v, wq, wk, al = to_dev(x, dev)
    kk = S.topk(p)
    idx_r, O_r = S.attention(p, q, k, v, wq, wk, al)
    idx_n = torch.full_like(idx_r, -1)
    O_n = torch.full_like(O_r, float("nan"))
    S.sla2_attention_noalloc(p, q, k, v, wq, wk, al, idx_n if kk > 0 else None, O_n)
    torch.cuda.synchronize()
    return idx_r, O_r, idx_n, O_n


def test_noalloc_two_calls_second_smaller(dev):
    big = wl("noalloc-big", "bf16", 8192, 128, 128, 0.05, H=2, seed=3)
    small = wl("noalloc-small", "bf16", 1500, 128, 128, 0.2, H=1, seed=4)
    for w in (big, small):
        idx_r, O_r, idx_n, O_n = run_both(I.make_inputs(w), dev)
        print(f"{w.name}: N={w.N} H={w.H}: noalloc output equal: {torch.equal(O_r, O_n)}",
              flush=True)
        assert torch.equal(idx_r, idx_n)
        assert torch.equal(O_r, O_n)


def test_noalloc_vector_alu_path(dev):
    """fp32 inputs with b_q = 64 take the vector-ALU kernels, which use the
    same array."""
    w = wl("noalloc-f32", "f32", 700, 64, 64, 0.25, H=2, seed=5)
    idx_r, O_r, idx_n, O_n = run_both(I.make_inputs(w), dev)
    assert torch.equal(idx_r, idx_n)
    assert torch.equal(O_r, O_n)
