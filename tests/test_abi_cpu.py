"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every entry point ``include/sla2.h`` declares,
and reject invalid arguments on the host before touching the device.
"""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

from sparse_linear_attention_amd import sla2 as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla2.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sla[12]_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = S.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(S.EXPORTS) == set(names)


def test_oracle_library_loads(orc):
    assert orc.topk(orc.problem(1, 1, 640, 64, 64, 64, 0.5)) == 5


def p_ok(**kw):
    base = dict(B=1, H=2, N=1000, d=128, bq=128, bkv=64, topk_frac=0.25, w_heads=1, dtype=S.BF16)
    base.update(kw)
    return S.problem(**base)


def test_block_counts_and_k():
    p = p_ok(N=75600, topk_frac=0.03)
    assert S.num_q_blocks(p) == 591 and S.num_kv_blocks(p) == 1182 and S.topk(p) == 36
    p = p_ok(N=32760, topk_frac=0.03)
    assert S.num_q_blocks(p) == 256 and S.num_kv_blocks(p) == 512 and S.topk(p) == 16


def test_topk_matches_oracle_table(orc):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "topk_counts.json")))
    for c in g["cases"]:
        p = p_ok(N=c["tkv"] * 64, topk_frac=c["frac"])
        assert S.topk(p) == c["k"]
        assert S.topk(p) == orc.topk(orc.problem(1, 2, c["tkv"] * 64, 128, 128, 64, c["frac"]))


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), S.EINVAL), (dict(H=-1), S.EINVAL), (dict(N=0), S.EINVAL),
    (dict(topk_frac=-0.1), S.EINVAL), (dict(topk_frac=1.5), S.EINVAL),
    (dict(topk_frac=float("nan")), S.EINVAL), (dict(w_heads=3), S.EINVAL),
    (dict(dtype=7), S.EINVAL), (dict(d=96), S.EUNSUPPORTED), (dict(bq=32), S.EUNSUPPORTED),
    (dict(bkv=128), S.EUNSUPPORTED), (dict(N=7681 * 64), S.EUNSUPPORTED),
    (dict(layout=2), S.EINVAL), (dict(alpha_mode=-1), S.EINVAL), (dict(out_dtype=5), S.EINVAL),
    (dict(lowbit=4), S.EINVAL),
    (dict(lowbit=-1), S.EINVAL),
])
def test_check_rejects(kw, code):
    assert S.check(p_ok(**kw), S.OP_ROUTE) == code
    assert S.workspace_bytes(p_ok(**kw), S.OP_ROUTE) == 0
    assert S.topk(p_ok(**kw)) == -1


def test_fp8_needs_bf16_and_bq128():
    assert S.check(p_ok(dtype=S.F32), S.OP_FORWARD_FP8) == S.EUNSUPPORTED
    assert S.check(p_ok(bq=64), S.OP_FORWARD_FP8) == S.EUNSUPPORTED
    assert S.check(p_ok(), S.OP_FORWARD_FP8) == S.OK
    # softmax phi: every forward shape; not the low-bit kernels nor the
    # backward (routing ignores phi)
    assert S.check(p_ok(phi=S.PHI_SOFTMAX), S.OP_FORWARD) == S.OK
    assert S.check(p_ok(phi=S.PHI_SOFTMAX), S.OP_ROUTE) == S.OK
    for kw in (dict(dtype=S.F32), dict(d=64), dict(bq=64)):
        assert S.check(p_ok(phi=S.PHI_SOFTMAX, **kw), S.OP_FORWARD) == S.OK
        assert S.check(p_ok(phi=S.PHI_SOFTMAX, **kw), S.OP_ATTENTION) == S.OK
    assert S.check(p_ok(phi=S.PHI_SOFTMAX), S.OP_FORWARD_FP8) == S.EUNSUPPORTED
    assert S.check(p_ok(phi=2), S.OP_FORWARD) == S.EUNSUPPORTED


def test_sla1_counts_and_checks(orc):
    """k_l as the oracle counts it; the v1 forward takes every shape the SLA2
    forward takes; its workspace adds the W_p fragments (32 KB per
    projection)."""
    for N, kh, low in ((32760, 0.05, 0.10), (75600, 0.05, 0.10), (640, 0.7, 0.5), (640, 1.0, 0.3),
                       (640, 0.0, 0.0), (1000, 0.2, 0.33)):
        p = p_ok(N=N, topk_frac=kh)
        want = orc.topk_low(orc.problem(1, 2, N, 128, 128, 64, kh, mode=1, low_frac=low))
        assert S.num_negligible(p, low) == want
    assert S.num_negligible(p_ok(), -0.1) == -1 and S.num_negligible(p_ok(), float("nan")) == -1
    assert S.num_negligible(p_ok(B=0), 0.1) == -1
    assert S.check(p_ok(), S.OP_SLA1_FORWARD) == S.OK
    for kw in (dict(dtype=S.F32), dict(bq=64), dict(d=64), dict(bq=64, phi=S.PHI_SOFTMAX)):
        assert S.check(p_ok(**kw), S.OP_SLA1_FORWARD) == S.OK
    assert S.check(p_ok(bkv=128), S.OP_SLA1_FORWARD) == S.EUNSUPPORTED
    assert S.check(p_ok(), S.OP_ROUTE_GRAD) == S.OK
    assert S.check(p_ok(), S.OP_BACKWARD) == S.OK
    assert S.check(p_ok(dtype=S.F32, d=64, bq=64), S.OP_BACKWARD) == S.OK
    assert S.check(p_ok(), S.OP_ATTENTION) == S.OK
    assert S.workspace_bytes(p_ok(), S.OP_ATTENTION) == (
        S.workspace_bytes(p_ok(), S.OP_ROUTE) + S.workspace_bytes(p_ok(), S.OP_FORWARD))
    assert S.check(p_ok(), S.OP_ATTENTION_FP8) == S.OK
    # the combined call keeps the column sums of K per KV block (16 rows per
    # head here) where the separate quantisation keeps them per 1024 tokens (1)
    extra = 2 * (S.num_kv_blocks(p_ok()) - 1) * 128 * 8
    assert S.workspace_bytes(p_ok(), S.OP_ATTENTION_FP8) == (
        S.workspace_bytes(p_ok(), S.OP_ROUTE) + S.workspace_bytes(p_ok(), S.OP_FORWARD_FP8) + extra)
    for kw in (dict(dtype=S.F32), dict(bq=64), dict(d=64), dict(phi=S.PHI_SOFTMAX)):
        assert S.check(p_ok(**kw), S.OP_ATTENTION_FP8) == S.EUNSUPPORTED
    assert S.check(p_ok(), 8) == S.EINVAL
    for wh in (1, 2):
        extra = S.workspace_bytes(p_ok(w_heads=wh), S.OP_SLA1_FORWARD) - S.workspace_bytes(
            p_ok(w_heads=wh), S.OP_FORWARD)
        assert extra == wh * 128 * 128 * 2
    assert S.check(p_ok(), 9) == S.EINVAL


def test_layouts_alpha_modes_and_output_dtypes_are_accepted():
    for layout in (S.LAYOUT_BHND, S.LAYOUT_BNHD):
        for am in (S.ALPHA_PER_HEAD, S.ALPHA_PER_QBLOCK):
            for od in (S.F32, S.BF16):
                for op in (S.OP_ROUTE, S.OP_FORWARD, S.OP_FORWARD_FP8):
                    p = p_ok(layout=layout, alpha_mode=am, out_dtype=od)
                    assert S.check(p, op) == S.OK
                    # the workspace does not depend on how Q/K/V/O are laid out
                    assert S.workspace_bytes(p, op) == S.workspace_bytes(p_ok(), op)
    # quantising V as well: its one-byte codes replace the fp16 V^T copy of
    # P V in the fp8 workspace (d = 128, bq = 128), and the plain forward's
    # workspace is unchanged
    pv = p_ok(lowbit=S.LOWBIT_QKV)
    assert S.workspace_bytes(pv, S.OP_FORWARD_FP8) < S.workspace_bytes(p_ok(), S.OP_FORWARD_FP8)
    assert S.workspace_bytes(pv, S.OP_FORWARD) == S.workspace_bytes(p_ok(), S.OP_FORWARD)
    # int8 Q/K codes take the same room as e4m3 ones
    for lb, same in ((S.LOWBIT_I8QK, p_ok()), (S.LOWBIT_I8QKV, pv)):
        assert S.check(p_ok(lowbit=lb), S.OP_FORWARD_FP8) == S.OK
        assert S.workspace_bytes(p_ok(lowbit=lb), S.OP_FORWARD_FP8) == S.workspace_bytes(
            same, S.OP_FORWARD_FP8)


def test_workspace_sizes_grow_with_the_problem():
    prev = {op: 0 for op in (S.OP_ROUTE, S.OP_FORWARD, S.OP_FORWARD_FP8)}
    for N in (64, 1000, 5000, 32760, 75600):
        for op in prev:
            n = S.workspace_bytes(p_ok(N=N, H=40), op)
            assert n > prev[op] and n % 256 == 0
            prev[op] = n
    assert S.workspace_bytes(p_ok(N=75600, H=40), S.OP_FORWARD_FP8) > S.workspace_bytes(
        p_ok(N=75600, H=40), S.OP_FORWARD)


def _call_route(p, ptrs):
    L = S.lib()
    return L.sla2_route(C.byref(p), *ptrs)


def test_entry_points_validate_before_launching():
    """Null / misaligned pointers and short workspaces are caught on the host."""
    L = S.lib()
    p = p_ok()
    good = 0x100000  # never dereferenced: every call below fails validation
    ws_need = S.workspace_bytes(p, S.OP_ROUTE)
    # null Q
    assert L.sla2_route(C.byref(p), None, good, good, good, good, None, good, ws_need, None) == S.EINVAL
    # misaligned K
    assert L.sla2_route(C.byref(p), good, good + 2, good, good, good, None, good, ws_need, None) == S.EINVAL
    # workspace too small
    assert L.sla2_route(C.byref(p), good, good, good, good, good, None, good, ws_need - 256, None) == S.EWORKSPACE
    # misaligned workspace
    assert L.sla2_route(C.byref(p), good, good, good, good, good, None, good + 16, ws_need, None) == S.EINVAL
    fw = S.workspace_bytes(p, S.OP_FORWARD)
    assert L.sla2_forward(C.byref(p), good, good, good, good, None, good, good, fw, None) == S.EINVAL
    assert L.sla2_forward(C.byref(p), good, good, good, good, good, good, good, fw - 1, None) == S.EWORKSPACE
    pf = p_ok(dtype=S.F32)
    f8 = S.workspace_bytes(p, S.OP_FORWARD_FP8)
    assert L.sla2_forward_fp8(C.byref(pf), good, good, good, good, good, good, good, f8, None) == S.EUNSUPPORTED
    assert L.sla2_quantize_fp8(C.byref(p), good, good, None, good, good, good, good, good, f8, None) == S.EINVAL
    # v1 entry points
    assert L.sla1_route(C.byref(p), good, good, C.c_float(0.1), good, None, None, good, ws_need,
                        None) == S.EINVAL  # k_l > 0 needs negl_idx
    assert L.sla1_route(C.byref(p), good, good, C.c_float(1.5), good, good, None, good, ws_need,
                        None) == S.EINVAL
    assert L.sla1_route(C.byref(p), good, good, C.c_float(0.1), good, good, None, good,
                        ws_need - 256, None) == S.EWORKSPACE
    v1w = S.workspace_bytes(p, S.OP_SLA1_FORWARD)
    assert L.sla1_forward(C.byref(p), good, good, good, good, good, C.c_float(0.1), None, good,
                          good, v1w, None) == S.EINVAL  # no W_p
    assert L.sla1_forward(C.byref(p), good, good, good, good, good, C.c_float(0.1), good, good,
                          good, fw, None) == S.EWORKSPACE
    pu = p_ok(d=96)
    assert L.sla1_forward(C.byref(pu), good, good, good, good, good, C.c_float(0.1), good, good,
                          good, v1w, None) == S.EUNSUPPORTED
    # backward
    bw = S.workspace_bytes(p, S.OP_BACKWARD)
    assert bw > 0
    assert L.sla2_backward(C.byref(p), good, good, good, good, good, None, good, good, good,
                           good, good, bw, None) == S.EINVAL  # no dO
    assert L.sla2_backward(C.byref(p), good, good, good, good, good, good, good, good, good,
                           good, good, bw - 256, None) == S.EWORKSPACE
    # softmax phi: the vector-ALU backward at every shape (its own workspace)
    psm = p_ok(phi=S.PHI_SOFTMAX)
    assert S.check(psm, S.OP_BACKWARD) == S.OK
    bsm = S.workspace_bytes(psm, S.OP_BACKWARD)
    assert bsm > 0 and bsm != bw
    assert L.sla2_backward(C.byref(psm), good, good, good, good, good, good, good, good, good,
                           good, good, bsm - 256, None) == S.EWORKSPACE
    # training-time router
    assert L.sla2_soft_topk(C.byref(p), good, good, good, good, C.c_float(0.0), good, None, good,
                            ws_need, None) == S.EINVAL  # tau must be > 0
    assert L.sla2_soft_topk(C.byref(p), good, good, good, good, C.c_float(0.1), None, None, good,
                            ws_need, None) == S.EINVAL  # no M
    assert L.sla2_soft_topk(C.byref(p), good, good, good, good, C.c_float(0.1), good, None, good,
                            ws_need - 256, None) == S.EWORKSPACE
    assert L.sla2_soft_topk_grad(C.byref(p), good, None, C.c_float(0.1), good, None) == S.EINVAL
    assert L.sla2_soft_topk_grad(C.byref(p), good, good, C.c_float(float("nan")), good,
                                 None) == S.EINVAL
    rg = S.workspace_bytes(p, S.OP_ROUTE_GRAD)
    assert rg > ws_need
    assert L.sla2_route_grad(C.byref(p), good, good, good, good, good, good, None, good, rg,
                             None) == S.EINVAL
    assert L.sla2_route_grad(C.byref(p), good, good, good, good, good, good, good, good,
                             rg - 256, None) == S.EWORKSPACE
    # idx may be null only when k == 0
    p0 = p_ok(topk_frac=0.0)
    assert L.sla2_route(C.byref(p), good, good, good, good, None, None, good, ws_need, None) == S.EINVAL
    assert S.topk(p0) == 0


def test_status_strings():
    for s in range(5):
        assert S.status_str(s) and S.status_str(s) != "unknown status"
    assert S.status_str(42) == "unknown status"
    assert "fused_mfma" in S.kernel_names()


def test_flags_rejected_outside_their_path():
    assert S.check(S.problem(1, 2, 1000, 64, 128, 64, 0.1, flags=1), S.OP_FORWARD) == S.EUNSUPPORTED
    assert S.check(S.problem(1, 2, 1000, 128, 64, 64, 0.1, flags=2), S.OP_FORWARD) == S.EUNSUPPORTED
    assert S.check(S.problem(1, 2, 1000, 128, 128, 64, 0.1, flags=4), S.OP_FORWARD) == S.EINVAL
    assert S.check(S.problem(1, 2, 1000, 128, 128, 64, 0.1, flags=1), S.OP_SLA1_FORWARD) == \
        S.EUNSUPPORTED
    assert S.check(S.problem(1, 2, 1000, 128, 128, 64, 0.1, flags=3), S.OP_ROUTE) == S.OK


def test_fp8_dot_tiles_rejects_bad_arguments():
    L = S.lib()
    good = 1 << 20
    assert L.sla2_fp8_dot_tiles(None, good, good, 1, None) == S.EINVAL
    assert L.sla2_fp8_dot_tiles(good, good + 8, good, 1, None) == S.EINVAL
    assert L.sla2_fp8_dot_tiles(good, good, good, 0, None) == S.EINVAL
    assert L.sla2_fp8_dot_tiles(good, good, good, (1 << 20) + 1, None) == S.EINVAL


def test_noalloc_rejects_problems_past_its_array():
    """The no-allocation entry point refuses, on the host and before any
    launch, a problem whose workspace exceeds its fixed device array."""
    L = S.lib()
    cap = S.noalloc_scratch_bytes()
    assert cap == 64 << 20
    small = p_ok(N=8192, H=2)
    assert S.workspace_bytes(small, S.OP_ATTENTION) <= cap
    big = p_ok(N=75600, H=40, topk_frac=0.03)
    assert S.workspace_bytes(big, S.OP_ATTENTION) > cap
    good = 1 << 20
    args = [good] * 8 + [None]
    assert L.sla2_attention_noalloc(C.byref(big), *args) == S.EWORKSPACE
    assert L.sla2_attention_noalloc(C.byref(small), None, *args[1:]) == S.EINVAL


def test_mfma_rate_probe_rejects_bad_arguments():
    L = S.lib()
    good = C.c_void_p(4096)
    assert L.sla2_mfma_rate_probe(4, 10, 1, good, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(-1, 10, 1, good, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(0, 0, 1, good, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(1, (1 << 24) + 1, 1, good, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(0, 10, 0, good, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(0, 10, (1 << 16) + 1, good, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(0, 10, 1, None, None) == S.EINVAL
    assert L.sla2_mfma_rate_probe(0, 10, 1, C.c_void_p(4096 + 4), None) == S.EINVAL
