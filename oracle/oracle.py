"""ctypes front end of the CPU oracle (``libsla2_oracle.so``).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``.  The GPU library and its Python binding
never import this module.  Arrays are numpy: Q/K/V [B,H,N,d] as float32 or as
uint16 bf16 bit patterns; Wq/Wk [w_heads,d,d] float32; alpha [H] float32.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sla2_oracle.c")
# a sanitizer build of the same source (tests/test_sanitizers.py) is loaded
# in place of the plain one when SLA2_ORACLE_LIB names it
_LIB = os.environ.get("SLA2_ORACLE_LIB") or os.path.join(_HERE, "libsla2_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("N", C.c_int32), ("d", C.c_int32),
                ("bq", C.c_int32), ("bkv", C.c_int32), ("topk_frac", C.c_float),
                ("w_heads", C.c_int32), ("dtype", C.c_int32), ("alpha_mode", C.c_int32),
                ("lowbit_v", C.c_int32), ("int8_qk", C.c_int32), ("phi", C.c_int32),
                ("mode", C.c_int32), ("low_frac", C.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P = C.POINTER(Problem)
        vp, ip, dp = C.c_void_p, C.c_void_p, C.c_void_p
        L.orc_topk.argtypes = [P]
        L.orc_topk_low.argtypes = [P]
        L.orc_route_grad.argtypes = [P, vp, vp, vp, vp, dp, dp, dp]
        L.orc_backward.argtypes = [P, vp, vp, vp, ip, vp, dp, dp, dp, dp, dp, C.c_int]
        L.orc_soft_topk_rows.argtypes = [dp, C.c_long, C.c_int, C.c_int, C.c_double, dp, dp]
        L.orc_soft_topk_grad_rows.argtypes = [vp, vp, C.c_long, C.c_int, C.c_double, dp]
        L.orc_route_v1.argtypes = [P, vp, vp, ip, C.c_int, ip, ip, vp, dp, dp, C.c_int]
        L.orc_forward_v1.argtypes = [P, vp, vp, vp, ip, ip, vp, ip, C.c_int, dp, C.c_int]
        L.orc_num_blocks.argtypes = [C.c_int, C.c_int]
        L.orc_route.argtypes = [P, vp, vp, vp, vp, ip, C.c_int, ip, vp, dp, dp, C.c_int]
        L.orc_forward.argtypes = [P, vp, vp, vp, ip, vp, ip, C.c_int, dp, C.c_int]
        L.orc_forward_fp8.argtypes = [P, vp, vp, vp, ip, vp, ip, C.c_int, C.c_int, dp, dp,
                                      C.c_double, C.c_int]
        L.orc_quant_fp8.argtypes = [P, vp, vp, C.c_long, vp, vp, vp, vp, vp]
        L.orc_quant_v_fp8.argtypes = [P, vp, C.c_long, vp, vp]
        L.orc_e4m3_encode.argtypes = [C.c_float]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_decode.restype = C.c_float
        L.orc_i8_encode.argtypes = [C.c_float]
        L.orc_i8_encode.restype = C.c_int8
        L.orc_bf16_encode.argtypes = [C.c_float]
        L.orc_bf16_encode.restype = C.c_uint16
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def problem(B, H, N, d, bq, bkv, frac, w_heads=1, dtype="f32", alpha_mode=0,
            lowbit_v=0, int8_qk=0, phi=0, mode=0, low_frac=0.0) -> Problem:
    """alpha_mode 0: alpha [H]; 1: alpha [H][T_q] (one per query block).
    lowbit_v 1: the low-bit variant quantises V too (per channel).
    int8_qk 1: the low-bit variant takes int8 Q/K codes instead of e4m3.
    phi 0: elu + 1; 1: softmax over the d channels of a row.
    mode 1: SLA (v1) with low_frac of the blocks negligible per row."""
    return Problem(B, H, N, d, bq, bkv, float(frac), w_heads, 0 if dtype == "f32" else 1,
                   alpha_mode, lowbit_v, int8_qk, phi, mode, float(low_frac))


def problem_of(x) -> Problem:
    """Problem for an ``inputs.Inputs`` bundle."""
    w = x.wl
    return problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, x.wq.shape[0], w.dtype)


def _arr(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _qkv(p: Problem, a):
    return _arr(a, np.float32 if p.dtype == 0 else np.uint16)


def topk(p: Problem) -> int:
    return lib().orc_topk(C.byref(p))


def topk_low(p: Problem) -> int:
    """v1: number of negligible blocks per row (0 in SLA2 mode)."""
    return lib().orc_topk_low(C.byref(p))


def num_blocks(n: int, b: int) -> int:
    return lib().orc_num_blocks(n, b)


def route(p: Problem, q, k, wq, wk, heads=None, nthreads=0, want_scores=False):
    """Router (pool -> project -> score -> top-k) for the listed heads.

    Returns (idx [B,H,Tq,k] int32 ascending, mask [B,H,Tq,Tkv] uint8,
    gap_rel [B,H,Tq] float64, scores or None).  Rows of unlisted heads are
    left at -1 / 0 / nan."""
    L = lib()
    B, H, N = p.B, p.H, p.N
    Tq, Tkv = num_blocks(N, p.bq), num_blocks(N, p.bkv)
    kk = topk(p)
    heads = np.arange(B * H, dtype=np.int32) if heads is None else np.asarray(heads, np.int32)
    q, k = _qkv(p, q), _qkv(p, k)
    wq, wk = _arr(wq, np.float32), _arr(wk, np.float32)
    idx = np.full((B, H, Tq, kk), -1, np.int32)
    mask = np.zeros((B, H, Tq, Tkv), np.uint8)
    gap = np.full((B, H, Tq), np.nan)
    sc = np.full((B, H, Tq, Tkv), np.nan) if want_scores else None
    L.orc_route(C.byref(p), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(heads), len(heads),
                _ptr(idx), _ptr(mask), _ptr(gap), _ptr(sc), nthreads)
    return idx, mask, gap, sc


def backward(p: Problem, q, k, v, idx, alpha, dO, nthreads=0):
    """Gradients of sum(dO * O) for the SLA2 forward with idx fixed:
    (dQ, dK, dV [B,H,N,d] fp64, dalpha [H] or [H,Tq])."""
    q, k, v = _qkv(p, q), _qkv(p, k), _qkv(p, v)
    idx = _arr(idx, np.int32)
    alpha = _arr(alpha, np.float32)
    dO = _arr(dO, np.float64)
    shape = (p.B, p.H, p.N, p.d)
    dQ, dK, dV = np.zeros(shape), np.zeros(shape), np.zeros(shape)
    Tq = num_blocks(p.N, p.bq)
    da = np.zeros((p.H, Tq) if p.alpha_mode else (p.H,))
    rc = lib().orc_backward(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(alpha),
                            _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(da), nthreads)
    if rc != 0:
        raise ValueError(f"oracle: backward failed ({rc})")
    return dQ, dK, dV, da


def route_grad(p: Problem, q, k, wq, wk, dS):
    """dL/dWq, dL/dWk [w_heads, d, d] (fp64) from dL/dS [B, H, Tq, Tkv]."""
    q, k = _qkv(p, q), _qkv(p, k)
    wq, wk = _arr(wq, np.float32), _arr(wk, np.float32)
    dS = _arr(dS, np.float64)
    gq = np.zeros((p.w_heads, p.d, p.d))
    gk = np.zeros((p.w_heads, p.d, p.d))
    lib().orc_route_grad(C.byref(p), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(dS), _ptr(gq),
                         _ptr(gk))
    return gq, gk


def soft_topk(scores, k: int, tau: float = 0.1):
    """SoftTop-k of score rows [..., Tkv] (fp64): (M, lambda)."""
    S = np.ascontiguousarray(scores, np.float64)
    Tkv = S.shape[-1]
    rows = S.size // Tkv
    M = np.zeros_like(S)
    lam = np.zeros(S.shape[:-1])
    lib().orc_soft_topk_rows(_ptr(S), rows, Tkv, int(k), float(tau), _ptr(M), _ptr(lam))
    return M, lam


def soft_topk_grad(M, dM, tau: float = 0.1):
    """dL/dS through SoftTop-k from the fp32 mask M and fp32 dL/dM: fp64."""
    M = np.ascontiguousarray(M, np.float32)
    dM = np.ascontiguousarray(dM, np.float32)
    Tkv = M.shape[-1]
    dS = np.zeros(M.shape)
    lib().orc_soft_topk_grad_rows(_ptr(M), _ptr(dM), M.size // Tkv, Tkv, float(tau), _ptr(dS))
    return dS


def route_v1(p: Problem, q, k, heads=None, nthreads=0, want_scores=False):
    """SLA (v1) router (p.mode == 1): returns (crit [B,H,Tq,k_h], negl
    [B,H,Tq,k_l], both int32 ascending; mask [B,H,Tq,Tkv] uint8 with 1 / 0xFF
    / 0 for critical / negligible / marginal; gap_rel; scores or None)."""
    L = lib()
    B, H, N = p.B, p.H, p.N
    Tq, Tkv = num_blocks(N, p.bq), num_blocks(N, p.bkv)
    kh, kl = topk(p), topk_low(p)
    heads = np.arange(B * H, dtype=np.int32) if heads is None else np.asarray(heads, np.int32)
    q, k = _qkv(p, q), _qkv(p, k)
    crit = np.full((B, H, Tq, kh), -1, np.int32)
    negl = np.full((B, H, Tq, kl), -1, np.int32)
    mask = np.zeros((B, H, Tq, Tkv), np.uint8)
    gap = np.full((B, H, Tq), np.nan)
    sc = np.full((B, H, Tq, Tkv), np.nan) if want_scores else None
    rc = L.orc_route_v1(C.byref(p), _ptr(q), _ptr(k), _ptr(heads), len(heads), _ptr(crit),
                        _ptr(negl), _ptr(mask), _ptr(gap), _ptr(sc), nthreads)
    if rc < 0:
        raise ValueError("oracle: route_v1 needs mode 1")
    return crit, negl, mask, gap, sc


def forward_v1(p: Problem, q, k, v, crit, negl, wp, blocks, nthreads=0):
    """SLA (v1) forward for the query blocks ``blocks``: [n_blocks, bq, d]."""
    L = lib()
    blocks = np.ascontiguousarray(np.asarray(blocks, np.int32).reshape(-1, 2))
    out = np.zeros((blocks.shape[0], p.bq, p.d))
    q, k, v = _qkv(p, q), _qkv(p, k), _qkv(p, v)
    crit, negl = _arr(crit, np.int32), _arr(negl, np.int32)
    wp = _arr(wp, np.float32)
    rc = L.orc_forward_v1(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(crit), _ptr(negl),
                          _ptr(wp), _ptr(blocks), blocks.shape[0], _ptr(out), nthreads)
    if rc != 0:
        raise ValueError(f"oracle: forward_v1 failed ({rc})")
    return out


def forward_v1_full(p: Problem, q, k, v, crit, negl, wp, nthreads=0):
    out = forward_v1(p, q, k, v, crit, negl, wp, all_blocks(p), nthreads)
    Tq = num_blocks(p.N, p.bq)
    o = out.reshape(p.B, p.H, Tq * p.bq, p.d)[:, :, : p.N]
    return np.ascontiguousarray(o)


def forward(p: Problem, q, k, v, idx, alpha, blocks, nthreads=0, variant="exact",
            quantize=True, acc_eps=None):
    """Forward for the query blocks ``blocks`` (list of (bh, i)).

    Returns out [n_blocks, bq, d] float64 (rows past N are 0).  With acc_eps
    (low-bit variant) also returns the per-row bound [n_blocks, bq] on the
    effect of the P-quantisation decisions that an implementation whose
    quantised dot products carry a relative accumulation error up to
    acc_eps * sum|q^ k^| may round the other way."""
    L = lib()
    blocks = np.ascontiguousarray(np.asarray(blocks, np.int32).reshape(-1, 2))
    out = np.zeros((blocks.shape[0], p.bq, p.d))
    q, k, v = _qkv(p, q), _qkv(p, k), _qkv(p, v)
    idx = _arr(idx, np.int32)
    alpha = _arr(alpha, np.float32)
    if variant == "exact":
        rc = L.orc_forward(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(alpha),
                           _ptr(blocks), blocks.shape[0], _ptr(out), nthreads)
    else:
        bound = np.zeros((blocks.shape[0], p.bq)) if acc_eps is not None else None
        rc = L.orc_forward_fp8(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(alpha),
                               _ptr(blocks), blocks.shape[0], 1 if quantize else 0,
                               _ptr(out), _ptr(bound), float(acc_eps or 0.0), nthreads)
        if rc != 0:
            raise ValueError("oracle: bad block list")
        return (out, bound) if acc_eps is not None else out
    if rc != 0:
        raise ValueError("oracle: bad block list")
    return out


def all_blocks(p: Problem):
    Tq = num_blocks(p.N, p.bq)
    return [(bh, i) for bh in range(p.B * p.H) for i in range(Tq)]


def forward_full(p: Problem, q, k, v, idx, alpha, nthreads=0, variant="exact",
                 quantize=True):
    """Whole output [B,H,N,d] float64 (small problems only)."""
    out = forward(p, q, k, v, idx, alpha, all_blocks(p), nthreads, variant, quantize)
    Tq = num_blocks(p.N, p.bq)
    o = out.reshape(p.B, p.H, Tq * p.bq, p.d)[:, :, : p.N]
    return np.ascontiguousarray(o)


def quant_fp8(p: Problem, q, k, bh):
    """Low-bit inputs of one head: (qhat [N,d] u8, khat [N,d] u8, sq [Tq],
    sk [Tkv], mu [d])."""
    L = lib()
    Tq, Tkv = num_blocks(p.N, p.bq), num_blocks(p.N, p.bkv)
    qh = np.zeros((p.N, p.d), np.uint8)
    kh = np.zeros((p.N, p.d), np.uint8)
    sq = np.zeros(Tq, np.float32)
    sk = np.zeros(Tkv, np.float32)
    mu = np.zeros(p.d, np.float32)
    q, k = _qkv(p, q), _qkv(p, k)
    L.orc_quant_fp8(C.byref(p), _ptr(q), _ptr(k), bh, _ptr(qh), _ptr(kh), _ptr(sq),
                    _ptr(sk), _ptr(mu))
    return qh, kh, sq, sk, mu


def quant_v_fp8(p: Problem, v, bh):
    """Per-channel quantised V of one head: (vhat [N,d] u8, sv [d])."""
    vh = np.zeros((p.N, p.d), np.uint8)
    sv = np.zeros(p.d, np.float32)
    lib().orc_quant_v_fp8(C.byref(p), _ptr(_qkv(p, v)), bh, _ptr(vh), _ptr(sv))
    return vh, sv


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def i8_encode(x: float) -> int:
    return int(lib().orc_i8_encode(float(x)))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


def bf16_encode(x: float) -> int:
    return int(lib().orc_bf16_encode(float(x)))
