"""ctypes binding of libsla2.so (C ABI in include/sla2.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  Tensors are torch tensors on the GPU (PyTorch supplies device memory
and the stream); names follow the C entry points.  Loading fails loudly if the
library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsla2.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = range(5)
F32, BF16 = 0, 1
PHI_ELU1, PHI_SOFTMAX = 0, 1
(OP_ROUTE, OP_FORWARD, OP_FORWARD_FP8, OP_SLA1_FORWARD, OP_ROUTE_GRAD, OP_BACKWARD,
 OP_ATTENTION, OP_ATTENTION_FP8) = range(8)
LAYOUT_BHND, LAYOUT_BNHD = 0, 1
ALPHA_PER_HEAD, ALPHA_PER_QBLOCK = 0, 1
LOWBIT_QK, LOWBIT_QKV, LOWBIT_I8QK, LOWBIT_I8QKV = 0, 1, 2, 3
FLAG_SKIP_LINEAR, FLAG_SKIP_SPARSE = 1, 2


class Problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("N", C.c_int32), ("d", C.c_int32),
                ("bq", C.c_int32), ("bkv", C.c_int32), ("topk_frac", C.c_float),
                ("w_heads", C.c_int32), ("phi", C.c_int32), ("dtype", C.c_int32),
                ("layout", C.c_int32), ("alpha_mode", C.c_int32), ("out_dtype", C.c_int32),
                ("lowbit", C.c_int32), ("flags", C.c_uint32)]


class SLA2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run sparse_linear_attention_amd/build.py "
                "(or __graft_entry__.build()) first")
        L = C.CDLL(LIB_PATH)
        P = C.POINTER(Problem)
        vp = C.c_void_p
        L.sla2_num_q_blocks.argtypes = [P]
        L.sla2_num_kv_blocks.argtypes = [P]
        L.sla2_topk.argtypes = [P]
        L.sla2_workspace_bytes.argtypes = [P, C.c_int32]
        L.sla2_workspace_bytes.restype = C.c_size_t
        L.sla2_check.argtypes = [P, C.c_int32]
        L.sla2_status_str.argtypes = [C.c_int32]
        L.sla2_status_str.restype = C.c_char_p
        L.sla2_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_forward_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_quantize_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_quantize_v_fp8.argtypes = [P, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_timing_start.argtypes = [C.c_int32]
        L.sla2_timing_stop.argtypes = [vp, vp, C.c_int32]
        L.sla2_kernel_name.argtypes = [C.c_int32]
        L.sla2_kernel_name.restype = C.c_char_p
        L.sla1_num_negligible.argtypes = [P, C.c_float]
        L.sla2_soft_topk.argtypes = [P, vp, vp, vp, vp, C.c_float, vp, vp, vp, C.c_size_t, vp]
        L.sla2_soft_topk_grad.argtypes = [P, vp, vp, C.c_float, vp, vp]
        L.sla2_route_grad.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_attention_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla2_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla1_route.argtypes = [P, vp, vp, C.c_float, vp, vp, vp, vp, C.c_size_t, vp]
        L.sla1_forward.argtypes = [P, vp, vp, vp, vp, vp, C.c_float, vp, vp, vp, C.c_size_t, vp]
        L.sla2_fp8_dot_tiles.argtypes = [vp, vp, vp, C.c_int32, vp]
        L.sla2_mfma_rate_probe.argtypes = [C.c_int32, C.c_int32, C.c_int32, vp, vp]
        L.sla2_attention_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sla2_noalloc_scratch_bytes.restype = C.c_size_t
        _lib = L
    return _lib


EXPORTS = ("sla2_num_q_blocks", "sla2_num_kv_blocks", "sla2_topk", "sla2_workspace_bytes",
           "sla2_check", "sla2_status_str", "sla2_route", "sla2_forward", "sla2_forward_fp8",
           "sla2_quantize_fp8", "sla2_quantize_v_fp8", "sla2_timing_start", "sla2_timing_stop",
           "sla2_kernel_kinds", "sla2_kernel_name", "sla1_num_negligible", "sla1_route",
           "sla1_forward", "sla2_soft_topk", "sla2_soft_topk_grad", "sla2_route_grad",
           "sla2_backward", "sla2_attention", "sla2_attention_fp8", "sla2_fp8_dot_tiles",
           "sla2_mfma_rate_probe", "sla2_attention_noalloc", "sla2_noalloc_scratch_bytes")


def _dtype(x):
    if isinstance(x, str):
        return F32 if x == "f32" else BF16
    return x


def problem(B, H, N, d, bq=128, bkv=64, topk_frac=0.03, w_heads=1, dtype=BF16,
            phi=PHI_ELU1, layout=LAYOUT_BHND, alpha_mode=ALPHA_PER_HEAD,
            out_dtype=F32, lowbit=LOWBIT_QK, flags=0) -> Problem:
    return Problem(B, H, N, d, bq, bkv, float(topk_frac), w_heads, phi, _dtype(dtype),
                   layout, alpha_mode, _dtype(out_dtype), lowbit, flags)


def status_str(s: int) -> str:
    return lib().sla2_status_str(int(s)).decode()


def num_q_blocks(p: Problem) -> int:
    return lib().sla2_num_q_blocks(C.byref(p))


def num_kv_blocks(p: Problem) -> int:
    return lib().sla2_num_kv_blocks(C.byref(p))


def topk(p: Problem) -> int:
    return lib().sla2_topk(C.byref(p))


def workspace_bytes(p: Problem, op: int) -> int:
    return int(lib().sla2_workspace_bytes(C.byref(p), op))


def check(p: Problem, op: int) -> int:
    return int(lib().sla2_check(C.byref(p), op))


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _raise(st, what):
    if st != OK:
        raise SLA2Error(st, what)


def sla2_route(p, Q, K, Wq, Wk, topk_idx, block_mask=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_route(C.byref(p), _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(topk_idx),
                            _ptr(block_mask), wp, wb, _stream(stream)), "sla2_route")


def sla2_forward(p, Q, K, V, topk_idx, alpha, O, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_forward(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(topk_idx),
                              _ptr(alpha), _ptr(O), wp, wb, _stream(stream)), "sla2_forward")


def sla2_forward_fp8(p, Q, K, V, topk_idx, alpha, O, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_forward_fp8(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(topk_idx),
                                  _ptr(alpha), _ptr(O), wp, wb, _stream(stream)),
           "sla2_forward_fp8")


def sla2_quantize_fp8(p, Q, K, Qhat, Khat, sQ, sK, mu, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_quantize_fp8(C.byref(p), _ptr(Q), _ptr(K), _ptr(Qhat), _ptr(Khat),
                                   _ptr(sQ), _ptr(sK), _ptr(mu), wp, wb, _stream(stream)),
           "sla2_quantize_fp8")


def sla2_quantize_v_fp8(p, V, Vhat, sV, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_quantize_v_fp8(C.byref(p), _ptr(V), _ptr(Vhat), _ptr(sV), wp, wb,
                                     _stream(stream)), "sla2_quantize_v_fp8")


def num_negligible(p: Problem, low_frac: float) -> int:
    return int(lib().sla1_num_negligible(C.byref(p), float(low_frac)))


def sla1_route(p, Q, K, low_frac, crit_idx, negl_idx, block_mask=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla1_route(C.byref(p), _ptr(Q), _ptr(K), float(low_frac), _ptr(crit_idx),
                            _ptr(negl_idx), _ptr(block_mask), wp, wb, _stream(stream)),
           "sla1_route")


def sla1_forward(p, Q, K, V, crit_idx, negl_idx, low_frac, Wp, O, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla1_forward(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(crit_idx),
                              _ptr(negl_idx), float(low_frac), _ptr(Wp), _ptr(O), wp, wb,
                              _stream(stream)), "sla1_forward")


def sla2_attention(p, Q, K, V, Wq, Wk, alpha, topk_idx, O, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_attention(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Wq), _ptr(Wk),
                                _ptr(alpha), _ptr(topk_idx), _ptr(O), wp, wb, _stream(stream)),
           "sla2_attention")


def sla2_attention_noalloc(p, Q, K, V, Wq, Wk, alpha, topk_idx, O, stream=None):
    _raise(lib().sla2_attention_noalloc(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Wq),
                                        _ptr(Wk), _ptr(alpha), _ptr(topk_idx), _ptr(O),
                                        _stream(stream)), "sla2_attention_noalloc")


def noalloc_scratch_bytes() -> int:
    return int(lib().sla2_noalloc_scratch_bytes())


def sla2_attention_fp8(p, Q, K, V, Wq, Wk, alpha, topk_idx, O, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_attention_fp8(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Wq), _ptr(Wk),
                                    _ptr(alpha), _ptr(topk_idx), _ptr(O), wp, wb,
                                    _stream(stream)), "sla2_attention_fp8")


def attention(p: Problem, Q, K, V, Wq, Wk, alpha, ws=None, stream=None, fp8=False):
    """Allocates idx, O and the workspace; runs sla2_attention (route +
    forward), or sla2_attention_fp8 (route + low-bit forward) with fp8;
    returns (idx, O)."""
    import torch
    dev = Q.device
    idx = torch.empty((p.B, p.H, num_q_blocks(p), max(topk(p), 0)), dtype=torch.int32,
                      device=dev)
    shape = (p.B, p.H, p.N, p.d) if p.layout == LAYOUT_BHND else (p.B, p.N, p.H, p.d)
    O = torch.empty(shape, dtype=torch.float32 if p.out_dtype == F32 else torch.bfloat16,
                    device=dev)
    if ws is None:
        ws = workspace(p, OP_ATTENTION_FP8 if fp8 else OP_ATTENTION, dev)
    fn = sla2_attention_fp8 if fp8 else sla2_attention
    fn(p, Q, K, V, Wq, Wk, alpha, idx if topk(p) > 0 else None, O, ws, stream)
    return idx, O


def sla2_mfma_rate_probe(kind, iters, groups, out, stream=None):
    _raise(lib().sla2_mfma_rate_probe(int(kind), int(iters), int(groups), _ptr(out),
                                      _stream(stream)), "sla2_mfma_rate_probe")


def sla2_fp8_dot_tiles(A, B, Cout, ntiles, stream=None):
    _raise(lib().sla2_fp8_dot_tiles(_ptr(A), _ptr(B), _ptr(Cout), int(ntiles), _stream(stream)),
           "sla2_fp8_dot_tiles")


def sla2_backward(p, Q, K, V, topk_idx, alpha, dO, dQ, dK, dV, dalpha, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_backward(C.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(topk_idx),
                               _ptr(alpha), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV),
                               _ptr(dalpha), wp, wb, _stream(stream)), "sla2_backward")


def backward(p: Problem, Q, K, V, topk_idx, alpha, dO, ws=None, stream=None):
    """Allocates dQ, dK, dV (fp32, the problem's layout), dalpha and the
    workspace; runs sla2_backward."""
    import torch
    f = lambda t: torch.empty(t.shape, dtype=torch.float32, device=t.device)
    dQ, dK, dV = f(Q), f(K), f(V)
    dal = torch.empty_like(alpha, dtype=torch.float32)
    if ws is None:
        ws = workspace(p, OP_BACKWARD, Q.device)
    sla2_backward(p, Q, K, V, topk_idx if topk(p) > 0 else None, alpha, dO, dQ, dK, dV, dal,
                  ws, stream)
    return dQ, dK, dV, dal


def sla2_soft_topk(p, Q, K, Wq, Wk, tau, M, lam=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_soft_topk(C.byref(p), _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), float(tau),
                                _ptr(M), _ptr(lam), wp, wb, _stream(stream)), "sla2_soft_topk")


def sla2_soft_topk_grad(p, M, dM, tau, dS, stream=None):
    _raise(lib().sla2_soft_topk_grad(C.byref(p), _ptr(M), _ptr(dM), float(tau), _ptr(dS),
                                     _stream(stream)), "sla2_soft_topk_grad")


def sla2_route_grad(p, Q, K, Wq, Wk, dS, dWq, dWk, ws=None, stream=None):
    wp, wb = _ws(ws)
    _raise(lib().sla2_route_grad(C.byref(p), _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(dS),
                                 _ptr(dWq), _ptr(dWk), wp, wb, _stream(stream)),
           "sla2_route_grad")


def soft_topk(p: Problem, Q, K, Wq, Wk, tau=0.1, ws=None, stream=None):
    """Allocates outputs, runs sla2_soft_topk; returns (M fp32, lambda fp64)."""
    import torch
    dev = Q.device
    M = torch.empty((p.B, p.H, num_q_blocks(p), num_kv_blocks(p)), dtype=torch.float32,
                    device=dev)
    lam = torch.empty((p.B, p.H, num_q_blocks(p)), dtype=torch.float64, device=dev)
    if ws is None:
        ws = workspace(p, OP_ROUTE, dev)
    sla2_soft_topk(p, Q, K, Wq, Wk, tau, M, lam, ws, stream)
    return M, lam


def soft_topk_grad(p: Problem, M, dM, tau=0.1, stream=None):
    import torch
    dS = torch.empty_like(M)
    sla2_soft_topk_grad(p, M, dM, tau, dS, stream)
    return dS


def route_grad(p: Problem, Q, K, Wq, Wk, dS, ws=None, stream=None):
    """Allocates dWq, dWk and the workspace; runs sla2_route_grad."""
    import torch
    dWq = torch.empty_like(Wq)
    dWk = torch.empty_like(Wk)
    if ws is None:
        ws = workspace(p, OP_ROUTE_GRAD, Q.device)
    sla2_route_grad(p, Q, K, Wq, Wk, dS, dWq, dWk, ws, stream)
    return dWq, dWk


def kernel_names():
    L = lib()
    return [L.sla2_kernel_name(i).decode() for i in range(L.sla2_kernel_kinds())]


def timing_start(max_launches: int = 4096):
    _raise(lib().sla2_timing_start(max_launches), "sla2_timing_start")


def timing_stop():
    """Returns {kernel name: (total ms, launches)} for the recorded launches."""
    import numpy as np
    n = lib().sla2_kernel_kinds()
    ms = np.zeros(n, np.float32)
    cnt = np.zeros(n, np.int32)
    _raise(lib().sla2_timing_stop(ms.ctypes.data, cnt.ctypes.data, n), "sla2_timing_stop")
    return {name: (float(ms[i]), int(cnt[i])) for i, name in enumerate(kernel_names())
            if cnt[i] > 0}


# ---------------------------------------------------------------------------
# convenience wrappers around the entry points (allocation with torch)
# ---------------------------------------------------------------------------
def workspace(p: Problem, op: int, device="cuda"):
    import torch
    n = workspace_bytes(p, op)
    if n == 0:
        st = check(p, op)
        _raise(st if st != OK else EINVAL, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def route(p: Problem, Q, K, Wq, Wk, want_mask=True, ws=None, stream=None):
    """Allocates outputs, runs sla2_route; returns (topk_idx, block_mask)."""
    import torch
    dev = Q.device
    Tq, Tkv, k = num_q_blocks(p), num_kv_blocks(p), topk(p)
    idx = torch.empty((p.B, p.H, Tq, max(k, 0)), dtype=torch.int32, device=dev)
    mask = torch.empty((p.B, p.H, Tq, Tkv), dtype=torch.uint8, device=dev) if want_mask else None
    if ws is None:
        ws = workspace(p, OP_ROUTE, dev)
    sla2_route(p, Q, K, Wq, Wk, idx if k > 0 else None, mask, ws, stream)
    return idx, mask


def route_v1(p: Problem, Q, K, low_frac, want_mask=True, ws=None, stream=None):
    """Allocates outputs, runs sla1_route; returns (crit_idx, negl_idx, mask)."""
    import torch
    dev = Q.device
    Tq, Tkv, kh, kl = num_q_blocks(p), num_kv_blocks(p), topk(p), num_negligible(p, low_frac)
    crit = torch.empty((p.B, p.H, Tq, max(kh, 0)), dtype=torch.int32, device=dev)
    negl = torch.empty((p.B, p.H, Tq, max(kl, 0)), dtype=torch.int32, device=dev)
    mask = torch.empty((p.B, p.H, Tq, Tkv), dtype=torch.uint8, device=dev) if want_mask else None
    if ws is None:
        ws = workspace(p, OP_ROUTE, dev)
    sla1_route(p, Q, K, low_frac, crit if kh > 0 else None, negl if kl > 0 else None, mask, ws,
               stream)
    return crit, negl, mask


def forward_v1(p: Problem, Q, K, V, crit, negl, low_frac, Wp, ws=None, out=None, stream=None):
    """Allocates O and the workspace if not given; runs sla1_forward."""
    import torch
    dev = Q.device
    shape = (p.B, p.H, p.N, p.d) if p.layout == LAYOUT_BHND else (p.B, p.N, p.H, p.d)
    dt = torch.float32 if p.out_dtype == F32 else torch.bfloat16
    O = out if out is not None else torch.empty(shape, dtype=dt, device=dev)
    if ws is None:
        ws = workspace(p, OP_SLA1_FORWARD, dev)
    sla1_forward(p, Q, K, V, crit if topk(p) > 0 else None,
                 negl if num_negligible(p, low_frac) > 0 else None, low_frac, Wp, O, ws, stream)
    return O


def forward(p: Problem, Q, K, V, topk_idx, alpha, fp8=False, ws=None, out=None, stream=None):
    """Allocates O (fp32 or bf16, in the problem's layout) and the workspace if
    not given; runs the forward."""
    import torch
    dev = Q.device
    shape = (p.B, p.H, p.N, p.d) if p.layout == LAYOUT_BHND else (p.B, p.N, p.H, p.d)
    dt = torch.float32 if p.out_dtype == F32 else torch.bfloat16
    O = out if out is not None else torch.empty(shape, dtype=dt, device=dev)
    op = OP_FORWARD_FP8 if fp8 else OP_FORWARD
    if ws is None:
        ws = workspace(p, op, dev)
    fn = sla2_forward_fp8 if fp8 else sla2_forward
    fn(p, Q, K, V, topk_idx if topk(p) > 0 else None, alpha, O, ws, stream)
    return O
