// Host side of libsla2: argument validation, block counts, workspace
// layout, kernel sequencing and the optional kernel timing records.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "sla2_internal.h"

#define SLA2_API extern "C" __attribute__((visibility("default")))

namespace sla2 {

static constexpr int kMaxTkv = 7680;

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// k = clamp(ceil(frac * T_kv - 1e-6), 0, T_kv)  (the pages give k% only)
static int topk_of(float frac, int tkv) {
    double k = ceil((double)frac * (double)tkv - 1e-6);
    if (k < 0) k = 0;
    if (k > tkv) k = tkv;
    return (int)k;
}

static sla2_status make_dims(const sla2_problem* p, int op, Dims* D) {
    if (!p) return SLA2_EINVAL;
    if (p->B <= 0 || p->H <= 0 || p->N <= 0 || p->d <= 0 || p->bq <= 0 || p->bkv <= 0)
        return SLA2_EINVAL;
    if (!(p->topk_frac >= 0.0f && p->topk_frac <= 1.0f)) return SLA2_EINVAL;  // also NaN
    if (p->w_heads != 1 && p->w_heads != p->H) return SLA2_EINVAL;
    if (p->dtype != SLA2_F32 && p->dtype != SLA2_BF16) return SLA2_EINVAL;
    if (p->layout != SLA2_LAYOUT_BHND && p->layout != SLA2_LAYOUT_BNHD) return SLA2_EINVAL;
    if (p->alpha_mode != SLA2_ALPHA_PER_HEAD && p->alpha_mode != SLA2_ALPHA_PER_QBLOCK)
        return SLA2_EINVAL;
    if (p->out_dtype != SLA2_F32 && p->out_dtype != SLA2_BF16) return SLA2_EINVAL;
    if (p->lowbit < SLA2_LOWBIT_QK || p->lowbit > SLA2_LOWBIT_I8QKV) return SLA2_EINVAL;
    if (p->flags & ~(uint32_t)(SLA2_FLAG_SKIP_LINEAR | SLA2_FLAG_SKIP_SPARSE)) return SLA2_EINVAL;
    if (op < SLA2_OP_ROUTE || op > SLA2_OP_ATTENTION_FP8) return SLA2_EINVAL;
    if (p->d != 64 && p->d != 128) return SLA2_EUNSUPPORTED;
    if (p->bq != 64 && p->bq != 128) return SLA2_EUNSUPPORTED;
    if (p->bkv != 64) return SLA2_EUNSUPPORTED;
    if (p->phi != SLA2_PHI_ELU1 && p->phi != SLA2_PHI_SOFTMAX) return SLA2_EUNSUPPORTED;
    const bool fast = p->dtype == SLA2_BF16 && p->bq == 128 && p->d == 128;
    const bool lowbit_op = op == SLA2_OP_FORWARD_FP8 || op == SLA2_OP_ATTENTION_FP8;
    if (lowbit_op && !fast) return SLA2_EUNSUPPORTED;
    const bool routing = op == SLA2_OP_ROUTE || op == SLA2_OP_ROUTE_GRAD;
    // the low-bit kernels take elu + 1 only (routing ignores phi)
    if (p->phi == SLA2_PHI_SOFTMAX && lowbit_op) return SLA2_EUNSUPPORTED;
    long bh = (long)p->B * p->H;
    if (bh > 65535) return SLA2_EUNSUPPORTED;
    D->B = p->B;
    D->H = p->H;
    D->N = p->N;
    D->d = p->d;
    D->bq = p->bq;
    D->bkv = p->bkv;
    D->Tq = ceil_div(p->N, p->bq);
    D->Tkv = ceil_div(p->N, p->bkv);
    if (D->Tkv > kMaxTkv) return SLA2_EUNSUPPORTED;
    D->k = topk_of(p->topk_frac, D->Tkv);
    D->w_heads = p->w_heads;
    D->dtype = p->dtype;
    D->BH = bh;
    const long nd = (long)p->N * p->d;
    if (p->layout == SLA2_LAYOUT_BHND) {
        D->st.b = (long)p->H * nd;
        D->st.h = nd;
        D->st.t = p->d;
    } else {
        D->st.b = (long)p->H * nd;
        D->st.h = p->d;
        D->st.t = p->H * p->d;
    }
    D->alpha_qblock = p->alpha_mode == SLA2_ALPHA_PER_QBLOCK;
    D->out_bf16 = p->out_dtype == SLA2_BF16;
    D->lowbit_v = (p->lowbit & SLA2_LOWBIT_QKV) != 0;
    D->int8_qk = (p->lowbit & SLA2_LOWBIT_I8QK) != 0;
    D->phi_sm = p->phi == SLA2_PHI_SOFTMAX;
    D->v1 = op == SLA2_OP_SLA1_FORWARD;
    D->kl = 0;
    D->skip_lin = (p->flags & SLA2_FLAG_SKIP_LINEAR) != 0;
    D->skip_sparse = (p->flags & SLA2_FLAG_SKIP_SPARSE) != 0;
    // stage switches: forward-type calls on the d = 128, bq = 128 bf16 path only
    if (p->flags && !routing && op != SLA2_OP_FORWARD && op != SLA2_OP_FORWARD_FP8 &&
        op != SLA2_OP_ATTENTION && op != SLA2_OP_ATTENTION_FP8)
        return SLA2_EUNSUPPORTED;
    if (p->flags && !routing && !fast) return SLA2_EUNSUPPORTED;
    if (routing) D->skip_lin = D->skip_sparse = 0;
    // the fused kernels address a head's rows with 32-bit byte offsets
    if ((double)p->N * D->st.t * 4.0 >= 2147483648.0) return SLA2_EUNSUPPORTED;
    return SLA2_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
template <typename T>
static T* carve(char* base, size_t& off, size_t bytes) {
    off = align256(off);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += bytes;
    return p;
}

size_t layout_route(const Dims& D, char* base, RouteWS* ws) {
    size_t off = 0;
    RouteWS w;
    w.qt = carve<double>(base, off, sizeof(double) * D.BH * D.Tq * D.d);
    w.kt = carve<double>(base, off, sizeof(double) * D.BH * D.Tkv * D.d);
    w.S = carve<double>(base, off, sizeof(double) * D.BH * D.Tq * D.Tkv);
    w.xq = carve<double>(base, off, sizeof(double) * D.BH * D.Tq * D.d);
    w.xk = carve<double>(base, off, sizeof(double) * D.BH * D.Tkv * D.d);
    if (ws) *ws = w;
    return align256(off);
}

size_t layout_backward(const Dims& D, char* base, FwdWS* ws, BwdWS* bw) {
    size_t off = 0;
    FwdWS w;
    memset(&w, 0, sizeof(w));
    BwdWS b;
    memset(&b, 0, sizeof(b));
    const size_t bh = (size_t)D.BH, d = D.d, n = (size_t)D.N;
    const bool mf = bwd_mfma_path(D);
    w.htot = carve<float>(base, off, 4 * bh * d * d);
    w.ztot = carve<float>(base, off, 4 * bh * d);
    if (mf) {
        b.hblk = carve<float>(base, off, 4 * bh * D.Tkv * d * d);
        b.zblk = carve<float>(base, off, 4 * bh * D.Tkv * d);
        b.dHq = carve<float>(base, off, 4 * bh * D.Tq * d * d);
        b.dZq = carve<float>(base, off, 4 * bh * D.Tq * d);
        b.hb16 = carve<uint16_t>(base, off, 2 * bh * D.Tkv * d * d);
        b.dHb16 = carve<uint16_t>(base, off, 2 * bh * D.Tq * d * d);
        const size_t np = (size_t)D.Tq * 128;
        b.gh = carve<uint16_t>(base, off, 2 * bh * np * d);
        b.gl = carve<uint16_t>(base, off, 2 * bh * np * d);
        b.lse = carve<float>(base, off, 4 * bh * np);
        b.D = carve<float>(base, off, 4 * bh * np);
        b.sbits = carve<uint8_t>(base, off, sel_product_bits_bytes(D));
        b.zpart = carve<float>(base, off, 4 * bh * bwd_summ_chunks(D) * d);
    } else {
        const int nch = summ_chunks(D);
        w.hpart = carve<float>(base, off, 4 * bh * nch * d * d);
        w.zpart = carve<float>(base, off, 4 * bh * nch * d);
        b.ds = carve<float>(base, off, 4 * bh * n);
        b.dn = carve<float>(base, off, 4 * bh * n * d);
        b.lse = carve<float>(base, off, 4 * bh * n);
        b.D = carve<float>(base, off, 4 * bh * n);
    }
    b.da = carve<float>(base, off, 4 * bh * n);
    b.dHt = carve<float>(base, off, 4 * bh * d * d);
    b.dZt = carve<float>(base, off, 4 * bh * d);
    b.off = carve<int32_t>(base, off, 4 * bh * (D.Tkv + 1));
    b.cnt = carve<int32_t>(base, off, 4 * bh * D.Tkv);
    b.list = carve<int32_t>(base, off, 4 * bh * (size_t)D.Tq * (D.k > 0 ? D.k : 1));
    if (ws) *ws = w;
    if (bw) *bw = b;
    return align256(off);
}

size_t layout_route_grad(const Dims& D, char* base, RouteWS* ws, GradWS* gw) {
    size_t off = layout_route(D, base, ws);
    GradWS g;
    g.dq = carve<double>(base, off, sizeof(double) * D.BH * D.Tq * D.d);
    g.dk = carve<double>(base, off, sizeof(double) * D.BH * D.Tkv * D.d);
    g.pq = carve<double>(base, off, sizeof(double) * D.BH * D.d * D.d);
    g.pk = carve<double>(base, off, sizeof(double) * D.BH * D.d * D.d);
    if (gw) *gw = g;
    return align256(off);
}

size_t layout_forward(const Dims& D, int op, char* base, FwdWS* ws) {
    size_t off = 0;
    FwdWS w;
    memset(&w, 0, sizeof(w));
    const size_t bh = (size_t)D.BH, d = D.d;
    const int nch = summ_chunks(D);
    const bool lowbit_op = op == SLA2_OP_FORWARD_FP8 || op == SLA2_OP_ATTENTION_FP8;
    if (hz_path(D)) {
        // V^T for P V (not needed when P V runs on the e4m3 codes of V), the
        // per-block summaries, U and the linear-branch product
        if (!(lowbit_op && D.lowbit_v)) w.vt = carve<uint16_t>(base, off, 2 * bh * D.Tkv * d * 64);
        w.hz = carve<uint16_t>(base, off, 2 * bh * D.Tkv * (size_t)kHzPitch);
        w.usel = carve<uint8_t>(base, off, bh * (size_t)(tkv_pad(D) / 64) * ubit_rows(D) * 8);
        w.HZ = carve<char>(base, off, bh * D.Tq * (size_t)kHzRowBytes);
    } else {
        if (D.dtype == SLA2_BF16) {
            w.vt = carve<uint16_t>(base, off, 2 * bh * D.Tkv * d * 64);
            w.pkt = carve<uint16_t>(base, off, 2 * bh * D.Tkv * d * 64);
            w.zb = carve<float>(base, off, 4 * bh * D.Tkv * d);
        }
        w.hpart = carve<float>(base, off, 4 * bh * nch * d * d);
        w.zpart = carve<float>(base, off, 4 * bh * nch * d);
        w.htot = carve<float>(base, off, 4 * bh * d * d);
        w.ztot = carve<float>(base, off, 4 * bh * d);
    }
    if (lowbit_op) {
        w.qhat = carve<uint8_t>(base, off, bh * (size_t)D.Tq * D.bq * d);
        w.khat = carve<uint8_t>(base, off, bh * (size_t)D.Tkv * 64 * d);
        w.sq = carve<float>(base, off, 4 * bh * D.Tq);
        w.sk = carve<float>(base, off, 4 * bh * D.Tkv);
        w.mu = carve<float>(base, off, 4 * bh * d);
        // the combined call keeps one row of column sums per KV block
        const size_t krows = op == SLA2_OP_ATTENTION_FP8
                                 ? (size_t)std::max(D.Tkv, (D.N + 1023) / 1024)
                                 : (size_t)((D.N + 1023) / 1024);
        w.ksum = carve<double>(base, off, 8 * bh * krows * d);
        if (D.lowbit_v) {
            w.vhat = carve<uint8_t>(base, off, bh * (size_t)D.Tkv * d * 64);
            w.vmax = carve<float>(base, off, 4 * bh * ((D.N + 1023) / 1024) * d);
            w.sv = carve<float>(base, off, 4 * bh * d);
        }
    }
    if (op == SLA2_OP_SLA1_FORWARD)
        w.wpf = carve<uint16_t>(base, off, 2 * (size_t)D.w_heads * d * d);
    if (ws) *ws = w;
    return align256(off);
}

static size_t ws_bytes_of(const Dims& D, int op) {
    if (op == SLA2_OP_ROUTE) return layout_route(D, nullptr, nullptr);
    if (op == SLA2_OP_ROUTE_GRAD) return layout_route_grad(D, nullptr, nullptr, nullptr);
    if (op == SLA2_OP_BACKWARD) return layout_backward(D, nullptr, nullptr, nullptr);
    if (op == SLA2_OP_ATTENTION)  // route region, then the forward's
        return layout_route(D, nullptr, nullptr) +
               layout_forward(D, SLA2_OP_FORWARD, nullptr, nullptr);
    if (op == SLA2_OP_ATTENTION_FP8)
        return layout_route(D, nullptr, nullptr) +
               layout_forward(D, SLA2_OP_ATTENTION_FP8, nullptr, nullptr);
    return layout_forward(D, op, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// timing records
// ---------------------------------------------------------------------------
namespace {
struct Rec {
    hipEvent_t a, b;
    int kind;
};
struct Timing {
    bool on = false;
    int max = 0;
    int used = 0;
    std::vector<Rec> recs;
} g_timing;

const char* kKindNames[K_NUM_KINDS] = {
    "pool_project", "score",       "topk_select", "summaries_valu",
    "summaries_reduce", "fused_valu", "summaries_mfma", "fused_mfma",
    "quant_mean",   "quant_fp8",   "fused_fp8",  "quant_v_fp8",
    "quant_i8",     "fused_i8",    "fused_sla1",  "bwd_rows",
    "bwd_dh",       "bwd_keys",    "bwd_lin_rows", "bwd_lin_keys",
    "bwd_rows_mfma", "bwd_keys_mfma", "bwd_blk_summ", "bwd_sum_parts", "pool_quant",
    "lin_gemm",     "score_topk",  "bwd_lin_product",
};
}  // namespace

void timing_before(hipStream_t s, int kind) {
    if (!g_timing.on || g_timing.used >= g_timing.max) return;
    Rec& r = g_timing.recs[g_timing.used];
    r.kind = kind;
    (void)hipEventRecord(r.a, s);
}

void timing_after(hipStream_t s, int kind) {
    (void)kind;
    if (!g_timing.on || g_timing.used >= g_timing.max) return;
    Rec& r = g_timing.recs[g_timing.used++];
    (void)hipEventRecord(r.b, s);
}

}  // namespace sla2

using namespace sla2;

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------
SLA2_API int32_t sla2_num_q_blocks(const sla2_problem* p) {
    Dims D;
    return make_dims(p, SLA2_OP_ROUTE, &D) == SLA2_OK ? D.Tq : -1;
}

SLA2_API int32_t sla2_num_kv_blocks(const sla2_problem* p) {
    Dims D;
    return make_dims(p, SLA2_OP_ROUTE, &D) == SLA2_OK ? D.Tkv : -1;
}

SLA2_API int32_t sla2_topk(const sla2_problem* p) {
    Dims D;
    return make_dims(p, SLA2_OP_ROUTE, &D) == SLA2_OK ? D.k : -1;
}

SLA2_API size_t sla2_workspace_bytes(const sla2_problem* p, int32_t op) {
    Dims D;
    if (make_dims(p, op, &D) != SLA2_OK) return 0;
    return ws_bytes_of(D, op);
}

SLA2_API sla2_status sla2_check(const sla2_problem* p, int32_t op) {
    Dims D;
    return make_dims(p, op, &D);
}

SLA2_API const char* sla2_status_str(int32_t s) {
    switch (s) {
        case SLA2_OK: return "ok";
        case SLA2_EINVAL: return "invalid argument";
        case SLA2_EUNSUPPORTED: return "unsupported configuration";
        case SLA2_EWORKSPACE: return "workspace too small";
        case SLA2_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

static sla2_status check_ws(const Dims& D, int op, void* ws, size_t ws_bytes) {
    size_t need = ws_bytes_of(D, op);
    if (need > 0 && (!ws || !aligned(ws, 256))) return SLA2_EINVAL;
    if (ws_bytes < need) return SLA2_EWORKSPACE;
    return SLA2_OK;
}

static bool ok_ptr(const void* p) { return p && aligned(p, 16); }

SLA2_API sla2_status sla2_route(const sla2_problem* p, const void* Q, const void* K,
                                const float* Wq, const float* Wk, int32_t* topk_idx,
                                uint8_t* block_mask, void* ws, size_t ws_bytes,
                                void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ROUTE, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(Wq) || !ok_ptr(Wk)) return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(topk_idx)) return SLA2_EINVAL;
    if (block_mask && !aligned(block_mask, 16)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_ROUTE, ws, ws_bytes)) != SLA2_OK) return st;
    RouteWS w;
    layout_route(D, (char*)ws, &w);
    hipError_t e = launch_route(D, Q, K, Wq, Wk, topk_idx, block_mask, w, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

static sla2_status forward_args(const sla2_problem* p, int op, const void* Q, const void* K,
                                const void* V, const int32_t* idx, const float* alpha,
                                void* O, void* ws, size_t ws_bytes, Dims* D, FwdWS* w) {
    sla2_status st = make_dims(p, op, D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(V) || !ok_ptr(alpha) || !ok_ptr(O))
        return SLA2_EINVAL;
    if (D->k > 0 && !ok_ptr(idx)) return SLA2_EINVAL;
    if ((st = check_ws(*D, op, ws, ws_bytes)) != SLA2_OK) return st;
    layout_forward(*D, op, (char*)ws, w);
    return SLA2_OK;
}

// hz_path: U from the selection, then the linear-branch product (skipped when
// every block is selected: the fused kernel then has no linear branch)
static hipError_t linear_product(const Dims& D, const int32_t* idx, const int32_t* negl,
                                 int kl, const FwdWS& w, hipStream_t s) {
    if (D.k + kl >= D.Tkv || D.skip_lin) return hipSuccess;
    hipError_t e = launch_unsel(D, idx, negl, kl, w, s);
    if (e == hipSuccess) e = launch_lin_gemm(D, w, s);
    return e;
}

SLA2_API sla2_status sla2_forward(const sla2_problem* p, const void* Q, const void* K,
                                  const void* V, const int32_t* topk_idx, const float* alpha,
                                  void* O, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    FwdWS w;
    sla2_status st = forward_args(p, SLA2_OP_FORWARD, Q, K, V, topk_idx, alpha, O, ws,
                                  ws_bytes, &D, &w);
    if (st != SLA2_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (valu_path(D)) {
        e = launch_forward_valu(D, Q, K, V, topk_idx, alpha, O, w, s);
    } else {
        e = launch_summaries_mfma(D, K, V, w, s);
        if (e == hipSuccess && hz_path(D)) e = linear_product(D, topk_idx, nullptr, 0, w, s);
        if (e == hipSuccess) e = launch_fused_mfma(D, Q, K, topk_idx, alpha, O, w, s);
    }
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

// ---------------------------------------------------------------------------
// route + forward in one call, the block summaries on a helper stream
// ---------------------------------------------------------------------------
namespace {
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, pooled = nullptr;
};
constexpr int kMaxDevices = 64;
Side g_side[kMaxDevices];
std::mutex g_side_mu;

// The caller holds g_side_mu from here until its last event record or wait
// is enqueued: the fork / join events are shared by every call on the device,
// so the sequence record(fork) .. wait(join) of one call must not interleave
// with another's.
hipError_t side_stream(Side** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    Side& sd = g_side[dev];
    if (!sd.s) {
        // default priority (no priority argument), independent of the null stream.
        // Kept only once all four handles exist, so that a failure here is
        // retried by the next call instead of leaving some of them null.
        Side n;
        if ((e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking)) == hipSuccess &&
            (e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) == hipSuccess &&
            (e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) == hipSuccess &&
            (e = hipEventCreateWithFlags(&n.pooled, hipEventDisableTiming)) == hipSuccess) {
            sd = n;
        } else {
            if (n.pooled) (void)hipEventDestroy(n.pooled);
            if (n.join) (void)hipEventDestroy(n.join);
            if (n.fork) (void)hipEventDestroy(n.fork);
            if (n.s) (void)hipStreamDestroy(n.s);
            return e;
        }
    }
    *out = &sd;
    return hipSuccess;
}
}  // namespace

SLA2_API sla2_status sla2_attention(const sla2_problem* p, const void* Q, const void* K,
                                    const void* V, const float* Wq, const float* Wk,
                                    const float* alpha, int32_t* topk_idx, void* O, void* ws,
                                    size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ATTENTION, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(V) || !ok_ptr(Wq) || !ok_ptr(Wk) || !ok_ptr(alpha) ||
        !ok_ptr(O))
        return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(topk_idx)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_ATTENTION, ws, ws_bytes)) != SLA2_OK) return st;
    RouteWS rw;
    FwdWS fw;
    const size_t roff = layout_route(D, (char*)ws, &rw);
    layout_forward(D, SLA2_OP_FORWARD, (char*)ws + roff, &fw);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (valu_path(D)) {  // vector-ALU path: in sequence
        e = launch_route(D, Q, K, Wq, Wk, topk_idx, nullptr, rw, s);
        if (e == hipSuccess) e = launch_forward_valu(D, Q, K, V, topk_idx, alpha, O, fw, s);
        return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
    }
    Side* sd = nullptr;
    std::lock_guard<std::mutex> lk(g_side_mu);  // see side_stream
    if ((e = side_stream(&sd)) != hipSuccess) return SLA2_EHIP;
    if ((e = hipEventRecord(sd->fork, s)) != hipSuccess) return SLA2_EHIP;
    if ((e = hipStreamWaitEvent(sd->s, sd->fork, 0)) != hipSuccess) return SLA2_EHIP;
    if (hz_path(D)) {
        // K is read once: the block-summaries pass (helper stream) also
        // writes the router's pooled keys, while the caller's stream pools
        // and projects the queries; the keys' projections, the scores and
        // top-k follow the join
        e = launch_summaries_mfma(D, K, V, fw, sd->s, D.k > 0 ? rw.xk : nullptr);
        if (e == hipSuccess) e = hipEventRecord(sd->join, sd->s);
        if (e == hipSuccess) e = launch_pool_queries(D, Q, rw, s, Wq);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, sd->join, 0);
        if (e == hipSuccess)
            e = launch_route(D, Q, K, Wq, Wk, topk_idx, nullptr, rw, s, true, true);
        const bool lin = D.k < D.Tkv && !D.skip_lin;
        if (e == hipSuccess && lin) e = launch_unsel(D, topk_idx, nullptr, 0, fw, s);
        if (e == hipSuccess && lin) e = launch_lin_gemm(D, fw, s);
        if (e == hipSuccess) e = launch_fused_mfma(D, Q, K, topk_idx, alpha, O, fw, s);
        return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
    }
    // summaries (K, V) on the helper stream, the router (Q, K) on the caller's
    e = launch_summaries_mfma(D, K, V, fw, sd->s);
    if (e == hipSuccess) e = hipEventRecord(sd->join, sd->s);
    if (e == hipSuccess) e = launch_route(D, Q, K, Wq, Wk, topk_idx, nullptr, rw, s);
    const bool lin = hz_path(D) && D.k < D.Tkv && !D.skip_lin;
    if (e == hipSuccess && lin) e = launch_unsel(D, topk_idx, nullptr, 0, fw, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, sd->join, 0);
    if (e == hipSuccess && lin) e = launch_lin_gemm(D, fw, s);
    if (e == hipSuccess) e = launch_fused_mfma(D, Q, K, topk_idx, alpha, O, fw, s);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

// ---------------------------------------------------------------------------
// route + forward with no allocation of any kind: the workspace is a
// file-scope device array, one copy per GPU (the code object's data, loaded
// with the library's kernels), addressed through hipGetSymbolAddress once per
// device; everything runs on the caller's stream (no helper stream, no
// events).  The array keeps the previous call's contents; nothing in the
// path reads workspace it did not write in the same call, so nothing is
// cleared.
// ---------------------------------------------------------------------------
static constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
void* g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

// the calling thread's current device's copy of scratch
hipError_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}
}  // namespace

SLA2_API size_t sla2_noalloc_scratch_bytes(void) { return kScratchBytes; }

SLA2_API sla2_status sla2_attention_noalloc(const sla2_problem* p, const void* Q, const void* K,
                                            const void* V, const float* Wq, const float* Wk,
                                            const float* alpha, int32_t* topk_idx, void* O,
                                            void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ATTENTION, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(V) || !ok_ptr(Wq) || !ok_ptr(Wk) || !ok_ptr(alpha) ||
        !ok_ptr(O))
        return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(topk_idx)) return SLA2_EINVAL;
    if (ws_bytes_of(D, SLA2_OP_ATTENTION) > kScratchBytes) return SLA2_EWORKSPACE;
    void* ws = nullptr;
    if (scratch_ptr(&ws) != hipSuccess) return SLA2_EHIP;
    RouteWS rw;
    FwdWS fw;
    const size_t roff = layout_route(D, (char*)ws, &rw);
    layout_forward(D, SLA2_OP_FORWARD, (char*)ws + roff, &fw);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_route(D, Q, K, Wq, Wk, topk_idx, nullptr, rw, s);
    if (e == hipSuccess) {
        if (valu_path(D)) {
            e = launch_forward_valu(D, Q, K, V, topk_idx, alpha, O, fw, s);
        } else {
            e = launch_summaries_mfma(D, K, V, fw, s);
            if (e == hipSuccess && hz_path(D)) e = linear_product(D, topk_idx, nullptr, 0, fw, s);
            if (e == hipSuccess) e = launch_fused_mfma(D, Q, K, topk_idx, alpha, O, fw, s);
        }
    }
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_attention_fp8(const sla2_problem* p, const void* Q, const void* K,
                                        const void* V, const float* Wq, const float* Wk,
                                        const float* alpha, int32_t* topk_idx, void* O,
                                        void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ATTENTION_FP8, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(V) || !ok_ptr(Wq) || !ok_ptr(Wk) || !ok_ptr(alpha) ||
        !ok_ptr(O))
        return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(topk_idx)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_ATTENTION_FP8, ws, ws_bytes)) != SLA2_OK) return st;
    RouteWS rw;
    FwdWS fw;
    const size_t roff = layout_route(D, (char*)ws, &rw);
    layout_forward(D, SLA2_OP_ATTENTION_FP8, (char*)ws + roff, &fw);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    Side* sd = nullptr;
    std::lock_guard<std::mutex> lk(g_side_mu);  // see side_stream
    if ((e = side_stream(&sd)) != hipSuccess) return SLA2_EHIP;
    // K is read by the block-summaries pass (helper stream), which also
    // writes the router's pooled keys and each KV block's column sums; the
    // caller's stream pools the queries, writes their codes and projects
    // them, then (once the summaries are done) runs the keys' projections,
    // the scores and top-k while
    // the helper stream takes the K mean from the block sums and writes the
    // key codes (and the V codes).  The same codes as sla2_quantize_fp8
    // (exact fp64 sums).
    if ((e = hipEventRecord(sd->fork, s)) != hipSuccess) return SLA2_EHIP;
    if ((e = hipStreamWaitEvent(sd->s, sd->fork, 0)) != hipSuccess) return SLA2_EHIP;
    e = launch_summaries_mfma(D, K, V, fw, sd->s, rw.xk, fw.ksum);
    if (e == hipSuccess) e = hipEventRecord(sd->pooled, sd->s);
    if (e == hipSuccess) e = launch_quantize_k(D, K, V, fw, sd->s);
    if (e == hipSuccess) e = hipEventRecord(sd->join, sd->s);
    if (e == hipSuccess) e = launch_pool_quant(D, Q, K, rw, fw, s, true);
    if (e == hipSuccess) e = launch_project_queries(D, Wq, rw, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, sd->pooled, 0);
    if (e == hipSuccess)
        e = launch_route(D, Q, K, Wq, Wk, topk_idx, nullptr, rw, s, true, true);
    const bool lin = D.k < D.Tkv && !D.skip_lin;
    if (e == hipSuccess && lin) e = launch_unsel(D, topk_idx, nullptr, 0, fw, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, sd->join, 0);
    if (e == hipSuccess && lin) e = launch_lin_gemm(D, fw, s);
    if (e == hipSuccess) e = launch_fused128(D, Q, K, topk_idx, alpha, O, fw, true, s);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_forward_fp8(const sla2_problem* p, const void* Q, const void* K,
                                      const void* V, const int32_t* topk_idx,
                                      const float* alpha, void* O, void* ws,
                                      size_t ws_bytes, void* stream) {
    Dims D;
    FwdWS w;
    sla2_status st = forward_args(p, SLA2_OP_FORWARD_FP8, Q, K, V, topk_idx, alpha, O, ws,
                                  ws_bytes, &D, &w);
    if (st != SLA2_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_quantize_fp8(D, Q, K, V, w, s);
    if (e == hipSuccess) e = launch_summaries_mfma(D, K, V, w, s);
    if (e == hipSuccess) e = linear_product(D, topk_idx, nullptr, 0, w, s);
    if (e == hipSuccess) e = launch_fused128(D, Q, K, topk_idx, alpha, O, w, true, s);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_quantize_fp8(const sla2_problem* p, const void* Q, const void* K,
                                       uint8_t* Qhat, uint8_t* Khat, float* sQ, float* sK,
                                       float* mu, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_FORWARD_FP8, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(Qhat) || !ok_ptr(Khat) || !ok_ptr(sQ) ||
        !ok_ptr(sK) || !ok_ptr(mu))
        return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_FORWARD_FP8, ws, ws_bytes)) != SLA2_OK) return st;
    FwdWS w;
    layout_forward(D, SLA2_OP_FORWARD_FP8, (char*)ws, &w);
    w.qhat = Qhat;
    w.khat = Khat;
    w.sq = sQ;
    w.sk = sK;
    w.mu = mu;
    hipError_t e = launch_quantize_fp8(D, Q, K, nullptr, w, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_quantize_v_fp8(const sla2_problem* p, const void* V, uint8_t* Vhat,
                                         float* sV, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_FORWARD_FP8, &D);
    if (st != SLA2_OK) return st;
    if (!D.lowbit_v) return SLA2_EUNSUPPORTED;
    if (!ok_ptr(V) || !ok_ptr(Vhat) || !ok_ptr(sV)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_FORWARD_FP8, ws, ws_bytes)) != SLA2_OK) return st;
    FwdWS w;
    layout_forward(D, SLA2_OP_FORWARD_FP8, (char*)ws, &w);
    w.sv = sV;
    hipError_t e = launch_quantize_v_rows(D, V, Vhat, w, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

// ---------------------------------------------------------------------------
// SLA (v1) compatibility
// ---------------------------------------------------------------------------
// k_l = clamp(ceil(low_frac * T_kv - 1e-6), 0, T_kv - k_h); -1 if low_frac is bad
static int low_of(const Dims& D, float low_frac) {
    if (!(low_frac >= 0.0f && low_frac <= 1.0f)) return -1;
    double k = ceil((double)low_frac * (double)D.Tkv - 1e-6);
    if (k < 0) k = 0;
    if (k > D.Tkv - D.k) k = D.Tkv - D.k;
    return (int)k;
}

SLA2_API int32_t sla1_num_negligible(const sla2_problem* p, float low_frac) {
    Dims D;
    if (make_dims(p, SLA2_OP_ROUTE, &D) != SLA2_OK) return -1;
    return low_of(D, low_frac);
}

SLA2_API sla2_status sla1_route(const sla2_problem* p, const void* Q, const void* K,
                                float low_frac, int32_t* crit_idx, int32_t* negl_idx,
                                uint8_t* block_mask, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ROUTE, &D);
    if (st != SLA2_OK) return st;
    const int kl = low_of(D, low_frac);
    if (kl < 0) return SLA2_EINVAL;
    if (!ok_ptr(Q) || !ok_ptr(K)) return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(crit_idx)) return SLA2_EINVAL;
    if (kl > 0 && !ok_ptr(negl_idx)) return SLA2_EINVAL;
    if (block_mask && !aligned(block_mask, 16)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_ROUTE, ws, ws_bytes)) != SLA2_OK) return st;
    RouteWS w;
    layout_route(D, (char*)ws, &w);
    hipError_t e = launch_route_v1(D, Q, K, kl, crit_idx, negl_idx, block_mask, w,
                                   (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla1_forward(const sla2_problem* p, const void* Q, const void* K,
                                  const void* V, const int32_t* crit_idx,
                                  const int32_t* negl_idx, float low_frac, const float* Wp,
                                  void* O, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_SLA1_FORWARD, &D);
    if (st != SLA2_OK) return st;
    D.kl = low_of(D, low_frac);
    if (D.kl < 0) return SLA2_EINVAL;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(V) || !ok_ptr(Wp) || !ok_ptr(O)) return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(crit_idx)) return SLA2_EINVAL;
    if (D.kl > 0 && !ok_ptr(negl_idx)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_SLA1_FORWARD, ws, ws_bytes)) != SLA2_OK) return st;
    FwdWS w;
    layout_forward(D, SLA2_OP_SLA1_FORWARD, (char*)ws, &w);
    hipStream_t s = (hipStream_t)stream;
    if (!hz_path(D)) {  // fp32, b_q = 64 or d = 64: the vector-ALU kernels
        hipError_t e = launch_forward_valu(D, Q, K, V, crit_idx, nullptr, O, w, s, negl_idx, Wp);
        return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
    }
    hipError_t e = launch_summaries_mfma(D, K, V, w, s);
    if (e == hipSuccess) e = launch_wp_frag(D, Wp, w, s);
    if (e == hipSuccess) e = linear_product(D, crit_idx, negl_idx, D.kl, w, s);
    if (e == hipSuccess) e = launch_fused128(D, Q, K, crit_idx, nullptr, O, w, false, s);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

// ---------------------------------------------------------------------------
// training-time router (Stage 1)
// ---------------------------------------------------------------------------
SLA2_API sla2_status sla2_soft_topk(const sla2_problem* p, const void* Q, const void* K,
                                    const float* Wq, const float* Wk, float tau, float* M,
                                    double* lambda, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ROUTE, &D);
    if (st != SLA2_OK) return st;
    if (!(tau > 0.0f) || !isfinite(tau)) return SLA2_EINVAL;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(Wq) || !ok_ptr(Wk) || !ok_ptr(M)) return SLA2_EINVAL;
    if (lambda && !aligned(lambda, 16)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_ROUTE, ws, ws_bytes)) != SLA2_OK) return st;
    RouteWS w;
    layout_route(D, (char*)ws, &w);
    hipError_t e = launch_soft_topk(D, Q, K, Wq, Wk, (double)tau, M, lambda, w,
                                    (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_soft_topk_grad(const sla2_problem* p, const float* M, const float* dM,
                                         float tau, float* dS, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ROUTE, &D);
    if (st != SLA2_OK) return st;
    if (!(tau > 0.0f) || !isfinite(tau)) return SLA2_EINVAL;
    if (!ok_ptr(M) || !ok_ptr(dM) || !ok_ptr(dS)) return SLA2_EINVAL;
    hipError_t e = launch_soft_topk_grad(D, M, dM, (double)tau, dS, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_route_grad(const sla2_problem* p, const void* Q, const void* K,
                                     const float* Wq, const float* Wk, const float* dS,
                                     float* dWq, float* dWk, void* ws, size_t ws_bytes,
                                     void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_ROUTE_GRAD, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(Wq) || !ok_ptr(Wk) || !ok_ptr(dS) || !ok_ptr(dWq) ||
        !ok_ptr(dWk))
        return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_ROUTE_GRAD, ws, ws_bytes)) != SLA2_OK) return st;
    RouteWS w;
    GradWS g;
    layout_route_grad(D, (char*)ws, &w, &g);
    hipError_t e = launch_route_grad(D, Q, K, Wq, Wk, dS, dWq, dWk, w, g, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_backward(const sla2_problem* p, const void* Q, const void* K,
                                   const void* V, const int32_t* topk_idx, const float* alpha,
                                   const float* dO, float* dQ, float* dK, float* dV,
                                   float* dalpha, void* ws, size_t ws_bytes, void* stream) {
    Dims D;
    sla2_status st = make_dims(p, SLA2_OP_BACKWARD, &D);
    if (st != SLA2_OK) return st;
    if (!ok_ptr(Q) || !ok_ptr(K) || !ok_ptr(V) || !ok_ptr(alpha) || !ok_ptr(dO) ||
        !ok_ptr(dQ) || !ok_ptr(dK) || !ok_ptr(dV) || !ok_ptr(dalpha))
        return SLA2_EINVAL;
    if (D.k > 0 && !ok_ptr(topk_idx)) return SLA2_EINVAL;
    if ((st = check_ws(D, SLA2_OP_BACKWARD, ws, ws_bytes)) != SLA2_OK) return st;
    FwdWS w;
    BwdWS b;
    layout_backward(D, (char*)ws, &w, &b);
    hipError_t e = launch_backward(D, Q, K, V, dO, topk_idx, alpha, dQ, dK, dV, dalpha, w, b,
                                   (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_fp8_dot_tiles(const uint8_t* A, const uint8_t* B, float* C,
                                        int32_t ntiles, void* stream) {
    if (!ok_ptr(A) || !ok_ptr(B) || !ok_ptr(C)) return SLA2_EINVAL;
    if (ntiles <= 0 || ntiles > (1 << 20)) return SLA2_EINVAL;
    hipError_t e = launch_fp8_dot(A, B, C, ntiles, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_mfma_rate_probe(int32_t kind, int32_t iters, int32_t groups,
                                          float* out, void* stream) {
    if (kind < 0 || kind > 3) return SLA2_EINVAL;
    if (iters <= 0 || iters > (1 << 24) || groups <= 0 || groups > (1 << 16)) return SLA2_EINVAL;
    if (!ok_ptr(out)) return SLA2_EINVAL;
    hipError_t e = launch_mfma_rate(kind, iters, groups, out, (hipStream_t)stream);
    return e == hipSuccess ? SLA2_OK : SLA2_EHIP;
}

SLA2_API sla2_status sla2_timing_start(int32_t max_launches) {
    if (max_launches <= 0) return SLA2_EINVAL;
    if ((int)g_timing.recs.size() < max_launches) {
        size_t old = g_timing.recs.size();
        g_timing.recs.resize(max_launches);
        for (size_t i = old; i < g_timing.recs.size(); ++i) {
            if (hipEventCreate(&g_timing.recs[i].a) != hipSuccess ||
                hipEventCreate(&g_timing.recs[i].b) != hipSuccess) {
                g_timing.recs.resize(i);
                return SLA2_EHIP;
            }
        }
    }
    g_timing.max = max_launches;
    g_timing.used = 0;
    g_timing.on = true;
    return SLA2_OK;
}

SLA2_API sla2_status sla2_timing_stop(float* total_ms, int32_t* launches, int32_t n_kinds) {
    if (!total_ms || !launches || n_kinds <= 0) return SLA2_EINVAL;
    for (int i = 0; i < n_kinds; ++i) {
        total_ms[i] = 0.0f;
        launches[i] = 0;
    }
    sla2_status st = SLA2_OK;
    for (int i = 0; i < g_timing.used; ++i) {
        Rec& r = g_timing.recs[i];
        if (hipEventSynchronize(r.b) != hipSuccess) {
            st = SLA2_EHIP;
            continue;
        }
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            st = SLA2_EHIP;
            continue;
        }
        if (r.kind >= 0 && r.kind < n_kinds) {
            total_ms[r.kind] += ms;
            launches[r.kind] += 1;
        }
    }
    g_timing.on = false;
    g_timing.used = 0;
    return st;
}

SLA2_API int32_t sla2_kernel_kinds(void) { return K_NUM_KINDS; }

SLA2_API const char* sla2_kernel_name(int32_t kind) {
    if (kind < 0 || kind >= K_NUM_KINDS) return "";
    return kKindNames[kind];
}
