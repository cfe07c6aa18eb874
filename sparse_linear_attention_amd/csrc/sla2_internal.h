// Internal declarations of libsla2: problem dimensions, workspace layout,
// kernel launchers and the timing hooks.  Host and device code of the
// library only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sla2.h"
#include "hz_layout.h"

namespace sla2 {

// kinds of kernels, for the timing records
enum KernelKind {
    K_POOL_PROJECT = 0,
    K_SCORE,
    K_TOPK,
    K_SUMM_VALU,
    K_SUMM_REDUCE,
    K_FUSED_VALU,
    K_SUMM_MFMA,
    K_FUSED_MFMA,
    K_QUANT_MEAN,
    K_QUANT,
    K_FUSED_FP8,
    K_QUANT_V,
    K_QUANT_I8,
    K_FUSED_I8,
    K_FUSED_SLA1,
    K_BWD_ROWS,
    K_BWD_DH,
    K_BWD_KEYS,
    K_BWD_LIN_ROWS,
    K_BWD_LIN_KEYS,
    K_BWD_ROWS_MFMA,
    K_BWD_KEYS_MFMA,
    K_BWD_BLK_SUMM,
    K_BWD_SUM_PARTS,
    K_POOL_QUANT,
    K_LIN_GEMM,
    K_SCORE_TOPK,
    K_BWD_LIN_PRODUCT,
    K_NUM_KINDS
};

// Element strides of a Q/K/V/O tensor: batch, head, token (d innermost).
// [B,H,N,d]: (H N d, N d, d); [B,N,H,d]: (N H d, d, H d).
struct Strides {
    long b, h;
    int t;
};

// offset of row 0 of head bh (= b * H + h)
__host__ __device__ inline long head_base(const Strides& s, long bh, int H) {
    return (bh / H) * s.b + (bh % H) * s.h;
}

struct Dims {
    int B, H, N, d, bq, bkv;
    int Tq, Tkv, k, w_heads;
    int dtype;  // sla2_dtype of Q, K, V
    long BH;
    Strides st;          // layout of Q, K, V and O
    int alpha_qblock;    // alpha is [H][Tq] (else [H])
    int out_bf16;        // O is bf16 (else fp32)
    int lowbit_v;        // the low-bit forward quantises V too
    int int8_qk;         // the low-bit forward takes int8 Q/K codes (else e4m3)
    int phi_sm;          // phi = softmax over the channels of a row (else elu + 1)
    int v1;              // SLA (v1) forward: ternary blocks, O = O_s + O_l W_p
    int kl;              // v1: negligible blocks per query block
    int skip_lin;        // SLA2_FLAG_SKIP_LINEAR: no linear branch (O = alpha O_s)
    int skip_sparse;     // SLA2_FLAG_SKIP_SPARSE: no sparse branch (O = (1 - alpha) O_l)
};

// Four consecutive outputs (element offset off, a multiple of 4) as fp32, or
// rounded once to bf16 (nearest even).
__device__ inline void store_out4(void* O, size_t off, float x, float y, float z, float w,
                                  int out_bf16) {
    if (out_bf16) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        bf16x4_t b;
        b[0] = (__bf16)x;
        b[1] = (__bf16)y;
        b[2] = (__bf16)z;
        b[3] = (__bf16)w;
        *reinterpret_cast<bf16x4_t*>(static_cast<uint16_t*>(O) + off) = b;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(O) + off) = make_float4(x, y, z, w);
    }
}

// alpha of a row of head bh in query block qb
__device__ inline float alpha_of(const float* alpha, long bh, int H, int qb, int Tq,
                                 int per_qblock) {
    const int h = (int)(bh % H);
    return per_qblock ? alpha[(size_t)h * Tq + qb] : alpha[h];
}

// chunking of the token axis for the block-summary pass
constexpr int kSummBlocksPerChunk = 16;  // KV blocks of 64 tokens per work-group
inline int summ_chunks(const Dims& D) {
    return (D.Tkv + kSummBlocksPerChunk - 1) / kSummBlocksPerChunk;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The d = 128, b_q = 128 bf16 path evaluates the linear branch as one dense
// matrix-core product per head: H_i, Z_i = sum over KV blocks j of
// U[i][j] (h_j, z_j), U the 0/1 indicator of the blocks query block i leaves
// to the linear branch (linear.hip).  Rows of the block summaries and of the
// products hold the d*d entries of h^T (V channel major) and then the d of z.
constexpr int kHzCols = 128 * 128 + 128;  // entries of a row
// bytes of a product row: H_i^T in bf16 (the fp32 exponent range, so no
// scaling), then Z_i in fp32
constexpr int kHzRowBytes = 128 * 128 * 2 + 128 * 4;
constexpr int kHzPitch = 65 * 256;        // bf16 elements per summaries row
constexpr int kGemmM = 320;               // query blocks per product tile
inline bool hz_path(const Dims& D) { return D.dtype == SLA2_BF16 && D.d == 128 && D.bq == 128; }
// forward on the vector-ALU kernels: fp32 inputs, b_q = 64, or d = 64 with
// the softmax feature map (the d = 64 matrix-core kernel takes elu + 1 only)
inline bool valu_path(const Dims& D) {
    return D.dtype == SLA2_F32 || D.bq != 128 || (D.d != 128 && D.phi_sm);
}
// KV blocks of U: Tkv rounded up to a multiple of 64 (one k-step of the product)
inline int tkv_pad(const Dims& D) { return (D.Tkv + 63) & ~63; }
// rows of U per head and k-step: whole product tiles plus a 64-row tail (the
// last tile's U loads run past its 320 rows)
inline int ubit_rows(const Dims& D) { return (D.Tq + kGemmM - 1) / kGemmM * kGemmM + 64; }

// ---------------------------------------------------------------------------
// workspace layout.  Every region starts 256-byte aligned.
// ---------------------------------------------------------------------------
struct RouteWS {
    double* qt;  // [BH][Tq][d]   projected pooled queries
    double* kt;  // [BH][Tkv][d]  projected pooled keys
    double* S;   // [BH][Tq][Tkv] compressed scores
    double* xq;  // [BH][Tq][d]   pooled queries (before the projection)
    double* xk;  // [BH][Tkv][d]  pooled keys
};

struct FwdWS {
    // bf16 path: block-transposed fp16 copies, kv order permuted inside each
    // group of 16 (see the fused kernel), padding tokens are 0
    uint16_t* vt;    // [BH][Tkv][d][64]  V^T      (fp16 bits)
    uint16_t* pkt;   // [BH][Tkv][d][64]  phi(K)^T (fp16 bits)
    float* zb;       // [BH][Tkv][d]      per-block z_j
    float* hpart;    // [BH][chunks][d][d] partial h per chunk
    float* zpart;    // [BH][chunks][d]
    float* htot;     // [BH][d][d]        h_tot[c][e] = sum phi(K)[.,c] V[.,e]
    float* ztot;     // [BH][d]
    // low-bit inputs
    uint8_t* qhat;   // [BH][Tq*bq][d]
    uint8_t* khat;   // [BH][Tkv*64][d]
    float* sq;       // [BH][Tq]
    float* sk;       // [BH][Tkv]
    float* mu;       // [BH][d]
    double* ksum;    // [BH][ceil(N/1024)][d] partial column sums of K (in the
                     // combined low-bit call: [BH][Tkv][d], one row per KV block)
    // fully low-bit (V quantised per channel)
    uint8_t* vhat;   // [BH][Tkv][d][64] e4m3 codes of V / s_V, keys in the order
                     // of the e4m3 P V product's k operand (see fused128.hip)
    float* vmax;     // [BH][ceil(N/1024)][d] partial max |V|
    float* sv;       // [BH][d]
    // SLA (v1): W_p as fp16 A-operand fragments of the projection product
    uint16_t* wpf;   // [w_heads][4 m-tiles][8 k-steps][64 lanes][8]
    // d = 128, b_q = 128 bf16 path (hz_path): the linear branch as a product
    uint16_t* hz;    // [BH][Tkv][kHzPitch] bf16: h_j^T (units at hz_unit), then z_j
    uint8_t* usel;   // [BH][tkv_pad / 64][ubit_rows][8] bits: block j left to the linear branch
    char* HZ;        // [BH][Tq][kHzRowBytes]: H_i^T (units at hz_unit) bf16, then Z_i fp32
};

// backward (SLA2_OP_BACKWARD: the forward's summary buffers, then these)
struct BwdWS {
    float* lse;     // [BH][N]  log-sum-exp of each row's selected logits
                    //          (matrix-core path: [BH][Tq * 128], log2 domain)
    float* D;       // [BH][N]  alpha dO . O_s (matrix-core path: [BH][Tq * 128])
    float* ds;      // [BH][N]  dL/d(denominator of O_l)
    float* dn;      // [BH][N][d] dL/d(numerator of O_l)
    float* da;      // [BH][N]  dO . (O_s - O_l)
    float* dHt;     // [BH][d][d] sum_t phi(q_t)^T dn_t
    float* dZt;     // [BH][d]    sum_t phi(q_t) ds_t
    int32_t* off;   // [BH][Tkv + 1] query blocks selecting each KV block:
    int32_t* cnt;   // [BH][Tkv]     offsets, counts,
    int32_t* list;  // [BH][Tq * k]  and the lists (ascending)
    // matrix-core path only (bwd_mfma_path): per-block summaries and the
    // per-query-block gradients of H_i, Z_i
    float* hblk;    // [BH][Tkv][d][d]: the per-chunk h partials, then the keys
                    //                product's rows
    float* zblk;    // [BH][Tkv][d]    z_j
    float* dHq;     // [BH][Tq][d][d]  dL/dH_i
    float* dZq;     // [BH][Tq][d]     dL/dZ_i
    uint16_t* hb16; // [BH][Tkv][d][d] h_j rounded to bf16 (for the per-pair gathers)
    uint16_t* dHb16;// [BH][Tq][d][d]  dH_i rounded to bf16
    uint16_t* gh;   // [BH][Tq * 128][d] bf16 high part of alpha dO (rows past N: 0)
    uint16_t* gl;   // [BH][Tq * 128][d] bf16 rest of alpha dO
    uint8_t* sbits; // 0/1 rows of the selection products (sel_product_bits_bytes)
    float* zpart;   // [BH][bwd_summ_chunks][d] z summed per chunk of KV blocks
                    // (the h partials go to the front of hblk)
};
// chunks of 8 KV blocks of the matrix-core backward's block summaries
inline int bwd_summ_chunks(const Dims& D) { return (D.Tkv + 7) / 8; }
// the backward runs on the matrix cores for bf16 inputs with d = b_q = 128
// (b_kv = 64) and phi = elu + 1; other problems take the vector-ALU kernels
inline bool bwd_mfma_path(const Dims& D) {
    return D.dtype == SLA2_BF16 && D.d == 128 && D.bq == 128 && D.bkv == 64 && !D.phi_sm;
}
size_t layout_backward(const Dims& D, char* base, FwdWS* ws, BwdWS* bw);

// router gradient (SLA2_OP_ROUTE_GRAD: the route layout, then these)
struct GradWS {
    double* dq;  // [BH][Tq][d]   dL/dqt
    double* dk;  // [BH][Tkv][d]  dL/dkt
    double* pq;  // [BH][d][d]    per-head dL/dWq
    double* pk;  // [BH][d][d]    per-head dL/dWk
};

// Lays out the workspace of `op` starting at `base` (may be null to size
// only); returns the bytes needed.
size_t layout_route(const Dims& D, char* base, RouteWS* ws);
size_t layout_route_grad(const Dims& D, char* base, RouteWS* ws, GradWS* gw);
size_t layout_forward(const Dims& D, int op, char* base, FwdWS* ws);

// ---------------------------------------------------------------------------
// timing hooks (no-ops unless sla2_timing_start was called)
// ---------------------------------------------------------------------------
void timing_before(hipStream_t s, int kind);
void timing_after(hipStream_t s, int kind);

// ---------------------------------------------------------------------------
// launchers (each returns hipGetLastError() after its launches)
// ---------------------------------------------------------------------------
// pooled: ws.xq / ws.xk already hold the pooled means (launch_pool_quant),
// so the pooling pass is skipped; q_projected: ws.qt holds the queries'
// projections as well (launch_pool_queries with Wq), only the keys are
// projected
hipError_t launch_route(const Dims& D, const void* Q, const void* K, const float* Wq,
                        const float* Wk, int32_t* idx, uint8_t* mask, const RouteWS& ws,
                        hipStream_t s, bool pooled = false, bool q_projected = false);

// the pooling pass over the query blocks only (ws.xq), for a caller that
// has the key blocks' means from the block-summaries pass; with Wq also
// their projections (ws.qt)
hipError_t launch_pool_queries(const Dims& D, const void* Q, const RouteWS& ws, hipStream_t s,
                               const float* Wq = nullptr);
// the queries' projections alone (ws.xq -> ws.qt), e.g. after launch_pool_quant
hipError_t launch_project_queries(const Dims& D, const float* Wq, const RouteWS& ws,
                                  hipStream_t s);

// router stages: pooled rows and their projections (ws.xq/xk, ws.qt/kt);
// then the scores (ws.S)
hipError_t launch_pool_project(const Dims& D, const void* Q, const void* K, const float* Wq,
                               const float* Wk, const RouteWS& ws, hipStream_t s,
                               bool pooled = false, bool q_projected = false);
hipError_t launch_scores(const Dims& D, const void* Q, const void* K, const float* Wq,
                         const float* Wk, const RouteWS& ws, hipStream_t s,
                         bool pooled = false, bool q_projected = false);

// training-time router: SoftTop-k, its gradient, the projections' gradient
hipError_t launch_soft_topk(const Dims& D, const void* Q, const void* K, const float* Wq,
                            const float* Wk, double tau, float* M, double* lambda,
                            const RouteWS& ws, hipStream_t s);
hipError_t launch_soft_topk_grad(const Dims& D, const float* M, const float* dM, double tau,
                                 float* dS, hipStream_t s);
hipError_t launch_route_grad(const Dims& D, const void* Q, const void* K, const float* Wq,
                             const float* Wk, const float* dS, float* dWq, float* dWk,
                             const RouteWS& ws, const GradWS& gw, hipStream_t s);

// SLA (v1) router: critical (top k) and negligible (bottom kl) blocks
hipError_t launch_route_v1(const Dims& D, const void* Q, const void* K, int kl, int32_t* crit,
                           int32_t* negl, uint8_t* mask, const RouteWS& ws, hipStream_t s);

// vector-ALU path (fp32 inputs, b_q = 64, d = 64): block summaries + fused
// kernel; with D.v1, negl [BH][Tq][D.kl] and Wp [w_heads][d][d] (alpha unused)
// matrix-core rate probe: kind 0 bf16 32x32x16, 1 e4m3 32x32x64, 2 bf16
// 16x16x32, 3 fp16 32x32x16; groups
// work-groups of 4 waves, each wave iters x 4 products; out [groups * 4]
hipError_t launch_mfma_rate(int kind, int iters, int groups, float* out, hipStream_t s);

hipError_t launch_forward_valu(const Dims& D, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const float* alpha, void* O,
                               const FwdWS& ws, hipStream_t s, const int32_t* negl = nullptr,
                               const float* Wp = nullptr);

// fp32 block summaries (h_tot, z_tot via the chunk partials)
hipError_t launch_summaries_valu(const Dims& D, const void* K, const void* V, const FwdWS& ws,
                                 hipStream_t s);

// backward of the SLA2 forward (selection fixed)
hipError_t launch_backward(const Dims& D, const void* Q, const void* K, const void* V,
                           const float* dO, const int32_t* idx, const float* alpha, float* dQ,
                           float* dK, float* dV, float* dalpha, const FwdWS& ws,
                           const BwdWS& bw, hipStream_t s);

// deterministic reduction of the per-chunk summary partials
hipError_t launch_summaries_reduce(const Dims& D, const FwdWS& ws, hipStream_t s);
// tot[bh] = sum over c < nch of part[bh][c] (d x d), ztot likewise (d), in order
hipError_t launch_partials_reduce(const Dims& D, const float* part, const float* zpart,
                                  float* tot, float* ztot, int nch, hipStream_t s);
// per-KV-block summaries h_j, z_j (fp32) into hblk [BH][Tkv][d][d], zblk [BH][Tkv][d]
hipError_t launch_summaries_blocks(const Dims& D, const void* K, const void* V, float* hblk,
                                   float* zblk, hipStream_t s);
// matrix-core backward (bwd_mfma_path)
hipError_t launch_backward_mfma(const Dims& D, const void* Q, const void* K, const void* V,
                                const float* dO, const int32_t* idx, const float* alpha,
                                float* dQ, float* dK, float* dV, const FwdWS& ws,
                                const BwdWS& bw, hipStream_t s);
// the selection inverted per KV block (bw.off, bw.cnt, bw.list)
hipError_t launch_invert(const Dims& D, const int32_t* idx, const BwdWS& bw, hipStream_t s);
// dalpha from the per-row values bw.da
hipError_t launch_dalpha(const Dims& D, const BwdWS& bw, float* dalpha, hipStream_t s);

// bf16 path: MFMA block summaries + MFMA fused kernel (bq = 128).  xk (d =
// 128, b_q = 128 path only): also write the router's pooled keys there, and
// with kblk the fp64 column sums of each KV block of K (xk must be given)
hipError_t launch_summaries_mfma(const Dims& D, const void* K, const void* V,
                                 const FwdWS& ws, hipStream_t s, double* xk = nullptr,
                                 double* kblk = nullptr);
hipError_t launch_fused_mfma(const Dims& D, const void* Q, const void* K,
                             const int32_t* idx, const float* alpha, void* O,
                             const FwdWS& ws, hipStream_t s);

// low bit
hipError_t launch_quantize_fp8(const Dims& D, const void* Q, const void* K, const void* V,
                               const FwdWS& ws, hipStream_t s);
// The same codes in two parts that share the router's reads:
// launch_pool_quant pools Q and K for the router (rw.xq, rw.xk), writes the
// query codes and scales and each KV block's column sums of K (fw.ksum, Tkv
// rows per head); launch_quantize_k then takes the K mean from those sums,
// writes the key codes and scales, and the V codes with lowbit_v.  With
// queries_only, launch_pool_quant takes the query blocks alone (the block
// summaries pass writes xk and the K block sums).
hipError_t launch_pool_quant(const Dims& D, const void* Q, const void* K, const RouteWS& rw,
                             const FwdWS& fw, hipStream_t s, bool queries_only = false);
hipError_t launch_quantize_k(const Dims& D, const void* K, const void* V, const FwdWS& fw,
                             hipStream_t s);
// V codes in rows [BH][Tkv*64][d] (inspection; s_V into ws.sv)
hipError_t launch_quantize_v_rows(const Dims& D, const void* V, uint8_t* vhat_rows,
                                  const FwdWS& ws, hipStream_t s);
// d = 128, b_q = 128 fused kernel (bf16, or the low-bit Q K^T with lowbit);
// reads ws.HZ (launch_lin_gemm) when some block is left to the linear branch
// (D.v1: the SLA (v1) forward, ws.wpf filled)
hipError_t launch_fused128(const Dims& D, const void* Q, const void* K, const int32_t* idx,
                           const float* alpha, void* O, const FwdWS& ws, bool lowbit,
                           hipStream_t s);
// hz_path: U (ws.usel) from the selected blocks idx [BH][Tq][D.k] and, for
// SLA v1, the negligible ones negl [BH][Tq][kl]; then ws.HZ = U * ws.hz
hipError_t launch_unsel(const Dims& D, const int32_t* idx, const int32_t* negl, int kl,
                        const FwdWS& ws, hipStream_t s);
hipError_t launch_lin_gemm(const Dims& D, const FwdWS& ws, hipStream_t s);
// backward (d = b_q = 128): out = sum of the bf16 d x d matrices B selected
// per row, fp32: keys = false: rows = query blocks, S_i = sum over the KV
// blocks i selects of B_j; keys = true: rows = KV blocks, D_j = sum over the
// query blocks selecting j (off / list) of B_i.  bits: the 0/1 rows
// (sel_product_bits_bytes); out: [BH][rows][d * d] fp32.
size_t sel_product_bits_bytes(const Dims& D);
// blocks of the k dimension that a 0/1 product row (unsel_kernel,
// csr_bits_kernel) holds at most
constexpr int kMaxBitBlocks = 7680;
inline bool sel_product_fits(const Dims& D) {
    return ((D.Tkv + 63) & ~63) <= kMaxBitBlocks && ((D.Tq + 63) & ~63) <= kMaxBitBlocks;
}
hipError_t launch_sel_product(const Dims& D, bool keys, const int32_t* idx, const int32_t* off,
                              const int32_t* list, uint8_t* bits, const uint16_t* B, float* out,
                              hipStream_t s);
// diagnostic: C[t] = A[t] B[t]^T, 32 x 128 e4m3 tiles, fp8 matrix cores
hipError_t launch_fp8_dot(const uint8_t* A, const uint8_t* B, float* C, int ntiles,
                          hipStream_t s);
// W_p [w_heads][d][d] fp32 -> ws.wpf (d = 128)
hipError_t launch_wp_frag(const Dims& D, const float* Wp, const FwdWS& ws, hipStream_t s);
}  // namespace sla2
