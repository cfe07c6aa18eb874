/*
 * sla2.h -- C ABI of libsla2.so, the SLA2 sparse-linear attention forward
 * pass for AMD MI355X (gfx950).
 *
 * What is computed (sources are the SLA2 pages; section names as printed):
 *   router   Qbar = pool(Q), Kbar = pool(K) (block means), P_c =
 *            proj_q(Qbar) proj_k(Kbar)^T, M_c = Top-k(k%, P_c) per row
 *            ["SLA2 深度解读" 05, "Learnable Router 到底学什么"];
 *   sparse   FlashAttention-style online softmax of Q K^T / sqrt(d) over the
 *            selected KV blocks only, O_s row-normalised
 *            ["SLA2 深度解读" 04 and 08];
 *   linear   O_l = phi(Q_i) H_i / (phi(Q_i) Z_i) with H_i, Z_i summed over the
 *            unselected blocks, phi = elu + 1
 *            ["SLA: Beyond Sparsity ..." notes, key design 3 and 4];
 *   combine  O = alpha O_s + (1 - alpha) O_l ["SLA2 深度解读" 04; gist.science
 *            explainer, section 2A];
 *   low bit  Q, K quantised to fp8 e4m3 with per-block scales, K smoothed by
 *            its channel mean, P quantised before P V ["SLA2 深度解读" 07];
 *   SLA v1   the predecessor's ternary routing (critical / marginal /
 *            negligible blocks), linear branch over the marginal blocks, O =
 *            O_s + Proj(O_l), softmax feature map ["SLA: Beyond Sparsity ..."
 *            notes, key designs 2 and 3, training section] -- sla1_* below.
 *
 * Conventions (all entry points):
 *  - Q, K, V, O, topk_idx, block_mask, alpha, Wq, Wk and ws are DEVICE
 *    pointers owned by the caller.  The library never allocates, frees or
 *    synchronises device memory; all work is enqueued on `stream` (a
 *    hipStream_t; NULL = the default stream) in call order.
 *  - Q, K, V and O share one memory layout (problem.layout): [B, H, N, d]
 *    (SLA2_LAYOUT_BHND) or [B, N, H, d] (SLA2_LAYOUT_BNHD, the token-major
 *    layout of a DiT block's attention), contiguous, d innermost.  Q, K, V
 *    share one dtype (problem.dtype); O is fp32 or bf16 (problem.out_dtype).
 *  - Every argument is validated on the host before anything is launched; on
 *    any error nothing is launched and no output is written.
 *  - Returned codes: SLA2_OK; SLA2_EINVAL (null or misaligned pointer,
 *    B/H/N <= 0, topk_frac outside [0,1] or NaN, w_heads not in {1,H}, an
 *    unknown layout, alpha mode, output dtype or low-bit mode);
 *    SLA2_EUNSUPPORTED (a valid but unbuilt combination: d not in {64,128},
 *    bq not in {64,128}, bkv != 64, phi softmax with the low-bit forward,
 *    fp8 with fp32 inputs or with bq or d other than 128, more than 65535
 *    heads or a number of blocks outside the limits below); SLA2_EWORKSPACE (ws_bytes smaller than sla2_workspace_bytes);
 *    SLA2_EHIP (a HIP launch error, reported right after the launch;
 *    asynchronous faults surface at the caller's next synchronisation).
 *  - Device-resident values are not inspected: Q, K, V must be finite, alpha
 *    values should lie in [0,1], for the bf16 paths |V| < 65504 (V is
 *    carried in fp16 inside the kernels), and every logit |q.k|/sqrt(d) must
 *    stay below 2^20 (the softmax exponent is evaluated as one fused
 *    multiply-add of the logit against the running maximum).
 *  - Pointers must be 16-byte aligned (ws: 256-byte aligned).
 *  - Calls on one stream are ordered; the library keeps no state between calls
 *    (except the optional timing records below), so concurrent calls on
 *    different streams with different workspaces are safe.
 */
#ifndef SLA2_H
#define SLA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SLA2_OK = 0,
    SLA2_EINVAL = 1,
    SLA2_EUNSUPPORTED = 2,
    SLA2_EWORKSPACE = 3,
    SLA2_EHIP = 4
} sla2_status;

typedef enum { SLA2_F32 = 0, SLA2_BF16 = 1 } sla2_dtype;

/* feature map of the linear branch: elu(x) + 1, elementwise on raw Q and K,
 * or the softmax of each raw Q or K row over its d channels, max-subtracted
 * (the SLA notes' training section picks softmax).  SLA2_PHI_SOFTMAX is taken
 * by every forward shape (sla2_forward, sla2_attention, sla1_forward), not by
 * sla2_forward_fp8 or sla2_attention_fp8. */
typedef enum { SLA2_PHI_ELU1 = 0, SLA2_PHI_SOFTMAX = 1 } sla2_phi;

/* memory layout of Q, K, V and O */
typedef enum { SLA2_LAYOUT_BHND = 0, SLA2_LAYOUT_BNHD = 1 } sla2_layout;

/* granularity of the combine weight alpha ("SLA2 深度解读" 08 gives alpha per
 * query block in the algorithm and per query in the text): one value per head
 * (alpha [H]) or one per head and query block (alpha [H][T_q]) */
typedef enum { SLA2_ALPHA_PER_HEAD = 0, SLA2_ALPHA_PER_QBLOCK = 1 } sla2_alpha_mode;

/* what sla2_forward_fp8 quantises ("SLA2 深度解读" 07: low-bit Q K^T and
 * P V, INT8 or FP8 for Q K^T): a bit mask.  Q, K and P always; bit 0: V as
 * well, per channel; bit 1: Q and K as int8 codes instead of e4m3 */
typedef enum {
    SLA2_LOWBIT_QK = 0,    /* e4m3 Q, K; V bf16           */
    SLA2_LOWBIT_QKV = 1,   /* e4m3 Q, K; e4m3 V           */
    SLA2_LOWBIT_I8QK = 2,  /* int8 Q, K; V bf16           */
    SLA2_LOWBIT_I8QKV = 3  /* int8 Q, K; e4m3 V           */
} sla2_lowbit;

/* operations, for sla2_workspace_bytes */
typedef enum {
    SLA2_OP_ROUTE = 0,         /* sla2_route, sla1_route     */
    SLA2_OP_FORWARD = 1,       /* sla2_forward               */
    SLA2_OP_FORWARD_FP8 = 2,   /* sla2_forward_fp8           */
    SLA2_OP_SLA1_FORWARD = 3,  /* sla1_forward               */
    SLA2_OP_ROUTE_GRAD = 4,    /* sla2_route_grad            */
    SLA2_OP_BACKWARD = 5,      /* sla2_backward              */
    SLA2_OP_ATTENTION = 6,     /* sla2_attention             */
    SLA2_OP_ATTENTION_FP8 = 7  /* sla2_attention_fp8         */
} sla2_op;

/* stage-timing switches (problem.flags): SKIP_LINEAR leaves the linear
 * branch out (O = alpha O_s: no block summaries h_j / z_j, no U product, no
 * epilogue product), SKIP_SPARSE the sparse branch (O = (1 - alpha) O_l: no
 * Q K^T, softmax or P V; the selection still decides which blocks the
 * linear branch covers).  Both at once give O = 0.  Taken by sla2_forward,
 * sla2_attention, sla2_forward_fp8 and sla2_attention_fp8 on the bf16,
 * d = 128, bq = 128 path (SLA2_EUNSUPPORTED elsewhere; the router and
 * sla2_workspace_bytes ignore them).  With SKIP_LINEAR, alpha = 1 and
 * k = T_kv the call is dense softmax attention, the bench's baseline. */
typedef enum { SLA2_FLAG_SKIP_LINEAR = 1, SLA2_FLAG_SKIP_SPARSE = 2 } sla2_flags;

typedef struct {
    int32_t B, H, N, d;  /* batch, heads, tokens, head dim (64 or 128)       */
    int32_t bq, bkv;     /* query / KV block sizes: bq in {64,128}, bkv = 64   */
    float topk_frac;     /* k% as a fraction in [0,1]; see sla2_topk           */
    int32_t w_heads;     /* 1: one Wq/Wk pair for all heads; H: one per head    */
    int32_t phi;         /* sla2_phi                                            */
    int32_t dtype;       /* sla2_dtype of Q, K, V                               */
    int32_t layout;      /* sla2_layout of Q, K, V and O                        */
    int32_t alpha_mode;  /* sla2_alpha_mode                                     */
    int32_t out_dtype;   /* sla2_dtype of O (SLA2_F32 or SLA2_BF16)             */
    int32_t lowbit;      /* sla2_lowbit (sla2_forward_fp8 only)                 */
    uint32_t flags;      /* 0, or sla2_flags bits (stage timing only)           */
} sla2_problem;

/* T_q = ceil(N / bq) and T_kv = ceil(N / bkv).  The last block of each kind
 * may be ragged; tokens past N are excluded from every mean, logit and sum. */
int32_t sla2_num_q_blocks(const sla2_problem* p);
int32_t sla2_num_kv_blocks(const sla2_problem* p);

/* Number of KV blocks kept per query block ("SLA2 深度解读" 05 gives k% only):
 * k = clamp(ceil(topk_frac * T_kv - 1e-6), 0, T_kv).  Returns -1 if the
 * problem is invalid. */
int32_t sla2_topk(const sla2_problem* p);

/* Bytes of device workspace an operation needs (0 if the problem is
 * invalid).  Limits: T_kv <= 7680. */
size_t sla2_workspace_bytes(const sla2_problem* p, int32_t op);

/* Validate a problem for an operation without launching anything. */
sla2_status sla2_check(const sla2_problem* p, int32_t op);

const char* sla2_status_str(int32_t status);

/*
 * sla2_route -- the block router ("SLA2 深度解读" 05).  Q, K in problem.layout.
 *   Qbar_i = mean of the valid rows of query block i, Kbar_j likewise;
 *   qt_i = Qbar_i Wq[h'], kt_j = Kbar_j Wk[h'] (h' = 0 if w_heads == 1,
 *   else h; W row-major [d][d], proj(x) = x W, no bias);
 *   S_ij = qt_i . kt_j (plain product: a 1/sqrt(d) scale or a softmax would
 *   not change a per-row top-k); the k largest S_ij of each row are
 *   selected, ties going to the lower block index.  All router arithmetic is
 *   fp64, so the selection does not depend on fp32 rounding.
 * In : Q, K (dtype, problem.layout); Wq, Wk [w_heads,d,d] fp32.
 * Out: topk_idx [B,H,T_q,k] int32, each row ascending (may be NULL if k = 0);
 *      block_mask [B,H,T_q,T_kv] uint8 0/1, or NULL if not wanted.
 * ws : sla2_workspace_bytes(p, SLA2_OP_ROUTE) bytes.
 */
sla2_status sla2_route(const sla2_problem* p, const void* Q, const void* K,
                       const float* Wq, const float* Wk, int32_t* topk_idx,
                       uint8_t* block_mask, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_forward -- sparse branch + linear branch + combine.
 *   O_s: softmax(Q_t K_u^T / sqrt(d)) V over the tokens u of the selected
 *        blocks ("SLA2 深度解读" 04, 08); O_s = 0 when k = 0.
 *   O_l: phi(Q_t) H_i / (phi(Q_t) . Z_i), H_i = sum over unselected blocks of
 *        h_j = phi(K_j)^T V_j, Z_i = sum of z_j = colsum phi(K_j) (SLA notes,
 *        key design 3 and 4); O_l = 0 when k = T_kv.  On the bf16 d = 128,
 *        bq = 128 path the sums run over the unselected blocks directly (a
 *        dense product of the 0/1 matrix of unselected blocks with the
 *        per-block summaries); elsewhere they are the head totals minus the
 *        selected blocks.
 *   O   = alpha O_s + (1 - alpha) O_l, written for the N valid rows; alpha is
 *        that of the row's head (and query block, with SLA2_ALPHA_PER_QBLOCK).
 * In : Q, K, V in problem.layout; topk_idx [B,H,T_q,k] from sla2_route
 *      (ascending, values in [0,T_kv), not checked on the device); alpha fp32
 *      [H] or [H][T_q] (problem.alpha_mode).
 * Out: O in problem.layout, fp32 or bf16 (problem.out_dtype; bf16 is O
 *      computed in fp32 and rounded to nearest even once).
 * ws : sla2_workspace_bytes(p, SLA2_OP_FORWARD) bytes.
 * Precision: fp32 inputs are computed in fp32 throughout (vector ALU), and
 * so are bf16 inputs with bq = 64.  bf16 inputs with bq = 128: Q K^T on bf16
 * matrix cores with fp32 accumulation, P rounded to fp16 for P V (V
 * converted to fp16, exact for |V| < 65504 apart from fp16 subnormals), each
 * block summary h_j = phi(K_j)^T V_j on fp16 matrix cores (phi(K_j) and V_j
 * in fp16, fp32 accumulation).  With d = 128 the summaries h_j, z_j are then
 * rounded to bf16, summed on bf16 matrix cores with fp32 accumulation, H_i
 * rounded to bf16 (Z_i kept in fp32), and phi(Q) . H_i taken on bf16 matrix
 * cores with phi(Q) rounded to bf16 (also in the denominator); with d = 64
 * H_i is formed in fp32 and enters phi(Q) H_i in fp16 (scaled by a power of
 * two).  Everything else is fp32.  Bound reached in the tests: 2e-3 max-abs
 * against an fp64 evaluation of the same definition.
 */
sla2_status sla2_forward(const sla2_problem* p, const void* Q, const void* K,
                         const void* V, const int32_t* topk_idx, const float* alpha,
                         void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_attention -- sla2_route followed by sla2_forward in one call (same
 *   kernels, bit-identical O and topk_idx).  On the bf16 bq = 128 path the
 *   block summaries (which read only K and V, and also write the router's
 *   pooled keys) run on a helper stream, concurrently with the pooling of
 *   the queries; the projections, scores and top-k follow once they are
 *   joined (events); other paths run in sequence.  The helper stream and its
 *   events are created once per device on first use (default priority) and
 *   kept until the process ends.  Calls from several host threads (on
 *   different streams, with different workspaces) are safe: a lock keeps
 *   each call's enqueue sequence on the shared helper stream whole, and the
 *   helper-stream work of concurrent calls runs one after the other.
 * In : Q, K, V, Wq, Wk, alpha as sla2_route / sla2_forward.
 * Out: topk_idx [B,H,T_q,k] (NULL allowed when k = 0); O as sla2_forward.
 * ws : sla2_workspace_bytes(p, SLA2_OP_ATTENTION) bytes.
 */
sla2_status sla2_attention(const sla2_problem* p, const void* Q, const void* K, const void* V,
                           const float* Wq, const float* Wk, const float* alpha,
                           int32_t* topk_idx, void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_attention_noalloc -- for callers that cannot allocate device memory
 *   or create HIP objects (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid allocation): sla2_attention with no workspace
 *   argument.  Its workspace is a file-scope device array of the library,
 *   sla2_noalloc_scratch_bytes() = 64 MiB, one copy on each GPU the library
 *   runs on, held until the process ends (addressed once per device, on the
 *   first call there).  Everything is enqueued on `stream`, in order (no
 *   helper stream, no events); the call itself allocates nothing.  Same
 *   results as sla2_attention (bit-identical O and topk_idx).
 *   Limit: sla2_workspace_bytes(p, SLA2_OP_ATTENTION) <= 64 MiB (for example
 *   B = 1, H = 2, N = 8192, d = 128 uses about 17 MiB); larger problems
 *   return SLA2_EWORKSPACE and launch nothing.
 *   Calls on one GPU share the array: calls that overlap in time on that GPU
 *   (different streams, or threads) race on it and give undefined results;
 *   order them (one stream, or events) when using this entry point.
 * In / Out: as sla2_attention.
 */
sla2_status sla2_attention_noalloc(const sla2_problem* p, const void* Q, const void* K,
                                   const void* V, const float* Wq, const float* Wk,
                                   const float* alpha, int32_t* topk_idx, void* O,
                                   void* stream);
size_t sla2_noalloc_scratch_bytes(void);

/*
 * sla2_forward_fp8 -- as sla2_forward, with the low-bit sparse branch
 * ("SLA2 深度解读" 07).  Requires dtype == SLA2_BF16, bq == 128 and d == 128
 * (SLA2_EUNSUPPORTED otherwise).
 *   mu = mean of K over the N valid tokens (per head, per channel; summed in
 *   fp64, rounded to fp32); K' = K - mu (fp32);
 *   s_K(j) = max|K'| over KV block j / 448, s_Q(i) = max|Q| over query block
 *   i / 448 (1 if the maximum is 0); Khat = e4m3(K' / s_K), Qhat = e4m3(Q /
 *   s_Q) (OCP e4m3, round to nearest even, saturating at 448);
 *   logits = (Qhat Khat^T) s_Q s_K / sqrt(d) on fp8 matrix cores;
 *   online softmax over the selected blocks in ascending block order, with
 *   P~ = exp(logit - running max) quantised as e4m3(256 P~) / 256 before
 *   P V (V unquantised, fp16) and the row sum taken over the quantised
 *   values.  Router and linear branch are those of sla2_forward.
 *   With bit 1 of lowbit set (SLA2_LOWBIT_I8QK, SLA2_LOWBIT_I8QKV) Q and K'
 *   take int8 codes instead: s = block max / 127, code = round-half-even(x /
 *   s) clamped to +-127 (fp32 division), and the logits are the exact int32
 *   dot products of the codes (int8 matrix cores) times s_Q s_K / sqrt(d).
 *   With bit 0 of lowbit set (SLA2_LOWBIT_QKV, SLA2_LOWBIT_I8QKV), V is
 *   quantised too: s_V(c) = max over the
 *   N valid tokens of |V(., c)| / 448 per head and channel (1 if 0), Vhat =
 *   e4m3(V / s_V) (fp32 division, round to nearest even, saturating), and
 *   P V runs on the e4m3 matrix cores as (256 P^) Vhat, scaled by s_V(c) per
 *   output channel; the linear branch keeps V in fp16.
 *   The fp8 matrix cores do not sum their products exactly (the error of a
 *   dot product reaches about 2^-15 of the sum of the absolute products), so
 *   a P~ lying that close to an e4m3 rounding midpoint may take either
 *   neighbouring code: results agree with an exact evaluation of the same
 *   steps up to such flips.
 * ws : sla2_workspace_bytes(p, SLA2_OP_FORWARD_FP8) bytes.
 */
sla2_status sla2_forward_fp8(const sla2_problem* p, const void* Q, const void* K,
                             const void* V, const int32_t* topk_idx, const float* alpha,
                             void* O, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_attention_fp8 -- sla2_route followed by sla2_forward_fp8 in one call
 *   (bit-identical O and topk_idx; same requirements as sla2_forward_fp8).
 *   The router's pooling pass also writes the query codes and the column
 *   sums of K per KV block, so Q is read once; the block summaries run on
 *   the helper stream of sla2_attention from the start, then (after the
 *   pooling pass, through an event) the K mean, the key codes and, with the
 *   low-bit V, the V codes, concurrently with the rest of the router; both
 *   streams join before the fused kernel.  The helper stream is shared with
 *   sla2_attention (the same conditions apply).
 * In : Q, K, V, Wq, Wk, alpha as sla2_route / sla2_forward_fp8.
 * Out: topk_idx [B,H,T_q,k] (NULL allowed when k = 0); O as sla2_forward_fp8.
 * ws : sla2_workspace_bytes(p, SLA2_OP_ATTENTION_FP8) bytes.
 */
sla2_status sla2_attention_fp8(const sla2_problem* p, const void* Q, const void* K,
                               const void* V, const float* Wq, const float* Wk,
                               const float* alpha, int32_t* topk_idx, void* O, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * sla2_quantize_fp8 -- the low-bit inputs alone (the quantisation step that
 * sla2_forward_fp8 runs first), for inspection.  Requires dtype == SLA2_BF16.
 * Out (device): Qhat [B,H,T_q*bq,d] and Khat [B,H,T_kv*bkv,d] e4m3 codes, or
 * int8 codes (two's complement) with bit 1 of lowbit set
 * (always head-major, whatever the layout of Q and K)
 * (rows past N are 0), s_Q [B,H,T_q], s_K [B,H,T_kv], mu [B,H,d] fp32.
 * ws : sla2_workspace_bytes(p, SLA2_OP_FORWARD_FP8) bytes.
 */
sla2_status sla2_quantize_fp8(const sla2_problem* p, const void* Q, const void* K,
                              uint8_t* Qhat, uint8_t* Khat, float* sQ, float* sK,
                              float* mu, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_quantize_v_fp8 -- the per-channel V quantisation of the fully low-bit
 * sparse branch alone (what sla2_forward_fp8 runs with lowbit ==
 * SLA2_LOWBIT_QKV), for inspection.  Requires dtype == SLA2_BF16, d == 128
 * and bit 0 of lowbit (SLA2_LOWBIT_QKV or SLA2_LOWBIT_I8QKV).
 * Out (device): Vhat [B,H,T_kv*bkv,d] e4m3 codes (head-major, rows past N are
 * 0), s_V [B,H,d] fp32.
 * ws : sla2_workspace_bytes(p, SLA2_OP_FORWARD_FP8) bytes.
 */
sla2_status sla2_quantize_v_fp8(const sla2_problem* p, const void* V, uint8_t* Vhat,
                                float* sV, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_fp8_dot_tiles -- diagnostic of the fp8 matrix cores the low-bit
 * logits run on: C[t] = A[t] B[t]^T for t < ntiles, A[t] and B[t] 32 x 128
 * OCP e4m3 codes (row-major, device), C[t] 32 x 32 fp32 (row-major), on the
 * same instruction and operand layout as sla2_forward_fp8's Q K^T (two
 * chained 32x32x64 products, unit scales).  The hardware does not sum the
 * 128 products exactly; the parity tests measure that error with this call.
 * Errors: SLA2_EINVAL for a null or misaligned pointer or ntiles outside
 * [1, 2^20].
 */
sla2_status sla2_fp8_dot_tiles(const uint8_t* A, const uint8_t* B, float* C, int32_t ntiles,
                               void* stream);

/*
 * sla2_mfma_rate_probe -- measurement aid: the matrix-core instruction rate
 * this GPU reaches, with no memory traffic.  groups work-groups of 4 waves;
 * every wave runs iters rounds of 4 independent products of one form: kind
 * 0 bf16 32x32x16 (32768 flop each), kind 1 e4m3 32x32x64 with unit scales
 * (131072 flop each), kind 2 bf16 16x16x32 (16384 flop each), kind 3 fp16
 * 32x32x16 (32768 flop each).  Total flop = groups * 4 * iters * 4 * (flop each);
 * the caller times the call (events on `stream`).  out: device fp32
 * [groups * 4], one value per wave (meaningless; keeps the work live).
 * Errors: SLA2_EINVAL for kind not in {0, 1, 2, 3}, iters outside [1, 2^24],
 * groups outside [1, 2^16], or a null or misaligned out.
 */
sla2_status sla2_mfma_rate_probe(int32_t kind, int32_t iters, int32_t groups, float* out,
                                 void* stream);

/*
 * Kernel timing (diagnostics, host-side state).  sla2_timing_start(n) makes
 * the library bracket each of its next n kernel launches with a pair of
 * hipEvents on the launch stream (the events are created here, not device
 * memory).  sla2_timing_stop() waits for those events and reports, per
 * kernel kind, the summed duration in ms and the launch count, then stops
 * recording.  Not thread-safe; meant for benchmarks.
 */
sla2_status sla2_timing_start(int32_t max_launches);
sla2_status sla2_timing_stop(float* total_ms, int32_t* launches, int32_t n_kinds);
int32_t sla2_kernel_kinds(void);
const char* sla2_kernel_name(int32_t kind);

/*
 * sla2_backward -- gradients of L = sum dO . O for sla2_forward with the
 *   selection topk_idx held fixed (the hard top-k has no gradient; "SLA2
 *   深度解读" 06 fine-tunes the model and alpha with it in Stage 2):
 *   sparse branch as FlashAttention's backward restricted to the selected
 *   tokens (p = exp(l - LSE), dl = p (alpha dO . v - alpha dO . O_s));
 *   linear branch through O_l = n / s with n = phi(q) H_i, s = phi(q) . Z_i,
 *   so that each block summary h_j, z_j collects the gradients of every
 *   query block that does not select it (evaluated as the head's total
 *   minus the selecting query blocks); dalpha = sum of dO . (O_s - O_l) over
 *   the rows alpha applies to.  Through phi (SLA notes, key design 4):
 *   dx = dphi * phi'(x) for elu + 1; for the row softmax p = phi(x), dx =
 *   p * (dphi - p . dphi).  bf16 inputs with d = bq = 128 and phi = elu + 1
 *   run on the matrix cores: the sparse passes with bf16 Q, K, V and every
 *   fp32 operand split into a bf16 high part and the bf16 rounding of the
 *   rest; the selected blocks' bf16 summaries (and the selecting query
 *   blocks' bf16 dH_i) summed by dense 0/1 products, fp32 accumulation; the
 *   linear passes' own products in fp32.  Every other problem (softmax phi
 *   included) in fp32 on the vector ALU.
 * In : Q, K, V, topk_idx, alpha as sla2_forward; dO fp32 in problem.layout.
 * Out: dQ, dK, dV fp32 in problem.layout; dalpha [H] or [H][T_q] fp32
 *      (problem.alpha_mode).  All overwritten.
 * ws : sla2_workspace_bytes(p, SLA2_OP_BACKWARD) bytes.
 */
sla2_status sla2_backward(const sla2_problem* p, const void* Q, const void* K, const void* V,
                          const int32_t* topk_idx, const float* alpha, const float* dO,
                          float* dQ, float* dK, float* dV, float* dalpha, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Training-time router ("SLA2 深度解读" 06, Stage 1: proj_q, proj_k and alpha
 * are fitted against full attention with a differentiable SoftTop-k in place
 * of the hard top-k; inference keeps the hard top-k).
 *
 * sla2_soft_topk -- M_ij = sigma(S_ij / tau + lambda_i) for the router scores
 *   S of sla2_route (same pooling, projections and fp64 arithmetic), with
 *   lambda_i found by bisection so that sum_j M_ij = k (k = sla2_topk(p)):
 *   f(lambda) = sum_j sigma(S_ij / tau + lambda) - k over the bracket
 *   [-max_j S_ij / tau - 50, -min_j S_ij / tau + 50], 100 halvings (stopped
 *   early once the midpoint equals an end of the bracket, after which no
 *   halving can move it), lambda = the final midpoint.  k = 0 gives M = 0 (lambda = -inf), k = T_kv M = 1
 *   (lambda = +inf).  The pages use tau = 0.1.
 * Out: M [B,H,T_q,T_kv] fp32; lambda [B,H,T_q] fp64, or NULL.
 * ws : sla2_workspace_bytes(p, SLA2_OP_ROUTE) bytes.  tau <= 0 or not finite:
 *      SLA2_EINVAL.
 */
sla2_status sla2_soft_topk(const sla2_problem* p, const void* Q, const void* K,
                           const float* Wq, const float* Wk, float tau, float* M,
                           double* lambda, void* ws, size_t ws_bytes, void* stream);

/*
 * sla2_soft_topk_grad -- dL/dS from dL/dM through SoftTop-k, lambda moving
 *   with S so that every row keeps its sum k: with s = M (1 - M),
 *   dS_ij = s_ij / tau * (dM_ij - sum_l dM_il s_il / sum_l s_il) (the second
 *   term 0 when sum_l s_il = 0).  fp64 arithmetic from the fp32 M and dM.
 * In : M (from sla2_soft_topk), dM [B,H,T_q,T_kv] fp32.  Out: dS, same shape.
 *      No workspace.
 */
sla2_status sla2_soft_topk_grad(const sla2_problem* p, const float* M, const float* dM,
                                float tau, float* dS, void* stream);

/*
 * sla2_route_grad -- dL/dWq and dL/dWk from dL/dS for the router scores
 *   S = (Qbar Wq[h']) (Kbar Wk[h'])^T: dqt = dS kt, dkt = dS^T qt,
 *   dWq = Qbar^T dqt, dWk = Kbar^T dkt per head, summed in head order over
 *   the heads that share a projection (w_heads == 1: all).  fp64 inside.
 * In : Q, K, Wq, Wk as sla2_route; dS [B,H,T_q,T_kv] fp32.
 * Out: dWq, dWk [w_heads,d,d] fp32 (overwritten).
 * ws : sla2_workspace_bytes(p, SLA2_OP_ROUTE_GRAD) bytes.
 */
sla2_status sla2_route_grad(const sla2_problem* p, const void* Q, const void* K,
                            const float* Wq, const float* Wk, const float* dS, float* dWq,
                            float* dWk, void* ws, size_t ws_bytes, void* stream);

/*
 * SLA (v1) compatibility ("SLA: Beyond Sparsity ..." notes: key design 2,
 * the three-way block classification; key design 3, the linear branch over
 * the marginal blocks and O = O_s + Proj(O_l); training section: phi =
 * softmax, k_h = 5 %, k_l = 10 %).  Same problem struct: topk_frac is k_h %,
 * low_frac (an argument) is k_l %, problem.phi picks the feature map;
 * w_heads applies to W_p; alpha_mode and lowbit are not used.
 *
 * sla1_num_negligible -- k_l = clamp(ceil(low_frac * T_kv - 1e-6), 0,
 * T_kv - k_h), k_h = sla2_topk(p).  -1 if the problem is invalid or low_frac
 * is outside [0,1].
 */
int32_t sla1_num_negligible(const sla2_problem* p, float low_frac);

/*
 * sla1_route -- ternary router.  Pools as sla2_route but without
 * projections (P_c = softmax(Qbar Kbar^T / sqrt(d)) keeps the row order of
 * the plain product Qbar . Kbar, computed in fp64).  One total order per row:
 * score descending, then block index ascending; its first k_h blocks are
 * critical, its last k_l negligible (so ties at the negligible cut drop the
 * higher index), the rest marginal.
 * In : Q, K (dtype, problem.layout).
 * Out: crit_idx [B,H,T_q,k_h] and negl_idx [B,H,T_q,k_l] int32, rows
 *      ascending (either may be NULL when its count is 0); block_mask
 *      [B,H,T_q,T_kv] int8 stored as uint8: 1 critical, 0 marginal, 0xFF (-1)
 *      negligible, or NULL.
 * ws : sla2_workspace_bytes(p, SLA2_OP_ROUTE) bytes.
 * Errors as sla2_route; low_frac outside [0,1] or NaN is SLA2_EINVAL.
 */
sla2_status sla1_route(const sla2_problem* p, const void* Q, const void* K, float low_frac,
                       int32_t* crit_idx, int32_t* negl_idx, uint8_t* block_mask, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * sla1_forward -- SLA (v1) forward.  Takes the shapes sla2_forward takes:
 * bf16 with d = bq = 128 on the matrix cores; bq = 64 (the notes' b_q = b_kv
 * = 64), d = 64 or fp32 inputs on the vector ALU in fp32.
 *   O_s: the sparse branch of sla2_forward over the critical blocks.
 *   O_l: phi(Q_t) H_i / (phi(Q_t) . Z_i) with H_i, Z_i summed over the
 *        marginal blocks (neither critical nor negligible): directly on the
 *        matrix-core path, as the totals minus the critical and the
 *        negligible blocks on the vector ALU; O_l = 0 when no block is
 *        marginal.
 *   O  = O_s + O_l W_p[h'] (Proj(x) = x W_p, W_p row-major [d][d], no bias;
 *        h' = 0 if w_heads == 1, else h).  On the matrix-core path O_l enters
 *        the projection on the fp16 matrix cores as the sum of two fp16 terms
 *        (high part + rest), W_p rounded to fp16; fp32 on the vector ALU.
 * In : Q, K, V (dtype, problem.layout); crit_idx / negl_idx from sla1_route
 *      (ascending rows; NULL allowed when the count is 0); Wp [w_heads,d,d]
 *      fp32.
 * Out: O in problem.layout, fp32 or bf16 (problem.out_dtype).
 * ws : sla2_workspace_bytes(p, SLA2_OP_SLA1_FORWARD) bytes.
 * Precision as sla2_forward's path for the same shape; phi = softmax is
 * evaluated in fp32 (max-subtracted), and carried in fp16 on the matrix-core
 * path.
 */
sla2_status sla1_forward(const sla2_problem* p, const void* Q, const void* K, const void* V,
                         const int32_t* crit_idx, const int32_t* negl_idx, float low_frac,
                         const float* Wp, void* O, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA2_H */
