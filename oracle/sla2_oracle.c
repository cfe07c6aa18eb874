/*
 * sla2_oracle.c -- plain, slow CPU reference of the SLA2 forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU library never links,
 * includes or calls it, and it shares no source with the GPU path.
 *
 * All floating point is fp64 (inputs converted exactly from fp32 / bf16),
 * except where a float decides an integer code in the low-bit variant: there
 * the code is decided in fp32, the precision the GPU kernel uses (see
 * orc_quant_fp8 and the P quantisation in orc_forward_fp8).
 *
 * Sources (the pages; section names as printed on them):
 *  [SLA2-zh] "SLA2 深度解读" (jefxiong.cn): 04 (P = softmax(QK^T/sqrt d),
 *            P1 = P.M, alpha = P1 1, O = alpha O_s + (1-alpha) O_l),
 *            05 (pool, proj_q / proj_k, P_c, hard Top-k, b_q=128, b_kv=64),
 *            07 (low-bit Q/K and P, K column-mean smoothing, online softmax
 *            over mask-hit blocks only), 08 (what runs for hit / missed blocks).
 *  [SLA-zh]  "SLA: Beyond Sparsity ..." notes (papernotes.org), key design 2
 *            (P_c = softmax(pool(Q) pool(K)^T / sqrt d); per row the top k_h %
 *            of blocks critical, the bottom k_l % negligible, the rest
 *            marginal), key design 3 (H_i, Z_i over the marginal blocks,
 *            O_i^l = phi(Q_i) H_i / phi(Q_i) Z_i, O = O^s + Proj(O^l)), key
 *            design 4 (per-block h_j = phi(K_j)^T V_j and z_j, H_i += h_j),
 *            and the training-strategy section (phi = softmax, k_h = 5 %,
 *            k_l = 10 %).
 *  [SLA2-en] gist.science explainer, section 2A (O = alpha O_s + (1-alpha) O_l,
 *            both branches row-normalised).
 *  [SLA2-zh] 06 also gives the training-time router: SoftTop-k(P_c)_ij =
 *            sigma((P_c)_ij / tau + lambda_i), tau = 0.1, lambda_i found by
 *            bisection so that each row's soft selections sum to the budget.
 *
 * Readings where the pages are silent or ambiguous:
 *  - router score is the plain product proj_q(Qbar) . proj_k(Kbar), no 1/sqrt(d)
 *    and no softmax (both are monotone per row and cannot change a hard top-k);
 *  - proj(x) = x W, no bias; W is [w_heads][d][d] row-major, w_heads in {1,H};
 *  - k = clamp(ceil(frac * T_kv - 1e-6), 0, T_kv); ties broken by lower index;
 *  - tokens beyond N in a ragged last block are excluded everywhere (means
 *    divide by the valid count, no logit, no phi term);
 *  - phi = elu + 1 elementwise on raw Q and K, or (phi = 1) softmax over the
 *    d channels of each raw Q or K row;
 *  - SLA (v1) mode (mode = 1): the router pools without projections (the
 *    softmax and 1/sqrt d of P_c keep the row order of the plain product);
 *    one total order per row, score descending then index ascending: the
 *    first k_h blocks are critical, the last k_l negligible, k_h as k above
 *    and k_l = clamp(ceil(low_frac * T_kv - 1e-6), 0, T_kv - k_h); the
 *    sparse branch runs over the critical blocks, the linear branch over the
 *    marginal ones (neither critical nor negligible), O = O_s + O_l W_p with
 *    W_p [w_heads][d][d] (Proj = x W_p, no bias, like the router's
 *    projections); alpha is not used;
 *  - empty selected set -> O_s = 0; empty unselected set -> O_l = 0;
 *  - alpha is per head, or per head and query block (the algorithm's
 *    granularity; alpha_mode 1);
 *  - low bit: OCP fp8 e4m3 (max 448), RNE, saturating; per-block absmax
 *    scales (Q: b_q tokens, K: b_kv tokens); K smoothed by its mean over the N
 *    valid tokens (sparse-branch QK^T only); P quantised as e4m3(256 P~)/256
 *    with P~ = exp(l - running max) and the row sum taken over the quantised
 *    values; tiles visited in ascending KV-block order; V stays bf16, or
 *    (lowbit_v) is quantised as well: s_V(c) = max over the N valid tokens
 *    of |V(.,c)| / 448 per head and channel (1 if 0), Vhat = e4m3(V / s_V),
 *    and P V uses Vhat s_V -- the pages quantise P and V for P V;
 *  - backward (SLA2 mode, exact sparse branch, the hard selection held
 *    fixed): the chain rule through O = alpha O_s + (1 - alpha) O_l --
 *    softmax attention over the selected tokens for O_s, and for O_l the
 *    linear branch's H_i, Z_i summed over the unselected blocks, so that
 *    block j's summary h_j, z_j receives the gradients of every query block
 *    that does not select it; alpha's gradient is summed over its rows;
 *  - SoftTop-k: the budget is the hard router's k; lambda_i by bisection on
 *    f(lambda) = sum_j sigma(S_ij / tau + lambda) - k over the bracket
 *    [-max_j S_ij / tau - 50, -min_j S_ij / tau + 50], a fixed 100 halvings,
 *    lambda = the final midpoint; k = 0 gives M = 0 (lambda = -inf) and
 *    k = T_kv gives M = 1 (lambda = +inf); its gradient is the implicit one
 *    (lambda moves so that the row sum stays k), evaluated from the mask M;
 *  - the pages allow INT8 or FP8 for Q K^T: with int8_qk the Q and smoothed K
 *    codes are int8, s = absmax / 127 per block (1 if 0), code =
 *    round-half-even(x / s) clamped to +-127, and the dot products of the
 *    codes are exact integers.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int32_t B, H, N, d;
    int32_t bq, bkv;
    float topk_frac;
    int32_t w_heads;
    int32_t dtype; /* 0: Q,K,V are float32; 1: Q,K,V are bf16 bit patterns */
    int32_t alpha_mode; /* 0: alpha [H]; 1: alpha [H][T_q], one per query block */
    int32_t lowbit_v;   /* low-bit variant: 1 = V also quantised (per channel) */
    int32_t int8_qk;    /* low-bit variant: 1 = Q, K as int8 codes (else e4m3) */
    int32_t phi;        /* 0: elu + 1; 1: softmax over the d channels of a row */
    int32_t mode;       /* 0: SLA2; 1: SLA (v1), ternary blocks and Proj combine */
    float low_frac;     /* v1: fraction of negligible blocks per row */
} orc_problem;

/* ------------------------------------------------------------------ */
/* small helpers                                                       */
/* ------------------------------------------------------------------ */
static int ceil_div(int a, int b) { return (a + b - 1) / b; }

int orc_num_blocks(int n, int b) { return ceil_div(n, b); }

/* step 5 reading: k = clamp(ceil(frac * T_kv - 1e-6), 0, T_kv) */
int orc_topk(const orc_problem* p) {
    int tkv = ceil_div(p->N, p->bkv);
    double k = ceil((double)p->topk_frac * (double)tkv - 1e-6);
    if (k < 0) k = 0;
    if (k > tkv) k = tkv;
    return (int)k;
}

/* v1: k_l = clamp(ceil(low_frac * T_kv - 1e-6), 0, T_kv - k_h); 0 in SLA2 mode */
int orc_topk_low(const orc_problem* p) {
    if (p->mode != 1) return 0;
    int tkv = ceil_div(p->N, p->bkv);
    double k = ceil((double)p->low_frac * (double)tkv - 1e-6);
    int kh = orc_topk(p);
    if (k < 0) k = 0;
    if (k > tkv - kh) k = tkv - kh;
    return (int)k;
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* element (bh, t, c) of a [B*H][N][d] input */
static double elem(const orc_problem* p, const void* X, long bh, long t, long c) {
    size_t off = ((size_t)bh * p->N + t) * p->d + c;
    if (p->dtype == 0) return (double)((const float*)X)[off];
    return bf16_to_double(((const uint16_t*)X)[off]);
}

/* phi = elu + 1: x + 1 for x > 0, exp(x) otherwise */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* phi of row t of X (head bh): elu + 1 per element, or the softmax of the
   row over its d channels */
static void phi_row(const orc_problem* p, const void* X, long bh, long t, double* out) {
    int d = p->d;
    if (p->phi == 0) {
        for (int c = 0; c < d; ++c) out[c] = phi(elem(p, X, bh, t, c));
        return;
    }
    double m = -INFINITY, s = 0.0;
    for (int c = 0; c < d; ++c) {
        out[c] = elem(p, X, bh, t, c);
        if (out[c] > m) m = out[c];
    }
    for (int c = 0; c < d; ++c) {
        out[c] = exp(out[c] - m);
        s += out[c];
    }
    for (int c = 0; c < d; ++c) out[c] /= s;
}

/* ------------------------------------------------------------------ */
/* OCP fp8 E4M3 (bias 7, no infinities, S.1111.111 = NaN, max 448)      */
/* ------------------------------------------------------------------ */
float orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);          /* subnormal: m/8 * 2^-6 */
    else v = ldexpf((float)(8 + m), e - 10);       /* (1 + m/8) * 2^(e-7)   */
    return s ? -v : v;
}

/* Round-to-nearest-even onto the e4m3 grid, saturating at +-448.
 * Works on the exact value of the fp32 input: the grid spacing in the binade
 * [2^e, 2^(e+1)) is 2^(e-3) for e >= -6, and 2^-9 below 2^-6. */
uint8_t orc_e4m3_encode(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7E;
    int e;
    frexp(a, &e);             /* a = f * 2^e, f in [0.5,1) -> binade 2^(e-1) */
    int be = e - 1;
    if (be < -6) be = -6;     /* subnormal range shares the 2^-9 spacing */
    double q = ldexp(1.0, be - 3);
    double n = a / q;         /* exact: scaling by a power of two */
    double r = floor(n);
    double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double v = r * q;
    if (v > 448.0) v = 448.0;
    /* encode v exactly */
    if (v == 0.0) return sign;
    int ve;
    double vf = frexp(v, &ve);           /* v = vf * 2^ve */
    int E = ve - 1 + 7;                  /* biased exponent of 1.m form */
    if (E <= 0) {                        /* subnormal: v = m * 2^-9 */
        int m = (int)llround(v / ldexp(1.0, -9));
        return sign | (uint8_t)m;
    }
    int m = (int)llround((vf * 2.0 - 1.0) * 8.0);
    return sign | (uint8_t)((E << 3) | m);
}

/* Round-half-to-even onto the integers, saturating at +-127: the int8 codes
 * of the int8 Q K^T variant, decided on the exact fp32 quotient. */
int8_t orc_i8_encode(float x) {
    double a = (double)x;
    double r = floor(a);
    double frac = a - r;
    if (frac > 0.5 || (frac == 0.5 && ((long long)r & 1) != 0)) r += 1.0;
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (int8_t)r;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs) */
uint16_t orc_bf16_encode(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* a tiny work pool                                                    */
/* ------------------------------------------------------------------ */
typedef void (*work_fn)(void* ctx, long item);
typedef struct {
    work_fn fn;
    void* ctx;
    long n;
    long next;
    pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* P = (pool_t*)arg;
    for (;;) {
        pthread_mutex_lock(&P->mu);
        long it = P->next++;
        pthread_mutex_unlock(&P->mu);
        if (it >= P->n) break;
        P->fn(P->ctx, it);
    }
    return NULL;
}

static int resolve_threads(int nthreads) {
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static void run_pool(work_fn fn, void* ctx, long n, int nthreads) {
    pool_t P = {fn, ctx, n, 0, PTHREAD_MUTEX_INITIALIZER};
    int nt = resolve_threads(nthreads);
    if (nt > n) nt = (int)n;
    if (nt <= 1) {
        for (long i = 0; i < n; ++i) fn(ctx, i);
        return;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nt);
    for (int i = 0; i < nt; ++i) pthread_create(&th[i], NULL, pool_worker, &P);
    for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
    free(th);
}

/* ------------------------------------------------------------------ */
/* Router: pool -> project -> score -> hard top-k  ([SLA2-zh] 05)      */
/* ------------------------------------------------------------------ */
typedef struct {
    double s;
    int j;
} scored_t;

static int cmp_scored(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1; /* larger score first */
    if (x->s < y->s) return 1;
    return x->j - y->j;         /* equal scores: lower index first */
}

typedef struct {
    const orc_problem* p;
    const void *Q, *K;
    const float *Wq, *Wk;
    const int32_t* heads;
    int32_t* idx;
    uint8_t* mask;
    double* gap_rel;
    double* scores; /* optional [B*H][Tq][Tkv] */
    int32_t* nidx;  /* v1: negligible blocks [B*H][Tq][k_l] (optional) */
} route_ctx;

/* mean of the valid rows of block `blk` (size bs) of head bh, in fp64 */
static void pool_block(const orc_problem* p, const void* X, long bh, int blk, int bs,
                       double* out) {
    int d = p->d;
    int t0 = blk * bs;
    int n = p->N - t0 < bs ? p->N - t0 : bs;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int t = t0; t < t0 + n; ++t)
        for (int c = 0; c < d; ++c) out[c] += elem(p, X, bh, t, c);
    for (int c = 0; c < d; ++c) out[c] /= (double)n;
}

/* y = x W  with W [d][d] row-major (W[c][e]) */
static void project(int d, const double* x, const float* W, double* y) {
    for (int e = 0; e < d; ++e) y[e] = 0.0;
    for (int c = 0; c < d; ++c)
        for (int e = 0; e < d; ++e) y[e] += x[c] * (double)W[(size_t)c * d + e];
}

static void route_head(void* vctx, long item) {
    route_ctx* C = (route_ctx*)vctx;
    const orc_problem* p = C->p;
    long bh = C->heads[item];
    int h = (int)(bh % p->H);
    int d = p->d;
    int Tq = ceil_div(p->N, p->bq), Tkv = ceil_div(p->N, p->bkv);
    int k = orc_topk(p);
    int kl = orc_topk_low(p);
    const int v1 = p->mode == 1; /* no projections in the v1 router */
    const float* Wq = v1 ? NULL : C->Wq + (p->w_heads == 1 ? 0 : (size_t)h * d * d);
    const float* Wk = v1 ? NULL : C->Wk + (p->w_heads == 1 ? 0 : (size_t)h * d * d);

    double* bar = (double*)malloc(sizeof(double) * d);
    double* qt = (double*)malloc(sizeof(double) * (size_t)Tq * d);
    double* kt = (double*)malloc(sizeof(double) * (size_t)Tkv * d);
    scored_t* row = (scored_t*)malloc(sizeof(scored_t) * Tkv);

    /* step 2 (pool) and step 3 (project) */
    for (int i = 0; i < Tq; ++i) {
        pool_block(p, C->Q, bh, i, p->bq, bar);
        if (v1) memcpy(qt + (size_t)i * d, bar, sizeof(double) * d);
        else project(d, bar, Wq, qt + (size_t)i * d);
    }
    for (int j = 0; j < Tkv; ++j) {
        pool_block(p, C->K, bh, j, p->bkv, bar);
        if (v1) memcpy(kt + (size_t)j * d, bar, sizeof(double) * d);
        else project(d, bar, Wk, kt + (size_t)j * d);
    }
    for (int i = 0; i < Tq; ++i) {
        /* step 4: compressed score row P_c[i, :] */
        double smax = 0.0;
        for (int j = 0; j < Tkv; ++j) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += qt[(size_t)i * d + e] * kt[(size_t)j * d + e];
            row[j].s = s;
            row[j].j = j;
            if (fabs(s) > smax) smax = fabs(s);
            if (C->scores) C->scores[((size_t)bh * Tq + i) * Tkv + j] = s;
        }
        /* step 5: hard top-k, ties to the lower index */
        qsort(row, Tkv, sizeof(scored_t), cmp_scored);
        uint8_t* mrow = C->mask ? C->mask + ((size_t)bh * Tq + i) * Tkv : NULL;
        if (mrow) memset(mrow, 0, Tkv);
        for (int r = 0; r < k; ++r)
            if (mrow) mrow[row[r].j] = 1;
        /* v1: the last k_l blocks of the order are negligible (mask -1) */
        for (int r = Tkv - kl; r < Tkv; ++r)
            if (mrow) mrow[row[r].j] = 0xFF;
        if (C->nidx && kl > 0) {
            int32_t* nrow = C->nidx + ((size_t)bh * Tq + i) * kl;
            uint8_t* tmp = (uint8_t*)calloc(Tkv, 1);
            for (int r = Tkv - kl; r < Tkv; ++r) tmp[row[r].j] = 1;
            int w = 0;
            for (int j = 0; j < Tkv; ++j)
                if (tmp[j]) nrow[w++] = j;
            free(tmp);
        }
        /* emit selected indices ascending */
        if (C->idx) {
            int32_t* irow = C->idx + ((size_t)bh * Tq + i) * k;
            int w = 0;
            /* a mask-ordered walk gives ascending order */
            uint8_t* tmp = (uint8_t*)calloc(Tkv, 1);
            for (int r = 0; r < k; ++r) tmp[row[r].j] = 1;
            for (int j = 0; j < Tkv; ++j)
                if (tmp[j]) irow[w++] = j;
            free(tmp);
        }
        /* step 10: margin between the k-th and (k+1)-th scores */
        if (C->gap_rel) {
            double g = 1.0;
            if (k > 0 && k < Tkv) {
                double gap = row[k - 1].s - row[k].s;
                g = smax > 0.0 ? gap / smax : 0.0;
            }
            if (kl > 0 && kl + k < Tkv) { /* v1: also the negligible cut */
                double gap = row[Tkv - kl - 1].s - row[Tkv - kl].s;
                double gl = smax > 0.0 ? gap / smax : 0.0;
                if (gl < g) g = gl;
            }
            C->gap_rel[(size_t)bh * Tq + i] = g;
        }
    }
    free(bar);
    free(qt);
    free(kt);
    free(row);
}

/* Route the listed heads (bh = b*H + h).  idx: [B*H][Tq][k] (ascending),
 * mask: [B*H][Tq][Tkv] (0/1), gap_rel: [B*H][Tq], scores: optional.
 * Returns k. */
int orc_route(const orc_problem* p, const void* Q, const void* K, const float* Wq,
              const float* Wk, const int32_t* heads, int n_heads, int32_t* idx,
              uint8_t* mask, double* gap_rel, double* scores, int nthreads) {
    route_ctx C = {p, Q, K, Wq, Wk, heads, idx, mask, gap_rel, scores, NULL};
    run_pool(route_head, &C, n_heads, nthreads);
    return orc_topk(p);
}

/* SLA (v1) router (p->mode == 1): idx [B*H][Tq][k_h] critical and nidx
 * [B*H][Tq][k_l] negligible blocks, both ascending; mask 1 / 0xFF (-1) / 0
 * for critical / negligible / marginal.  gap_rel: the smaller relative margin
 * of the two cuts.  Returns k_l, or -1 if p is not in v1 mode. */
int orc_route_v1(const orc_problem* p, const void* Q, const void* K, const int32_t* heads,
                 int n_heads, int32_t* idx, int32_t* nidx, uint8_t* mask, double* gap_rel,
                 double* scores, int nthreads) {
    if (p->mode != 1) return -1;
    route_ctx C = {p, Q, K, NULL, NULL, heads, idx, mask, gap_rel, scores, nidx};
    run_pool(route_head, &C, n_heads, nthreads);
    return orc_topk_low(p);
}

/* Gradient of the router scores S = proj_q(Qbar) proj_k(Kbar)^T with
 * respect to the projections ([SLA2-zh] 05, 06: Stage 1 trains proj_q and
 * proj_k): qt = Qbar Wq, kt = Kbar Wk, dqt = dS kt, dkt = dS^T qt,
 * dWq = Qbar^T dqt, dWk = Kbar^T dkt, summed over the heads that share a
 * projection.  dS [B*H][Tq][Tkv]; dWq, dWk [w_heads][d][d], overwritten. */
void orc_route_grad(const orc_problem* p, const void* Q, const void* K, const float* Wq,
                    const float* Wk, const double* dS, double* dWq, double* dWk) {
    int d = p->d, Tq = ceil_div(p->N, p->bq), Tkv = ceil_div(p->N, p->bkv);
    long nbh = (long)p->B * p->H;
    memset(dWq, 0, sizeof(double) * (size_t)p->w_heads * d * d);
    memset(dWk, 0, sizeof(double) * (size_t)p->w_heads * d * d);
    double* qb = (double*)malloc(sizeof(double) * (size_t)Tq * d);
    double* kb = (double*)malloc(sizeof(double) * (size_t)Tkv * d);
    double* qt = (double*)malloc(sizeof(double) * (size_t)Tq * d);
    double* kt = (double*)malloc(sizeof(double) * (size_t)Tkv * d);
    double* dq = (double*)malloc(sizeof(double) * (size_t)Tq * d);
    double* dk = (double*)malloc(sizeof(double) * (size_t)Tkv * d);
    for (long bh = 0; bh < nbh; ++bh) {
        int hw = p->w_heads == 1 ? 0 : (int)(bh % p->H);
        const float* wq = Wq + (size_t)hw * d * d;
        const float* wk = Wk + (size_t)hw * d * d;
        for (int i = 0; i < Tq; ++i) {
            pool_block(p, Q, bh, i, p->bq, qb + (size_t)i * d);
            project(d, qb + (size_t)i * d, wq, qt + (size_t)i * d);
        }
        for (int j = 0; j < Tkv; ++j) {
            pool_block(p, K, bh, j, p->bkv, kb + (size_t)j * d);
            project(d, kb + (size_t)j * d, wk, kt + (size_t)j * d);
        }
        const double* g = dS + (size_t)bh * Tq * Tkv;
        memset(dq, 0, sizeof(double) * (size_t)Tq * d);
        memset(dk, 0, sizeof(double) * (size_t)Tkv * d);
        for (int i = 0; i < Tq; ++i)
            for (int j = 0; j < Tkv; ++j) {
                double gij = g[(size_t)i * Tkv + j];
                for (int e = 0; e < d; ++e) {
                    dq[(size_t)i * d + e] += gij * kt[(size_t)j * d + e];
                    dk[(size_t)j * d + e] += gij * qt[(size_t)i * d + e];
                }
            }
        double* gq = dWq + (size_t)hw * d * d;
        double* gk = dWk + (size_t)hw * d * d;
        for (int c = 0; c < d; ++c)
            for (int e = 0; e < d; ++e) {
                double a = 0.0, b = 0.0;
                for (int i = 0; i < Tq; ++i) a += qb[(size_t)i * d + c] * dq[(size_t)i * d + e];
                for (int j = 0; j < Tkv; ++j) b += kb[(size_t)j * d + c] * dk[(size_t)j * d + e];
                gq[(size_t)c * d + e] += a;
                gk[(size_t)c * d + e] += b;
            }
    }
    free(qb);
    free(kb);
    free(qt);
    free(kt);
    free(dq);
    free(dk);
}

/* ------------------------------------------------------------------ */
/* SoftTop-k ([SLA2-zh] 06, Stage 1)                                   */
/* ------------------------------------------------------------------ */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* rows of scores S [rows][Tkv] -> M = sigma(S / tau + lambda_row) with
 * sum_j M = k per row; lambda [rows] (+-inf at k = T_kv / 0). */
void orc_soft_topk_rows(const double* S, long rows, int Tkv, int k, double tau, double* M,
                        double* lambda) {
    for (long r = 0; r < rows; ++r) {
        const double* x = S + (size_t)r * Tkv;
        double* m = M + (size_t)r * Tkv;
        if (k <= 0 || k >= Tkv) {
            for (int j = 0; j < Tkv; ++j) m[j] = k <= 0 ? 0.0 : 1.0;
            lambda[r] = k <= 0 ? -INFINITY : INFINITY;
            continue;
        }
        double smax = -INFINITY, smin = INFINITY;
        for (int j = 0; j < Tkv; ++j) {
            if (x[j] / tau > smax) smax = x[j] / tau;
            if (x[j] / tau < smin) smin = x[j] / tau;
        }
        double lo = -smax - 50.0, hi = -smin + 50.0;
        for (int it = 0; it < 100; ++it) {
            double mid = 0.5 * (lo + hi), f = -(double)k;
            for (int j = 0; j < Tkv; ++j) f += sigmoid(x[j] / tau + mid);
            if (f > 0.0) hi = mid;
            else lo = mid;
        }
        double lam = 0.5 * (lo + hi);
        lambda[r] = lam;
        for (int j = 0; j < Tkv; ++j) m[j] = sigmoid(x[j] / tau + lam);
    }
}

/* Gradient through SoftTop-k: with s_j = M_j (1 - M_j) and lambda implicit
 * (sum_j M_j = k), dS_l = s_l / tau * (dM_l - sum_j dM_j s_j / sum_j s_j);
 * the second term is 0 when sum_j s_j = 0.  M and dM fp32 (as the mask is
 * stored), arithmetic fp64. */
void orc_soft_topk_grad_rows(const float* M, const float* dM, long rows, int Tkv, double tau,
                             double* dS) {
    for (long r = 0; r < rows; ++r) {
        const float* m = M + (size_t)r * Tkv;
        const float* g = dM + (size_t)r * Tkv;
        double a = 0.0, b = 0.0;
        for (int j = 0; j < Tkv; ++j) {
            double sj = (double)m[j] * (1.0 - (double)m[j]);
            a += (double)g[j] * sj;
            b += sj;
        }
        double c = b > 0.0 ? a / b : 0.0;
        for (int j = 0; j < Tkv; ++j) {
            double sj = (double)m[j] * (1.0 - (double)m[j]);
            dS[(size_t)r * Tkv + j] = sj / tau * ((double)g[j] - c);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Per-KV-block linear summaries  ([SLA-zh] key design 4)              */
/*   h_j = sum_{u in block j} phi(K_u)^T V_u   (d x d)                  */
/*   z_j = sum_{u in block j} phi(K_u)          (d)                     */
/* ------------------------------------------------------------------ */
typedef struct {
    const orc_problem* p;
    const void *K, *V;
    long bh;
    double* h; /* [Tkv][d][d] */
    double* z; /* [Tkv][d] */
} summ_ctx;

static void summary_block(void* vctx, long j) {
    summ_ctx* S = (summ_ctx*)vctx;
    const orc_problem* p = S->p;
    int d = p->d;
    double* h = S->h + (size_t)j * d * d;
    double* z = S->z + (size_t)j * d;
    double* pk = (double*)malloc(sizeof(double) * d);
    double* vv = (double*)malloc(sizeof(double) * d);
    memset(h, 0, sizeof(double) * d * d);
    memset(z, 0, sizeof(double) * d);
    int t0 = (int)j * p->bkv;
    int n = p->N - t0 < p->bkv ? p->N - t0 : p->bkv;
    for (int u = t0; u < t0 + n; ++u) {
        phi_row(p, S->K, S->bh, u, pk);
        for (int e = 0; e < d; ++e) vv[e] = elem(p, S->V, S->bh, u, e);
        for (int c = 0; c < d; ++c) {
            z[c] += pk[c];
            for (int e = 0; e < d; ++e) h[(size_t)c * d + e] += pk[c] * vv[e];
        }
    }
    free(pk);
    free(vv);
}

/* ------------------------------------------------------------------ */
/* Backward of the SLA2 forward (hard selection fixed)                  */
/* ------------------------------------------------------------------ */
/* dx from dphi for row t of X: elu + 1 has phi' = 1 (x > 0) or exp(x);
   softmax has dx = phi (dphi - phi . dphi) */
static void phi_row_backward(const orc_problem* p, const void* X, long bh, long t,
                             const double* ph, const double* dph, double* dx) {
    int d = p->d;
    if (p->phi == 0) {
        for (int c = 0; c < d; ++c) {
            double x = elem(p, X, bh, t, c);
            dx[c] = dph[c] * (x > 0.0 ? 1.0 : exp(x));
        }
        return;
    }
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += ph[c] * dph[c];
    for (int c = 0; c < d; ++c) dx[c] = ph[c] * (dph[c] - dot);
}

typedef struct {
    const orc_problem* p;
    const void *Q, *K, *V;
    const int32_t* idx;
    const float* alpha;
    const double* dO;          /* [B*H][N][d] */
    double *dQ, *dK, *dV;      /* [B*H][N][d], accumulated (zeroed by the caller) */
    double* dalpha_part;       /* [B*H][Tq] per-(head, query block) partials */
} bwd_ctx;

static void backward_head(void* vctx, long bh) {
    bwd_ctx* C = (bwd_ctx*)vctx;
    const orc_problem* p = C->p;
    int d = p->d, N = p->N, Tq = ceil_div(N, p->bq), Tkv = ceil_div(N, p->bkv);
    int k = orc_topk(p), h = (int)(bh % p->H);
    double inv = 1.0 / sqrt((double)d);
    size_t dd = (size_t)d * d;
    double* hj = (double*)malloc(sizeof(double) * Tkv * dd);
    double* zj = (double*)malloc(sizeof(double) * Tkv * d);
    summ_ctx S = {p, C->K, C->V, bh, hj, zj};
    for (int j = 0; j < Tkv; ++j) summary_block(&S, j);
    double* dH = (double*)calloc((size_t)Tq * dd, sizeof(double));
    double* dZ = (double*)calloc((size_t)Tq * d, sizeof(double));
    uint8_t* hit = (uint8_t*)malloc((size_t)Tq * Tkv);
    double* Hi = (double*)malloc(sizeof(double) * dd);
    double* Zi = (double*)malloc(sizeof(double) * d);
    double* pq = (double*)malloc(sizeof(double) * d);
    double* os = (double*)malloc(sizeof(double) * d);
    double* olin = (double*)malloc(sizeof(double) * d);
    double* g = (double*)malloc(sizeof(double) * d);
    double* dq = (double*)malloc(sizeof(double) * d);
    double* dph = (double*)malloc(sizeof(double) * d);
    double* dx = (double*)malloc(sizeof(double) * d);
    double* dn = (double*)malloc(sizeof(double) * d);
    double* lw = (double*)malloc(sizeof(double) * ((size_t)k * p->bkv + 1));
    int n_unsel = Tkv - k;
    for (int i = 0; i < Tq; ++i) {
        const int32_t* sel = C->idx + ((size_t)bh * Tq + i) * k;
        uint8_t* hrow = hit + (size_t)i * Tkv;
        memset(hrow, 0, Tkv);
        for (int r = 0; r < k; ++r) hrow[sel[r]] = 1;
        memset(Hi, 0, sizeof(double) * dd);
        memset(Zi, 0, sizeof(double) * d);
        for (int j = 0; j < Tkv; ++j) {
            if (hrow[j]) continue;
            for (size_t x = 0; x < dd; ++x) Hi[x] += hj[(size_t)j * dd + x];
            for (int c = 0; c < d; ++c) Zi[c] += zj[(size_t)j * d + c];
        }
        double a = (double)(p->alpha_mode ? C->alpha[(size_t)h * Tq + i] : C->alpha[h]);
        int t0 = i * p->bq, nq = N - t0 < p->bq ? N - t0 : p->bq;
        for (int t = t0; t < t0 + nq; ++t) {
            const double* gt = C->dO + ((size_t)bh * N + t) * d;
            for (int e = 0; e < d; ++e) g[e] = gt[e];
            for (int e = 0; e < d; ++e) dq[e] = 0.0;
            /* forward of the row: sparse branch (two-pass softmax) */
            long nu = 0;
            double m = -INFINITY, l = 0.0;
            for (int r = 0; r < k; ++r) {
                int u0 = sel[r] * p->bkv, n = N - u0 < p->bkv ? N - u0 : p->bkv;
                for (int u = u0; u < u0 + n; ++u) {
                    double sc = 0.0;
                    for (int c = 0; c < d; ++c)
                        sc += elem(p, C->Q, bh, t, c) * elem(p, C->K, bh, u, c);
                    lw[nu++] = sc * inv;
                    if (sc * inv > m) m = sc * inv;
                }
            }
            for (long x = 0; x < nu; ++x) {
                lw[x] = exp(lw[x] - m);
                l += lw[x];
            }
            for (int e = 0; e < d; ++e) os[e] = 0.0;
            nu = 0;
            for (int r = 0; r < k; ++r) {
                int u0 = sel[r] * p->bkv, n = N - u0 < p->bkv ? N - u0 : p->bkv;
                for (int u = u0; u < u0 + n; ++u, ++nu) {
                    lw[nu] /= l; /* p_tu */
                    for (int e = 0; e < d; ++e) os[e] += lw[nu] * elem(p, C->V, bh, u, e);
                }
            }
            /* linear branch */
            phi_row(p, C->Q, bh, t, pq);
            double den = 0.0;
            for (int c = 0; c < d; ++c) den += Zi[c] * pq[c];
            for (int e = 0; e < d; ++e) {
                double num = 0.0;
                if (n_unsel > 0)
                    for (int c = 0; c < d; ++c) num += Hi[(size_t)c * d + e] * pq[c];
                olin[e] = n_unsel > 0 ? num / den : 0.0;
            }
            /* alpha: dO . (O_s - O_l) */
            double da = 0.0;
            for (int e = 0; e < d; ++e) da += g[e] * (os[e] - olin[e]);
            C->dalpha_part[(size_t)bh * Tq + i] += da;
            /* sparse branch: dO_s = a dO, D = dO_s . O_s, dl = p (dO_s . v - D) */
            double D = 0.0;
            for (int e = 0; e < d; ++e) D += a * g[e] * os[e];
            nu = 0;
            for (int r = 0; r < k; ++r) {
                int u0 = sel[r] * p->bkv, n = N - u0 < p->bkv ? N - u0 : p->bkv;
                for (int u = u0; u < u0 + n; ++u, ++nu) {
                    double dp = 0.0;
                    for (int e = 0; e < d; ++e) dp += a * g[e] * elem(p, C->V, bh, u, e);
                    double dl = lw[nu] * (dp - D);
                    double* dku = C->dK + ((size_t)bh * N + u) * d;
                    double* dvu = C->dV + ((size_t)bh * N + u) * d;
                    for (int c = 0; c < d; ++c) {
                        dq[c] += dl * elem(p, C->K, bh, u, c) * inv;
                        dku[c] += dl * elem(p, C->Q, bh, t, c) * inv;
                    }
                    for (int e = 0; e < d; ++e) dvu[e] += lw[nu] * a * g[e];
                }
            }
            /* linear branch: dn = (1-a) dO / den, ds = -((1-a) dO . O_l) / den */
            if (n_unsel > 0) {
                double dsv = 0.0;
                for (int e = 0; e < d; ++e) {
                    dn[e] = (1.0 - a) * g[e] / den;
                    dsv -= (1.0 - a) * g[e] * olin[e] / den;
                }
                for (int c = 0; c < d; ++c) {
                    double v = Zi[c] * dsv;
                    for (int e = 0; e < d; ++e) v += Hi[(size_t)c * d + e] * dn[e];
                    dph[c] = v;
                    for (int e = 0; e < d; ++e) dH[(size_t)i * dd + (size_t)c * d + e] += pq[c] * dn[e];
                    dZ[(size_t)i * d + c] += pq[c] * dsv;
                }
                phi_row_backward(p, C->Q, bh, t, pq, dph, dx);
                for (int c = 0; c < d; ++c) dq[c] += dx[c];
            }
            double* dqt = C->dQ + ((size_t)bh * N + t) * d;
            for (int c = 0; c < d; ++c) dqt[c] += dq[c];
        }
    }
    /* block summaries: dh_j, dz_j gather every query block not selecting j */
    double* dhj = (double*)malloc(sizeof(double) * dd);
    double* dzj = (double*)malloc(sizeof(double) * d);
    double* pk = (double*)malloc(sizeof(double) * d);
    for (int j = 0; j < Tkv; ++j) {
        memset(dhj, 0, sizeof(double) * dd);
        memset(dzj, 0, sizeof(double) * d);
        for (int i = 0; i < Tq; ++i) {
            if (hit[(size_t)i * Tkv + j]) continue;
            for (size_t x = 0; x < dd; ++x) dhj[x] += dH[(size_t)i * dd + x];
            for (int c = 0; c < d; ++c) dzj[c] += dZ[(size_t)i * d + c];
        }
        int u0 = j * p->bkv, n = N - u0 < p->bkv ? N - u0 : p->bkv;
        for (int u = u0; u < u0 + n; ++u) {
            phi_row(p, C->K, bh, u, pk);
            double* dvu = C->dV + ((size_t)bh * N + u) * d;
            for (int e = 0; e < d; ++e) {
                double v = 0.0;
                for (int c = 0; c < d; ++c) v += pk[c] * dhj[(size_t)c * d + e];
                dvu[e] += v;
            }
            for (int c = 0; c < d; ++c) {
                double v = dzj[c];
                for (int e = 0; e < d; ++e) v += dhj[(size_t)c * d + e] * elem(p, C->V, bh, u, e);
                dph[c] = v;
            }
            phi_row_backward(p, C->K, bh, u, pk, dph, dx);
            double* dku = C->dK + ((size_t)bh * N + u) * d;
            for (int c = 0; c < d; ++c) dku[c] += dx[c];
        }
    }
    free(hj); free(zj); free(dH); free(dZ); free(hit); free(Hi); free(Zi); free(pq); free(os);
    free(olin); free(g); free(dq); free(dph); free(dx); free(dn); free(lw); free(dhj);
    free(dzj); free(pk);
}

/* Gradients of L = sum dO . O for the SLA2 forward with the selection idx
 * held fixed (exact sparse branch).  dO [B*H][N][d] fp64; dQ, dK, dV
 * [B*H][N][d] fp64 (overwritten); dalpha [H] or [H][Tq] (alpha_mode),
 * overwritten.  Returns 0, -2 if p is not in SLA2 mode. */
int orc_backward(const orc_problem* p, const void* Q, const void* K, const void* V,
                 const int32_t* idx, const float* alpha, const double* dO, double* dQ,
                 double* dK, double* dV, double* dalpha, int nthreads) {
    if (p->mode != 0) return -2;
    int d = p->d, N = p->N, Tq = ceil_div(N, p->bq);
    long nbh = (long)p->B * p->H;
    size_t n = (size_t)nbh * N * d;
    memset(dQ, 0, sizeof(double) * n);
    memset(dK, 0, sizeof(double) * n);
    memset(dV, 0, sizeof(double) * n);
    double* part = (double*)calloc((size_t)nbh * Tq, sizeof(double));
    bwd_ctx C = {p, Q, K, V, idx, alpha, dO, dQ, dK, dV, part};
    run_pool(backward_head, &C, nbh, nthreads);
    int na = p->alpha_mode ? p->H * Tq : p->H;
    for (int x = 0; x < na; ++x) dalpha[x] = 0.0;
    for (long bh = 0; bh < nbh; ++bh) {
        int h = (int)(bh % p->H);
        for (int i = 0; i < Tq; ++i)
            dalpha[p->alpha_mode ? (size_t)h * Tq + i : (size_t)h] += part[(size_t)bh * Tq + i];
    }
    free(part);
    return 0;
}

/* ------------------------------------------------------------------ */
/* low-bit inputs of one head (fp32 decisions, as the kernel takes them) */
/* ------------------------------------------------------------------ */
typedef struct {
    uint8_t* qh; /* [N][d] e4m3 codes (int8 codes with int8_qk) */
    uint8_t* kh; /* [N][d] */
    float* sq;   /* [Tq] */
    float* sk;   /* [Tkv] */
    float* mu;   /* [d] */
    uint8_t* vh; /* [N][d] e4m3 codes of V / s_V (lowbit_v only) */
    float* sv;   /* [d] per-channel V scales (lowbit_v only) */
} quant_t;

static float elemf(const orc_problem* p, const void* X, long bh, long t, long c) {
    return (float)elem(p, X, bh, t, c); /* exact: fp32 or bf16 inputs */
}

static void quant_head(const orc_problem* p, const void* Q, const void* K, long bh,
                       quant_t* o) {
    int d = p->d, N = p->N;
    int Tq = ceil_div(N, p->bq), Tkv = ceil_div(N, p->bkv);
    const float qmax = p->int8_qk ? 127.0f : 448.0f; /* largest code magnitude */
    /* K channel mean over the N valid tokens (column-mean smoothing,
       [SLA2-zh] 07): summed in fp64, rounded once to fp32 */
    for (int c = 0; c < d; ++c) {
        double s = 0.0;
        for (int t = 0; t < N; ++t) s += elem(p, K, bh, t, c);
        o->mu[c] = (float)(s / (double)N);
    }
    for (int j = 0; j < Tkv; ++j) {
        int t0 = j * p->bkv, n = N - t0 < p->bkv ? N - t0 : p->bkv;
        float amax = 0.0f;
        for (int t = t0; t < t0 + n; ++t)
            for (int c = 0; c < d; ++c) {
                float ks = elemf(p, K, bh, t, c) - o->mu[c];
                if (fabsf(ks) > amax) amax = fabsf(ks);
            }
        float s = amax > 0.0f ? amax / qmax : 1.0f;
        o->sk[j] = s;
        for (int t = t0; t < t0 + n; ++t)
            for (int c = 0; c < d; ++c) {
                float ks = elemf(p, K, bh, t, c) - o->mu[c];
                o->kh[(size_t)t * d + c] = p->int8_qk ? (uint8_t)orc_i8_encode(ks / s)
                                                      : orc_e4m3_encode(ks / s);
            }
    }
    for (int i = 0; i < Tq; ++i) {
        int t0 = i * p->bq, n = N - t0 < p->bq ? N - t0 : p->bq;
        float amax = 0.0f;
        for (int t = t0; t < t0 + n; ++t)
            for (int c = 0; c < d; ++c) {
                float x = elemf(p, Q, bh, t, c);
                if (fabsf(x) > amax) amax = fabsf(x);
            }
        float s = amax > 0.0f ? amax / qmax : 1.0f;
        o->sq[i] = s;
        for (int t = t0; t < t0 + n; ++t)
            for (int c = 0; c < d; ++c) {
                float x = elemf(p, Q, bh, t, c) / s;
                o->qh[(size_t)t * d + c] = p->int8_qk ? (uint8_t)orc_i8_encode(x)
                                                      : orc_e4m3_encode(x);
            }
    }
}

/* Per-channel V scales and codes of head bh (the fully low-bit variant:
   [SLA2-zh] 07 quantises P and V before P V).  The per-channel maximum is
   exact in fp32; the code is decided in fp32, as the kernel decides it. */
static void quant_v_head(const orc_problem* p, const void* V, long bh, quant_t* o) {
    int d = p->d, N = p->N;
    for (int c = 0; c < d; ++c) {
        float amax = 0.0f;
        for (int t = 0; t < N; ++t) {
            float v = fabsf(elemf(p, V, bh, t, c));
            if (v > amax) amax = v;
        }
        o->sv[c] = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    for (int t = 0; t < N; ++t)
        for (int c = 0; c < d; ++c)
            o->vh[(size_t)t * d + c] = orc_e4m3_encode(elemf(p, V, bh, t, c) / o->sv[c]);
}

/* Quantised V of head bh: vhat [N][d] codes, sv [d] scales. */
void orc_quant_v_fp8(const orc_problem* p, const void* V, long bh, uint8_t* vhat, float* sv) {
    quant_t o = {0};
    o.vh = vhat;
    o.sv = sv;
    quant_v_head(p, V, bh, &o);
}

/* Quantised inputs of head bh (step a4 of the low-bit variant). */
void orc_quant_fp8(const orc_problem* p, const void* Q, const void* K, long bh,
                   uint8_t* qhat, uint8_t* khat, float* sq, float* sk, float* mu) {
    quant_t o = {qhat, khat, sq, sk, mu, NULL, NULL};
    quant_head(p, Q, K, bh, &o);
}

/* ------------------------------------------------------------------ */
/* Forward for a list of query blocks                                  */
/* ------------------------------------------------------------------ */
typedef struct {
    const orc_problem* p;
    const void *Q, *K, *V;
    const int32_t* idx;
    const float* alpha;
    const int32_t* blocks; /* pairs (bh, i) */
    double* out;           /* [n_blocks][bq][d] */
    long bh;               /* head being processed */
    const long* items;     /* block-list positions belonging to this head */
    const double *h, *z;   /* this head's per-block summaries (or NULL) */
    int variant;           /* 0: bf16/fp32 sparse branch, 1: low bit */
    int quantize;          /* low bit: 1 = e4m3, 0 = identity quantiser */
    const quant_t* qt;     /* this head's quantised inputs (low bit) */
    double* bound;         /* low bit, optional: [n_blocks][bq] near-midpoint bound */
    double acc_eps;        /* relative accumulation error assumed for the bound */
    const int32_t* nidx;   /* v1: negligible blocks [B*H][Tq][k_l] */
    const float* Wp;       /* v1: Proj weights [w_heads][d][d] */
} fwd_ctx;

/* Ambiguous P-quantisation decisions.  A second implementation computes the
 * same logits with its own dot-product accumulation and exp(); when it sums
 * the products of a quantised dot product with a relative error of at most
 * acc_eps * sum|q^ k^|, the logit l_u and the running maximum m can each move
 * by that much (times the block scales), and 256 P~ = 256 exp(l_u - m) by the
 * sum of the two in relative terms, plus a few fp32 rounding steps.  A
 * decision whose input lies that close to an e4m3 rounding midpoint may be
 * taken the other way; it is recorded so that the effect of the other code on
 * the output row can be bounded. */
#define ORC_MAX_AMBIG 8192

typedef struct {
    int u;       /* token */
    double m;    /* running max (natural log units) when it was quantised */
    double step; /* distance to the neighbouring code value (256-scaled) */
} ambig_t;

/* V(u, e) as the low-bit P V sees it: the decoded code times the channel
   scale when V is quantised (and the quantiser is on), else V itself. */
static double v_lowbit(const fwd_ctx* F, long u, int e) {
    const orc_problem* p = F->p;
    if (p->lowbit_v && F->quantize)
        return (double)orc_e4m3_decode(F->qt->vh[(size_t)u * p->d + e]) * (double)F->qt->sv[e];
    return elem(p, F->V, F->bh, u, e);
}

/* Sparse branch, exact: O_s[t] = softmax(l) V over the selected tokens
   ([SLA2-zh] 04 and 08), as a two-pass max-subtracted softmax. */
static void sparse_exact(const fwd_ctx* F, int i, const int32_t* sel, int k, int t,
                         double* os, double* lbuf) {
    const orc_problem* p = F->p;
    int d = p->d;
    double inv = 1.0 / sqrt((double)d);
    for (int e = 0; e < d; ++e) os[e] = 0.0;
    if (k == 0) return;
    long nu = 0;
    double m = -INFINITY;
    for (int r = 0; r < k; ++r) {
        int t0 = sel[r] * p->bkv, n = p->N - t0 < p->bkv ? p->N - t0 : p->bkv;
        for (int u = t0; u < t0 + n; ++u) {
            double s = 0.0;
            for (int c = 0; c < d; ++c) s += elem(p, F->Q, F->bh, t, c) * elem(p, F->K, F->bh, u, c);
            s *= inv;
            lbuf[nu++] = s;
            if (s > m) m = s;
        }
    }
    double l = 0.0;
    nu = 0;
    for (int r = 0; r < k; ++r) {
        int t0 = sel[r] * p->bkv, n = p->N - t0 < p->bkv ? p->N - t0 : p->bkv;
        for (int u = t0; u < t0 + n; ++u) {
            double w = exp(lbuf[nu++] - m);
            l += w;
            for (int e = 0; e < d; ++e) os[e] += w * elem(p, F->V, F->bh, u, e);
        }
    }
    for (int e = 0; e < d; ++e) os[e] /= l;
    (void)i;
}

/* Sparse branch, low bit ([SLA2-zh] 07): quantised Q^K^T with per-block
   scales, online softmax over the selected tiles in ascending order, P
   quantised per tile against the running max, V unquantised. */
/* distance from f (> 0) to the nearest e4m3 rounding midpoint, and the
 * size of the code step across that midpoint */
static void e4m3_midpoint(float f, double* dist, double* step) {
    uint8_t c = orc_e4m3_encode(f);
    double v = orc_e4m3_decode(c);
    double best = INFINITY, st = 0.0;
    if (c > 0) {
        double lo = orc_e4m3_decode((uint8_t)(c - 1));
        double d = fabs((double)f - 0.5 * (lo + v));
        if (d < best) { best = d; st = v - lo; }
    }
    if (c < 0x7E) {
        double hi = orc_e4m3_decode((uint8_t)(c + 1));
        double d = fabs((double)f - 0.5 * (v + hi));
        if (d < best) { best = d; st = hi - v; }
    }
    *dist = best;
    *step = st;
}

static void sparse_lowbit(const fwd_ctx* F, int i, const int32_t* sel, int k, int t,
                          double* os, double* lbuf, double* bound) {
    const orc_problem* p = F->p;
    int d = p->d;
    double inv = 1.0 / sqrt((double)d);
    const quant_t* Qt = F->qt;
    for (int e = 0; e < d; ++e) os[e] = 0.0;
    if (bound) *bound = 0.0;
    if (k == 0) return;
    ambig_t* amb = bound ? (ambig_t*)malloc(sizeof(ambig_t) * ORC_MAX_AMBIG) : NULL;
    double abuf[512];
    int n_amb = 0;
    double m = -INFINITY, l = 0.0;
    double mA = 0.0; /* largest logit movement seen so far: bounds the max's */
    for (int r = 0; r < k; ++r) {
        int j = sel[r];
        int t0 = j * p->bkv, n = p->N - t0 < p->bkv ? p->N - t0 : p->bkv;
        double sc = (double)Qt->sq[i] * (double)Qt->sk[j] * inv;
        double mt = -INFINITY;
        for (int u = t0; u < t0 + n; ++u) {
            double s = 0.0, sa = 0.0;
            for (int c = 0; c < d; ++c) {
                double a, b;
                if (F->quantize && p->int8_qk) {
                    a = (double)(int8_t)Qt->qh[(size_t)t * d + c];
                    b = (double)(int8_t)Qt->kh[(size_t)u * d + c];
                } else if (F->quantize) {
                    a = orc_e4m3_decode(Qt->qh[(size_t)t * d + c]);
                    b = orc_e4m3_decode(Qt->kh[(size_t)u * d + c]);
                } else { /* identity quantiser: x / s exactly */
                    a = elem(p, F->Q, F->bh, t, c) / (double)Qt->sq[i];
                    b = (elem(p, F->K, F->bh, u, c) - (double)Qt->mu[c]) / (double)Qt->sk[j];
                }
                s += a * b;
                sa += fabs(a * b);
            }
            s *= sc;
            lbuf[u - t0] = s;
            abuf[u - t0] = F->acc_eps * sa * sc; /* how far l_u may move */
            if (s > mt) mt = s;
            if (abuf[u - t0] > mA) mA = abuf[u - t0];
        }
        double mn = mt > m ? mt : m;
        double resc = (m == -INFINITY) ? 0.0 : exp(m - mn);
        l *= resc;
        for (int e = 0; e < d; ++e) os[e] *= resc;
        for (int u = t0; u < t0 + n; ++u) {
            double pt = exp(lbuf[u - t0] - mn);
            double ph;
            if (F->quantize) {
                float f = (float)(256.0 * pt);
                ph = (double)orc_e4m3_decode(orc_e4m3_encode(f)) / 256.0;
                if (amb && f > 0.0f) {
                    double dist, step;
                    e4m3_midpoint(f, &dist, &step);
                    /* relative movement of 256 P~: logit and max, then the
                       fp32 rounding of the exponent argument (magnitude up
                       to |m| + 8 in log2 units) and of exp2 itself */
                    double win = abuf[u - t0] + mA +
                                 ldexp(fabs(mn) * 1.4426950408889634 + 16.0, -21) + ldexp(1.0, -21);
                    if (dist <= win * (double)f && n_amb < ORC_MAX_AMBIG) {
                        amb[n_amb].u = u;
                        amb[n_amb].m = mn;
                        amb[n_amb].step = step;
                        ++n_amb;
                    }
                }
            } else {
                ph = pt;
            }
            l += ph;
            for (int e = 0; e < d; ++e) os[e] += ph * v_lowbit(F, u, e);
        }
        m = mn;
    }
    for (int e = 0; e < d; ++e) os[e] /= l;
    if (amb) {
        /* moving one ambiguous P^ by its code step changes O_s by at most
           (step/256) e^(m_q - m) / l * max_e |V_u - O_s| (to first order; a
           factor 2 covers the change of l) */
        double b = 0.0;
        for (int a = 0; a < n_amb; ++a) {
            double wgt = amb[a].step / 256.0 * exp(amb[a].m - m) / l;
            double dv = 0.0;
            for (int e = 0; e < d; ++e) {
                double x = fabs(v_lowbit(F, amb[a].u, e) - os[e]);
                if (x > dv) dv = x;
            }
            b += 2.0 * wgt * dv;
        }
        *bound = b;
        free(amb);
    }
}

static void forward_block(void* vctx, long it) {
    const fwd_ctx* F = (const fwd_ctx*)vctx;
    const orc_problem* p = F->p;
    long pos = F->items[it];
    int i = F->blocks[2 * pos + 1];
    int d = p->d, Tq = ceil_div(p->N, p->bq), Tkv = ceil_div(p->N, p->bkv);
    int k = orc_topk(p);
    int h = (int)(F->bh % p->H);
    const int v1 = p->mode == 1;
    int kl = orc_topk_low(p);
    /* step 8 weight: per head, or per head and query block (SLA2 only) */
    double a = v1 ? 1.0
                  : (double)(p->alpha_mode ? F->alpha[(size_t)h * Tq + i] : F->alpha[h]);
    const int32_t* sel = F->idx + ((size_t)F->bh * Tq + i) * k;
    double* out = F->out + (size_t)pos * p->bq * d;
    memset(out, 0, sizeof(double) * (size_t)p->bq * d);

    /* linear set, H_i and Z_i ([SLA-zh] key design 3): the unselected
       blocks; in v1 mode the marginal ones (neither critical nor negligible) */
    uint8_t* hit = (uint8_t*)calloc(Tkv, 1);
    for (int r = 0; r < k; ++r) hit[sel[r]] = 1;
    if (v1)
        for (int r = 0; r < kl; ++r) hit[F->nidx[((size_t)F->bh * Tq + i) * kl + r]] = 1;
    int n_unsel = Tkv - k - (v1 ? kl : 0);
    const float* Wp = v1 ? F->Wp + (p->w_heads == 1 ? 0 : (size_t)h * d * d) : NULL;
    double* ol = (double*)malloc(sizeof(double) * d);
    double* Hi = (double*)calloc((size_t)d * d, sizeof(double));
    double* Zi = (double*)calloc(d, sizeof(double));
    if (n_unsel > 0) {
        for (int j = 0; j < Tkv; ++j) {
            if (hit[j]) continue;
            const double* hj = F->h + (size_t)j * d * d;
            const double* zj = F->z + (size_t)j * d;
            for (size_t x = 0; x < (size_t)d * d; ++x) Hi[x] += hj[x];
            for (int c = 0; c < d; ++c) Zi[c] += zj[c];
        }
    }
    double* os = (double*)malloc(sizeof(double) * d);
    double* pq = (double*)malloc(sizeof(double) * d);
    double* lbuf = (double*)malloc(sizeof(double) * ((size_t)k * p->bkv + 1));
    int t0 = i * p->bq, nq = p->N - t0 < p->bq ? p->N - t0 : p->bq;
    for (int t = t0; t < t0 + nq; ++t) {
        double* o = out + (size_t)(t - t0) * d;
        /* step 6: sparse branch */
        double* bnd = F->bound ? F->bound + (size_t)pos * p->bq + (t - t0) : NULL;
        if (F->variant == 0) sparse_exact(F, i, sel, k, t, os, lbuf);
        else sparse_lowbit(F, i, sel, k, t, os, lbuf, bnd);
        if (bnd) *bnd *= a; /* the combine scales O_s by alpha */
        /* step 7: linear branch O_l = phi(q) H_i / (phi(q) . Z_i) */
        phi_row(p, F->Q, F->bh, t, pq);
        if (n_unsel > 0) {
            double den = 0.0;
            for (int c = 0; c < d; ++c) den += pq[c] * Zi[c];
            for (int e = 0; e < d; ++e) {
                double num = 0.0;
                for (int c = 0; c < d; ++c) num += pq[c] * Hi[(size_t)c * d + e];
                ol[e] = num / den;
            }
        } else {
            for (int e = 0; e < d; ++e) ol[e] = 0.0;
        }
        /* step 8: combine; v1: O = O_s + O_l W_p ([SLA-zh] key design 3) */
        for (int e = 0; e < d; ++e) {
            if (v1) {
                double pr = 0.0;
                for (int c = 0; c < d; ++c) pr += ol[c] * (double)Wp[(size_t)c * d + e];
                o[e] = os[e] + pr;
            } else {
                o[e] = a * os[e] + (1.0 - a) * ol[e];
            }
        }
    }
    free(ol);
    free(hit);
    free(Hi);
    free(Zi);
    free(os);
    free(pq);
    free(lbuf);
}

static int forward_common(const orc_problem* p, const void* Q, const void* K, const void* V,
                          const int32_t* idx, const float* alpha, const int32_t* blocks,
                          int n_blocks, double* out, int nthreads, int variant,
                          int quantize, double* bound, double acc_eps, const int32_t* nidx,
                          const float* Wp) {
    int d = p->d, Tq = ceil_div(p->N, p->bq), Tkv = ceil_div(p->N, p->bkv);
    int k = orc_topk(p) + orc_topk_low(p); /* blocks outside the linear branch */
    long nbh = (long)p->B * p->H;
    /* process heads one at a time: the per-block summaries of a head are
       large (T_kv * d * d doubles) */
    long* items = (long*)malloc(sizeof(long) * (n_blocks > 0 ? n_blocks : 1));
    for (long bh = 0; bh < nbh; ++bh) {
        long n_it = 0;
        for (long b = 0; b < n_blocks; ++b)
            if (blocks[2 * b] == bh) {
                if (blocks[2 * b + 1] < 0 || blocks[2 * b + 1] >= Tq) {
                    free(items);
                    return -1;
                }
                items[n_it++] = b;
            }
        if (n_it == 0) continue;
        double *h = NULL, *z = NULL;
        if (k < Tkv) {
            h = (double*)malloc(sizeof(double) * (size_t)Tkv * d * d);
            z = (double*)malloc(sizeof(double) * (size_t)Tkv * d);
            summ_ctx S = {p, K, V, bh, h, z};
            run_pool(summary_block, &S, Tkv, nthreads);
        }
        quant_t qt = {0};
        if (variant == 1) {
            qt.qh = (uint8_t*)malloc((size_t)p->N * d);
            qt.kh = (uint8_t*)malloc((size_t)p->N * d);
            qt.sq = (float*)malloc(sizeof(float) * Tq);
            qt.sk = (float*)malloc(sizeof(float) * Tkv);
            qt.mu = (float*)malloc(sizeof(float) * d);
            quant_head(p, Q, K, bh, &qt);
            if (p->lowbit_v) {
                qt.vh = (uint8_t*)malloc((size_t)p->N * d);
                qt.sv = (float*)malloc(sizeof(float) * d);
                quant_v_head(p, V, bh, &qt);
            }
        }
        fwd_ctx F = {p, Q, K, V, idx, alpha, blocks, out, bh, items, h, z,
                     variant, quantize, &qt, bound, acc_eps, nidx, Wp};
        run_pool(forward_block, &F, n_it, nthreads);
        free(h);
        free(z);
        if (variant == 1) {
            free(qt.qh);
            free(qt.kh);
            free(qt.sq);
            free(qt.sk);
            free(qt.mu);
            free(qt.vh);
            free(qt.sv);
        }
    }
    free(items);
    return 0;
}

/* Forward (exact sparse branch) for the listed query blocks.
 * blocks: n_blocks pairs (bh, i); out: [n_blocks][bq][d] fp64, rows past
 * the valid tokens of a ragged block are 0.  idx: the router's
 * [B*H][Tq][k] ascending selection.  Returns 0, or -1 on a bad block. */
int orc_forward(const orc_problem* p, const void* Q, const void* K, const void* V,
                const int32_t* idx, const float* alpha, const int32_t* blocks,
                int n_blocks, double* out, int nthreads) {
    if (p->mode != 0) return -2;
    return forward_common(p, Q, K, V, idx, alpha, blocks, n_blocks, out, nthreads, 0, 1, NULL,
                          0.0, NULL, NULL);
}

/* SLA (v1) forward (p->mode == 1): sparse branch over the critical blocks
 * idx [B*H][Tq][k_h], linear branch over the marginal blocks (neither in idx
 * nor in nidx [B*H][Tq][k_l]), O = O_s + O_l Wp.  Same block list and output
 * as orc_forward.  Returns 0, -1 on a bad block, -2 if p is not in v1 mode. */
int orc_forward_v1(const orc_problem* p, const void* Q, const void* K, const void* V,
                   const int32_t* idx, const int32_t* nidx, const float* Wp,
                   const int32_t* blocks, int n_blocks, double* out, int nthreads) {
    if (p->mode != 1) return -2;
    return forward_common(p, Q, K, V, idx, NULL, blocks, n_blocks, out, nthreads, 0, 1, NULL,
                          0.0, nidx, Wp);
}

/* Forward with the low-bit sparse branch (quantize=1: e4m3; 0: identity).
 * bound (optional, [n_blocks][bq]): per output row, a bound on how far the
 * row can move if the P-quantisation decisions that an implementation with
 * relative dot-product accumulation error acc_eps could take the other way
 * are all flipped (0 for rows without such a decision). */
int orc_forward_fp8(const orc_problem* p, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* alpha, const int32_t* blocks,
                    int n_blocks, int quantize, double* out, double* bound, double acc_eps,
                    int nthreads) {
    if (bound) memset(bound, 0, sizeof(double) * (size_t)n_blocks * p->bq);
    if (p->bkv > 512 || p->mode != 0) return -2;
    return forward_common(p, Q, K, V, idx, alpha, blocks, n_blocks, out, nthreads, 1,
                          quantize, bound, acc_eps, NULL, NULL);
}
