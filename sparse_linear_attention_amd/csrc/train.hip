// Training-time router ("SLA2 深度解读" 06, Stage 1: the router projections
// and alpha are fitted with a differentiable SoftTop-k in place of the hard
// top-k):
//   SoftTop-k(S)_ij = sigma(S_ij / tau + lambda_i), lambda_i by bisection so
//   that every row's soft selections sum to the budget k;
//   its gradient, lambda moving with S so that the row sum stays k;
//   the gradient of S = proj_q(Qbar) proj_k(Kbar)^T with respect to the two
//   projections.
// Everything in fp64 except the stored mask and gradients (fp32).
#include "sla2_internal.h"

namespace sla2 {
namespace {

constexpr int kSoftIters = 100;  // bisection halvings

// deterministic sum of one double per thread over the work-group (256
// threads): each wave reduces in a fixed butterfly order, then wave sums in
// wave order; every thread gets the result
__device__ inline double block_sum(double v, double* red) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int t = threadIdx.x;
    __syncthreads();
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ inline double block_max(double v, double* red) {
    for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
    const int t = threadIdx.x;
    __syncthreads();
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    return fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

__device__ inline double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

// one work-group per score row (grid (Tq, BH)), 256 threads
__global__ __launch_bounds__(256) void soft_topk_kernel(const double* __restrict__ S, int Tq,
                                                        int Tkv, int k, double tau,
                                                        float* __restrict__ M,
                                                        double* __restrict__ lambda) {
    extern __shared__ double x[];  // [Tkv]: S / tau
    __shared__ double red[4];
    const int t = threadIdx.x;
    const size_t row = (size_t)blockIdx.y * Tq + blockIdx.x;
    float* mrow = M + row * Tkv;
    if (k <= 0 || k >= Tkv) {
        for (int j = t; j < Tkv; j += 256) mrow[j] = k <= 0 ? 0.0f : 1.0f;
        if (t == 0 && lambda) lambda[row] = k <= 0 ? -INFINITY : INFINITY;
        return;
    }
    double mx = -INFINITY, mn = INFINITY;
    for (int j = t; j < Tkv; j += 256) {
        const double v = S[row * Tkv + j] / tau;
        x[j] = v;
        mx = fmax(mx, v);
        mn = fmin(mn, v);
    }
    mx = block_max(mx, red);
    mn = -block_max(-mn, red);
    double lo = -mx - 50.0, hi = -mn + 50.0;
    for (int it = 0; it < kSoftIters; ++it) {
        const double mid = 0.5 * (lo + hi);
        // once the midpoint equals an end, no halving can move lambda (the
        // final midpoint) any more: the rest of the 100 would be no-ops
        if (mid == lo || mid == hi) break;
        double f = 0.0;
        for (int j = t; j < Tkv; j += 256) f += sigmoid(x[j] + mid);
        f = block_sum(f, red) - (double)k;
        if (f > 0.0) hi = mid;
        else lo = mid;
    }
    const double lam = 0.5 * (lo + hi);
    for (int j = t; j < Tkv; j += 256) mrow[j] = (float)sigmoid(x[j] + lam);
    if (t == 0 && lambda) lambda[row] = lam;
}

// The same bisection with one wave per score row (four rows per work-group
// of 256), for rows of at most 64 SLOTS blocks: the row's S / tau stays in
// registers (block j in lane j % 64, slot j / 64) and the sums are wave
// reductions, so no work-group barrier is needed.
__device__ inline double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
template <int SLOTS>
__global__ __launch_bounds__(256) void soft_topk_wave_kernel(const double* __restrict__ S,
                                                             long rows, int Tkv, int k,
                                                             double tau, float* __restrict__ M,
                                                             double* __restrict__ lambda) {
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // the whole wave
    float* mrow = M + (size_t)row * Tkv;
    if (k <= 0 || k >= Tkv) {
        for (int j = lane; j < Tkv; j += 64) mrow[j] = k <= 0 ? 0.0f : 1.0f;
        if (lane == 0 && lambda) lambda[row] = k <= 0 ? -INFINITY : INFINITY;
        return;
    }
    double x[SLOTS];
    double mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int t = 0; t < SLOTS; ++t) {
        const int j = lane + 64 * t;
        x[t] = 0.0;
        if (j < Tkv) {
            x[t] = S[(size_t)row * Tkv + j] / tau;
            mx = fmax(mx, x[t]);
            mn = fmin(mn, x[t]);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        mx = fmax(mx, __shfl_xor(mx, off));
        mn = fmin(mn, __shfl_xor(mn, off));
    }
    double lo = -mx - 50.0, hi = -mn + 50.0;
    for (int it = 0; it < kSoftIters; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;  // (as in soft_topk_kernel)
        double f = 0.0;
#pragma unroll
        for (int t = 0; t < SLOTS; ++t)
            if (lane + 64 * t < Tkv) f += sigmoid(x[t] + mid);
        f = wave_sum_f64(f) - (double)k;
        if (f > 0.0) hi = mid;
        else lo = mid;
    }
    const double lam = 0.5 * (lo + hi);
#pragma unroll
    for (int t = 0; t < SLOTS; ++t) {
        const int j = lane + 64 * t;
        if (j < Tkv) mrow[j] = (float)sigmoid(x[t] + lam);
    }
    if (lane == 0 && lambda) lambda[row] = lam;
}

// dS = s / tau (dM - sum dM s / sum s), s = M (1 - M); grid (Tq, BH)
__global__ __launch_bounds__(256) void soft_topk_grad_kernel(const float* __restrict__ M,
                                                             const float* __restrict__ dM,
                                                             int Tq, int Tkv, double tau,
                                                             float* __restrict__ dS) {
    __shared__ double red[4];
    const int t = threadIdx.x;
    const size_t row = ((size_t)blockIdx.y * Tq + blockIdx.x) * Tkv;
    double a = 0.0, b = 0.0;
    for (int j = t; j < Tkv; j += 256) {
        const double m = (double)M[row + j];
        const double s = m * (1.0 - m);
        a += (double)dM[row + j] * s;
        b += s;
    }
    a = block_sum(a, red);
    b = block_sum(b, red);
    const double c = b > 0.0 ? a / b : 0.0;
    for (int j = t; j < Tkv; j += 256) {
        const double m = (double)M[row + j];
        dS[row + j] = (float)(m * (1.0 - m) / tau * ((double)dM[row + j] - c));
    }
}

// C[z] (M x N, ldc) = A[z] (M x K) B[z] (K x N) in fp64, batched over z =
// blockIdx.z.  A element (m, kk) at a[z * sa + (TA ? kk * lda + m : m * lda + kk)]
// (float or double), B element (kk, n) at b[z * sb + kk * ldb + n].  64x64
// tiles, 4x4 per thread, each output accumulated over kk in order.
template <typename TA, bool TRANS_A>
__global__ __launch_bounds__(256) void gemm64_kernel(const TA* __restrict__ a, long sa, int lda,
                                                     const double* __restrict__ b, long sb,
                                                     int ldb, double* __restrict__ c, long sc,
                                                     int ldc, int Mr, int Nc, int Kd) {
    __shared__ double As[16][65];
    __shared__ double Bs[16][65];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const long z = blockIdx.z;
    const TA* A = a + z * sa;
    const double* B = b + z * sb;
    double acc[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = 0.0;
    for (int k0 = 0; k0 < Kd; k0 += 16) {
        for (int x = threadIdx.x; x < 1024; x += 256) {
            // A tile: row r (0..63), column kk (0..15)
            int r, kk;
            if (TRANS_A) {  // contiguous along m
                r = x & 63;
                kk = x >> 6;
            } else {        // contiguous along k
                r = x >> 4;
                kk = x & 15;
            }
            const int gm = m0 + r, gk = k0 + kk;
            As[kk][r] = (gm < Mr && gk < Kd)
                            ? (double)(TRANS_A ? A[(size_t)gk * lda + gm] : A[(size_t)gm * lda + gk])
                            : 0.0;
            const int col = x & 63, kr = x >> 6;
            const int bn = n0 + col, bk = k0 + kr;
            Bs[kr][col] = (bn < Nc && bk < Kd) ? B[(size_t)bk * ldb + bn] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            double av[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                av[q] = As[kk][ty + 16 * q];
                bv[q] = Bs[kk][tx + 16 * q];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fma(av[p], bv[q], acc[p][q]);
        }
        __syncthreads();
    }
    double* C = c + z * sc;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int m = m0 + ty + 16 * p;
        if (m >= Mr) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx + 16 * q;
            if (n < Nc) C[(size_t)m * ldc + n] = acc[p][q];
        }
    }
}

// dW[h'] = sum over the heads sharing projection h' of part[bh], in head
// order; fp32 out.  grid (d*d/256, w_heads)
__global__ __launch_bounds__(256) void head_sum_kernel(const double* __restrict__ part,
                                                       float* __restrict__ out, int BH, int H,
                                                       int w_heads, int dd) {
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x >= dd) return;
    const int hw = blockIdx.y;
    double s = 0.0;
    for (int bh = 0; bh < BH; ++bh)
        if (w_heads == 1 || bh % H == hw) s += part[(size_t)bh * dd + x];
    out[(size_t)hw * dd + x] = (float)s;
}

template <typename TA, bool TR>
hipError_t gemm64(const TA* a, long sa, int lda, const double* b, long sb, int ldb, double* c,
                  long sc, int ldc, int Mr, int Nc, int Kd, int batch, hipStream_t s) {
    dim3 g((Nc + 63) / 64, (Mr + 63) / 64, batch);
    gemm64_kernel<TA, TR><<<g, 256, 0, s>>>(a, sa, lda, b, sb, ldb, c, sc, ldc, Mr, Nc, Kd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_soft_topk(const Dims& D, const void* Q, const void* K, const float* Wq,
                            const float* Wk, double tau, float* M, double* lambda,
                            const RouteWS& ws, hipStream_t s) {
    hipError_t e = launch_scores(D, Q, K, Wq, Wk, ws, s);
    if (e != hipSuccess) return e;
    constexpr int kWaveSlots = 19;  // rows of up to 1216 blocks: one wave each
    if (D.Tkv <= 64 * kWaveSlots) {
        const long rows = D.BH * (long)D.Tq;
        soft_topk_wave_kernel<kWaveSlots><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(
            ws.S, rows, D.Tkv, D.k, tau, M, lambda);
    } else {
        soft_topk_kernel<<<dim3(D.Tq, (unsigned)D.BH), 256, sizeof(double) * D.Tkv, s>>>(
            ws.S, D.Tq, D.Tkv, D.k, tau, M, lambda);
    }
    return hipGetLastError();
}

hipError_t launch_soft_topk_grad(const Dims& D, const float* M, const float* dM, double tau,
                                 float* dS, hipStream_t s) {
    soft_topk_grad_kernel<<<dim3(D.Tq, (unsigned)D.BH), 256, 0, s>>>(M, dM, D.Tq, D.Tkv, tau,
                                                                     dS);
    return hipGetLastError();
}

hipError_t launch_route_grad(const Dims& D, const void* Q, const void* K, const float* Wq,
                             const float* Wk, const float* dS, float* dWq, float* dWk,
                             const RouteWS& ws, const GradWS& gw, hipStream_t s) {
    // pooled rows (xq, xk) and their projections (qt, kt)
    hipError_t e = launch_pool_project(D, Q, K, Wq, Wk, ws, s);
    const int d = D.d, Tq = D.Tq, Tkv = D.Tkv, BH = (int)D.BH;
    // dqt = dS kt  [Tq x d];  dkt = dS^T qt  [Tkv x d]
    if (e == hipSuccess)
        e = gemm64<float, false>(dS, (long)Tq * Tkv, Tkv, ws.kt, (long)Tkv * d, d, gw.dq,
                                 (long)Tq * d, d, Tq, d, Tkv, BH, s);
    if (e == hipSuccess)
        e = gemm64<float, true>(dS, (long)Tq * Tkv, Tkv, ws.qt, (long)Tq * d, d, gw.dk,
                                (long)Tkv * d, d, Tkv, d, Tq, BH, s);
    // per-head dWq = xq^T dqt, dWk = xk^T dkt  [d x d]
    if (e == hipSuccess)
        e = gemm64<double, true>(ws.xq, (long)Tq * d, d, gw.dq, (long)Tq * d, d, gw.pq,
                                 (long)d * d, d, d, d, Tq, BH, s);
    if (e == hipSuccess)
        e = gemm64<double, true>(ws.xk, (long)Tkv * d, d, gw.dk, (long)Tkv * d, d, gw.pk,
                                 (long)d * d, d, d, d, Tkv, BH, s);
    if (e != hipSuccess) return e;
    const dim3 gs((d * d + 255) / 256, D.w_heads);
    head_sum_kernel<<<gs, 256, 0, s>>>(gw.pq, dWq, BH, D.H, D.w_heads, d * d);
    head_sum_kernel<<<gs, 256, 0, s>>>(gw.pk, dWk, BH, D.H, D.w_heads, d * d);
    return hipGetLastError();
}

}  // namespace sla2
