// fp32 forward path (vector ALU): linear-branch block summaries and a fused
// sparse + linear + combine kernel, for every d, b_q and input type the
// matrix-core kernels do not take (fp32 inputs, b_q = 64, d = 64).
//
// Sparse branch ("SLA2 深度解读" 04/08): online softmax of q.k/sqrt(d) over
// the tokens of the selected KV blocks.  Linear branch (SLA notes, key
// design 3/4): O_l = phi(q) H_i / (phi(q) . Z_i) with H_i = h_tot - sum over
// the blocks outside the linear set; that part is evaluated per token as
// sum_u (phi(q) . phi(k_u)) v_u, which equals phi(q) (sum_u phi(k_u)^T v_u).
// Combine: O = alpha O_s + (1 - alpha) O_l.
// SLA (v1) (SLA notes, key design 3): the critical blocks run the softmax,
// the negligible ones are left out of both branches, the linear set is the
// marginal rest, and O = O_s + O_l W_p.
// phi: elu + 1, or the softmax of each row over its d channels (SLA notes'
// training section), max-subtracted.
#include "sla2_internal.h"

namespace sla2 {
namespace {

__device__ inline float ld1(const float* p) { return *p; }
__device__ inline float ld1(const uint16_t* p) { return __uint_as_float((unsigned)(*p) << 16); }

__device__ inline float phi_f(float x) { return x > 0.0f ? x + 1.0f : expf(x); }

// phi of one row held by the 8 consecutive lanes of a group, each lane CS
// (of 16) channels: elu + 1 per channel, or the softmax over the row's d
// channels.  Every lane of the group takes part (shuffles).
__device__ inline void phi_row8(const float* x, float* y, int CS, int phi_sm) {
    if (!phi_sm) {
#pragma unroll
        for (int c = 0; c < 16; ++c) y[c] = phi_f(x[c]);
        return;
    }
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        if (c < CS) m = fmaxf(m, x[c]);
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        y[c] = c < CS ? __expf(x[c] - m) : 0.0f;
        sum += y[c];
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < 16; ++c) y[c] *= inv;
}

// row t of a head (CS channels from c0; zeros where !ok)
template <typename T>
__device__ inline void load_row(const T* X, size_t t, size_t stride, int c0, int CS, bool ok,
                                float* x) {
#pragma unroll
    for (int c = 0; c < 16; ++c) x[c] = (ok && c < CS) ? ld1(X + t * stride + c0 + c) : 0.0f;
}

// Per-chunk partial h[c][e] = sum_u phi(K_u)[c] V_u[e] and z[c] = sum_u phi(K_u)[c]
// over the valid tokens of the chunk (bpc KV blocks).  grid (chunks, BH), 256
// threads.
template <typename T>
__global__ __launch_bounds__(256) void summaries_valu_kernel(
    const T* __restrict__ K, const T* __restrict__ V, float* __restrict__ hpart,
    float* __restrict__ zpart, int N, int d, int nch, int H, Strides st, int bpc, int phi_sm) {
    __shared__ float pk[32 * 128];
    __shared__ float vv[32 * 128];
    const int chunk = blockIdx.x;
    const long bh = blockIdx.y;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int SB = d >> 4;  // 8 or 4
    const int t_begin = chunk * bpc * 64;
    const int t_end = min(N, t_begin + bpc * 64);
    const T* Kh = K + head_base(st, bh, H);
    const T* Vh = V + head_base(st, bh, H);
    float acc[8][8];
    float z[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        z[a] = 0.0f;
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.0f;
    }
    // loads: token u = thread / 8, channels c0 .. c0 + d/8 (as in the fused
    // kernel, so both evaluate phi(k) the same way)
    const int lu = threadIdx.x >> 3, CS = d >> 3, c0 = (threadIdx.x & 7) * CS;
    for (int u0 = t_begin; u0 < t_end; u0 += 32) {
        {
            const int t = u0 + lu;
            const bool ok = t < t_end;
            float kx[16], px[16], vx[16];
            load_row(Kh, t, st.t, c0, CS, ok, kx);
            load_row(Vh, t, st.t, c0, CS, ok, vx);
            phi_row8(kx, px, CS, phi_sm);
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (c < CS) {
                    pk[lu * d + c0 + c] = ok ? px[c] : 0.0f;
                    vv[lu * d + c0 + c] = vx[c];
                }
        }
        __syncthreads();
        for (int u = 0; u < 32; ++u) {
            float a[8], b[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                a[q] = q < SB ? pk[u * d + ty * SB + q] : 0.0f;
                b[q] = q < SB ? vv[u * d + tx * SB + q] : 0.0f;
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                z[p] += a[p];
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
            }
        }
        __syncthreads();
    }
    float* hp = hpart + ((size_t)bh * nch + chunk) * d * d;
    for (int p = 0; p < SB; ++p)
        for (int q = 0; q < SB; ++q) hp[(size_t)(ty * SB + p) * d + tx * SB + q] = acc[p][q];
    if (tx == 0) {
        float* zp = zpart + ((size_t)bh * nch + chunk) * d;
        for (int p = 0; p < SB; ++p) zp[ty * SB + p] = z[p];
    }
}

// h_tot = sum of the chunk partials in chunk order (deterministic).
__global__ __launch_bounds__(256) void summaries_reduce_kernel(
    const float* __restrict__ hpart, const float* __restrict__ zpart, float* __restrict__ htot,
    float* __restrict__ ztot, int d, int nch) {
    const long bh = blockIdx.y;
    const int x = blockIdx.x * 256 + threadIdx.x;
    const int dd = d * d;
    if (x < dd) {
        float s = 0.0f;
        // loads issued ahead, additions in chunk order
#pragma unroll 8
        for (int c = 0; c < nch; ++c) s += hpart[((size_t)bh * nch + c) * dd + x];
        htot[(size_t)bh * dd + x] = s;
    }
    if (blockIdx.x == 0 && threadIdx.x < d) {
        float s = 0.0f;
        for (int c = 0; c < nch; ++c) s += zpart[((size_t)bh * nch + c) * d + threadIdx.x];
        ztot[(size_t)bh * d + threadIdx.x] = s;
    }
}

// Fused sparse + linear + combine.  A work-group handles 32 query rows of one
// query block; 8 threads per row, each owning d/8 channels.  KV tiles are
// visited 32 tokens at a time.  grid (Tq * bq/32, BH), 256 threads.
// v1: negl [BH][Tq][kl] are the negligible blocks (outside both branches),
// Wp [w_heads][d][d] the projection of the linear branch's output.
template <typename T>
__global__ __launch_bounds__(256) void fused_valu_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ negl,
    const float* __restrict__ alpha, const float* __restrict__ Wp,
    const float* __restrict__ htot, const float* __restrict__ ztot, void* __restrict__ O,
    int N, int d, int bq, int Tq, int Tkv, int k, int kl, int H, int w_heads, Strides st,
    int alpha_qblock, int out_bf16, int phi_sm, int v1) {
    __shared__ float Kt[32 * 128];
    __shared__ float Vt[32 * 128];
    __shared__ float Pk[32 * 128];
    const int per_blk = bq >> 5;
    const int qb = blockIdx.x / per_blk;
    const int row = threadIdx.x >> 3, sub = threadIdx.x & 7;
    const int CS = d >> 3;  // 16 or 8
    const int c0 = sub * CS;
    const long bh = blockIdx.y;
    const int tq = qb * bq + (blockIdx.x % per_blk) * 32 + row;
    const bool valid_q = tq < N;
    const T* Qh = Q + head_base(st, bh, H);
    const T* Kh = K + head_base(st, bh, H);
    const T* Vh = V + head_base(st, bh, H);
    const float inv_sqrt_d = 1.0f / sqrtf((float)d);

    float q[16], pq[16], acc[16], corr[16];
    load_row(Qh, tq, st.t, c0, CS, valid_q, q);
    phi_row8(q, pq, CS, phi_sm);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        acc[c] = 0.0f;
        corr[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f, zc = 0.0f;
    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;
    const int32_t* nsel = kl > 0 ? negl + ((size_t)bh * Tq + qb) * kl : nullptr;
    // the linear set is not empty: T_kv - k blocks (SLA2), T_kv - k - kl (v1)
    const bool lin = k + kl < Tkv;

    // tokens u0 .. u0 + 31 (nu of them valid): K, phi(K) and V into LDS
    auto load_tile = [&](int u0, int nu) {
        const bool ok = row < nu;
        float kx[16], px[16], vx[16];
        load_row(Kh, u0 + row, st.t, c0, CS, ok, kx);
        load_row(Vh, u0 + row, st.t, c0, CS, ok, vx);
        phi_row8(kx, px, CS, phi_sm);
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) {
                Kt[row * d + c0 + c] = kx[c];
                Pk[row * d + c0 + c] = ok ? px[c] : 0.0f;
                Vt[row * d + c0 + c] = vx[c];
            }
    };
    // phi(q) . phi(k_u) for the tile's token u (whole row, after the shuffles)
    auto phi_dot = [&](int u) {
        float ap = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) ap = fmaf(pq[c], Pk[u * d + c0 + c], ap);
        ap += __shfl_xor(ap, 1);
        ap += __shfl_xor(ap, 2);
        ap += __shfl_xor(ap, 4);
        return ap;
    };

    for (int r = 0; r < k; ++r) {
        const int j = sel[r];
        for (int half = 0; half < 2; ++half) {
            const int u0 = j * 64 + half * 32;
            const int nu = min(32, N - u0);
            if (nu <= 0) break;
            load_tile(u0, nu);
            __syncthreads();
            float s[32];
            float tmax = -INFINITY;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                float sp = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) sp = fmaf(q[c], Kt[u * d + c0 + c], sp);
                sp += __shfl_xor(sp, 1);
                sp += __shfl_xor(sp, 2);
                sp += __shfl_xor(sp, 4);
                const float ap = phi_dot(u);
                const bool ok = u < nu;
                s[u] = ok ? sp * inv_sqrt_d : -INFINITY;
                tmax = fmaxf(tmax, s[u]);
                if (ok) {
                    zc += ap;
#pragma unroll
                    for (int c = 0; c < 16; ++c)
                        if (c < CS) corr[c] = fmaf(ap, Vt[u * d + c0 + c], corr[c]);
                }
            }
            const float mn = fmaxf(m, tmax);
            const float resc = (m == -INFINITY) ? 0.0f : expf(m - mn);
            l *= resc;
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[c] *= resc;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const float p = expf(s[u] - mn);
                l += p;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) acc[c] = fmaf(p, Vt[u * d + c0 + c], acc[c]);
            }
            m = mn;
            __syncthreads();
        }
    }
    // v1: the negligible blocks leave the linear set too (no softmax for them)
    if (lin) {
        for (int r = 0; r < kl; ++r) {
            const int j = nsel[r];
            for (int half = 0; half < 2; ++half) {
                const int u0 = j * 64 + half * 32;
                const int nu = min(32, N - u0);
                if (nu <= 0) break;
                load_tile(u0, nu);
                __syncthreads();
                for (int u = 0; u < nu; ++u) {
                    const float ap = phi_dot(u);
                    zc += ap;
#pragma unroll
                    for (int c = 0; c < 16; ++c)
                        if (c < CS) corr[c] = fmaf(ap, Vt[u * d + c0 + c], corr[c]);
                }
                __syncthreads();
            }
        }
    }

    // linear branch: phi(q) (h_tot - left out) / (phi(q) . (z_tot - left out))
    float ol[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) ol[c] = 0.0f;
    if (lin) {
        const float* hT = htot + (size_t)bh * d * d;
        const float* zT = ztot + (size_t)bh * d;
        // full phi(q) of each row into LDS
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) Kt[row * d + c0 + c] = pq[c];
        float den = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) den = fmaf(pq[c], zT[c0 + c], den);
        den += __shfl_xor(den, 1);
        den += __shfl_xor(den, 2);
        den += __shfl_xor(den, 4);
        den -= zc;
        float num[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) num[c] = 0.0f;
        for (int cb = 0; cb < d; cb += 32) {
            __syncthreads();
            for (int x = threadIdx.x; x < 32 * d; x += 256) Vt[x] = hT[(size_t)cb * d + x];
            __syncthreads();
            for (int cc = 0; cc < 32; ++cc) {
                const float a = Kt[row * d + cb + cc];
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) num[c] = fmaf(a, Vt[cc * d + c0 + c], num[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) ol[c] = (num[c] - corr[c]) / den;
        if (v1) {
            // O_l W_p: the whole row of O_l through LDS
            __syncthreads();
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (c < CS) Kt[row * d + c0 + c] = ol[c];
            __syncthreads();
            const float* W = Wp + (w_heads == 1 ? 0 : (size_t)(bh % H) * d * d);
            float pr[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) pr[c] = 0.0f;
            for (int cc = 0; cc < d; ++cc) {
                const float a = Kt[row * d + cc];
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) pr[c] = fmaf(a, W[(size_t)cc * d + c0 + c], pr[c]);
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) ol[c] = pr[c];
        }
    }
    if (valid_q) {
        const float a = v1 ? 1.0f : alpha_of(alpha, bh, H, qb, Tq, alpha_qblock);
        const float b = v1 ? 1.0f : 1.0f - a;
        const float inv_l = (k > 0) ? 1.0f / l : 0.0f;
        const size_t o = head_base(st, bh, H) + (size_t)tq * st.t + c0;
        float v[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) v[c] = a * (acc[c] * inv_l) + b * ol[c];
#pragma unroll
        for (int c = 0; c < 16; c += 4)
            if (c < CS) store_out4(O, o + c, v[c], v[c + 1], v[c + 2], v[c + 3], out_bf16);
    }
}

}  // namespace

hipError_t launch_partials_reduce(const Dims& D, const float* part, const float* zpart,
                                  float* tot, float* ztot, int nch, hipStream_t s) {
    timing_before(s, K_SUMM_REDUCE);
    summaries_reduce_kernel<<<dim3((D.d * D.d + 255) / 256, (unsigned)D.BH), 256, 0, s>>>(
        part, zpart, tot, ztot, D.d, nch);
    timing_after(s, K_SUMM_REDUCE);
    return hipGetLastError();
}

hipError_t launch_summaries_reduce(const Dims& D, const FwdWS& ws, hipStream_t s) {
    return launch_partials_reduce(D, ws.hpart, ws.zpart, ws.htot, ws.ztot, summ_chunks(D), s);
}

// per-chunk partials over chunks of bpc KV blocks
static hipError_t summaries_chunks(const Dims& D, const void* K, const void* V, float* hpart,
                                   float* zpart, int bpc, hipStream_t s) {
    const int nch = (D.Tkv + bpc - 1) / bpc;
    timing_before(s, K_SUMM_VALU);
    if (D.dtype == SLA2_F32)
        summaries_valu_kernel<float><<<dim3(nch, (unsigned)D.BH), 256, 0, s>>>(
            (const float*)K, (const float*)V, hpart, zpart, D.N, D.d, nch, D.H, D.st, bpc,
            D.phi_sm);
    else
        summaries_valu_kernel<uint16_t><<<dim3(nch, (unsigned)D.BH), 256, 0, s>>>(
            (const uint16_t*)K, (const uint16_t*)V, hpart, zpart, D.N, D.d, nch, D.H, D.st,
            bpc, D.phi_sm);
    timing_after(s, K_SUMM_VALU);
    return hipGetLastError();
}

hipError_t launch_summaries_valu(const Dims& D, const void* K, const void* V, const FwdWS& ws,
                                 hipStream_t s) {
    hipError_t e = summaries_chunks(D, K, V, ws.hpart, ws.zpart, kSummBlocksPerChunk, s);
    if (e != hipSuccess) return e;
    return launch_summaries_reduce(D, ws, s);
}

hipError_t launch_summaries_blocks(const Dims& D, const void* K, const void* V, float* hblk,
                                   float* zblk, hipStream_t s) {
    return summaries_chunks(D, K, V, hblk, zblk, 1, s);
}

hipError_t launch_forward_valu(const Dims& D, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const float* alpha, void* O,
                               const FwdWS& ws, hipStream_t s, const int32_t* negl,
                               const float* Wp) {
    const int kl = D.v1 ? D.kl : 0;
    if (D.k + kl < D.Tkv) {
        hipError_t e = launch_summaries_valu(D, K, V, ws, s);
        if (e != hipSuccess) return e;
    }
    dim3 g(D.Tq * (D.bq / 32), (unsigned)D.BH);
    timing_before(s, K_FUSED_VALU);
    if (D.dtype == SLA2_F32)
        fused_valu_kernel<float><<<g, 256, 0, s>>>(
            (const float*)Q, (const float*)K, (const float*)V, idx, negl, alpha, Wp, ws.htot,
            ws.ztot, O, D.N, D.d, D.bq, D.Tq, D.Tkv, D.k, kl, D.H, D.w_heads, D.st,
            D.alpha_qblock, D.out_bf16, D.phi_sm, D.v1);
    else
        fused_valu_kernel<uint16_t><<<g, 256, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, idx, negl, alpha, Wp,
            ws.htot, ws.ztot, O, D.N, D.d, D.bq, D.Tq, D.Tkv, D.k, kl, D.H, D.w_heads, D.st,
            D.alpha_qblock, D.out_bf16, D.phi_sm, D.v1);
    timing_after(s, K_FUSED_VALU);
    return hipGetLastError();
}

}  // namespace sla2
