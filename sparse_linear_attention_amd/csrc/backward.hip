// Backward of the SLA2 forward with the hard selection held fixed, vector-ALU
// form (fp32 arithmetic) for the problems the matrix-core backward
// (backward_mfma.hip: bf16 with d = b_q = 128, phi = elu + 1) does not take:
// fp32 inputs, d = 64, b_q = 64, or phi = the softmax of each row.  L = sum dO . O with O = alpha O_s + (1 -
// alpha) O_l ("SLA2 深度解读" 04; the SLA notes' key designs 3 and 4 for O_l).
//
// Per query row t of block i, with g = dO_t, gs = alpha g, e = (1 - alpha) g:
//   sparse  D = gs . O_s; for every selected token u: p = exp(l_tu - LSE_t),
//           dl = p (gs . v_u - D); dq_t += dl k_u / sqrt d; dk_u += dl q_t /
//           sqrt d; dv_u += p gs;
//   linear  O_l = n / s with n = phi(q) h_tot - sum_u a_tu v_u and s =
//           phi(q) . z_tot - sum_u a_tu over the selected tokens (a_tu =
//           phi(q_t) . phi(k_u), the same total-minus-selected form as the
//           forward); dn = e / s, ds = -(e . O_l) / s;
//           dphi(q_t) = h_tot dn + z_tot ds - sum_u phi(k_u) (v_u . dn + ds);
//           for the selected tokens dphi(k_u) -= phi(q_t) (v_u . dn + ds) and
//           dv_u -= a_tu dn; every token u gets dv_u += phi(k_u) dH_tot and
//           dphi(k_u) += dH_tot v_u + dZ_tot with dH_tot = sum_t phi(q_t)^T
//           dn_t, dZ_tot = sum_t phi(q_t) ds_t over the whole head;
//   dalpha  sum over its rows of g . (O_s - O_l).
// Through phi (SLA notes, key design 4: the backward runs through the feature
// map): dx = dphi * phi'(x) for elu + 1; for the row softmax p = phi(x),
// dx = p * (dphi - p . dphi).
// Kernels: block summaries (h_tot, z_tot) as the fp32 forward; a query-row
// pass (dQ and the per-row values the key pass needs); dH_tot, dZ_tot; the
// selection inverted per KV block; a key pass over the query blocks that
// select each KV block (dK, dV); dalpha summed in a fixed order.
#include "sla2_internal.h"

namespace sla2 {
namespace {

__device__ inline float ldx(const float* p) { return *p; }
__device__ inline float ldx(const uint16_t* p) { return __uint_as_float((unsigned)(*p) << 16); }
__device__ inline float phi_e(float x) { return x > 0.0f ? x + 1.0f : expf(x); }
__device__ inline float dphi_e(float x) { return x > 0.0f ? 1.0f : expf(x); }

// sum over the 8 consecutive lanes that share a row, with DPP lane moves
// (VALU speed): quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2),
// then the half-row mirror (lane i <-> 7 - i) adds the other quad's sum; every
// lane of the 8 ends with the same value
template <int CTRL>
__device__ inline float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ inline float row8(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    return v;
}
__device__ inline float row8max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    return v;
}

// phi of one row held by the 8 lanes of a group (CS channels each, any
// assignment of channels to lanes): elu + 1, or the softmax over the row
__device__ inline void phi_row(const float* x, float* y, int CS, int sm) {
    if (!sm) {
#pragma unroll
        for (int c = 0; c < 16; ++c) y[c] = phi_e(x[c]);
        return;
    }
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        if (c < CS) m = fmaxf(m, x[c]);
    m = row8max(m);
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        y[c] = c < CS ? __expf(x[c] - m) : 0.0f;
        sum += y[c];
    }
    const float inv = 1.0f / row8(sum);
#pragma unroll
    for (int c = 0; c < 16; ++c) y[c] *= inv;
}

// dx from dphi through phi at x (y = phi(x)), row held as in phi_row
__device__ inline void dphi_row(const float* x, const float* y, const float* g, float* dx,
                                int CS, int sm) {
    if (!sm) {
#pragma unroll
        for (int c = 0; c < 16; ++c) dx[c] = g[c] * dphi_e(x[c]);
        return;
    }
    float pg = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c)
        if (c < CS) pg = fmaf(y[c], g[c], pg);
    pg = row8(pg);
#pragma unroll
    for (int c = 0; c < 16; ++c) dx[c] = y[c] * (g[c] - pg);
}

// Query rows: 32 rows per work-group, 8 threads per row; thread `sub` of a
// row owns channels sub, sub + 8, ... (d / 8 of them), so that the 8 threads
// read 8 different LDS banks.  grid (Tq * bq / 32, BH), 256 threads.
template <typename T>
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ dO, const int32_t* __restrict__ idx,
    const float* __restrict__ alpha, const float* __restrict__ htot,
    const float* __restrict__ ztot, float* __restrict__ dQ, float* __restrict__ lse,
    float* __restrict__ Dv, float* __restrict__ dsv, float* __restrict__ dn_out,
    float* __restrict__ da_row, int N, int d, int bq, int Tq, int Tkv, int k, int H,
    Strides st, int alpha_qblock, int phi_sm) {
    __shared__ float Kt[32 * 128];
    __shared__ float Pk[32 * 128];
    __shared__ float Vt[32 * 128];
    __shared__ float Rw[32 * 128];  // per-row vectors (phi(q), then dn)
    const int per_blk = bq >> 5;
    const int qb = blockIdx.x / per_blk;
    const int row = threadIdx.x >> 3, sub = threadIdx.x & 7;
    const int CS = d >> 3;  // channels sub, sub + 8, ... (conflict-free LDS reads)
    const long bh = blockIdx.y;
    const int tq = qb * bq + (blockIdx.x % per_blk) * 32 + row;
    const bool valid_q = tq < N;
    const T* Qh = Q + head_base(st, bh, H);
    const T* Kh = K + head_base(st, bh, H);
    const T* Vh = V + head_base(st, bh, H);
    const float* dOh = dO + head_base(st, bh, H);
    const float isd = 1.0f / sqrtf((float)d);
    const bool lin = k < Tkv;

    float q[16], pq[16], g[16], acc[16], corr[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const bool ok = c < CS && valid_q;
        q[c] = ok ? ldx(Qh + (size_t)tq * st.t + sub + 8 * c) : 0.0f;
        g[c] = ok ? dOh[(size_t)tq * st.t + sub + 8 * c] : 0.0f;
        acc[c] = 0.0f;
        corr[c] = 0.0f;
    }
    phi_row(q, pq, CS, phi_sm);
    float m = -INFINITY, l = 0.0f, zc = 0.0f;
    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;

    // stage 32 tokens (K, phi(K), V) of selected block j starting at u0;
    // token `row` by the 8 threads of that row (phi of a whole row)
    auto stage = [&](int u0, int nu) {
        const bool ok = row < nu;
        float kx[16], px[16];
#pragma unroll
        for (int c = 0; c < 16; ++c)
            kx[c] = (ok && c < CS) ? ldx(Kh + (size_t)(u0 + row) * st.t + sub + 8 * c) : 0.0f;
        phi_row(kx, px, CS, phi_sm);
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) {
                const int x = row * d + sub + 8 * c;
                Kt[x] = kx[c];
                Pk[x] = ok ? px[c] : 0.0f;
                Vt[x] = ok ? ldx(Vh + (size_t)(u0 + row) * st.t + sub + 8 * c) : 0.0f;
            }
        __syncthreads();
    };

    // ---- pass 1: the forward quantities of the row
    for (int r = 0; r < k; ++r) {
        const int j = sel[r];
        for (int half = 0; half < 2; ++half) {
            const int u0 = j * 64 + half * 32;
            const int nu = min(32, N - u0);
            if (nu <= 0) break;
            stage(u0, nu);
            float s[32];
            float tmax = -INFINITY;
            for (int u = 0; u < 32; ++u) {
                float sp = 0.0f, ap = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        sp = fmaf(q[c], Kt[u * d + sub + 8 * c], sp);
                        ap = fmaf(pq[c], Pk[u * d + sub + 8 * c], ap);
                    }
                sp = row8(sp);
                ap = row8(ap);
                const bool ok = u < nu;
                s[u] = ok ? sp * isd : -INFINITY;
                tmax = fmaxf(tmax, s[u]);
                if (ok) {
                    zc += ap;
#pragma unroll
                    for (int c = 0; c < 16; ++c)
                        if (c < CS) corr[c] = fmaf(ap, Vt[u * d + sub + 8 * c], corr[c]);
                }
            }
            const float mn = fmaxf(m, tmax);
            const float resc = (m == -INFINITY) ? 0.0f : expf(m - mn);
            l *= resc;
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[c] *= resc;
            for (int u = 0; u < 32; ++u) {
                const float p = expf(s[u] - mn);
                l += p;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) acc[c] = fmaf(p, Vt[u * d + sub + 8 * c], acc[c]);
            }
            m = mn;
            __syncthreads();
        }
    }
    const float a = alpha_of(alpha, bh, H, qb, Tq, alpha_qblock);
    const float inv_l = k > 0 ? 1.0f / l : 0.0f;
    const float L = k > 0 ? m + logf(l) : 0.0f;
    float os[16], ol[16], dph[16], dn[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        os[c] = acc[c] * inv_l;
        ol[c] = 0.0f;
        dph[c] = 0.0f;
        dn[c] = 0.0f;
    }
    float den = 1.0f, ds = 0.0f;
    const float* hT = htot + (size_t)bh * d * d;
    const float* zT = ztot + (size_t)bh * d;
    if (lin) {
        // O_l = (phi(q) h_tot - corr) / (phi(q) . z_tot - zc); phi(q) rows in LDS
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) Rw[row * d + sub + 8 * c] = pq[c];
        float dz = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) dz = fmaf(pq[c], zT[sub + 8 * c], dz);
        den = row8(dz) - zc;
        float num[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) num[c] = 0.0f;
        for (int cb = 0; cb < d; cb += 32) {
            __syncthreads();
            for (int x = threadIdx.x; x < 32 * d; x += 256) Vt[x] = hT[(size_t)cb * d + x];
            __syncthreads();
            for (int cc = 0; cc < 32; ++cc) {
                const float pv = Rw[row * d + cb + cc];
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) num[c] = fmaf(pv, Vt[cc * d + sub + 8 * c], num[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) ol[c] = (num[c] - corr[c]) / den;
        // dn = (1 - a) g / den, ds = -((1 - a) g . O_l) / den
        float eo = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            dn[c] = (1.0f - a) * g[c] / den;
            eo = fmaf((1.0f - a) * g[c], ol[c], eo);
        }
        ds = -row8(eo) / den;
        // dphi(q) = h_tot dn + z_tot ds (the selected tokens come off in pass 2);
        // dn rows in LDS, h_tot in chunks of 32 columns
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) Rw[row * d + sub + 8 * c] = dn[c];
        for (int eb = 0; eb < d; eb += 16) {
            __syncthreads();
            for (int x = threadIdx.x; x < 16 * d; x += 256) {
                const int cr = x / 16, ec = x % 16;  // Vt[cr][ec] = h_tot[cr][eb + ec]
                Vt[cr * 17 + ec] = hT[(size_t)cr * d + eb + ec];
            }
            __syncthreads();
            for (int ec = 0; ec < 16; ++ec) {
                const float w = Rw[row * d + eb + ec];
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) dph[c] = fmaf(Vt[(sub + 8 * c) * 17 + ec], w, dph[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) dph[c] = fmaf(zT[sub + 8 * c], ds, dph[c]);
        __syncthreads();
    }
    // D = a g . O_s; dalpha row value g . (O_s - O_l)
    float Dp = 0.0f, dap = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        Dp = fmaf(a * g[c], os[c], Dp);
        dap = fmaf(g[c], os[c] - ol[c], dap);
    }
    const float D = row8(Dp);
    const float da = row8(dap);

    // ---- pass 2: dq from the selected tokens
    float dq[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) dq[c] = 0.0f;
    for (int r = 0; r < k; ++r) {
        const int j = sel[r];
        for (int half = 0; half < 2; ++half) {
            const int u0 = j * 64 + half * 32;
            const int nu = min(32, N - u0);
            if (nu <= 0) break;
            stage(u0, nu);
            for (int u = 0; u < nu; ++u) {
                float sp = 0.0f, dp = 0.0f, vd = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        const float kv = Kt[u * d + sub + 8 * c], vv = Vt[u * d + sub + 8 * c];
                        sp = fmaf(q[c], kv, sp);
                        dp = fmaf(a * g[c], vv, dp);
                        vd = fmaf(vv, dn[c], vd);
                    }
                sp = row8(sp);
                dp = row8(dp);
                vd = row8(vd);
                const float p = expf(sp * isd - L);
                const float dl = p * (dp - D) * isd;
                const float cc = vd + ds;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        dq[c] = fmaf(dl, Kt[u * d + sub + 8 * c], dq[c]);
                        if (lin) dph[c] = fmaf(-cc, Pk[u * d + sub + 8 * c], dph[c]);
                    }
            }
            __syncthreads();
        }
    }
    float dqp[16];
    dphi_row(q, pq, dph, dqp, CS, phi_sm);
    if (valid_q) {
        const size_t o = head_base(st, bh, H) + (size_t)tq * st.t + sub;
        const size_t rr = (size_t)bh * N + tq;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) {
                dQ[o + 8 * c] = dq[c] + (lin ? dqp[c] : 0.0f);
                dn_out[rr * d + sub + 8 * c] = dn[c];
            }
        if (sub == 0) {
            lse[rr] = L;
            Dv[rr] = D;
            dsv[rr] = ds;
            da_row[rr] = da;
        }
    }
}

// dH_tot[c][e] = sum_t phi(q_t)[c] dn_t[e], dZ_tot[c] = sum_t phi(q_t)[c] ds_t
// per chunk of rows (partials, then summed in chunk order).  grid (chunks,
// BH), 256 threads: 16 x 16 threads, d/16 rows and columns each.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dh_kernel(const T* __restrict__ Q,
                                                     const float* __restrict__ dn,
                                                     const float* __restrict__ dsv,
                                                     float* __restrict__ hpart,
                                                     float* __restrict__ zpart, int N, int d,
                                                     int nch, int H, Strides st, int phi_sm) {
    __shared__ float pq[32 * 128];
    __shared__ float dv[32 * 128];
    __shared__ float sds[32];
    const int chunk = blockIdx.x;
    const long bh = blockIdx.y;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int SB = d >> 4;
    const int t_begin = chunk * kSummBlocksPerChunk * 64;
    const int t_end = min(N, t_begin + kSummBlocksPerChunk * 64);
    const T* Qh = Q + head_base(st, bh, H);
    float acc[8][8];
    float z[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        z[p] = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[p][q] = 0.0f;
    }
    const int lr = threadIdx.x >> 3, lsub = threadIdx.x & 7, CS = d >> 3;
    for (int u0 = t_begin; u0 < t_end; u0 += 32) {
        {  // row lr by the 8 threads of that row (phi of a whole row)
            const int t = u0 + lr;
            const bool ok = t < t_end;
            float qx[16], px[16];
#pragma unroll
            for (int c = 0; c < 16; ++c)
                qx[c] = (ok && c < CS) ? ldx(Qh + (size_t)t * st.t + lsub + 8 * c) : 0.0f;
            phi_row(qx, px, CS, phi_sm);
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (c < CS) {
                    const int ch = lsub + 8 * c;
                    pq[lr * d + ch] = ok ? px[c] : 0.0f;
                    dv[lr * d + ch] = ok ? dn[((size_t)bh * N + t) * d + ch] : 0.0f;
                }
        }
        if (threadIdx.x < 32) {
            const int t = u0 + threadIdx.x;
            sds[threadIdx.x] = t < t_end ? dsv[(size_t)bh * N + t] : 0.0f;
        }
        __syncthreads();
        for (int u = 0; u < 32; ++u) {
            float av[8], bv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                av[q] = q < SB ? pq[u * d + ty * SB + q] : 0.0f;
                bv[q] = q < SB ? dv[u * d + tx * SB + q] : 0.0f;
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                z[p] = fmaf(av[p], sds[u], z[p]);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[p][q] = fmaf(av[p], bv[q], acc[p][q]);
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

// For every KV block, the query blocks that select it, ascending: offsets
// off[bh][j .. j+1] into list[bh][...].  One work-group per head.
__global__ __launch_bounds__(256) void invert_kernel(const int32_t* __restrict__ idx, int Tq,
                                                     int Tkv, int k, int32_t* __restrict__ off,
                                                     int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ list) {
    const long bh = blockIdx.x;
    const int32_t* I = idx + (size_t)bh * Tq * k;
    int32_t* o = off + (size_t)bh * (Tkv + 1);
    int32_t* c = cnt + (size_t)bh * Tkv;
    int32_t* L = list + (size_t)bh * Tq * k;
    for (int j = threadIdx.x; j < Tkv; j += 256) c[j] = 0;
    __syncthreads();
    for (int x = threadIdx.x; x < Tq * k; x += 256) atomicAdd(&c[I[x]], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = 0;
        for (int j = 0; j < Tkv; ++j) {
            o[j] = s;
            s += c[j];
            c[j] = 0;
        }
        o[Tkv] = s;
    }
    __syncthreads();
    // query blocks in ascending order; the k entries of a row are distinct
    for (int i = 0; i < Tq; ++i) {
        for (int r = threadIdx.x; r < k; r += 256) {
            const int j = I[(size_t)i * k + r];
            L[o[j] + c[j]] = i;
            c[j] += 1;
        }
        __syncthreads();
    }
}

// Keys: 32 keys per work-group (half of a KV block), 8 threads per key.
// grid (Tkv * 2, BH), 256 threads.  Rows of the query blocks that select the
// block are staged 16 at a time.
template <typename T>
__global__ __launch_bounds__(256) void bwd_keys_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ alpha,
    const float* __restrict__ lse, const float* __restrict__ Dv, const float* __restrict__ dsv,
    const float* __restrict__ dn, const float* __restrict__ dHt, const float* __restrict__ dZt,
    const int32_t* __restrict__ off, const int32_t* __restrict__ list, float* __restrict__ dK,
    float* __restrict__ dV, int N, int d, int bq, int Tq, int Tkv, int k, int H, Strides st,
    int alpha_qblock, int phi_sm) {
    __shared__ float sQ[16 * 128];
    __shared__ float sP[16 * 128];  // phi(q)
    __shared__ float sG[16 * 128];  // alpha dO
    __shared__ float sN[16 * 128];  // dn
    __shared__ float sL[16], sD[16], sS[16];
    __shared__ int sOk[16];
    const int j = blockIdx.x >> 1, half = blockIdx.x & 1;
    const long bh = blockIdx.y;
    const int key = threadIdx.x >> 3, sub = threadIdx.x & 7;
    const int CS = d >> 3;  // channels sub, sub + 8, ... (conflict-free LDS reads)
    const int u = j * 64 + half * 32 + key;
    const bool valid_k = u < N;
    const T* Qh = Q + head_base(st, bh, H);
    const T* Kh = K + head_base(st, bh, H);
    const T* Vh = V + head_base(st, bh, H);
    const float* dOh = dO + head_base(st, bh, H);
    const float isd = 1.0f / sqrtf((float)d);
    const bool lin = k < Tkv;

    float kv[16], pk[16], vv[16], dk[16], dv[16], dph[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const bool ok = c < CS && valid_k;
        kv[c] = ok ? ldx(Kh + (size_t)u * st.t + sub + 8 * c) : 0.0f;
        vv[c] = ok ? ldx(Vh + (size_t)u * st.t + sub + 8 * c) : 0.0f;
        dk[c] = 0.0f;
        dv[c] = 0.0f;
        dph[c] = 0.0f;
    }
    phi_row(kv, pk, CS, phi_sm);
    const int32_t* o = off + (size_t)bh * (Tkv + 1);
    const int32_t* L = list + (size_t)bh * Tq * k;
    const int n0 = k > 0 ? o[j] : 0, n1 = k > 0 ? o[j + 1] : 0;
    for (int n = n0; n < n1; ++n) {
        const int i = L[n];
        const float a = alpha_of(alpha, bh, H, i, Tq, alpha_qblock);
        for (int r0 = 0; r0 < bq; r0 += 16) {
            __syncthreads();
            for (int x = threadIdx.x; x < 16 * d; x += 256) {
                const int rr = x / d, c = x % d;
                const int t = i * bq + r0 + rr;
                const bool ok = t < N;
                sG[rr * d + c] = ok ? a * dOh[(size_t)t * st.t + c] : 0.0f;
                sN[rr * d + c] = ok ? dn[((size_t)bh * N + t) * d + c] : 0.0f;
            }
            if (threadIdx.x < 128) {  // 16 rows of q and phi(q), 8 threads a row
                const int rr = threadIdx.x >> 3;
                const int t = i * bq + r0 + rr;
                const bool ok = t < N;
                float qx[16], px[16];
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    qx[c] = (ok && c < CS) ? ldx(Qh + (size_t)t * st.t + sub + 8 * c) : 0.0f;
                phi_row(qx, px, CS, phi_sm);
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        sQ[rr * d + sub + 8 * c] = qx[c];
                        sP[rr * d + sub + 8 * c] = px[c];
                    }
            }
            if (threadIdx.x < 16) {
                const int t = i * bq + r0 + threadIdx.x;
                const bool ok = t < N;
                sOk[threadIdx.x] = ok;
                sL[threadIdx.x] = ok ? lse[(size_t)bh * N + t] : 0.0f;
                sD[threadIdx.x] = ok ? Dv[(size_t)bh * N + t] : 0.0f;
                sS[threadIdx.x] = ok ? dsv[(size_t)bh * N + t] : 0.0f;
            }
            __syncthreads();
            for (int rr = 0; rr < 16; ++rr) {
                if (!sOk[rr]) break;  // rows past N come last
                float sp = 0.0f, dp = 0.0f, ap = 0.0f, vd = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        sp = fmaf(kv[c], sQ[rr * d + sub + 8 * c], sp);
                        dp = fmaf(vv[c], sG[rr * d + sub + 8 * c], dp);
                        ap = fmaf(pk[c], sP[rr * d + sub + 8 * c], ap);
                        vd = fmaf(vv[c], sN[rr * d + sub + 8 * c], vd);
                    }
                sp = row8(sp);
                dp = row8(dp);
                ap = row8(ap);
                vd = row8(vd);
                const float p = expf(sp * isd - sL[rr]);
                const float dl = p * (dp - sD[rr]) * isd;
                const float cc = vd + sS[rr];
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        dk[c] = fmaf(dl, sQ[rr * d + sub + 8 * c], dk[c]);
                        dv[c] = fmaf(p, sG[rr * d + sub + 8 * c], dv[c]);
                        if (lin) {
                            dv[c] = fmaf(-ap, sN[rr * d + sub + 8 * c], dv[c]);
                            dph[c] = fmaf(-cc, sP[rr * d + sub + 8 * c], dph[c]);
                        }
                    }
            }
        }
    }
    if (lin) {
        // dv += phi(k) dH_tot (columns of this thread), dphi(k) += dH_tot v + dZ_tot
        // (rows of this thread); phi(k) and v of every key through LDS
        const float* H0 = dHt + (size_t)bh * d * d;
        const float* Z0 = dZt + (size_t)bh * d;
        for (int kh = 0; kh < 2; ++kh) {  // keys 16 kh .. 16 kh + 15 through LDS
            __syncthreads();
            if ((key >> 4) == kh) {
#pragma unroll
                for (int c = 0; c < 16; ++c)
                    if (c < CS) {
                        sP[(key & 15) * d + sub + 8 * c] = pk[c];
                        sN[(key & 15) * d + sub + 8 * c] = vv[c];
                    }
            }
            __syncthreads();
            if ((key >> 4) == kh) {
                const int kk = key & 15;
                for (int cc = 0; cc < d; ++cc) {
                    const float pc = sP[kk * d + cc], vc = sN[kk * d + cc];
#pragma unroll
                    for (int c = 0; c < 16; ++c)
                        if (c < CS) {
                            // dv[e] += phi(k)[cc] dH[cc][e];  dphi[c] += dH[c][cc] v[cc]
                            dv[c] = fmaf(pc, H0[(size_t)cc * d + sub + 8 * c], dv[c]);
                            dph[c] = fmaf(H0[(size_t)(sub + 8 * c) * d + cc], vc, dph[c]);
                        }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) dph[c] += Z0[sub + 8 * c];
    }
    float dkp[16];
    dphi_row(kv, pk, dph, dkp, CS, phi_sm);
    if (valid_k) {
        const size_t ob = head_base(st, bh, H) + (size_t)u * st.t + sub;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (c < CS) {
                dK[ob + 8 * c] = dk[c] + (lin ? dkp[c] : 0.0f);
                dV[ob + 8 * c] = dv[c];
            }
    }
}

// dalpha: per head (or per head and query block), the row values summed over
// batch and rows in a fixed order: 256 threads take interleaved rows (fp64
// partial sums), combined by a fixed tree.  grid (H or H * Tq).
__global__ __launch_bounds__(256) void dalpha_kernel(const float* __restrict__ da_row,
                                                     float* __restrict__ dalpha, int B, int H,
                                                     int N, int bq, int Tq, int per_qblock) {
    __shared__ double red[4];
    const int x = blockIdx.x;
    const int h = per_qblock ? x / Tq : x;
    const int qb = per_qblock ? x % Tq : 0;
    const int t0 = per_qblock ? qb * bq : 0, t1 = per_qblock ? min(N, t0 + bq) : N;
    double part = 0.0;
    for (int b = 0; b < B; ++b) {
        const float* r = da_row + ((size_t)b * H + h) * N;
        for (int t = t0 + (int)threadIdx.x; t < t1; t += 256) part += (double)r[t];
    }
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) dalpha[x] = (float)((red[0] + red[1]) + (red[2] + red[3]));
}

}  // namespace

hipError_t launch_invert(const Dims& D, const int32_t* idx, const BwdWS& bw, hipStream_t s) {
    invert_kernel<<<dim3((unsigned)D.BH), 256, 0, s>>>(idx, D.Tq, D.Tkv, D.k, bw.off, bw.cnt,
                                                       bw.list);
    return hipGetLastError();
}

hipError_t launch_dalpha(const Dims& D, const BwdWS& bw, float* dalpha, hipStream_t s) {
    const int na = D.alpha_qblock ? D.H * D.Tq : D.H;
    dalpha_kernel<<<dim3((unsigned)na), 256, 0, s>>>(bw.da, dalpha, D.B, D.H, D.N, D.bq, D.Tq,
                                                     D.alpha_qblock);
    return hipGetLastError();
}

hipError_t launch_backward(const Dims& D, const void* Q, const void* K, const void* V,
                           const float* dO, const int32_t* idx, const float* alpha, float* dQ,
                           float* dK, float* dV, float* dalpha, const FwdWS& ws,
                           const BwdWS& bw, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (bwd_mfma_path(D)) {
        e = launch_backward_mfma(D, Q, K, V, dO, idx, alpha, dQ, dK, dV, ws, bw, s);
        if (e != hipSuccess) return e;
        return launch_dalpha(D, bw, dalpha, s);
    }
    const int nch = summ_chunks(D);
    const bool f32 = D.dtype == SLA2_F32;
    if (D.k < D.Tkv) {
        e = launch_summaries_valu(D, K, V, ws, s);
        if (e != hipSuccess) return e;
    }
    dim3 gr(D.Tq * (D.bq / 32), (unsigned)D.BH);
    timing_before(s, K_BWD_ROWS);
    if (f32)
        bwd_rows_kernel<float><<<gr, 256, 0, s>>>(
            (const float*)Q, (const float*)K, (const float*)V, dO, idx, alpha, ws.htot, ws.ztot,
            dQ, bw.lse, bw.D, bw.ds, bw.dn, bw.da, D.N, D.d, D.bq, D.Tq, D.Tkv, D.k, D.H, D.st,
            D.alpha_qblock, D.phi_sm);
    else
        bwd_rows_kernel<uint16_t><<<gr, 256, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, dO, idx, alpha, ws.htot,
            ws.ztot, dQ, bw.lse, bw.D, bw.ds, bw.dn, bw.da, D.N, D.d, D.bq, D.Tq, D.Tkv, D.k, D.H,
            D.st, D.alpha_qblock, D.phi_sm);
    timing_after(s, K_BWD_ROWS);
    if (D.k < D.Tkv) {
        dim3 gh(nch, (unsigned)D.BH);
        timing_before(s, K_BWD_DH);
        if (f32)
            bwd_dh_kernel<float><<<gh, 256, 0, s>>>((const float*)Q, bw.dn, bw.ds, ws.hpart,
                                                    ws.zpart, D.N, D.d, nch, D.H, D.st,
                                                    D.phi_sm);
        else
            bwd_dh_kernel<uint16_t><<<gh, 256, 0, s>>>((const uint16_t*)Q, bw.dn, bw.ds,
                                                       ws.hpart, ws.zpart, D.N, D.d, nch, D.H,
                                                       D.st, D.phi_sm);
        timing_after(s, K_BWD_DH);
        // reduce into dH_tot / dZ_tot (the forward's totals are no longer needed)
        FwdWS r = ws;
        r.htot = bw.dHt;
        r.ztot = bw.dZt;
        e = launch_summaries_reduce(D, r, s);
        if (e != hipSuccess) return e;
    }
    if (D.k > 0) {
        e = launch_invert(D, idx, bw, s);
        if (e != hipSuccess) return e;
    }
    dim3 gk(D.Tkv * 2, (unsigned)D.BH);
    timing_before(s, K_BWD_KEYS);
    if (f32)
        bwd_keys_kernel<float><<<gk, 256, 0, s>>>(
            (const float*)Q, (const float*)K, (const float*)V, dO, alpha, bw.lse, bw.D, bw.ds,
            bw.dn, bw.dHt, bw.dZt, bw.off, bw.list, dK, dV, D.N, D.d, D.bq, D.Tq, D.Tkv, D.k, D.H,
            D.st, D.alpha_qblock, D.phi_sm);
    else
        bwd_keys_kernel<uint16_t><<<gk, 256, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, dO, alpha, bw.lse, bw.D,
            bw.ds, bw.dn, bw.dHt, bw.dZt, bw.off, bw.list, dK, dV, D.N, D.d, D.bq, D.Tq, D.Tkv,
            D.k, D.H, D.st, D.alpha_qblock, D.phi_sm);
    timing_after(s, K_BWD_KEYS);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dalpha(D, bw, dalpha, s);
}

}  // namespace sla2
