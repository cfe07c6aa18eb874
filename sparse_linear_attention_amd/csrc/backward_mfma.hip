// Backward of the SLA2 forward on the matrix cores: bf16 Q, K, V with
// d = b_q = 128, b_kv = 64, phi = elu + 1; fp32 dO and gradients; the hard
// selection is held fixed.  L = sum dO . O, O = alpha O_s + (1 - alpha) O_l
// ("SLA2 深度解读" 04; SLA notes, key designs 3 and 4: the sparse part
// backpropagates as in FlashAttention, the linear part by the chain rule with
// per-block dH, dZ collected by additions).
//
// Sparse part, per row t of query block i (g = dO_t, selected tokens u):
//   P_tu = exp(l_tu - LSE_t), D_t = alpha g . O_s,t,
//   dl_tu = P_tu (alpha g . v_u - D_t) / sqrt(d);
//   dq_t = sum_u dl_tu k_u, dk_u = sum_t dl_tu q_t, dv_u = sum_t P_tu alpha g_t.
// Linear part, per query block i, with H_i = h_tot - sum over the selected
// blocks of h_j (Z_i likewise), s_t = phi(q_t) . Z_i, O_l,t = phi(q_t) H_i / s_t,
// e = (1 - alpha) g, dn_t = e / s_t, ds_t = -(e . O_l,t) / s_t:
//   dphi(q_t) = H_i dn_t + Z_i ds_t;  dH_i = sum_t phi(q_t)^T dn_t,
//   dZ_i = sum_t phi(q_t) ds_t;  every block summary receives the dH_i of
//   the query blocks that do not select it, dh_j = dH_tot - sum over the
//   selecting i of dH_i (dz_j likewise), and passes it to its tokens:
//   dphi(k_u) = dh_j v_u + dz_j, dv_u += phi(k_u) dh_j.
//
// Kernels, in launch order: per-block summaries h_j, z_j and their totals;
// the linear rows pass (dQ's phi part, dH_i, dZ_i, g . O_l); dH_tot; the
// selection inverted per KV block; the linear keys pass (dK's phi part and
// dV's linear part); the sparse rows pass (recomputes LSE and O_s, then dQ);
// the sparse keys pass (dK, dV over the query blocks that select each KV
// block).  The two linear passes are fp32 vector-ALU products on LDS tiles.
// The sparse passes run every product on the bf16 matrix cores (32x32x16):
// Q, K, V enter exactly; every fp32 operand (P, dl, alpha dO) is split into
// a bf16 high part and the bf16 rounding of the rest, and the products keep
// the hi*hi, hi*lo and lo*hi terms (16 significant bits per operand).
#include <type_traits>

#include "cdna4.h"
#include "sla2_internal.h"

namespace sla2 {
namespace {
using namespace cdna4;

constexpr int kD = 128;
constexpr int kLd = 129;  // row stride of fp32 LDS matrices: rows and columns hit distinct banks
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float phi1(float x) { return x > 0.0f ? x + 1.0f : expf(x); }
// phi'(x) from y = phi(x): 1 where x > 0 (there y > 1), else e^x = y
__device__ inline float dphi_of(float y) { return fminf(y, 1.0f); }

// sum over the 16 lanes that share t >> 4 (fixed butterfly order)
__device__ inline float sum16(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

// NT side-by-side 32x32 tiles (columns n0 + 32 i) of C += A B over kk < K
// on the fp32 matrix cores (32x32x2, exact fp32 products): lane l supplies
// A(m0 + l%32, kk + l/32) and B(kk + l/32, n0 + 32 i + l%32), with A(m, kk)
// = A[m am + kk ak] and B(kk, n) = B[kk bk + n bn] in LDS.  Tile i's
// register r holds C(m0 + 8 (r/4) + 4 (l/32) + r%4, n0 + 32 i + l%32).
template <int NT>
__device__ inline void mfma_f32_row(f32x16 (&c)[NT], const float* A, int am, int ak,
                                    const float* B, int bk, int bn, int m0, int n0, int K,
                                    int lane) {
    const int l32 = lane & 31, h = lane >> 5;
    const float* pa = A + (m0 + l32) * am + h * ak;
    const float* pb = B + h * bk + (n0 + l32) * bn;
#pragma unroll 4
    for (int kk = 0; kk < K; kk += 2) {
        const float av = pa[kk * ak];
#pragma unroll
        for (int i = 0; i < NT; ++i)
            c[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, pb[kk * bk + 32 * i * bn], c[i], 0,
                                                        0, 0);
    }
}
// Work-groups run round-robin over the 8 XCDs (dispatch index g on XCD g % 8).
// For the per-KV-block passes, whose work grows with the number of query
// blocks selecting the block (the first and last blocks of a sequence are
// selected far more often), the blocks of a head are dealt to the XCDs
// interleaved (XCD x takes positions x, x + 8, ... of one head at a time),
// and position p is block p / 2 for even p and T - 1 - p / 2 for odd p, so
// both heavy ends come early and each head ends with light blocks.
__device__ inline bool head_interleaved_map(int g, int T, long* bh, int* j) {
    const int R = (T + 7) >> 3;
    const int x = g & 7, s = g >> 3;
    *bh = s / R;
    const int p = (s % R) * 8 + x;
    *j = (p & 1) ? T - 1 - (p >> 1) : (p >> 1);
    return p < T;
}

// row of register r of a 32x32 accumulator tile, relative to the tile
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// rows r0 .. r0 + 63 of a head's [rows][128] bf16 matrix (rows st_t elements
// apart) as fp32 into an LDS matrix with row stride kLd, through phi when
// PHI; rows at or past N are 0.  16-byte loads, 4 per thread.
template <bool PHI>
__device__ inline void fill64(float* dst, const uint16_t* src, int st_t, int r0, int N, int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x = t + 256 * i, u = x >> 4, c8 = (x & 15) * 8, tok = r0 + u;
        const bool ok = tok < N;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(src + (size_t)tok * st_t + c8);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float lo = __uint_as_float(wv[q] << 16), hi = __uint_as_float(wv[q] & 0xffff0000u);
            if (PHI) {
                lo = ok ? phi1(lo) : 0.0f;
                hi = ok ? phi1(hi) : 0.0f;
            }
            dst[u * kLd + c8 + 2 * q] = lo;
            dst[u * kLd + c8 + 2 * q + 1] = hi;
        }
    }
}
// base - sum of bf16 d x d matrices, per thread: floats 8 (t + 256 m) .. +7
// (m < 8) of the flattened matrix
__device__ inline void load_base8(float (&acc)[8][8], const float* base, int t) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 a = *reinterpret_cast<const float4*>(base + 8 * (t + 256 * m));
        const float4 b = *reinterpret_cast<const float4*>(base + 8 * (t + 256 * m) + 4);
        acc[m][0] = a.x;
        acc[m][1] = a.y;
        acc[m][2] = a.z;
        acc[m][3] = a.w;
        acc[m][4] = b.x;
        acc[m][5] = b.y;
        acc[m][6] = b.z;
        acc[m][7] = b.w;
    }
}
// z - src(0) - .. - src(n - 1), in that order, four loads at a time
template <typename F>
__device__ inline float sub_seq(float z, int n, F src) {
    int r = 0;
    for (; r + 4 <= n; r += 4) {
        const float a = src(r), b = src(r + 1), c = src(r + 2), d = src(r + 3);
        z -= a;
        z -= b;
        z -= c;
        z -= d;
    }
    for (; r < n; ++r) z -= src(r);
    return z;
}
// acc -= the fp32 d x d matrix src (the same entries as load_base8)
__device__ inline void sub_f32_8(float (&acc)[8][8], const float* src, int t) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 a = *reinterpret_cast<const float4*>(src + 8 * (t + 256 * m));
        const float4 b = *reinterpret_cast<const float4*>(src + 8 * (t + 256 * m) + 4);
        acc[m][0] -= a.x;
        acc[m][1] -= a.y;
        acc[m][2] -= a.z;
        acc[m][3] -= a.w;
        acc[m][4] -= b.x;
        acc[m][5] -= b.y;
        acc[m][6] -= b.z;
        acc[m][7] -= b.w;
    }
}
__device__ inline void put_dd8(float* dst, const float (&acc)[8][8], int t) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int x = 8 * (t + 256 * m), r = x >> 7, c = x & 127;
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[r * kLd + c + i] = acc[m][i];
    }
}

// ---------------------------------------------------------------------------
// Linear rows pass: one work-group per (head, query block), 256 threads.
// Writes dQ (the phi chain; the first writer of dQ), dH_i, dZ_i and g . O_l
// per row into gol.  H_i = h_tot - S_i with S_i the sum of the bf16 h_j of
// the selected blocks, row i of the selection product (fp32; k > 0 only;
// it may be the row of dHq that this work-group overwrites at its end).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_lin_rows_kernel(
    const uint16_t* __restrict__ Q, const float* __restrict__ dO,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha,
    const float* __restrict__ htot, const float* __restrict__ ztot,
    const float* __restrict__ zblk, float* __restrict__ dQ,
    float* __restrict__ dHq, uint16_t* __restrict__ dHb16, float* __restrict__ dZq,
    float* __restrict__ gol, int N, int Tq, int Tkv, int k, int H, Strides st,
    int alpha_qblock, const float* ssel) {
    __shared__ float sH[kD * kLd];  // H_i [c][e]
    __shared__ float sA[64 * kLd];  // phi(q) of 64 rows [m][c]
    __shared__ float sB[64 * kLd];  // dn of the same rows [m][e]
    __shared__ float sZ[kD], sS[64], sDs[64];
    const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
    long bh;
    int qb;
    if (!head_major_map(blockIdx.x, Tq, &bh, &qb)) return;
    const long hb = head_base(st, bh, H);
    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;
    {
        float acc[8][8];
        load_base8(acc, htot + (size_t)bh * kD * kD, t);
        if (k > 0) sub_f32_8(acc, ssel + ((size_t)bh * Tq + qb) * kD * kD, t);
        put_dd8(sH, acc, t);
        if (t < kD)
            sZ[t] = sub_seq(ztot[(size_t)bh * kD + t], k, [&](int r) {
                return zblk[((size_t)bh * Tkv + sel[r]) * kD + t];
            });
    }
    const float a = alpha_of(alpha, bh, H, qb, Tq, alpha_qblock);
    const float om = 1.0f - a;
    const int lane = t & 63, w = t >> 6, l32 = lane & 31;
    // this wave's tiles of the 64-row x 128 products: (rows 32 mt, columns n0 + 32 i)
    const int mt = w & 1, n0 = 64 * (w >> 1);
    f32x16 dh[4];  // dH_i rows 32 w .., columns 32 i ..
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[i] = zero16();
    float dzp[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) dzp[p] = 0.0f;
    for (int half = 0; half < 2; ++half) {
        const int m0 = qb * 128 + 64 * half;
        __syncthreads();  // sH, sZ written; the previous half's reads of sA, sB done
        fill64<true>(sA, Q + hb, st.t, m0, N, t);
        __syncthreads();
        if (t < 64) {
            float sv = 0.0f;
            for (int c = 0; c < kD; ++c) sv = fmaf(sA[t * kLd + c], sZ[c], sv);
            sS[t] = sv;
        }
        {  // numerator phi(q) H_i into sB
            f32x16 n[2] = {zero16(), zero16()};
            mfma_f32_row<2>(n, sA, kLd, 1, sH, kLd, 1, 32 * mt, n0, kD, lane);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sB[(32 * mt + acc_row(r, lane)) * kLd + n0 + 32 * i + l32] = n[i][r];
        }
        __syncthreads();  // sS and the numerators
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int m = ty + 16 * p, tq = m0 + m;
            const bool ok = tq < N;
            const float inv = ok ? 1.0f / sS[m] : 0.0f;
            const float* grow = dO + hb + (size_t)(ok ? tq : 0) * st.t;
            float d1 = 0.0f, d2 = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int e = tx + 16 * q;
                const float g = ok ? grow[e] : 0.0f;
                const float ol = sB[m * kLd + e] * inv, ee = om * g;
                d1 = fmaf(ee, ol, d1);
                d2 = fmaf(g, ol, d2);
                sB[m * kLd + e] = ee * inv;  // dn replaces the numerator
            }
            d1 = sum16(d1);
            d2 = sum16(d2);
            if (tx == 0) {
                sDs[m] = -d1 * inv;
                if (ok) gol[(size_t)bh * N + tq] = d2;
            }
        }
        __syncthreads();
        {  // dphi(q) = dn H_i^T + ds Z_i^T; dQ = dphi phi'(q)
            f32x16 dp[2] = {zero16(), zero16()};
            mfma_f32_row<2>(dp, sB, kLd, 1, sH, 1, kLd, 32 * mt, n0, kD, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * mt + acc_row(r, lane), tq = m0 + m;
                if (tq >= N) continue;
                float* qo = dQ + hb + (size_t)tq * st.t;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int c = n0 + 32 * i + l32;
                    qo[c] = fmaf(sZ[c], sDs[m], dp[i][r]) * dphi_of(sA[m * kLd + c]);
                }
            }
        }
        // dH_i += phi(Q)^T dn, dZ_i += phi(Q)^T ds over these 64 rows
        mfma_f32_row<4>(dh, sA, 1, kLd, sB, kLd, 1, 32 * w, 0, 64, lane);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int c = ty + 16 * p;
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int m = tx + 16 * mm;
                dzp[p] = fmaf(sA[m * kLd + c], sDs[m], dzp[p]);
            }
        }
    }
    float* dHo = dHq + ((size_t)bh * Tq + qb) * kD * kD;
    uint16_t* dHo16 = dHb16 + ((size_t)bh * Tq + qb) * kD * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o = (32 * w + acc_row(r, lane)) * kD + 32 * i + l32;
            dHo[o] = dh[i][r];
            dHo16[o] = __builtin_bit_cast(uint16_t, (__bf16)dh[i][r]);
        }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const float z = sum16(dzp[p]);
        if (tx == 0) dZq[((size_t)bh * Tq + qb) * kD + ty + 16 * p] = z;
    }
}

// ---------------------------------------------------------------------------
// Linear keys pass: one work-group per (head, KV block j), 256 threads.
// dh_j = dH_tot - sum over the query blocks selecting j of dH_i (bf16; row j
// of the transposed selection product dsel, fp32; k > 0 only), dz_j
// likewise (gathered, fp32); writes
// dK = (dh_j v_u + dz_j) phi'(k_u) and dV = phi(k_u) dh_j (the first writers
// of dK and dV).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_lin_keys_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ dHt, const float* __restrict__ dZt,
    const float* __restrict__ dZq, const int32_t* __restrict__ off,
    const int32_t* __restrict__ list, float* __restrict__ dK,
    float* __restrict__ dV, int N, int Tq, int Tkv, int k, int H, Strides st,
    const float* __restrict__ dsel) {
    __shared__ float sH[kD * kLd];  // dh_j [c][e]
    __shared__ float sA[64 * kLd];  // V_j [u][e]
    __shared__ float sB[64 * kLd];  // phi(K_j) [u][c]
    __shared__ float sZ[kD];
    const int t = threadIdx.x;
    long bh;
    int j;
    if (!head_interleaved_map(blockIdx.x, Tkv, &bh, &j)) return;
    const long hb = head_base(st, bh, H);
    const int n0 = k > 0 ? off[(size_t)bh * (Tkv + 1) + j] : 0;
    const int n1 = k > 0 ? off[(size_t)bh * (Tkv + 1) + j + 1] : 0;
    const int32_t* L = list + (size_t)bh * Tq * k;
    {
        float acc[8][8];
        load_base8(acc, dHt + (size_t)bh * kD * kD, t);
        if (k > 0) sub_f32_8(acc, dsel + ((size_t)bh * Tkv + j) * kD * kD, t);
        put_dd8(sH, acc, t);
        if (t < kD)
            sZ[t] = sub_seq(dZt[(size_t)bh * kD + t], n1 - n0, [&](int r) {
                return dZq[((size_t)bh * Tq + L[n0 + r]) * kD + t];
            });
    }
    fill64<false>(sA, V + hb, st.t, j * 64, N, t);
    fill64<true>(sB, K + hb, st.t, j * 64, N, t);
    __syncthreads();
    const int lane = t & 63, w = t >> 6, l32 = lane & 31;
    const int mt = w & 1, c0 = 64 * (w >> 1);
    f32x16 x[2] = {zero16(), zero16()}, y[2] = {zero16(), zero16()};
    // x = sum_e v[u][e] dh[c][e], y = sum_c phi(k)[u][c] dh[c][e]
    mfma_f32_row<2>(x, sA, kLd, 1, sH, 1, kLd, 32 * mt, c0, kD, lane);
    mfma_f32_row<2>(y, sB, kLd, 1, sH, kLd, 1, 32 * mt, c0, kD, lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int u = 32 * mt + acc_row(r, lane), tok = j * 64 + u;
        if (tok >= N) continue;
        float* ko = dK + hb + (size_t)tok * st.t;
        float* vo = dV + hb + (size_t)tok * st.t;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = c0 + 32 * i + l32;
            ko[c] = (x[i][r] + sZ[c]) * dphi_of(sB[u * kLd + c]);
            vo[c] = y[i][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Per-KV-block summaries on the fp32 matrix cores: h_j = phi(K_j)^T V_j
// ([c][e], over the block's tokens below N; written rounded to bf16) and
// z_j = colsum phi(K_j) (fp32).  One work-group per (head, chunk of
// kBlkChunk blocks), 256 threads; the chunk's h_j and z_j summed in fp32
// (ascending j) into hpart / zpart[bh][chunk], from which sum_parts forms
// the head's totals.
// ---------------------------------------------------------------------------
constexpr int kBlkChunk = 8;

__global__ __launch_bounds__(256, 2) void blk_summ_kernel(const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       float* __restrict__ hpart,
                                                       float* __restrict__ zpart,
                                                       uint16_t* __restrict__ hb16,
                                                       float* __restrict__ zblk, int N, int Tkv,
                                                       int nch, int H, Strides st) {
    __shared__ float sP[64 * kLd];  // phi(K_j) [u][c]
    __shared__ float sV[64 * kLd];  // V_j [u][e]
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, l32 = lane & 31;
    long bh;
    int ch;
    if (!head_major_map(blockIdx.x, nch, &bh, &ch)) return;
    const long hb = head_base(st, bh, H);
    f32x16 hs[4] = {zero16(), zero16(), zero16(), zero16()};
    float zs = 0.0f;
    const int j1 = min(Tkv, (ch + 1) * kBlkChunk);
    for (int j = ch * kBlkChunk; j < j1; ++j) {
        __syncthreads();  // the previous block's reads of sP, sV are done
        fill64<true>(sP, K + hb, st.t, j * 64, N, t);
        fill64<false>(sV, V + hb, st.t, j * 64, N, t);
        __syncthreads();
        f32x16 h[4] = {zero16(), zero16(), zero16(), zero16()};
        mfma_f32_row<4>(h, sP, 1, kLd, sV, kLd, 1, 32 * w, 0, 64, lane);
        uint16_t* ho16 = hb16 + ((size_t)bh * Tkv + j) * kD * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int o = (32 * w + acc_row(r, lane)) * kD + 32 * i + l32;
                ho16[o] = __builtin_bit_cast(uint16_t, (__bf16)h[i][r]);
                hs[i][r] += h[i][r];
            }
        if (t < kD) {
            float z = 0.0f;
            for (int u = 0; u < 64; ++u) z += sP[u * kLd + t];
            zblk[((size_t)bh * Tkv + j) * kD + t] = z;
            zs += z;
        }
    }
    float* ho = hpart + ((size_t)bh * nch + ch) * kD * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) ho[(32 * w + acc_row(r, lane)) * kD + 32 * i + l32] = hs[i][r];
    if (t < kD) zpart[((size_t)bh * nch + ch) * kD + t] = zs;
}

// tot[bh][e] = sum over c < nch of part[bh][c][e] for the d*d entries of the
// matrices and the d entries of the vectors (entries past d*d index zpart);
// 8 interleaved slices of c per entry, added in a fixed order.  grid
// ((d*d + d) / 32, BH), 256 threads.
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part,
                                                        const float* __restrict__ zpart,
                                                        float* __restrict__ tot,
                                                        float* __restrict__ ztot, int nch) {
    __shared__ float red[8][33];
    const int t = threadIdx.x, sl = t >> 5;
    const long bh = blockIdx.y;
    const int e = blockIdx.x * 32 + (t & 31);
    const bool mat = e < kD * kD;
    const float* src = mat ? part + (size_t)bh * nch * kD * kD + e
                           : zpart + (size_t)bh * nch * kD + (e - kD * kD);
    const size_t stride = mat ? (size_t)kD * kD : (size_t)kD;
    float acc = 0.0f;
#pragma unroll 4
    for (int c = sl; c < nch; c += 8) acc += src[(size_t)c * stride];
    red[sl][t & 31] = acc;
    __syncthreads();
    if (sl == 0) {
        const int i = t & 31;
        const float v = ((red[0][i] + red[1][i]) + (red[2][i] + red[3][i])) +
                        ((red[4][i] + red[5][i]) + (red[6][i] + red[7][i]));
        if (mat) tot[(size_t)bh * kD * kD + e] = v;
        else ztot[(size_t)bh * kD + e - kD * kD] = v;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core helpers for the sparse passes.
//
// Tiles of 64 rows x 128 bf16 channels sit in LDS as [64][256 B] with the
// 16-byte chunk c of row r at chunk c ^ (r & 15).  A "row operand" of a
// 32x32x16 product (lane: one row, 8 channels) is one 16-byte read; a
// "column operand" (lane: one channel, 8 rows) is two transposed 8-byte
// reads (ds_read_b64_tr_b16).  The column operand's k order (element e = row
// 8 (e/4) + 4 (lane/32) + e%4 of its 16) is the order in which a 32x32
// accumulator holds its rows, so registers 8 h .. 8 h + 7 of an accumulator
// are the matching operand of rows 16 h .. 16 h + 15 with no data movement.
// The per-lane parts of both addresses are computed once (LaneOffs).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t head_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
__device__ inline void load_lds16(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SLA2_LDS(dst), 16, voff, soff, 0, 0);
}
__device__ inline void load_lds4(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SLA2_LDS(dst), 4, voff, soff, 0, 0);
}

struct LaneOffs {
    int ro[8];     // row operand, row (base + l32), chunk 2 ks + hl
    int co[4][2];  // column operand of m-tile mt (channels 32 mt ..), rows +0 / +8
};
// row base rb (a multiple of 32) folded in
__device__ inline void lane_offsets(int lane, int rb, LaneOffs& o) {
    const int l32 = lane & 31, hl = lane >> 5, r = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        o.ro[ks] = (rb + l32) * 256 + (((2 * ks + hl) ^ (l32 & 15)) << 4);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 4 * hl + (r >> 2) + 8 * h;  // within a 16-row group
            const int chunk = 4 * mt + 2 * g1 + ((r & 3) >> 1);
            o.co[mt][h] = (rb + row) * 256 + ((chunk ^ row) << 4) + (r & 1) * 8;
        }
}
__device__ inline bf16x8 row_op(const char* tile, const LaneOffs& o, int ks) {
    return *reinterpret_cast<const bf16x8*>(tile + o.ro[ks]);
}
// Column operands of the four m-tiles (channels 32 mt ..) of rows 16 g ..
// 16 g + 15, for tiles whose LDS address is base (a per-stage VGPR offset,
// plus the per-lane offsets: a[2 mt + h] = base + co[mt][h]) plus the
// constant OFF (tile offset + 4096 g).  The eight transposed reads sit in one
// asm block that waits for them before it ends, so their results are
// complete when the block returns; the compiler does not see them as reads
// of the tiles that direct-to-LDS loads fill (it would otherwise wait for
// every tile load in flight, including the prefetched ones), and the
// kernels' own vmcnt waits and barriers order them after those loads.
template <int OFF>
__device__ inline void col_ops4(const uint32_t (&a)[8], bf16x8 (&out)[4]) {
    s16x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "i"(OFF));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x4 rr[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const s16x4 x = rr[2 * mt], y = rr[2 * mt + 1];
        const s16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        out[mt] = __builtin_bit_cast(bf16x8, v);
    }
}
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)SLA2_LDS(p);
}
// per-stage column-operand addresses
__device__ inline void col_addrs(const char* stage, const LaneOffs& o, uint32_t (&a)[8]) {
    const uint32_t b = lds_addr(stage);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        a[2 * mt] = b + (uint32_t)o.co[mt][0];
        a[2 * mt + 1] = b + (uint32_t)o.co[mt][1];
    }
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi), two values per conversion
__device__ inline void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const f32x2 v = {x[e], x[e + 1]};
        const b16x2 h = __builtin_convertvector(v, b16x2);
        const f32x2 hf = __builtin_convertvector(h, f32x2);
        const f32x2 r = {v[0] - hf[0], v[1] - hf[1]};
        const b16x2 l = __builtin_convertvector(r, b16x2);
        hi[e] = h[0];
        hi[e + 1] = h[1];
        lo[e] = l[0];
        lo[e + 1] = l[1];
    }
}

// Rows j*64 .. j*64+63 of a head's [rows][128] bf16 matrix (rows rp bytes
// apart) into a tile by direct-to-LDS loads: piece u = 4 i + w (1 KB) holds
// rows 4 u .. 4 u + 3; the lane's 16 bytes are chunk (lane & 15) ^ (row & 15)
// of row 4 u + lane / 16.  Rows at or past n repeat row n - 1.
__device__ inline uint32_t tile_lane_off(int w, int lane, uint32_t rp) {
    const int row = 4 * w + (lane >> 4);
    return (uint32_t)row * rp + ((uint32_t)((lane & 15) ^ (row & 15)) << 4);
}
__device__ inline void issue_tile(char* dst, rsrc_t r, int j, int n, int w, int lane,
                                  uint32_t loff, uint32_t rp) {
    if (j * 64 + 64 <= n) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            load_lds16(r, loff, (uint32_t)j * 64 * rp + 16 * rp * i, dst + (4 * i + w) * 1024);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * i + 4 * w + (lane >> 4);
            const int tok = min(j * 64 + row, n - 1);
            const uint32_t o = (uint32_t)tok * rp + ((uint32_t)((lane & 15) ^ (row & 15)) << 4);
            load_lds16(r, o, 0, dst + (4 * i + w) * 1024);
        }
    }
}

// ---------------------------------------------------------------------------
// Sparse rows pass: one work-group of 4 waves per (head, query block); wave
// w owns queries 32 w .. 32 w + 31 (one per lane column).  Two passes over
// the selected KV tiles, run as one sequence of 2 k steps whose K and V
// tiles arrive by direct-to-LDS loads two steps ahead (three buffers):
//   1. S^T = K Q^T, online softmax, O_s^T += V^T P^T  ->  LSE, D = alpha g . O_s
//   2. S^T again, P = exp(S - LSE), dP^T = V (alpha G)^T, dl = P (dP - D) /
//      sqrt(d), dQ^T += K^T dl^T.
// dQ is added to the linear part when `lin` (else written); da = g . O_s -
// (lin ? da : 0).  For the keys pass it leaves, over the query blocks' whole
// 128 rows (rows past N: LSE = +inf, D = 0, alpha dO = 0), the log2-domain
// LSE, D and alpha dO split into bf16 high and low parts.
// ---------------------------------------------------------------------------
constexpr int kRStage = 32768;  // K tile, V tile
constexpr int kRLoads = 8;      // direct loads per wave and step

__global__ __launch_bounds__(256) void bwd_rows_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ dO,
    const int32_t* __restrict__ idx, const float* __restrict__ alpha, float* __restrict__ dQ,
    float* __restrict__ l2se, float* __restrict__ Dv, float* __restrict__ da,
    uint16_t* __restrict__ Gh, uint16_t* __restrict__ Gl, int N, int Tq, int k, int H,
    Strides st, int alpha_qblock, int lin) {
    __shared__ __attribute__((aligned(1024))) char lds[3 * kRStage];
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    long bh;
    int qb;
    if (!head_major_map(blockIdx.x, Tq, &bh, &qb)) return;
    const int tq = qb * 128 + 32 * w + l32;
    const bool valid_q = tq < N;
    const long hb = head_base(st, bh, H);
    const float c2 = kLog2e / sqrtf(128.0f);
    const float isd = 1.0f / sqrtf(128.0f);
    LaneOffs lo;
    lane_offsets(lane, 0, lo);

    bf16x8 qf[8];  // Q^T operand: query tq, channels 16 ks + 8 hl ..
    {
        const uint16_t* qrow = Q + hb + (size_t)(valid_q ? tq : 0) * st.t;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid_q) v = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;
    const uint32_t rp = (uint32_t)st.t * 2;
    const rsrc_t rk = head_rsrc(K + hb), rv = head_rsrc(V + hb);
    const uint32_t loff = tile_lane_off(w, lane, rp);
    const int nsteps = 2 * k;
    // step r: tile sel[r] (pass 1) or sel[r - k] (pass 2) into buffer r % 3
    auto issue = [&](int r) {
        char* dst = lds + (r % 3) * kRStage;
        const int j = sel[r < k ? r : r - k];
        issue_tile(dst, rk, j, N, w, lane, loff, rp);
        issue_tile(dst + 16384, rv, j, N, w, lane, loff, rp);
    };
    // wait for step r's tiles (this wave's loads, then every wave's)
    auto arrive = [&](int r) {
        if (r + 1 < nsteps) wait_vmcnt<kRLoads>();
        else wait_vmcnt<0>();
        wg_barrier();  // all waves are also done with step r - 1
        if (r + 2 < nsteps) issue(r + 2);
    };
    auto scores = [&](const char* kt, int j, f32x16 (&s)[2]) {
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                s[mt] = mfma_bf16(row_op(kt + 8192 * mt, lo, ks), qf[ks], s[mt]);
        if (j * 64 + 64 > N) {  // the ragged last block only
            asm volatile("" ::: "memory");
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (j * 64 + 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3) >= N)
                        s[mt][i] = -INFINITY;
        }
    };
    if (nsteps > 0) issue(0);
    if (nsteps > 1) issue(1);

    // ---- pass 1: LSE and O_s
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = zero16();
    float m2 = -INFINITY, lsum = 0.0f;
    for (int r = 0; r < k; ++r) {
        arrive(r);
        const char* kt = lds + (r % 3) * kRStage;
        uint32_t ca[8];
        col_addrs(kt, lo, ca);
        f32x16 s[2];
        scores(kt, sel[r], s);
        float mx = s[0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float xm = mx * c2;
        if (xm > m2) {
            const float f = __builtin_amdgcn_exp2f(m2 - xm);
            lsum *= f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[i][e] *= f;
            m2 = xm;
        }
        // O_s^T += V^T P^T, k-step kq = keys 16 kq .. 16 kq + 15
        auto pv = [&](auto kq_c) {
            constexpr int kq = decltype(kq_c)::value;
            float pv8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv8[e] = __builtin_amdgcn_exp2f(fmaf(s[kq >> 1][8 * (kq & 1) + e], c2, -m2));
                lsum += pv8[e];
            }
            bf16x8 ph, pl, av[4];
            split8(pv8, ph, pl);
            col_ops4<16384 + 4096 * kq>(ca, av);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                o[mt] = mfma_bf16(av[mt], ph, o[mt]);
                o[mt] = mfma_bf16(av[mt], pl, o[mt]);
            }
        };
        pv(std::integral_constant<int, 0>{});
        pv(std::integral_constant<int, 1>{});
        pv(std::integral_constant<int, 2>{});
        pv(std::integral_constant<int, 3>{});
    }
    const float l_all = lsum + __shfl_xor(lsum, 32);
    const float L2 = k > 0 ? m2 + log2f(l_all) : 0.0f;
    const float inv_l = k > 0 ? 1.0f / l_all : 0.0f;
    const float* grow = dO + hb + (size_t)(valid_q ? tq : 0) * st.t;
    float go = 0.0f;  // g . O_s over this lane's channels 32 mt + 8 i4 + 4 hl + 0..3
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            float4 g = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (valid_q) g = *reinterpret_cast<const float4*>(grow + 32 * mt + 8 * i4 + 4 * hl);
            go = fmaf(g.x, o[mt][4 * i4], go);
            go = fmaf(g.y, o[mt][4 * i4 + 1], go);
            go = fmaf(g.z, o[mt][4 * i4 + 2], go);
            go = fmaf(g.w, o[mt][4 * i4 + 3], go);
        }
    go = (go + __shfl_xor(go, 32)) * inv_l;
    const float a = alpha_of(alpha, bh, H, qb, Tq, alpha_qblock);
    const float Dq = a * go;

    // ---- pass 2: dQ
    bf16x8 gh[8], gl[8];  // (alpha G)^T operand: query tq, channels 16 ks + 8 hl ..
    const size_t prow = (size_t)bh * Tq * 128 + (size_t)qb * 128 + 32 * w + l32;  // padded row
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        float gv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] = 0.0f;
        if (valid_q) {
            const float4 g0 = *reinterpret_cast<const float4*>(grow + 16 * ks + 8 * hl);
            const float4 g1 = *reinterpret_cast<const float4*>(grow + 16 * ks + 8 * hl + 4);
            gv[0] = a * g0.x;
            gv[1] = a * g0.y;
            gv[2] = a * g0.z;
            gv[3] = a * g0.w;
            gv[4] = a * g1.x;
            gv[5] = a * g1.y;
            gv[6] = a * g1.z;
            gv[7] = a * g1.w;
        }
        split8(gv, gh[ks], gl[ks]);
        *reinterpret_cast<bf16x8*>(Gh + prow * 128 + 16 * ks + 8 * hl) = gh[ks];
        *reinterpret_cast<bf16x8*>(Gl + prow * 128 + 16 * ks + 8 * hl) = gl[ks];
    }
    if (hl == 0) {
        l2se[prow] = valid_q ? L2 : INFINITY;
        Dv[prow] = valid_q ? Dq : 0.0f;
    }
    f32x16 dq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dq[i] = zero16();
    for (int r = k; r < nsteps; ++r) {
        arrive(r);
        const char* kt = lds + (r % 3) * kRStage;
        const char* vt = kt + 16384;
        uint32_t ca[8];
        col_addrs(kt, lo, ca);
        f32x16 s[2];
        scores(kt, sel[r - k], s);
        f32x16 dp[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 av = row_op(vt + 8192 * mt, lo, ks);
                dp[mt] = mfma_bf16(av, gh[ks], dp[mt]);
                dp[mt] = mfma_bf16(av, gl[ks], dp[mt]);
            }
        // dQ^T += K^T dl^T, k-step kq
        auto kd = [&](auto kq_c) {
            constexpr int kq = decltype(kq_c)::value;
            float dl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = 8 * (kq & 1) + e;
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kq >> 1][i], c2, -L2));
                dl[e] = p * (dp[kq >> 1][i] - Dq) * isd;
            }
            bf16x8 dh, dlo, ak[4];
            split8(dl, dh, dlo);
            col_ops4<4096 * kq>(ca, ak);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                dq[mt] = mfma_bf16(ak[mt], dh, dq[mt]);
                dq[mt] = mfma_bf16(ak[mt], dlo, dq[mt]);
            }
        };
        kd(std::integral_constant<int, 0>{});
        kd(std::integral_constant<int, 1>{});
        kd(std::integral_constant<int, 2>{});
        kd(std::integral_constant<int, 3>{});
    }
    if (valid_q) {
        float* qo = dQ + hb + (size_t)tq * st.t;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                float4* p4 = reinterpret_cast<float4*>(qo + 32 * mt + 8 * i4 + 4 * hl);
                float4 v = make_float4(dq[mt][4 * i4], dq[mt][4 * i4 + 1], dq[mt][4 * i4 + 2],
                                       dq[mt][4 * i4 + 3]);
                if (lin) {
                    const float4 old = *p4;
                    v.x += old.x;
                    v.y += old.y;
                    v.z += old.z;
                    v.w += old.w;
                }
                *p4 = v;
            }
        if (hl == 0) {
            const size_t rr = (size_t)bh * N + tq;
            da[rr] = lin ? go - da[rr] : go;
        }
    }
}

// ---------------------------------------------------------------------------
// Sparse keys pass: one work-group of 4 waves per (head, KV block j); wave
// w owns keys 32 (w & 1) .. +31 of the block (one per lane column) and rows
// 32 (w >> 1) .. +31 of every 64-row stage of the query blocks that select
// j.  A stage holds Q, the high and low parts of alpha dO, LSE and D of 64
// rows; stages arrive by direct-to-LDS loads two ahead (three buffers).  Per
// stage:  S = Q K^T, P = exp(S - LSE), dP = (alpha G) V^T,
//         dl = P (dP - D) / sqrt d,  dV^T += (alpha G)^T P,  dK^T += Q^T dl.
// The two row halves are summed at the end (fixed order); dK and dV are
// added to the linear parts when `lin` (else written).
// ---------------------------------------------------------------------------
constexpr int kKStage = 3 * 16384 + 512;
constexpr int kKLoads = 14;  // direct loads per wave and stage

__global__ __launch_bounds__(256) void bwd_keys_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ Gh,
    const uint16_t* __restrict__ Gl, const float* __restrict__ l2se,
    const float* __restrict__ Dv, const int32_t* __restrict__ off,
    const int32_t* __restrict__ list, float* __restrict__ dK, float* __restrict__ dV, int N,
    int Tq, int Tkv, int k, int H, Strides st, int lin) {
    __shared__ __attribute__((aligned(1024))) char lds[3 * kKStage];
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kh = w & 1, qh = w >> 1;
    long bh;
    int j;
    if (!head_interleaved_map(blockIdx.x, Tkv, &bh, &j)) return;
    const int n0 = k > 0 ? off[(size_t)bh * (Tkv + 1) + j] : 0;
    const int n1 = k > 0 ? off[(size_t)bh * (Tkv + 1) + j + 1] : 0;
    const int nst = 2 * (n1 - n0);
    if (nst == 0 && lin) return;  // nothing to add
    const long hb = head_base(st, bh, H);
    const int u = j * 64 + 32 * kh + l32;
    const bool valid_k = u < N;
    const float c2 = kLog2e / sqrtf(128.0f);
    const float isd = 1.0f / sqrtf(128.0f);
    const int rb = 32 * qh;
    LaneOffs lo;
    lane_offsets(lane, rb, lo);

    bf16x8 kf[8], vf[8];  // K^T and V^T operands: key u, channels 16 ks + 8 hl ..
    {
        const uint16_t* krow = K + hb + (size_t)(valid_k ? u : 0) * st.t;
        const uint16_t* vrow = V + hb + (size_t)(valid_k ? u : 0) * st.t;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
            if (valid_k) {
                a = *reinterpret_cast<const uint4*>(krow + 16 * ks + 8 * hl);
                b = *reinterpret_cast<const uint4*>(vrow + 16 * ks + 8 * hl);
            }
            kf[ks] = __builtin_bit_cast(bf16x8, a);
            vf[ks] = __builtin_bit_cast(bf16x8, b);
        }
    }
    const int32_t* Ls = list + (size_t)bh * Tq * k;
    const int Np = Tq * 128;
    const uint32_t rpq = (uint32_t)st.t * 2;
    const rsrc_t rq = head_rsrc(Q + hb);
    const rsrc_t rgh = head_rsrc(Gh + (size_t)bh * Np * 128);
    const rsrc_t rgl = head_rsrc(Gl + (size_t)bh * Np * 128);
    const rsrc_t rl = head_rsrc(l2se + (size_t)bh * Np);
    const rsrc_t rd = head_rsrc(Dv + (size_t)bh * Np);
    const uint32_t loffq = tile_lane_off(w, lane, rpq), loffg = tile_lane_off(w, lane, 256);
    // stage s: rows 64 (s & 1) .. of query block list[n0 + s / 2] (64-row tile tb)
    auto issue = [&](int s) {
        char* dst = lds + (s % 3) * kKStage;
        const int tb = 2 * Ls[n0 + (s >> 1)] + (s & 1);
        issue_tile(dst, rq, tb, N, w, lane, loffq, rpq);
        issue_tile(dst + 16384, rgh, tb, Np, w, lane, loffg, 256);
        issue_tile(dst + 32768, rgl, tb, Np, w, lane, loffg, 256);
        if (lane < 16) {  // LSE and D: 16 rows per wave
            load_lds4(rl, (uint32_t)(16 * w + lane) * 4, (uint32_t)tb * 256, dst + 49152 + 64 * w);
            load_lds4(rd, (uint32_t)(16 * w + lane) * 4, (uint32_t)tb * 256,
                      dst + 49152 + 256 + 64 * w);
        }
    };

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dk[i] = zero16();
        dv[i] = zero16();
    }
    if (nst > 0) issue(0);
    if (nst > 1) issue(1);
    for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) wait_vmcnt<kKLoads>();  // stage s has landed for this wave ...
        else wait_vmcnt<0>();
        wg_barrier();  // ... and for every wave; all waves are done with stage s - 1
        if (s + 2 < nst) issue(s + 2);
        const char* sQ = lds + (s % 3) * kKStage;
        const char* sGh = sQ + 16384;
        const char* sGl = sQ + 32768;
        const float* sL = reinterpret_cast<const float*>(sQ + 49152);
        const float* sD = sL + 64;
        f32x16 sc = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            sc = mfma_bf16(row_op(sQ, lo, ks), kf[ks], sc);
            dp = mfma_bf16(row_op(sGh, lo, ks), vf[ks], dp);
            dp = mfma_bf16(row_op(sGl, lo, ks), vf[ks], dp);
        }
        float p[16], dl[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qr = rb + 8 * (i >> 2) + 4 * hl + (i & 3);
            p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -sL[qr]));
            dl[i] = p[i] * (dp[i] - sD[qr]) * isd;
        }
        uint32_t ca[8];
        col_addrs(sQ, lo, ca);
        auto kv = [&](auto kq_c) {
            constexpr int kq = decltype(kq_c)::value;
            bf16x8 ph, pl, dh, dlo, gth[4], gtl[4], qt[4];
            split8(p + 8 * kq, ph, pl);
            split8(dl + 8 * kq, dh, dlo);
            col_ops4<16384 + 4096 * kq>(ca, gth);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                dv[mt] = mfma_bf16(gth[mt], ph, dv[mt]);
                dv[mt] = mfma_bf16(gth[mt], pl, dv[mt]);
            }
            col_ops4<4096 * kq>(ca, qt);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                dk[mt] = mfma_bf16(qt[mt], dh, dk[mt]);
                dk[mt] = mfma_bf16(qt[mt], dlo, dk[mt]);
            }
            col_ops4<32768 + 4096 * kq>(ca, gtl);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) dv[mt] = mfma_bf16(gtl[mt], ph, dv[mt]);
        };
        kv(std::integral_constant<int, 0>{});
        kv(std::integral_constant<int, 1>{});
    }
    // rows 32..63 of every stage (waves qh = 1) onto rows 0..31 (qh = 0)
    float* red = reinterpret_cast<float*>(lds);  // [kh][mt][16][64 lanes]: 32 KB
#pragma unroll
    for (int arr = 0; arr < 2; ++arr) {
        __syncthreads();
        if (qh == 1) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    red[((kh * 4 + mt) * 16 + i) * 64 + lane] = arr ? dv[mt][i] : dk[mt][i];
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float x = red[((kh * 4 + mt) * 16 + i) * 64 + lane];
                    if (arr) dv[mt][i] += x;
                    else dk[mt][i] += x;
                }
        }
    }
    if (qh == 0 && valid_k) {
        float* ko = dK + hb + (size_t)u * st.t;
        float* vo = dV + hb + (size_t)u * st.t;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int ch = 32 * mt + 8 * i4 + 4 * hl;
                float4 a = make_float4(dk[mt][4 * i4], dk[mt][4 * i4 + 1], dk[mt][4 * i4 + 2],
                                       dk[mt][4 * i4 + 3]);
                float4 b = make_float4(dv[mt][4 * i4], dv[mt][4 * i4 + 1], dv[mt][4 * i4 + 2],
                                       dv[mt][4 * i4 + 3]);
                if (lin) {
                    const float4 ao = *reinterpret_cast<const float4*>(ko + ch);
                    const float4 bo = *reinterpret_cast<const float4*>(vo + ch);
                    a.x += ao.x;
                    a.y += ao.y;
                    a.z += ao.z;
                    a.w += ao.w;
                    b.x += bo.x;
                    b.y += bo.y;
                    b.z += bo.z;
                    b.w += bo.w;
                }
                *reinterpret_cast<float4*>(ko + ch) = a;
                *reinterpret_cast<float4*>(vo + ch) = b;
            }
    }
}

inline dim3 head_major_grid(long BH, int T) { return dim3((unsigned)(BH * 8 * ((T + 7) / 8))); }

hipError_t sum_parts(const Dims& D, const float* part, const float* zpart, float* tot,
                     float* ztot, int nch, hipStream_t s) {
    timing_before(s, K_BWD_SUM_PARTS);
    sum_parts_kernel<<<dim3((kD * kD + kD) / 32, (unsigned)D.BH), 256, 0, s>>>(part, zpart, tot,
                                                                              ztot, nch);
    timing_after(s, K_BWD_SUM_PARTS);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_mfma(const Dims& D, const void* Q, const void* K, const void* V,
                                const float* dO, const int32_t* idx, const float* alpha,
                                float* dQ, float* dK, float* dV, const FwdWS& ws,
                                const BwdWS& bw, hipStream_t s) {
    const bool lin = D.k < D.Tkv;
    // the selected sums by dense products (every valid problem fits them)
    const bool prod = lin && D.k > 0;
    if (prod && !sel_product_fits(D)) return hipErrorInvalidValue;
    const uint16_t* q = static_cast<const uint16_t*>(Q);
    const uint16_t* kk = static_cast<const uint16_t*>(K);
    const uint16_t* v = static_cast<const uint16_t*>(V);
    hipError_t e = hipSuccess;
    if (lin) {
        const int nch = bwd_summ_chunks(D);
        timing_before(s, K_BWD_BLK_SUMM);
        blk_summ_kernel<<<head_major_grid(D.BH, nch), 256, 0, s>>>(
            kk, v, bw.hblk, bw.zpart, bw.hb16, bw.zblk, D.N, D.Tkv, nch, D.H, D.st);
        timing_after(s, K_BWD_BLK_SUMM);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = sum_parts(D, bw.hblk, bw.zpart, ws.htot, ws.ztot, nch, s)) != hipSuccess)
            return e;
        // S_i (the selected h_j summed) as a dense 0/1 product into dHq,
        // which the rows pass reads and then overwrites row by row
        if (prod && (e = launch_sel_product(D, false, idx, nullptr, nullptr, bw.sbits, bw.hb16,
                                            bw.dHq, s)) != hipSuccess)
            return e;
        timing_before(s, K_BWD_LIN_ROWS);
        bwd_lin_rows_kernel<<<head_major_grid(D.BH, D.Tq), 256, 0, s>>>(
            q, dO, idx, alpha, ws.htot, ws.ztot, bw.zblk, dQ, bw.dHq, bw.dHb16, bw.dZq,
            bw.da, D.N, D.Tq, D.Tkv, D.k, D.H, D.st, D.alpha_qblock, prod ? bw.dHq : nullptr);
        timing_after(s, K_BWD_LIN_ROWS);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = sum_parts(D, bw.dHq, bw.dZq, bw.dHt, bw.dZt, D.Tq, s)) != hipSuccess) return e;
    }
    if (D.k > 0 && (e = launch_invert(D, idx, bw, s)) != hipSuccess) return e;
    if (lin) {
        // the selecting query blocks' dH_i summed per KV block, into hblk
        // (free once h_tot is formed)
        if (prod && (e = launch_sel_product(D, true, nullptr, bw.off, bw.list, bw.sbits,
                                            bw.dHb16, bw.hblk, s)) != hipSuccess)
            return e;
        timing_before(s, K_BWD_LIN_KEYS);
        bwd_lin_keys_kernel<<<head_major_grid(D.BH, D.Tkv), 256, 0, s>>>(
            kk, v, bw.dHt, bw.dZt, bw.dZq, bw.off, bw.list, dK, dV, D.N, D.Tq, D.Tkv,
            D.k, D.H, D.st, prod ? bw.hblk : nullptr);
        timing_after(s, K_BWD_LIN_KEYS);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    timing_before(s, K_BWD_ROWS_MFMA);
    bwd_rows_mfma_kernel<<<head_major_grid(D.BH, D.Tq), 256, 0, s>>>(
        q, kk, v, dO, idx, alpha, dQ, bw.lse, bw.D, bw.da, bw.gh, bw.gl, D.N, D.Tq, D.k, D.H,
        D.st, D.alpha_qblock, lin ? 1 : 0);
    timing_after(s, K_BWD_ROWS_MFMA);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (D.k > 0) {
        timing_before(s, K_BWD_KEYS_MFMA);
        bwd_keys_mfma_kernel<<<head_major_grid(D.BH, D.Tkv), 256, 0, s>>>(
            q, kk, v, bw.gh, bw.gl, bw.lse, bw.D, bw.off, bw.list, dK, dV, D.N, D.Tq, D.Tkv, D.k,
            D.H, D.st, lin ? 1 : 0);
        timing_after(s, K_BWD_KEYS_MFMA);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sla2
