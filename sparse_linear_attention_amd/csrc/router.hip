// Router kernels: block mean-pool + projection, compressed score, hard top-k
// ("SLA2 深度解读" section 05: Qbar = pool(Q), Kbar = pool(K),
// P_c = proj_q(Qbar) proj_k(Kbar)^T, M_c = Top-k(k%, P_c)).  The SLA (v1)
// router ("SLA: Beyond Sparsity ..." notes, key design 2) pools without
// projections and also marks the bottom k_l % of each row negligible.
//
// All arithmetic is fp64.  Block sums of <= 128 bf16 values are exact in
// fp64, so the pooled means do not depend on summation order; the scores
// are exact to fp64 rounding, which keeps the selection identical to any
// other fp64 evaluation unless two scores of a row lie within ~1e-15
// relative of each other at the k-th place.
#include "sla2_internal.h"

namespace sla2 {
namespace {

__device__ inline void load8(const float* __restrict__ p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

__device__ inline void load8(const uint16_t* __restrict__ p, float* o) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// One work-group per (head, block); blocks [0, Tq) are query blocks, the
// rest KV blocks.  Output: proj(mean of the valid rows) in fp64, or the mean
// itself when Wq and Wk are null (SLA v1).
template <typename T>
__global__ __launch_bounds__(256) void pool_project_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ Wq,
    const float* __restrict__ Wk, double* __restrict__ qt, double* __restrict__ kt, int N,
    int d, int bq, int bkv, int Tq, int Tkv, int H, int w_heads, Strides st) {
    __shared__ double part[2048];  // [R][d], R * d == 2048
    __shared__ double xbar[128];
    const int blk = blockIdx.x;
    const long bh = blockIdx.y;
    const bool isq = blk < Tq;
    const int j = isq ? blk : blk - Tq;
    const int bs = isq ? bq : bkv;
    const T* X = (isq ? Q : K) + head_base(st, bh, H);
    const int t0 = j * bs;
    const int n = min(bs, N - t0);
    const int groups = d >> 3;  // channel groups of 8
    const int g = threadIdx.x % groups;
    const int r = threadIdx.x / groups;
    const int R = 256 / groups;

    double s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0;
    for (int row = r; row < n; row += R) {
        float v[8];
        load8(X + (size_t)(t0 + row) * st.t + g * 8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += (double)v[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r * d + g * 8 + e] = s[e];
    __syncthreads();
    if (threadIdx.x < d) {
        const int c = threadIdx.x;
        double acc = 0.0;
        for (int rr = 0; rr < R; ++rr) acc += part[rr * d + c];
        xbar[c] = acc / (double)n;
    }
    __syncthreads();
    if (threadIdx.x < d) {
        const int e = threadIdx.x;
        const int h = (int)(bh % H);
        double* out = isq ? qt + ((size_t)bh * Tq + j) * d : kt + ((size_t)bh * Tkv + j) * d;
        if (!Wq) {
            out[e] = xbar[e];
        } else {
            const float* W = (isq ? Wq : Wk) + (w_heads == 1 ? 0 : (size_t)h * d * d);
            double y = 0.0;
            for (int c = 0; c < d; ++c) y = fma(xbar[c], (double)W[(size_t)c * d + e], y);
            out[e] = y;
        }
    }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// S[bh][i][j] = qt[bh][i] . kt[bh][j] on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64: A[i][k] in lane i + 16 k, B[k][j] in lane
// j + 16 k, D[i][j] in lane j + 16 (i % 4), item i / 4).  A 64 x 64 tile
// per work-group, 32 x 32 (2 x 2 products) per wave, operands straight from
// L2 (a head's qt and kt are (Tq + Tkv) d 8 B).  For channels k0 .. k0+7
// lane i + 16 kq loads the pair k0 + 2 kq, k0 + 2 kq + 1 of its row in one
// 16-byte load; the first product of the step takes the first of each pair,
// the second the other, so every channel enters each score exactly once.
// Rows past Tq / Tkv read the last row and are not stored.  d = 64 or 128.
template <int d>
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ qt,
                                                    const double* __restrict__ kt,
                                                    double* __restrict__ S, int Tq, int Tkv) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const long bh = blockIdx.z;
    const int iw = blockIdx.y * 64 + 32 * (w >> 1), jw = blockIdx.x * 64 + 32 * (w & 1);
    const double* A = qt + (size_t)bh * Tq * d;
    const double* B = kt + (size_t)bh * Tkv * d;
    const double* ar[2];
    const double* br[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        ar[m] = A + (size_t)min(iw + 16 * m + r16, Tq - 1) * d + 2 * kq;
        br[m] = B + (size_t)min(jw + 16 * m + r16, Tkv - 1) * d + 2 * kq;
    }
    f64x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k0 = 0; k0 < d; k0 += 8) {
        double2 a[2], b[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            a[m] = *reinterpret_cast<const double2*>(ar[m] + k0);
            b[m] = *reinterpret_cast<const double2*>(br[m] + k0);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mt].x, b[nt].x, acc[mt][nt],
                                                                   0, 0, 0);
                acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mt].y, b[nt].y, acc[mt][nt],
                                                                   0, 0, 0);
            }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = iw + 16 * mt + kq + 4 * r, j = jw + 16 * nt + r16;
                if (i < Tq && j < Tkv) S[((size_t)bh * Tq + i) * Tkv + j] = acc[mt][nt][r];
            }
}

// y = x W for the pooled rows of one (head, side) on the fp64 matrix cores,
// with the operand layouts of score_kernel: grid (row tiles of 64, 2 d / 64,
// BH) with y = side * (d / 64) + column tile (side 0: queries with Wq, 1:
// keys with Wk); 32 x 32 outputs (2 x 2 products) per wave.  Lane i + 16 kq
// loads the pair of channels k0 + 2 kq, k0 + 2 kq + 1 of its x row in one
// 16-byte load and the matching two fp32 entries of its W column; the two
// products of a step of 8 channels take the first and the second of each
// pair.  Rows past the side's count read its last row and are not stored.
template <int d>
__global__ __launch_bounds__(256) void proj_kernel(const double* __restrict__ xq,
                                                   const double* __restrict__ xk,
                                                   const float* __restrict__ Wq,
                                                   const float* __restrict__ Wk,
                                                   double* __restrict__ qt, double* __restrict__ kt,
                                                   int Tq, int Tkv, int H, int w_heads, int side0) {
    constexpr int ct = d / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const long bh = blockIdx.z;
    const int side = side0 + (int)blockIdx.y / ct;  // 0: queries, 1: keys
    const int rows = side ? Tkv : Tq;
    const int iw = blockIdx.x * 64 + 32 * (w >> 1);
    const int ew = ((int)blockIdx.y % ct) * 64 + 32 * (w & 1);
    if ((int)blockIdx.x * 64 >= rows) return;
    const double* X = side ? xk + (size_t)bh * Tkv * d : xq + (size_t)bh * Tq * d;
    const float* W = (side ? Wk : Wq) + (w_heads == 1 ? 0 : (size_t)(bh % H) * d * d);
    double* Y = side ? kt + (size_t)bh * Tkv * d : qt + (size_t)bh * Tq * d;
    const double* xr[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) xr[m] = X + (size_t)min(iw + 16 * m + r16, rows - 1) * d + 2 * kq;
    f64x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k0 = 0; k0 < d; k0 += 8) {
        double2 a[2];
        double b0[2], b1[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) a[m] = *reinterpret_cast<const double2*>(xr[m] + k0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float* wc = W + (size_t)(k0 + 2 * kq) * d + ew + 16 * nt + r16;
            b0[nt] = (double)wc[0];
            b1[nt] = (double)wc[d];
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[mt][nt] =
                    __builtin_amdgcn_mfma_f64_16x16x4f64(a[mt].x, b0[nt], acc[mt][nt], 0, 0, 0);
                acc[mt][nt] =
                    __builtin_amdgcn_mfma_f64_16x16x4f64(a[mt].y, b1[nt], acc[mt][nt], 0, 0, 0);
            }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = iw + 16 * mt + kq + 4 * r;
                if (i < rows) Y[(size_t)i * d + ew + 16 * nt + r16] = acc[mt][nt][r];
            }
}

// Order-preserving map of an fp64 score to an unsigned key (-0 -> +0 first).
__device__ inline unsigned long long score_key(double v) {
    if (v == 0.0) v = 0.0;
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// One work-group per score row: radix-select the k-th largest key, then keep
// every larger key and the lowest-index keys equal to it; indices are emitted
// ascending.  Deterministic (counts only, no order-dependent arithmetic).
// low: the k LAST blocks of the order (score descending, index ascending)
// instead, i.e. the smallest scores with ties to the higher index; the mask
// then gets 0xFF at those blocks and is left alone elsewhere.
__global__ __launch_bounds__(256) void topk_kernel(const double* __restrict__ S, int Tq,
                                                   int Tkv, int k, int32_t* __restrict__ idx,
                                                   uint8_t* __restrict__ mask, int low) {
    extern __shared__ unsigned long long keys[];  // [Tkv]
    __shared__ unsigned hist[256];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_kr;
    __shared__ int s_done;
    __shared__ int s_cnt[4];
    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
    const size_t row = (size_t)blockIdx.y * Tq + blockIdx.x;
    const double* srow = S + row * Tkv;
    uint8_t* mrow = mask ? mask + row * Tkv : nullptr;
    int32_t* irow = idx + row * k;

    const uint8_t mark = low ? 0xFF : 1;
    if (k == Tkv) {  // everything selected
        for (int j = t; j < Tkv; j += 256) {
            if (mrow) mrow[j] = mark;
            irow[j] = j;
        }
        return;
    }
    // low: keys inverted and stored at position Tkv-1-j, so that the scan
    // below (positions ascending) meets equal keys from the higher index down
    for (int j = t; j < Tkv; j += 256) {
        if (low) keys[Tkv - 1 - j] = ~score_key(srow[j]);
        else keys[j] = score_key(srow[j]);
    }

    unsigned long long prefix = 0, pmask = 0;
    int kr = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
        hist[t] = 0u;
        __syncthreads();
        for (int j = t; j < Tkv; j += 256) {
            const unsigned long long key = keys[j];
            if ((key & pmask) == prefix) atomicAdd(&hist[(unsigned)(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wid == 0) {
            unsigned c[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[255 - 4 * lane - q];
                tot += c[q];
            }
            unsigned incl = tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            const unsigned excl = incl - tot;
            if (excl < (unsigned)kr && (unsigned)kr <= incl) {
                unsigned run = excl;
                int digit = -1;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (digit < 0) {
                        if (run + c[q] >= (unsigned)kr) {
                            digit = 255 - 4 * lane - q;
                            s_kr = kr - (int)run;
                            // the bucket holds exactly the keys still wanted:
                            // the prefix so far decides the selection
                            s_done = c[q] == (unsigned)(kr - (int)run);
                        } else {
                            run += c[q];
                        }
                    }
                }
                s_prefix = prefix | ((unsigned long long)digit << shift);
            }
        }
        __syncthreads();
        prefix = s_prefix;
        kr = s_kr;
        pmask |= 255ull << shift;
        if (s_done) break;
    }

    // keys compared on the decided prefix (all 64 bits unless a bucket held
    // exactly the remaining keys, in which case every key equal to the prefix
    // there is selected)
    const unsigned long long thr = prefix;
    int eq_base = 0, out_base = 0;
    for (int j0 = 0; j0 < Tkv; j0 += 256) {
        const int j = j0 + t;
        const unsigned long long key = j < Tkv ? (keys[j] & pmask) : 0ull;
        const bool gt = j < Tkv && key > thr;
        const bool eq = j < Tkv && key == thr;
        const unsigned long long below = (1ull << lane) - 1ull;
        const unsigned long long be = __ballot(eq);
        const int eq_rank = __popcll(be & below);
        __syncthreads();
        if (lane == 0) s_cnt[wid] = __popcll(be);
        __syncthreads();
        int eq_before = eq_base, eq_total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < wid) eq_before += s_cnt[w];
            eq_total += s_cnt[w];
        }
        const bool sel = gt || (eq && eq_before + eq_rank < kr);
        const unsigned long long bs = __ballot(sel);
        const int sel_rank = __popcll(bs & below);
        __syncthreads();
        if (lane == 0) s_cnt[wid] = __popcll(bs);
        __syncthreads();
        int sel_before = out_base, sel_total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < wid) sel_before += s_cnt[w];
            sel_total += s_cnt[w];
        }
        if (j < Tkv) {
            if (!low) {
                if (mrow) mrow[j] = sel ? 1 : 0;
                if (sel) irow[sel_before + sel_rank] = j;
            } else if (sel) {  // position j is block Tkv-1-j; emit ascending
                if (mrow) mrow[Tkv - 1 - j] = 0xFF;
                irow[k - 1 - (sel_before + sel_rank)] = Tkv - 1 - j;
            }
        }
        eq_base += eq_total;
        out_base += sel_total;
    }
}

// Scores and hard top-k in one pass, the score rows kept in LDS (S never
// reaches memory): one work-group per 16 query blocks of a head.
//
// Scores: the 8 waves take turns over the 16-column tiles of the row block;
// every 16 x 16 tile is the same chain of fp64 matrix-core products as a
// quarter of score_kernel's 32 x 32 (same operand split, same order over the
// channels), so the scores are bit for bit those of score_kernel.  They are
// stored as order-preserving keys.
//
// Selection: wave w takes rows w and w + 8.  Per row a radix
// select on a wave-private 256-bin histogram finds the k-th largest key; its
// digits start at the highest bit where the row's keys differ (the bits above
// are common to all keys, and the first 8-bit digit would otherwise put every
// key in one bin).  Then every larger key and the lowest-index keys equal to
// it are kept, as in topk_kernel, indices ascending.  For SLA v1 (kl > 0) a
// second selection takes the kl smallest scores, ties to the higher index
// (topk_kernel's low pass), and marks them 0xFF in the mask.
constexpr int kStRows = 16;
constexpr int kStMaxTkv = 1200;  // 16 rows of keys + 8 histograms fit 160 KiB of LDS

// LDS operations of one wave are done in order; this also keeps the compiler
// from moving them across (the histogram is written by other lanes)
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ inline unsigned long long wave_or64(unsigned long long v) {
    unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lo |= __shfl_xor(lo, o);
        hi |= __shfl_xor(hi, o);
    }
    return ((unsigned long long)hi << 32) | lo;
}

constexpr int kStSlots = (kStMaxTkv + 63) / 64;
// the filtered selection is tried for k up to this (on the Wan-shape scores
// about 46 keys pass the filter at k = 36 and 130 at k = 60)
constexpr int kFilterMaxK = 48;

// Radix select over one row's keys held by a wave (the key of position
// p = lane + 64 t in kv[t], positions below n, 0 < kk < n): the kk largest
// keys are those above thr on the bits pmask, and the first kr keys (lowest
// positions) equal to it there.  Digits of 8 bits start at the highest bit
// where the keys differ; h is the wave's 256-bin histogram in LDS.
__device__ inline void wave_radix_select(const unsigned long long (&kv)[kStSlots], int n, int kk,
                                         unsigned* h, int lane, unsigned long long& thr,
                                         unsigned long long& pmask_out, int& kr_out) {
    const unsigned long long key0 =
        ((unsigned long long)(unsigned)__shfl((int)(kv[0] >> 32), 0) << 32) |
        (unsigned)__shfl((int)(unsigned)kv[0], 0);
    unsigned long long diff = 0;
#pragma unroll
    for (int t = 0; t < kStSlots; ++t)
        if (lane + 64 * t < n) diff |= kv[t] ^ key0;
    diff = wave_or64(diff);
    int hi = diff ? 63 - __clzll((long long)diff) : -1;
    // bits above hi are common: the prefix starts as those bits of any key
    unsigned long long pmask = hi < 0 ? ~0ull : hi == 63 ? 0ull : ~((2ull << hi) - 1ull);
    unsigned long long prefix = key0 & pmask;
    int kr = kk;
    for (; hi >= 0; hi -= 8) {
        const int lo = hi >= 7 ? hi - 7 : 0;
        *reinterpret_cast<uint4*>(h + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < kStSlots; ++t)
            if (lane + 64 * t < n && (kv[t] & pmask) == prefix)
                atomicAdd(&h[(unsigned)(kv[t] >> lo) & 255u], 1u);
        wave_lds_sync();
        // lane l holds bins 255 - 4 l - q (descending); inclusive scan
        unsigned c[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c[q] = h[255 - 4 * lane - q];
            tot += c[q];
        }
        unsigned incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const unsigned o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        const unsigned excl = incl - tot;
        const bool found = excl < (unsigned)kr && (unsigned)kr <= incl;
        int digit = 0, nkr = 0, done = 0;
        if (found) {
            unsigned run = excl;
            digit = -1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (digit < 0) {
                    if (run + c[q] >= (unsigned)kr) {
                        digit = 255 - 4 * lane - q;
                        nkr = kr - (int)run;
                        // the bin holds exactly the keys still wanted
                        done = c[q] == (unsigned)nkr;
                    } else {
                        run += c[q];
                    }
                }
            }
        }
        const int src = __ffsll((unsigned long long)__ballot(found)) - 1;
        digit = __shfl(digit, src);
        nkr = __shfl(nkr, src);
        done = __shfl(done, src);
        // a last digit narrower than 8 bits also carries bits above hi,
        // which equal the prefix's there
        prefix |= (unsigned long long)(unsigned)digit << lo;
        pmask |= (unsigned long long)((2u << (hi - lo)) - 1u) << lo;
        kr = nkr;
        wave_lds_sync();  // the bins are read before the next clear
        if (done) break;
    }
    thr = prefix;
    pmask_out = pmask;
    kr_out = kr;
}

__device__ inline unsigned long long shfl_xor64(unsigned long long v, int m) {
    const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)v, m);
    const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(v >> 32), m);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ inline unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}
__device__ inline unsigned long long umin64(unsigned long long a, unsigned long long b) {
    return a < b ? a : b;
}

// The same result as wave_radix_select (thr on all 64 bits, kr) for kk <= 64,
// by a filter: every lane's largest key is an element of the row, so at
// least kk keys are >= tau, the kk-th largest of the 64 lane maxima, and so
// is the kk-th largest key of the row.  The keys >= tau (at most 128 of them)
// are gathered through the wave's LDS scratch sc (128 entries), sorted
// descending by a bitonic network over two slots per lane, and the kk-th of
// them is thr; kr counts the keys equal to thr among the first kk.  Returns
// false (nothing decided) when more than 128 keys pass the filter.
__device__ inline bool wave_filter_select(const unsigned long long (&kv)[kStSlots], int n,
                                          int kk, unsigned long long* sc, int lane,
                                          unsigned long long& thr, int& kr_out) {
    unsigned long long m = 0ull;  // below every key of a real score
#pragma unroll
    for (int t = 0; t < kStSlots; ++t)
        if (lane + 64 * t < n) m = umax64(m, kv[t]);
    // lane maxima sorted descending (bitonic; blocks with lane & size clear
    // run descending, the lower lane of a pair keeping the larger key)
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int j = size >> 1; j > 0; j >>= 1) {
            const unsigned long long o = shfl_xor64(m, j);
            const bool keep_max = ((lane & j) == 0) == ((lane & size) == 0);
            m = keep_max ? umax64(m, o) : umin64(m, o);
        }
    const unsigned long long tau = ((unsigned long long)(unsigned)__shfl((int)(m >> 32), kk - 1)
                                    << 32) |
                                   (unsigned)__shfl((int)(unsigned)m, kk - 1);
    // gather the keys >= tau (their order does not matter)
    const unsigned long long below = (1ull << lane) - 1ull;
    int c = 0;
#pragma unroll
    for (int t = 0; t < kStSlots; ++t) {
        const bool in = lane + 64 * t < n && kv[t] >= tau;
        const unsigned long long b = __ballot(in);
        const int r = c + __popcll(b & below);
        if (in && r < 128) sc[r] = kv[t];
        c += __popcll(b);
    }
    wave_lds_sync();
    if (c > 128) return false;
    unsigned long long a = lane < c ? sc[lane] : 0ull;        // element lane
    unsigned long long b = lane + 64 < c ? sc[lane + 64] : 0ull;  // element lane + 64
    wave_lds_sync();  // read before the scratch is written again
    // 128 elements (index lane and lane + 64) sorted descending
#pragma unroll
    for (int size = 2; size <= 128; size <<= 1)
#pragma unroll
        for (int j = size >> 1; j > 0; j >>= 1) {
            if (j == 64) {  // partners in the same lane; one descending block
                const unsigned long long x = umax64(a, b), y = umin64(a, b);
                a = x;
                b = y;
            } else {
                const unsigned long long oa = shfl_xor64(a, j), ob = shfl_xor64(b, j);
                const bool low = (lane & j) == 0;
                const bool da = (lane & size) == 0, db = ((lane + 64) & size) == 0;
                a = (low == da) ? umax64(a, oa) : umin64(a, oa);
                b = (low == db) ? umax64(b, ob) : umin64(b, ob);
            }
        }
    thr = ((unsigned long long)(unsigned)__shfl((int)(a >> 32), kk - 1) << 32) |
          (unsigned)__shfl((int)(unsigned)a, kk - 1);
    kr_out = __popcll(__ballot(lane < kk && a == thr));
    return true;
}

// f(p, selected, rank among the selected) for every position p < n, in
// ascending order, after wave_radix_select
template <typename F>
__device__ inline void wave_emit(const unsigned long long (&kv)[kStSlots], int n,
                                 unsigned long long thr, unsigned long long pmask, int kr,
                                 int lane, F f) {
    const unsigned long long below = (1ull << lane) - 1ull;
    int eq_base = 0, out_base = 0;
#pragma unroll
    for (int t = 0; t < kStSlots; ++t) {
        const int p = lane + 64 * t;
        const bool in = p < n;
        const unsigned long long key = kv[t] & pmask;
        const bool gt = in && key > thr;
        const bool eq = in && key == thr;
        const unsigned long long be = __ballot(eq);
        const bool sel = gt || (eq && eq_base + __popcll(be & below) < kr);
        const unsigned long long bs = __ballot(sel);
        if (in) f(p, sel, out_base + __popcll(bs & below));
        eq_base += __popcll(be);
        out_base += __popcll(bs);
    }
}

template <int d>
__global__ __launch_bounds__(512) void score_topk_kernel(const double* __restrict__ qt,
                                                         const double* __restrict__ kt, int Tq,
                                                         int Tkv, int k,
                                                         int32_t* __restrict__ idx,
                                                         uint8_t* __restrict__ mask, int kl,
                                                         int32_t* __restrict__ negl) {
    __shared__ unsigned long long keys[kStRows * kStMaxTkv];  // [row][Tkv]
    __shared__ unsigned hist[8][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    const long bh = blockIdx.y;
    const int i0 = blockIdx.x * kStRows;

    // ---- scores: A operand (16 query rows) held for the whole row block
    {
        const double* ar = qt + ((size_t)bh * Tq + min(i0 + r16, Tq - 1)) * d + 2 * kq;
        double2 a[d / 8];
#pragma unroll
        for (int s = 0; s < d / 8; ++s) a[s] = *reinterpret_cast<const double2*>(ar + 8 * s);
        const double* B = kt + (size_t)bh * Tkv * d + 2 * kq;
        const int ntiles = (Tkv + 15) >> 4;
        for (int t = w; t < ntiles; t += 16) {  // two tiles in flight: t and t + 8
            const int ja = 16 * t + r16, jb = ja + 128;
            const double* ba = B + (size_t)min(ja, Tkv - 1) * d;
            const double* bb = B + (size_t)min(jb, Tkv - 1) * d;
            f64x4 ca = {0.0, 0.0, 0.0, 0.0}, cb = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < d / 8; ++s) {
                const double2 x = *reinterpret_cast<const double2*>(ba + 8 * s);
                const double2 y = *reinterpret_cast<const double2*>(bb + 8 * s);
                ca = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s].x, x.x, ca, 0, 0, 0);
                cb = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s].x, y.x, cb, 0, 0, 0);
                ca = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s].y, x.y, ca, 0, 0, 0);
                cb = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s].y, y.y, cb, 0, 0, 0);
            }
            // element r of lane (kq, r16): row kq + 4 r, column r16 of the tile
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (ja < Tkv) keys[(kq + 4 * r) * Tkv + ja] = score_key(ca[r]);
                if (jb < Tkv) keys[(kq + 4 * r) * Tkv + jb] = score_key(cb[r]);
            }
        }
    }
    __syncthreads();

    // ---- selection, one row at a time per wave, the row's keys in registers
    // (position p in lane p % 64, slot p / 64)
    unsigned* h = hist[w];
    for (int rr = w; rr < kStRows; rr += 8) {
        const int i = i0 + rr;
        if (i >= Tq) break;
        const size_t row = (size_t)bh * Tq + i;
        uint8_t* mrow = mask ? mask + row * Tkv : nullptr;
        const unsigned long long* krow = keys + rr * Tkv;
        unsigned long long kv[kStSlots];
        if (k > 0) {  // the k largest, ties to the lower index; mask 1 / 0
            int32_t* irow = idx + row * k;
            if (k == Tkv) {  // everything selected
                for (int j = lane; j < Tkv; j += 64) {
                    if (mrow) mrow[j] = 1;
                    irow[j] = j;
                }
            } else {
#pragma unroll
                for (int t = 0; t < kStSlots; ++t) {
                    const int j = lane + 64 * t;
                    kv[t] = j < Tkv ? krow[j] : 0ull;
                }
                unsigned long long thr, pm = ~0ull;
                int kr;
                if (k > kFilterMaxK ||
                    !wave_filter_select(kv, Tkv, k, reinterpret_cast<unsigned long long*>(h),
                                        lane, thr, kr))
                    wave_radix_select(kv, Tkv, k, h, lane, thr, pm, kr);
                wave_emit(kv, Tkv, thr, pm, kr, lane, [&](int j, bool sel, int rank) {
                    if (mrow) mrow[j] = sel ? 1 : 0;
                    if (sel) irow[rank] = j;
                });
            }
        } else if (mrow) {
            for (int j = lane; j < Tkv; j += 64) mrow[j] = 0;
        }
        if (kl > 0) {
            // SLA v1: the kl LAST blocks of the order (score descending, index
            // ascending), i.e. the smallest scores with ties to the higher
            // index: the inverted keys at reversed positions p = Tkv - 1 - j,
            // selected like the k largest; the mask gets 0xFF there (the
            // stores above come first in this wave's order) and the indices
            // leave ascending
            int32_t* nrow = negl + row * kl;
            if (kl == Tkv) {
                for (int j = lane; j < Tkv; j += 64) {
                    if (mrow) mrow[j] = 0xFF;
                    nrow[j] = j;
                }
            } else {
#pragma unroll
                for (int t = 0; t < kStSlots; ++t) {
                    const int p = lane + 64 * t;
                    kv[t] = p < Tkv ? ~krow[Tkv - 1 - p] : 0ull;
                }
                unsigned long long thr, pm;
                int kr;
                wave_radix_select(kv, Tkv, kl, h, lane, thr, pm, kr);
                wave_emit(kv, Tkv, thr, pm, kr, lane, [&](int p, bool sel, int rank) {
                    if (!sel) return;
                    if (mrow) mrow[Tkv - 1 - p] = 0xFF;
                    nrow[kl - 1 - rank] = Tkv - 1 - p;
                });
            }
        }
    }
}

__global__ void zero_mask_kernel(uint8_t* __restrict__ mask, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        mask[i] = 0;
}

void launch_score_kernel(const Dims& D, const RouteWS& ws, hipStream_t s) {
    dim3 g2((D.Tkv + 63) / 64, (D.Tq + 63) / 64, (unsigned)D.BH);
    if (D.d == 128)
        score_kernel<128><<<g2, 256, 0, s>>>(ws.qt, ws.kt, ws.S, D.Tq, D.Tkv);
    else
        score_kernel<64><<<g2, 256, 0, s>>>(ws.qt, ws.kt, ws.S, D.Tq, D.Tkv);
}

}  // namespace

namespace {
// the projection product over the queries (sides = 1), the keys (2) or both (3)
void launch_proj(const Dims& D, const float* Wq, const float* Wk, const RouteWS& ws, int sides,
                 hipStream_t s) {
    const int rows = sides == 1 ? D.Tq : sides == 2 ? D.Tkv : max(D.Tq, D.Tkv);
    const int ns = sides == 3 ? 2 : 1, side0 = sides == 2 ? 1 : 0;
    dim3 gp((rows + 63) / 64, ns * (D.d / 64), (unsigned)D.BH);
    if (D.d == 128)
        proj_kernel<128><<<gp, 256, 0, s>>>(ws.xq, ws.xk, Wq, Wk, ws.qt, ws.kt, D.Tq, D.Tkv, D.H,
                                            D.w_heads, side0);
    else
        proj_kernel<64><<<gp, 256, 0, s>>>(ws.xq, ws.xk, Wq, Wk, ws.qt, ws.kt, D.Tq, D.Tkv, D.H,
                                           D.w_heads, side0);
}
}  // namespace

hipError_t launch_pool_project(const Dims& D, const void* Q, const void* K, const float* Wq,
                               const float* Wk, const RouteWS& ws, hipStream_t s, bool pooled,
                               bool q_projected) {
    // pool (means into ws.xq / ws.xk), then project them with a tiled product
    dim3 g1(D.Tq + D.Tkv, (unsigned)D.BH);
    timing_before(s, K_POOL_PROJECT);
    if (pooled) {
        // the means are there already
    } else if (D.dtype == SLA2_F32)
        pool_project_kernel<float><<<g1, 256, 0, s>>>(
            (const float*)Q, (const float*)K, nullptr, nullptr, ws.xq, ws.xk, D.N, D.d, D.bq,
            D.bkv, D.Tq, D.Tkv, D.H, D.w_heads, D.st);
    else
        pool_project_kernel<uint16_t><<<g1, 256, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, nullptr, nullptr, ws.xq, ws.xk, D.N, D.d,
            D.bq, D.bkv, D.Tq, D.Tkv, D.H, D.w_heads, D.st);
    launch_proj(D, Wq, Wk, ws, q_projected ? 2 : 3, s);
    timing_after(s, K_POOL_PROJECT);
    return hipGetLastError();
}

hipError_t launch_pool_queries(const Dims& D, const void* Q, const RouteWS& ws, hipStream_t s,
                               const float* Wq) {
    if (D.k == 0) return hipSuccess;
    // work-groups [0, Tq) of the pooling grid: the query blocks
    dim3 g1(D.Tq, (unsigned)D.BH);
    timing_before(s, K_POOL_PROJECT);
    if (D.dtype == SLA2_F32)
        pool_project_kernel<float><<<g1, 256, 0, s>>>(
            (const float*)Q, nullptr, nullptr, nullptr, ws.xq, ws.xk, D.N, D.d, D.bq, D.bkv,
            D.Tq, D.Tkv, D.H, D.w_heads, D.st);
    else
        pool_project_kernel<uint16_t><<<g1, 256, 0, s>>>(
            (const uint16_t*)Q, nullptr, nullptr, nullptr, ws.xq, ws.xk, D.N, D.d, D.bq,
            D.bkv, D.Tq, D.Tkv, D.H, D.w_heads, D.st);
    if (Wq) launch_proj(D, Wq, nullptr, ws, 1, s);
    timing_after(s, K_POOL_PROJECT);
    return hipGetLastError();
}

hipError_t launch_project_queries(const Dims& D, const float* Wq, const RouteWS& ws,
                                  hipStream_t s) {
    if (D.k == 0) return hipSuccess;
    timing_before(s, K_POOL_PROJECT);
    launch_proj(D, Wq, nullptr, ws, 1, s);
    timing_after(s, K_POOL_PROJECT);
    return hipGetLastError();
}

hipError_t launch_scores(const Dims& D, const void* Q, const void* K, const float* Wq,
                         const float* Wk, const RouteWS& ws, hipStream_t s, bool pooled,
                         bool q_projected) {
    hipError_t e = launch_pool_project(D, Q, K, Wq, Wk, ws, s, pooled, q_projected);
    if (e != hipSuccess) return e;
    timing_before(s, K_SCORE);
    launch_score_kernel(D, ws, s);
    timing_after(s, K_SCORE);
    return hipGetLastError();
}

hipError_t launch_route(const Dims& D, const void* Q, const void* K, const float* Wq,
                        const float* Wk, int32_t* idx, uint8_t* mask, const RouteWS& ws,
                        hipStream_t s, bool pooled, bool q_projected) {
    if (D.k == 0) {  // nothing is selected: only the mask (if wanted) is written
        if (mask) {
            const size_t n = (size_t)D.BH * D.Tq * D.Tkv;
            timing_before(s, K_TOPK);
            const size_t nb = (n + 255) / 256;
            zero_mask_kernel<<<dim3((unsigned)(nb < 65535 ? nb : 65535)), 256, 0, s>>>(mask, n);
            timing_after(s, K_TOPK);
        }
        return hipGetLastError();
    }
    if (D.Tkv <= kStMaxTkv) {  // scores and selection in one pass
        hipError_t e = launch_pool_project(D, Q, K, Wq, Wk, ws, s, pooled, q_projected);
        if (e != hipSuccess) return e;
        const dim3 g((D.Tq + kStRows - 1) / kStRows, (unsigned)D.BH);
        timing_before(s, K_SCORE_TOPK);
        if (D.d == 128)
            score_topk_kernel<128><<<g, 512, 0, s>>>(ws.qt, ws.kt, D.Tq, D.Tkv, D.k, idx, mask, 0,
                                                     nullptr);
        else
            score_topk_kernel<64><<<g, 512, 0, s>>>(ws.qt, ws.kt, D.Tq, D.Tkv, D.k, idx, mask, 0,
                                                    nullptr);
        timing_after(s, K_SCORE_TOPK);
        return hipGetLastError();
    }
    hipError_t e = launch_scores(D, Q, K, Wq, Wk, ws, s, pooled, q_projected);
    if (e != hipSuccess) return e;

    dim3 g3(D.Tq, (unsigned)D.BH);
    timing_before(s, K_TOPK);
    topk_kernel<<<g3, 256, sizeof(unsigned long long) * D.Tkv, s>>>(ws.S, D.Tq, D.Tkv, D.k,
                                                                    idx, mask, 0);
    timing_after(s, K_TOPK);
    return hipGetLastError();
}

hipError_t launch_route_v1(const Dims& D, const void* Q, const void* K, int kl, int32_t* crit,
                           int32_t* negl, uint8_t* mask, const RouteWS& ws, hipStream_t s) {
    if (D.k == 0 && kl == 0) {  // every block marginal
        if (mask) {
            const size_t n = (size_t)D.BH * D.Tq * D.Tkv;
            const size_t nb = (n + 255) / 256;
            timing_before(s, K_TOPK);
            zero_mask_kernel<<<dim3((unsigned)(nb < 65535 ? nb : 65535)), 256, 0, s>>>(mask, n);
            timing_after(s, K_TOPK);
        }
        return hipGetLastError();
    }
    dim3 g1(D.Tq + D.Tkv, (unsigned)D.BH);
    timing_before(s, K_POOL_PROJECT);
    if (D.dtype == SLA2_F32)
        pool_project_kernel<float><<<g1, 256, 0, s>>>(
            (const float*)Q, (const float*)K, nullptr, nullptr, ws.qt, ws.kt, D.N, D.d, D.bq,
            D.bkv, D.Tq, D.Tkv, D.H, D.w_heads, D.st);
    else
        pool_project_kernel<uint16_t><<<g1, 256, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, nullptr, nullptr, ws.qt, ws.kt, D.N, D.d,
            D.bq, D.bkv, D.Tq, D.Tkv, D.H, D.w_heads, D.st);
    timing_after(s, K_POOL_PROJECT);
    if (D.Tkv <= kStMaxTkv) {  // scores, both selections and the mask in one pass
        const dim3 g((D.Tq + kStRows - 1) / kStRows, (unsigned)D.BH);
        timing_before(s, K_SCORE_TOPK);
        if (D.d == 128)
            score_topk_kernel<128><<<g, 512, 0, s>>>(ws.qt, ws.kt, D.Tq, D.Tkv, D.k, crit, mask,
                                                     kl, negl);
        else
            score_topk_kernel<64><<<g, 512, 0, s>>>(ws.qt, ws.kt, D.Tq, D.Tkv, D.k, crit, mask,
                                                    kl, negl);
        timing_after(s, K_SCORE_TOPK);
        return hipGetLastError();
    }
    timing_before(s, K_SCORE);
    launch_score_kernel(D, ws, s);
    timing_after(s, K_SCORE);
    dim3 g3(D.Tq, (unsigned)D.BH);
    const size_t sh = sizeof(unsigned long long) * D.Tkv;
    timing_before(s, K_TOPK);
    if (D.k > 0) {
        topk_kernel<<<g3, 256, sh, s>>>(ws.S, D.Tq, D.Tkv, D.k, crit, mask, 0);
    } else if (mask) {
        const size_t n = (size_t)D.BH * D.Tq * D.Tkv;
        const size_t nb = (n + 255) / 256;
        zero_mask_kernel<<<dim3((unsigned)(nb < 65535 ? nb : 65535)), 256, 0, s>>>(mask, n);
    }
    if (kl > 0) topk_kernel<<<g3, 256, sh, s>>>(ws.S, D.Tq, D.Tkv, kl, negl, mask, 1);
    timing_after(s, K_TOPK);
    return hipGetLastError();
}

}  // namespace sla2
