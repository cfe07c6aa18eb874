// Low-bit inputs of the sparse branch ("SLA2 深度解读" 07: Q and K quantised
// for Q K^T, K smoothed by its column mean, scheme of SageAttention2++):
//   mu      = mean of K over the N valid tokens, per head and channel
//             (summed in fp64, rounded once to fp32; the sum is exact, hence
//             independent of its order, unless a head's K values span more
//             than about 2^27 in magnitude);
//   K'      = K - mu (fp32);
//   s_K(j)  = max |K'| over KV block j / 448, s_Q(i) = max |Q| over query
//             block i / 448 (1 when the maximum is 0);
//   Khat    = e4m3(K' / s_K), Qhat = e4m3(Q / s_Q): OCP e4m3, round to
//             nearest even, saturated at +-448.
// With int8 Q/K codes (the pages allow INT8 or FP8 for Q K^T) the scales are
// max / 127 and the codes round-half-even(x / s) clamped to +-127.
// Rows past N are written as code 0.  d = 128.
// Fully low-bit variant (P V on the e4m3 matrix cores as well): s_V(c) =
// max over the N valid tokens of |V(., c)| / 448 per head and channel (1 if
// 0), Vhat = e4m3(V / s_V) (fp32 division, nearest even, saturated).
#include "sla2_internal.h"

namespace sla2 {
namespace {

constexpr int kTokPerChunk = 1024;

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Column sums of K over chunks of 1024 tokens, in fp64.  grid (chunks, BH).
__global__ __launch_bounds__(256) void ksum_kernel(const uint16_t* __restrict__ K,
                                                   double* __restrict__ part, int N, int nch,
                                                   int H, Strides st) {
    __shared__ double red[16][128];
    const long bh = blockIdx.y;
    const int chunk = blockIdx.x;
    const int g = threadIdx.x & 15, r = threadIdx.x >> 4;  // 16 channel groups x 16 rows
    const int t0 = chunk * kTokPerChunk, t1 = min(N, t0 + kTokPerChunk);
    const uint16_t* Kh = K + head_base(st, bh, H);
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0;
    for (int t = t0 + r; t < t1; t += 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(Kh + (size_t)t * st.t + g * 8);
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] += (double)bf16_lo(w[e]);
            s[2 * e + 1] += (double)bf16_hi(w[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[r][g * 8 + e] = s[e];
    __syncthreads();
    if (threadIdx.x < 128) {
        double a = 0.0;
        for (int rr = 0; rr < 16; ++rr) a += red[rr][threadIdx.x];
        part[((size_t)bh * nch + chunk) * 128 + threadIdx.x] = a;
    }
}

// mu = (sum of the nch partial sums) / N, rounded to fp32.  grid (BH), 1024
// threads: 8 groups of 128 channels each sum every 8th partial, then the
// 8 group sums are added in order.
__global__ __launch_bounds__(1024) void kmean_kernel(const double* __restrict__ part,
                                                     float* __restrict__ mu, int N, int nch) {
    __shared__ double red[8][128];
    const long bh = blockIdx.x;
    const int c = threadIdx.x & 127, grp = threadIdx.x >> 7;
    double a = 0.0;
#pragma unroll 8
    for (int k = grp; k < nch; k += 8) a += part[((size_t)bh * nch + k) * 128 + c];
    red[grp][c] = a;
    __syncthreads();
    if (grp == 0) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) t += red[i][c];
        mu[bh * 128 + c] = (float)(t / (double)N);
    }
}

__device__ inline unsigned e4m3_pair(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// two int8 codes: nearest integer, ties to even (v_rndne), clamped to +-127
__device__ inline unsigned i8_pair(float a, float b) {
    const int ia = (int)fminf(fmaxf(__builtin_rintf(a), -127.0f), 127.0f);
    const int ib = (int)fminf(fmaxf(__builtin_rintf(b), -127.0f), 127.0f);
    return ((unsigned)ia & 0xffu) | (((unsigned)ib & 0xffu) << 8);
}

template <bool I8>
__device__ inline unsigned code_pair(float a, float b) {
    if constexpr (I8) return i8_pair(a, b);
    else return e4m3_pair(a, b);
}

// One work-group per (head, block): blocks [0, Tq) are query blocks of 128
// tokens, the rest KV blocks of 64.  Each thread handles rows r, r+R, ... of
// one 8-channel group.  I8: int8 codes (else e4m3).
template <bool I8>
__global__ __launch_bounds__(256) void quant_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const float* __restrict__ mu, uint8_t* __restrict__ qhat, uint8_t* __restrict__ khat,
    float* __restrict__ sq, float* __restrict__ sk, int N, int Tq, int Tkv, int H, Strides st,
    int blk0) {
    __shared__ float red[256];
    __shared__ float s_scale;
    const int blk = blockIdx.x + blk0;  // blk0 = Tq: key blocks only
    const long bh = blockIdx.y;
    const bool isq = blk < Tq;
    const int j = isq ? blk : blk - Tq;
    const int bs = isq ? 128 : 64;
    const int t0 = j * bs;
    const int n = min(bs, N - t0);
    const uint16_t* X = (isq ? Q : K) + head_base(st, bh, H);
    const int g = threadIdx.x & 15, r = threadIdx.x >> 4;  // 16 groups x 16 rows
    float m8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m8[e] = isq ? 0.0f : mu[bh * 128 + g * 8 + e];

    // pass 1: block absmax of Q or of K - mu
    float amax = 0.0f;
    for (int row = r; row < n; row += 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + (size_t)(t0 + row) * st.t + g * 8);
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax = fmaxf(amax, fabsf(bf16_lo(w[e]) - m8[2 * e]));
            amax = fmaxf(amax, fabsf(bf16_hi(w[e]) - m8[2 * e + 1]));
        }
    }
    red[threadIdx.x] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = 0.0f;
        for (int i = 0; i < 256; ++i) a = fmaxf(a, red[i]);
        const float s = a > 0.0f ? a / (I8 ? 127.0f : 448.0f) : 1.0f;
        s_scale = s;
        if (isq) sq[bh * Tq + j] = s;
        else sk[bh * Tkv + j] = s;
    }
    __syncthreads();
    const float s = s_scale;

    // pass 2: codes (the block is re-read from L2)
    uint8_t* out = isq ? qhat + ((size_t)bh * Tq * 128 + t0) * 128
                       : khat + ((size_t)bh * Tkv * 64 + t0) * 128;
    for (int row = r; row < bs; row += 16) {
        uint2 codes = make_uint2(0, 0);
        if (row < n) {
            const uint4 v = *reinterpret_cast<const uint4*>(X + (size_t)(t0 + row) * st.t + g * 8);
            const unsigned w[4] = {v.x, v.y, v.z, v.w};
            unsigned pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pk[e] = code_pair<I8>((bf16_lo(w[e]) - m8[2 * e]) / s,
                                      (bf16_hi(w[e]) - m8[2 * e + 1]) / s);
            codes.x = pk[0] | (pk[1] << 16);
            codes.y = pk[2] | (pk[3] << 16);
        }
        *reinterpret_cast<uint2*>(out + (size_t)row * 128 + g * 8) = codes;
    }
}

// The router's pooling pass with the query codes folded in, so that Q and K
// are read once for both ("SLA2 深度解读" 05 and 07).  One work-group per
// (head, block), blocks [0, Tq) query blocks of 128 tokens, the rest KV
// blocks of 64; thread (r, g) keeps rows r, r+16, ... of channel group g in
// registers.  Every block: the fp64 mean of its valid rows into xq / xk
// (the block sums of bf16 values are exact in fp64, so the means equal the
// router pooling pass's own).  Query block i also: s_Q(i) and its codes,
// exactly as quant_kernel computes them.  KV block j also: its fp64 column
// sums into kblk[bh][j], from which kmean_kernel takes the same mu as from
// ksum_kernel's chunk sums (both sums exact under the condition stated for
// mu above).  bf16, d = 128.
template <bool I8>
__global__ __launch_bounds__(256) void pool_quant_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, double* __restrict__ xq,
    double* __restrict__ xk, double* __restrict__ kblk, uint8_t* __restrict__ qhat,
    float* __restrict__ sq, int N, int Tq, int Tkv, int H, Strides st) {
    __shared__ double part[16][128];
    __shared__ float red[4];
    __shared__ float s_scale;
    const int blk = blockIdx.x;
    const long bh = blockIdx.y;
    const bool isq = blk < Tq;
    const int j = isq ? blk : blk - Tq;
    const int bs = isq ? 128 : 64;
    const int t0 = j * bs;
    const int n = min(bs, N - t0);
    const uint16_t* X = (isq ? Q : K) + head_base(st, bh, H);
    const int g = threadIdx.x & 15, r = threadIdx.x >> 4;  // 16 groups x 16 rows

    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = r + 16 * i;
        v[i] = make_uint4(0, 0, 0, 0);
        if (row < n) v[i] = *reinterpret_cast<const uint4*>(X + (size_t)(t0 + row) * st.t + g * 8);
    }
    double s8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = 0.0;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const unsigned w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};  // 0 past n
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s8[2 * e] += (double)bf16_lo(w[e]);
            s8[2 * e + 1] += (double)bf16_hi(w[e]);
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r][g * 8 + e] = s8[e];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x < 128) {
        const int c = threadIdx.x;
        double acc = 0.0;
        for (int rr = 0; rr < 16; ++rr) acc += part[rr][c];
        if (isq) {
            xq[((size_t)bh * Tq + j) * 128 + c] = acc / (double)n;
        } else {
            xk[((size_t)bh * Tkv + j) * 128 + c] = acc / (double)n;
            kblk[((size_t)bh * Tkv + j) * 128 + c] = acc;
        }
    } else if (isq && threadIdx.x == 128) {
        const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float sc = a > 0.0f ? a / (I8 ? 127.0f : 448.0f) : 1.0f;
        s_scale = sc;
        sq[bh * Tq + j] = sc;
    }
    if (!isq) return;  // uniform per work-group
    __syncthreads();
    const float sc = s_scale;
    uint8_t* out = qhat + ((size_t)bh * Tq * 128 + t0) * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = r + 16 * i;
        uint2 codes = make_uint2(0, 0);
        if (row < n) {
            const unsigned w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            unsigned pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pk[e] = code_pair<I8>((bf16_lo(w[e]) - 0.0f) / sc, (bf16_hi(w[e]) - 0.0f) / sc);
            codes.x = pk[0] | (pk[1] << 16);
            codes.y = pk[2] | (pk[3] << 16);
        }
        *reinterpret_cast<uint2*>(out + (size_t)row * 128 + g * 8) = codes;
    }
}

// Per-channel max |V| over chunks of 1024 tokens (fp32 max: exact and
// order independent).  grid (chunks, BH).
__global__ __launch_bounds__(256) void vmax_kernel(const uint16_t* __restrict__ V,
                                                   float* __restrict__ part, int N, int nch,
                                                   int H, Strides st) {
    __shared__ float red[16][128];
    const long bh = blockIdx.y;
    const int chunk = blockIdx.x;
    const int g = threadIdx.x & 15, r = threadIdx.x >> 4;
    const int t0 = chunk * kTokPerChunk, t1 = min(N, t0 + kTokPerChunk);
    const uint16_t* Vh = V + head_base(st, bh, H);
    float m8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m8[e] = 0.0f;
    for (int t = t0 + r; t < t1; t += 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(Vh + (size_t)t * st.t + g * 8);
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m8[2 * e] = fmaxf(m8[2 * e], fabsf(bf16_lo(w[e])));
            m8[2 * e + 1] = fmaxf(m8[2 * e + 1], fabsf(bf16_hi(w[e])));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[r][g * 8 + e] = m8[e];
    __syncthreads();
    if (threadIdx.x < 128) {
        float a = 0.0f;
        for (int rr = 0; rr < 16; ++rr) a = fmaxf(a, red[rr][threadIdx.x]);
        part[((size_t)bh * nch + chunk) * 128 + threadIdx.x] = a;
    }
}

// s_V = (max over the chunk maxima) / 448, 1 if the maximum is 0.
// grid (BH), 128 threads.
__global__ void vscale_kernel(const float* __restrict__ part, float* __restrict__ sv, int nch) {
    const long bh = blockIdx.x;
    const int c = threadIdx.x;
    float a = 0.0f;
#pragma unroll 8
    for (int k = 0; k < nch; ++k) a = fmaxf(a, part[((size_t)bh * nch + k) * 128 + c]);
    sv[bh * 128 + c] = a > 0.0f ? a / 448.0f : 1.0f;
}

// Key u of a 64-key block -> its position in the k operand of the e4m3 P V
// product: the lane holding query column q and k half h carries the codes of
// its S^T accumulators s[mt][i] (key 32 mt + 8 (i / 4) + 4 h + i % 4) at
// positions 32 h + 16 mt + i.
__device__ inline int pv8_pos(int u) {
    return 32 * ((u >> 2) & 1) + 16 * (u >> 5) + 4 * ((u >> 3) & 3) + (u & 3);
}

// Codes of V / s_V for KV block j (grid (Tkv, BH), 256 threads: token u =
// t % 64, channels 32 (t / 64) .. +31).  TILE: the block transposed, [128
// channels][64 positions] with key u at pv8_pos(u); otherwise rows [64][128].
// Rows past N are code 0.
template <bool TILE>
__global__ __launch_bounds__(256) void vquant_kernel(const uint16_t* __restrict__ V,
                                                     const float* __restrict__ sv,
                                                     uint8_t* __restrict__ out, int N, int Tkv,
                                                     int H, Strides st) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[128 * 64];
    const int j = blockIdx.x;
    const long bh = blockIdx.y;
    const int u = threadIdx.x & 63, cg = threadIdx.x >> 6;
    const int tok = j * 64 + u;
    const bool ok = tok < N;
    const uint16_t* vrow = V + head_base(st, bh, H) + (size_t)(ok ? tok : 0) * st.t + 32 * cg;
    const float* s = sv + bh * 128 + 32 * cg;
    unsigned words[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(vrow + 8 * q);
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
        unsigned pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pk[e] = e4m3_pair(bf16_lo(w[e]) / s[8 * q + 2 * e], bf16_hi(w[e]) / s[8 * q + 2 * e + 1]);
        words[2 * q] = pk[0] | (pk[1] << 16);
        words[2 * q + 1] = pk[2] | (pk[3] << 16);
    }
    if (TILE) {
        const int pos = pv8_pos(u);
#pragma unroll
        for (int b = 0; b < 32; ++b)
            tile[(32 * cg + b) * 64 + pos] = (uint8_t)(words[b >> 2] >> (8 * (b & 3)));
        __syncthreads();
        uint8_t* dst = out + ((size_t)bh * Tkv + j) * 8192;
        *reinterpret_cast<uint4*>(dst + threadIdx.x * 32) =
            *reinterpret_cast<const uint4*>(tile + threadIdx.x * 32);
        *reinterpret_cast<uint4*>(dst + threadIdx.x * 32 + 16) =
            *reinterpret_cast<const uint4*>(tile + threadIdx.x * 32 + 16);
    } else {
        uint8_t* dst = out + (((size_t)bh * Tkv + j) * 64 + u) * 128 + 32 * cg;
        *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(words[4], words[5], words[6], words[7]);
    }
}

}  // namespace

static hipError_t launch_vscale(const Dims& D, const void* V, const FwdWS& ws, hipStream_t s) {
    const int nch = (D.N + kTokPerChunk - 1) / kTokPerChunk;
    vmax_kernel<<<dim3(nch, (unsigned)D.BH), 256, 0, s>>>((const uint16_t*)V, ws.vmax, D.N, nch,
                                                          D.H, D.st);
    vscale_kernel<<<dim3((unsigned)D.BH), 128, 0, s>>>(ws.vmax, ws.sv, nch);
    return hipGetLastError();
}

hipError_t launch_quantize_v_rows(const Dims& D, const void* V, uint8_t* vhat_rows,
                                  const FwdWS& ws, hipStream_t s) {
    hipError_t e = launch_vscale(D, V, ws, s);
    if (e != hipSuccess) return e;
    vquant_kernel<false><<<dim3(D.Tkv, (unsigned)D.BH), 256, 0, s>>>(
        (const uint16_t*)V, ws.sv, vhat_rows, D.N, D.Tkv, D.H, D.st);
    return hipGetLastError();
}

// V codes for the fully low-bit P V (nothing without lowbit_v or V)
static hipError_t launch_quantize_v(const Dims& D, const void* V, const FwdWS& ws,
                                    hipStream_t s) {
    if (!D.lowbit_v || !V) return hipGetLastError();
    timing_before(s, K_QUANT_V);
    hipError_t e = launch_vscale(D, V, ws, s);
    if (e != hipSuccess) return e;
    vquant_kernel<true><<<dim3(D.Tkv, (unsigned)D.BH), 256, 0, s>>>(
        (const uint16_t*)V, ws.sv, ws.vhat, D.N, D.Tkv, D.H, D.st);
    timing_after(s, K_QUANT_V);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(const Dims& D, const void* Q, const void* K, const void* V,
                               const FwdWS& ws, hipStream_t s) {
    const int nch = (D.N + kTokPerChunk - 1) / kTokPerChunk;
    timing_before(s, K_QUANT_MEAN);
    ksum_kernel<<<dim3(nch, (unsigned)D.BH), 256, 0, s>>>((const uint16_t*)K, ws.ksum, D.N, nch,
                                                          D.H, D.st);
    kmean_kernel<<<dim3((unsigned)D.BH), 1024, 0, s>>>(ws.ksum, ws.mu, D.N, nch);
    timing_after(s, K_QUANT_MEAN);
    const KernelKind kq = D.int8_qk ? K_QUANT_I8 : K_QUANT;
    timing_before(s, kq);
    (D.int8_qk ? quant_kernel<true> : quant_kernel<false>)<<<dim3(D.Tq + D.Tkv, (unsigned)D.BH),
                                                             256, 0, s>>>(
        (const uint16_t*)Q, (const uint16_t*)K, ws.mu, ws.qhat, ws.khat, ws.sq, ws.sk, D.N, D.Tq,
        D.Tkv, D.H, D.st, 0);
    timing_after(s, kq);
    return launch_quantize_v(D, V, ws, s);
}

hipError_t launch_pool_quant(const Dims& D, const void* Q, const void* K, const RouteWS& rw,
                             const FwdWS& fw, hipStream_t s, bool queries_only) {
    timing_before(s, K_POOL_QUANT);
    (D.int8_qk ? pool_quant_kernel<true> : pool_quant_kernel<false>)<<<
        dim3(queries_only ? D.Tq : D.Tq + D.Tkv, (unsigned)D.BH), 256, 0, s>>>(
        (const uint16_t*)Q, (const uint16_t*)K, rw.xq, rw.xk, fw.ksum, fw.qhat, fw.sq, D.N, D.Tq,
        D.Tkv, D.H, D.st);
    timing_after(s, K_POOL_QUANT);
    return hipGetLastError();
}

hipError_t launch_quantize_k(const Dims& D, const void* K, const void* V, const FwdWS& ws,
                             hipStream_t s) {
    timing_before(s, K_QUANT_MEAN);
    kmean_kernel<<<dim3((unsigned)D.BH), 1024, 0, s>>>(ws.ksum, ws.mu, D.N, D.Tkv);
    timing_after(s, K_QUANT_MEAN);
    const KernelKind kq = D.int8_qk ? K_QUANT_I8 : K_QUANT;
    timing_before(s, kq);
    (D.int8_qk ? quant_kernel<true> : quant_kernel<false>)<<<dim3(D.Tkv, (unsigned)D.BH), 256, 0,
                                                             s>>>(
        nullptr, (const uint16_t*)K, ws.mu, ws.qhat, ws.khat, ws.sq, ws.sk, D.N, D.Tq, D.Tkv, D.H,
        D.st, D.Tq);
    timing_after(s, kq);
    return launch_quantize_v(D, V, ws, s);
}

}  // namespace sla2
