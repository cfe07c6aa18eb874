// Low-bit inputs of the sparse branch ("SLA2 深度解读" 07: Q and K quantised
// for Q K^T, K smoothed by its column mean, scheme of SageAttention2++):
//   mu      = mean of K over the N valid tokens, per head and channel
//             (summed in fp64, which is exact for bf16 inputs, rounded once
//             to fp32);
//   K'      = K - mu (fp32);
//   s_K(j)  = max |K'| over KV block j / 448, s_Q(i) = max |Q| over query
//             block i / 448 (1 when the maximum is 0);
//   Khat    = e4m3(K' / s_K), Qhat = e4m3(Q / s_Q): OCP e4m3, round to
//             nearest even, saturated at +-448.
// Rows past N are written as code 0.  d = 128.
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

// mu = (sum of the chunk sums) / N, rounded to fp32.  grid (BH), 128 threads.
__global__ void kmean_kernel(const double* __restrict__ part, float* __restrict__ mu, int N,
                             int nch) {
    const long bh = blockIdx.x;
    const int c = threadIdx.x;
    double a = 0.0;
    for (int k = 0; k < nch; ++k) a += part[((size_t)bh * nch + k) * 128 + c];
    mu[bh * 128 + c] = (float)(a / (double)N);
}

__device__ inline unsigned e4m3_pair(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// One work-group per (head, block): blocks [0, Tq) are query blocks of 128
// tokens, the rest KV blocks of 64.  Each thread handles rows r, r+R, ... of
// one 8-channel group.
__global__ __launch_bounds__(256) void quant_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const float* __restrict__ mu, uint8_t* __restrict__ qhat, uint8_t* __restrict__ khat,
    float* __restrict__ sq, float* __restrict__ sk, int N, int Tq, int Tkv, int H, Strides st) {
    __shared__ float red[256];
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
        const float s = a > 0.0f ? a / 448.0f : 1.0f;
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
                pk[e] = e4m3_pair((bf16_lo(w[e]) - m8[2 * e]) / s,
                                  (bf16_hi(w[e]) - m8[2 * e + 1]) / s);
            codes.x = pk[0] | (pk[1] << 16);
            codes.y = pk[2] | (pk[3] << 16);
        }
        *reinterpret_cast<uint2*>(out + (size_t)row * 128 + g * 8) = codes;
    }
}

}  // namespace

hipError_t launch_quantize_fp8(const Dims& D, const void* Q, const void* K, const FwdWS& ws,
                               hipStream_t s) {
    const int nch = (D.N + kTokPerChunk - 1) / kTokPerChunk;
    timing_before(s, K_QUANT_MEAN);
    ksum_kernel<<<dim3(nch, (unsigned)D.BH), 256, 0, s>>>((const uint16_t*)K, ws.ksum, D.N, nch,
                                                          D.H, D.st);
    kmean_kernel<<<dim3((unsigned)D.BH), 128, 0, s>>>(ws.ksum, ws.mu, D.N, nch);
    timing_after(s, K_QUANT_MEAN);
    timing_before(s, K_QUANT);
    quant_kernel<<<dim3(D.Tq + D.Tkv, (unsigned)D.BH), 256, 0, s>>>(
        (const uint16_t*)Q, (const uint16_t*)K, ws.mu, ws.qhat, ws.khat, ws.sq, ws.sk, D.N, D.Tq,
        D.Tkv, D.H, D.st);
    timing_after(s, K_QUANT);
    return hipGetLastError();
}

}  // namespace sla2
