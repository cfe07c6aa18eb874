// Matrix-core rate probe: the instruction throughput this GPU reaches on the
// two product forms the forward runs on, with no memory traffic, so that the
// fused kernel's rate can be set against what the chip delivers at the
// clocks it holds under that load (beside the datasheet peak).
//
// Every wave runs `iters` rounds of four independent accumulation chains of
// one form (bf16 32x32x16, e4m3 32x32x64 with unit scales, bf16 16x16x32 or
// fp16 32x32x16); operands come
// from the thread index (nothing is constant-folded) and one value per wave
// is stored (nothing is dead).
#include "cdna4.h"
#include "sla2_internal.h"

namespace sla2 {
namespace {
using namespace cdna4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* __restrict__ out) {
    const int t = threadIdx.x;
    f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
    if constexpr (KIND == 2) {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(1.0f + 0.001f * (float)((t + i) & 15));
            b[i] = (__bf16)(0.5f - 0.001f * (float)((t ^ i) & 15));
        }
        f32x4 d0 = {0, 0, 0, 0}, d1 = d0, d2 = d0, d3 = d0;
        for (int r = 0; r < iters; ++r) {
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d1, 0, 0, 0);
            d2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d2, 0, 0, 0);
            d3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d3, 0, 0, 0);
        }
        c0[0] = d0[0];
        c1[1] = d1[1];
        c2[2] = d2[2];
        c3[3] = d3[3];
    } else if constexpr (KIND == 3) {
        f16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (_Float16)(1.0f + 0.001f * (float)((t + i) & 15));
            b[i] = (_Float16)(0.5f - 0.001f * (float)((t ^ i) & 15));
        }
        for (int r = 0; r < iters; ++r) {
            c0 = mfma_f16(a, b, c0);
            c1 = mfma_f16(a, b, c1);
            c2 = mfma_f16(a, b, c2);
            c3 = mfma_f16(a, b, c3);
        }
    } else if constexpr (KIND == 1) {
        i32x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = 0x38383838 ^ (t & 7) ^ i;  // e4m3 codes near 1.0
            b[i] = 0x30303030 ^ ((t >> 3) & 7) ^ (i << 8);
        }
        for (int r = 0; r < iters; ++r) {
            c0 = mfma_fp8(a, b, c0);
            c1 = mfma_fp8(a, b, c1);
            c2 = mfma_fp8(a, b, c2);
            c3 = mfma_fp8(a, b, c3);
        }
    } else {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(1.0f + 0.001f * (float)((t + i) & 15));
            b[i] = (__bf16)(0.5f - 0.001f * (float)((t ^ i) & 15));
        }
        for (int r = 0; r < iters; ++r) {
            c0 = mfma_bf16(a, b, c0);
            c1 = mfma_bf16(a, b, c1);
            c2 = mfma_bf16(a, b, c2);
            c3 = mfma_bf16(a, b, c3);
        }
    }
    const float s = (c0[0] + c1[1]) + (c2[2] + c3[3]);
    if ((t & 63) == 0) out[blockIdx.x * 4 + (t >> 6)] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int kind, int iters, int groups, float* out, hipStream_t s) {
    if (kind == 1)
        mfma_rate_kernel<1><<<groups, 256, 0, s>>>(iters, out);
    else if (kind == 2)
        mfma_rate_kernel<2><<<groups, 256, 0, s>>>(iters, out);
    else if (kind == 3)
        mfma_rate_kernel<3><<<groups, 256, 0, s>>>(iters, out);
    else
        mfma_rate_kernel<0><<<groups, 256, 0, s>>>(iters, out);
    return hipGetLastError();
}

}  // namespace sla2
