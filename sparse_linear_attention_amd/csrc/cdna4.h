// Device helpers shared by the matrix-core kernels (gfx950 / CDNA4).
//
// MFMA operand layouts relied on (v_mfma_f32_32x32x16_{bf16,f16}): A (32 x 16)
// lane l holds row l%32 and k = 8*(l/32)+[0..7]; B (16 x 32) lane l holds
// column l%32 and the same k; C (32 x 32) lane l holds column l%32 and rows
// 8*(r/4) + 4*(l/32) + r%4, r = 0..15.  The scaled e4m3 form (32x32x64) takes
// 32 consecutive k per lane: k = 32*(l/32)+[0..31]; the int8 form
// (v_mfma_i32_32x32x32_i8) 16: k = 16*(l/32)+[0..15], with exact int32 sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla2 {
namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3 -> fp32 (32x32x64); E8M0 scale 127 = 1.0
__device__ inline f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// int8 x int8 -> int32 (32x32x32), exact
__device__ inline i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ inline f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// max of two floats (not NaN) in one instruction: the median of a, b and
// +inf.  fmaxf quiets each operand with an extra instruction first; written
// as a builtin (not inline asm) so that the compiler keeps the wait states
// between a matrix instruction and the reads of its result.
__device__ inline float max2f(float a, float b) {
    // +inf hidden from the compiler, which would otherwise turn the med3 into
    // a max with a canonicalising max per operand (IEEE mode)
    float inf = INFINITY;
    __asm__("" : "+v"(inf));
    return __builtin_amdgcn_fmed3f(a, b, inf);
}

__device__ inline float bf16_bits(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

// phi = elu + 1
__device__ inline float phi_fast(float x) { return x > 0.0f ? x + 1.0f : __expf(x); }

#define SLA2_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Transposed LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// r points at 4 consecutive 16-bit elements; lane j receives element j%4 of
// the chunks of lanes j/4, j/4+4, j/4+8, j/4+12 (in that order).
__device__ inline s16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ inline void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_barrier without the memory fence of __syncthreads (which would also wait
// for the prefetch in flight); the empty asm keeps the compiler from moving
// memory accesses across it.  LDS writes that other waves read after it must
// be complete first (wait_lgkm0).
__device__ inline void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Work-groups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  The grid is laid out as heads x (8 ranges of ceil(Tq/8) query
// blocks); dispatch index g runs on XCD g % 8, which this map gives query
// blocks x*R .. x*R+R-1 of one head at a time: all XCDs work on the same head
// together (its gathered KV tiles stay in the shared last-level cache) and
// each XCD walks a contiguous range.  Returns false for the padding slots.
__device__ inline bool head_major_map(int g, int Tq, long* bh, int* qb) {
    const int R = (Tq + 7) >> 3;
    const int x = g & 7, s = g >> 3;
    *bh = s / R;
    *qb = x * R + s % R;
    return *qb < Tq;
}

}  // namespace cdna4
}  // namespace sla2
