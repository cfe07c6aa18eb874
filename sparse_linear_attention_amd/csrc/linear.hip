// Linear branch of the d = 128, b_q = 128 bf16 path as one dense product per
// head.
//
// The linear branch of query block i needs H_i = sum of h_j = phi(K_j)^T V_j
// and Z_i = sum of z_j = colsum phi(K_j) over the KV blocks j that i does not
// select (SLA notes, key designs 3 and 4; "SLA2 深度解读" 04: every block the
// router leaves out goes to the linear branch).  With U[i][j] = 1 for those
// blocks and 0 otherwise, the rows (H_i, Z_i) of all query blocks of a head
// are the product U * [h | z]: T_q x T_kv times T_kv x (d*d + d).  Summing
// the left-out blocks directly (rather than the head total minus the
// selected ones) keeps H_i exact up to the bf16 rounding of each h_j even
// when only a few blocks are left out.
//
// unsel_kernel writes U as bits from the selected indices (and, for SLA v1,
// the negligible ones, which leave the linear branch as well).
// lin_gemm_kernel multiplies it with the per-block summaries written by the
// block-summaries pass (bf16 rows of h_j^T, then z_j) on the bf16 matrix
// cores (32x32x16, fp32 accumulation) into rows of H_i^T (rounded to bf16)
// and Z_i (fp32) that the fused kernel's epilogue reads.  The backward uses
// the same product in an fp32-output form (lin_gemm_kernel<true>) over the
// selection's bits (unsel_kernel with sel set) or over the bits of its
// transpose (csr_bits_kernel), summing bf16 d x d matrices per row.
//
// Product tiles: 320 query blocks x 128 columns per work-group of 4 waves
// (2 x 2: each wave 5 x 2 tiles of 32 x 32, 160 rows x 64 columns), 64 KV
// blocks per stage, two stages.  Every wave stages its own operands by
// direct-to-LDS loads one stage ahead (the summaries of a column range are
// loaded by the two waves that use them), so the loop has no barrier; 80 KB
// of LDS lets two work-groups share a compute unit.  LDS layouts, per wave
// and stage:
//   U bits   [160 rows][8 B]    bit b of byte g: KV block 8 g + b of the stage
//   hz tile  [64 rows][128 B]   32-byte unit u of row r at u ^ (r & 3)
//   table    [256][16 B]        byte v -> its 8 bits as bf16 0.0 / 1.0
// The U operand (row = query block, 8 consecutive KV blocks) is one 16-byte
// read from the table at the row's byte for those blocks (U is mostly ones,
// so most lanes read the same entry); the summaries operand (column, 8
// consecutive KV blocks) is two transposed reads (ds_read_b64_tr_b16).
#include "cdna4.h"
#include "sla2_internal.h"

namespace sla2 {
namespace {
using namespace cdna4;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t head_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
__device__ inline void load_lds16(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SLA2_LDS(dst), 16, voff, soff, 0, 0);
}
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)SLA2_LDS(p); }

constexpr int kMaxTkvPad = kMaxBitBlocks;
constexpr int kGN = 128;                 // columns per tile
constexpr int kGK = 64;                  // KV blocks per stage
constexpr int kNT = kHzPitch / kGN;      // column tiles (130)
// per wave and stage: U bits of its 160 rows (8 bytes each), then the
// summaries of its 64 columns (64 rows x 128 B)
constexpr int kWU = 160 * 8;
constexpr int kWB = kGK * 64 * 2;
constexpr int kWSt = kWU + kWB;
constexpr int kTbl = 4096;               // byte -> 8 bf16 0/1 values
static_assert(kGemmM == 320, "tile shape");
static_assert(4 * 2 * kWSt + kTbl <= 80 * 1024, "LDS budget: two work-groups per CU");

// One work-group per row of U: query block i of head bh (rows past T_q, up to
// the padded row count, are all zero).  Bit b of byte g of the row is KV
// block 8 g + b.  Stored k-step major, [BH][Tkvp / 64][rows][8 bytes], so
// that a product tile's 320 rows of one k-step are contiguous.
// sel: bits of the selected blocks instead (the backward's products).
__global__ __launch_bounds__(256) void unsel_kernel(const int32_t* __restrict__ idx, int k,
                                                    const int32_t* __restrict__ negl, int kl,
                                                    uint8_t* __restrict__ U, int Tq, int Tkv,
                                                    int Tkvp, int rows, int sel) {
    __shared__ uint32_t row[kMaxTkvPad / 32];
    const int t = threadIdx.x;
    const long bh = blockIdx.x / rows;
    const int i = blockIdx.x % rows;
    const int nw = Tkvp / 32;
    for (int x = t; x < nw; x += 256) {
        const int lo = 32 * x;
        uint32_t v = 0;
        if (i < Tq && !sel)
            v = Tkv >= lo + 32 ? 0xffffffffu : (Tkv > lo ? (1u << (Tkv - lo)) - 1u : 0u);
        row[x] = v;
    }
    __syncthreads();
    if (i < Tq) {
        const size_t r = (size_t)bh * Tq + i;
        for (int x = t; x < k; x += 256) {
            const int j = idx[r * k + x];
            if ((unsigned)j < (unsigned)Tkv) {
                if (sel) atomicOr(&row[j >> 5], 1u << (j & 31));
                else atomicAnd(&row[j >> 5], ~(1u << (j & 31)));
            }
        }
        for (int x = t; x < kl; x += 256) {
            const int j = negl[r * kl + x];
            if ((unsigned)j < (unsigned)Tkv) atomicAnd(&row[j >> 5], ~(1u << (j & 31)));
        }
    }
    __syncthreads();
    const int nks = Tkvp / 64;
    for (int x = t; x < nks; x += 256)
        *reinterpret_cast<uint2*>(U + (((size_t)bh * nks + x) * rows + i) * 8) =
            make_uint2(row[2 * x], row[2 * x + 1]);
}

// The transposed selection as product rows: row j (a KV block) has bit i
// set for every query block i in list[off[j] .. off[j + 1]) (the query
// blocks that select j; off per head [Tkv + 1], list per head [Tq * k]).
// Same layout as unsel_kernel's, with the query blocks as the k dimension.
__global__ __launch_bounds__(256) void csr_bits_kernel(const int32_t* __restrict__ off,
                                                       const int32_t* __restrict__ list, int k,
                                                       uint8_t* __restrict__ U, int Tq, int Tkv,
                                                       int Tqp, int rows) {
    __shared__ uint32_t row[kMaxTkvPad / 32];
    const int t = threadIdx.x;
    const long bh = blockIdx.x / rows;
    const int j = blockIdx.x % rows;
    const int nw = Tqp / 32;
    for (int x = t; x < nw; x += 256) row[x] = 0u;
    __syncthreads();
    if (j < Tkv) {
        const int32_t* o = off + (size_t)bh * (Tkv + 1);
        const int32_t* L = list + (size_t)bh * Tq * k;
        for (int x = o[j] + t; x < o[j + 1]; x += 256) {
            const int i = L[x];
            if ((unsigned)i < (unsigned)Tq) atomicOr(&row[i >> 5], 1u << (i & 31));
        }
    }
    __syncthreads();
    const int nks = Tqp / 64;
    for (int x = t; x < nks; x += 256)
        *reinterpret_cast<uint2*>(U + (((size_t)bh * nks + x) * rows + j) * 8) =
            make_uint2(row[2 * x], row[2 * x + 1]);
}

// operands of one 16-KV-block sub-step: U fragments of the wave's five row
// tiles, two transposed halves of the summaries fragments of its two column
// tiles
struct SubOps {
    i32x4 a[5];
    s16x4 b[4];
};

// the nine LDS reads of sub-step S (rows 16 S .. 16 S + 15 of the stage):
// five U fragments from the byte table at per-lane addresses u[m], four
// transposed summaries halves; waited for before returning
template <int S>
__device__ inline void read_sub(const uint32_t (&u)[5], uint32_t b0, uint32_t b1, SubOps& x) {
    asm volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %10\n\t"
        "ds_read_b128 %2, %11\n\t"
        "ds_read_b128 %3, %12\n\t"
        "ds_read_b128 %4, %13\n\t"
        "ds_read_b64_tr_b16 %5, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%17\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "ds_read_b64_tr_b16 %8, %15 offset:%17\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x.a[0]), "=&v"(x.a[1]), "=&v"(x.a[2]), "=&v"(x.a[3]), "=&v"(x.a[4]),
          "=&v"(x.b[0]), "=&v"(x.b[1]), "=&v"(x.b[2]), "=&v"(x.b[3])
        : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(b0), "v"(b1),
          "i"(2048 * S), "i"(2048 * S + 512));
}
// The same reads without the wait: their results arrive later, and
// wait_ops(x, .) must run before any use of x (it names the registers, so no
// use can move above it).  The previous sub-step's operands p pass through
// unchanged, which keeps that sub-step's products below these reads.
template <int S>
__device__ inline void read_sub_async(const uint32_t (&u)[5], uint32_t b0, uint32_t b1,
                                      SubOps& x, SubOps& p) {
    asm volatile(
        "ds_read_b128 %0, %18\n\t"
        "ds_read_b128 %1, %19\n\t"
        "ds_read_b128 %2, %20\n\t"
        "ds_read_b128 %3, %21\n\t"
        "ds_read_b128 %4, %22\n\t"
        "ds_read_b64_tr_b16 %5, %23 offset:%25\n\t"
        "ds_read_b64_tr_b16 %6, %23 offset:%26\n\t"
        "ds_read_b64_tr_b16 %7, %24 offset:%25\n\t"
        "ds_read_b64_tr_b16 %8, %24 offset:%26"
        : "=&v"(x.a[0]), "=&v"(x.a[1]), "=&v"(x.a[2]), "=&v"(x.a[3]), "=&v"(x.a[4]),
          "=&v"(x.b[0]), "=&v"(x.b[1]), "=&v"(x.b[2]), "=&v"(x.b[3]), "+v"(p.a[0]),
          "+v"(p.a[1]), "+v"(p.a[2]), "+v"(p.a[3]), "+v"(p.a[4]), "+v"(p.b[0]), "+v"(p.b[1]),
          "+v"(p.b[2]), "+v"(p.b[3])
        : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(b0), "v"(b1),
          "i"(2048 * S), "i"(2048 * S + 512));
}
// wait for the reads of x; the operands p of the products issued since pass
// through as well, which keeps those products above the wait
__device__ inline void wait_ops(SubOps& x, SubOps& p) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(x.a[0]), "+v"(x.a[1]), "+v"(x.a[2]), "+v"(x.a[3]), "+v"(x.a[4]),
                   "+v"(x.b[0]), "+v"(x.b[1]), "+v"(x.b[2]), "+v"(x.b[3]), "+v"(p.a[0]),
                   "+v"(p.a[1]), "+v"(p.a[2]), "+v"(p.a[3]), "+v"(p.a[4]), "+v"(p.b[0]),
                   "+v"(p.b[1]), "+v"(p.b[2]), "+v"(p.b[3]));
}

__device__ inline void load_lds4(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SLA2_LDS(dst), 4, voff, soff, 0, 0);
}

// Each wave stages its own operands (no barrier in the loop): waves of a
// work-group and the two work-groups of a compute unit run unsynchronised,
// so one wave's load and LDS waits are covered by the others' products.
// F32: the backward's form: B rows bp elements apart, nt column tiles, every
// output column in fp32 (rows of nt * 128 floats); otherwise the forward's
// summaries rows (kHzPitch, kNT tiles) and H_i bf16 / Z_i fp32 output rows.
template <bool F32>
__global__ __launch_bounds__(256, 2) void lin_gemm_kernel(const uint8_t* __restrict__ U,
                                                         const uint16_t* __restrict__ hz,
                                                         char* __restrict__ HZ, int Tq, int Tkv,
                                                         int Tkvp, int nM, int rows, int nt_,
                                                         int bp_) {
    // the forward's form keeps its sizes as constants
    const int nt = F32 ? nt_ : kNT, bp = F32 ? bp_ : kHzPitch;
    __shared__ __attribute__((aligned(1024))) char lds[4 * 2 * kWSt + kTbl];
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    int g = blockIdx.x;
    const int mi = g % nM;
    g /= nM;
    const int ni = g % nt;
    const long bh = g / nt;
    const int m0 = mi * kGemmM + 160 * wm;  // this wave's first row
    const int n0 = ni * kGN + 64 * wn;      // this wave's first column
    const int nk = Tkvp / kGK;
    const rsrc_t ru = head_rsrc(U + (size_t)bh * nk * rows * 8);
    const rsrc_t rh = head_rsrc(hz + (size_t)bh * Tkv * bp);

    // byte table: entry v holds the 8 bf16 values bit e of v (0 or 1)
    char* const tbl = lds + 4 * 2 * kWSt;
    {
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d[e] = (((t >> (2 * e)) & 1) ? 0x3F80u : 0u) | (((t >> (2 * e + 1)) & 1) ? 0x3F800000u : 0u);
        *reinterpret_cast<uint4*>(tbl + 16 * t) = make_uint4(d[0], d[1], d[2], d[3]);
    }
    wait_lgkm0();
    __syncthreads();  // the table, once; no barrier after this

    // U bits of a stage: this wave's rows m0 .. m0 + 159 of k-step kk, 1280
    // contiguous bytes (1 KB piece + 256 B); past T_q they are the padding
    // rows (zero), whose products are not stored
    const uint32_t uoff = (uint32_t)(m0 * 8 + 16 * lane), uoff2 = (uint32_t)(m0 * 8 + 1024 + 4 * lane);
    // summaries: 8 pieces of 8 rows x 128 B; lane fills 16-byte position
    // lane & 7 of row 8 q + lane / 8, holding 32-byte unit ((lane & 7) / 2) ^
    // (row & 3) of the wave's 64 columns
    const int brow = lane >> 3;  // + 8 q (row & 3 does not depend on q)
    const int bcol = n0 + 16 * (((lane & 7) >> 1) ^ (brow & 3)) + 8 * (lane & 1);
    const uint32_t boff = (uint32_t)(brow * bp + bcol) * 2;
    char* const wbase = lds + w * 2 * kWSt;
    auto issue = [&](int stage, int kk) {
        char* A = wbase + stage * kWSt;
        char* B = A + kWU;
        const uint32_t us = (uint32_t)kk * rows * 8;
        load_lds16(ru, uoff, us, A);
        load_lds4(ru, uoff2, us, A + 1024);
        const int j0 = kk * kGK;
        if (j0 + kGK <= Tkv) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                load_lds16(rh, boff, (uint32_t)(j0 + 8 * q) * bp * 2, B + 1024 * q);
        } else {  // rows past T_kv repeat row T_kv - 1, whose U bits are 0
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int jr = min(j0 + 8 * q + brow, Tkv - 1);
                load_lds16(rh, (uint32_t)(jr * bp + bcol) * 2, 0, B + 1024 * q);
            }
        }
    };

    // per-lane LDS addresses (stage 0): this lane's U bits (row 32 m + l32 of
    // the wave's, 8 bytes) and the summaries operand of column tile nt
    // (transposed reads; sub-step and half rows as immediates)
    const uint32_t tbase = lds_addr(tbl);
    const uint32_t ubit = lds_addr(wbase) + (uint32_t)(l32 * 8);
    const int r16 = lane & 15, G = lane >> 4;
    uint32_t aB[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
        aB[nt] = lds_addr(wbase) + kWU +
                 (uint32_t)((8 * (G >> 1) + (r16 >> 2)) * 128 +
                            (((2 * nt + (G & 1)) ^ (r16 >> 2)) << 5) + 8 * (r16 & 3));

    f32x16 acc[5][2];
#pragma unroll
    for (int m = 0; m < 5; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = zero16();
    auto mma = [&](const SubOps& x) {
        typedef short s16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const s16x4 p = x.b[2 * nt], q = x.b[2 * nt + 1];
            const s16x8 v = {p[0], p[1], p[2], p[3], q[0], q[1], q[2], q[3]};
            const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
            for (int m = 0; m < 5; ++m)
                acc[m][nt] = mfma_bf16(__builtin_bit_cast(bf16x8, x.a[m]), b, acc[m][nt]);
        }
    };

    issue(0, 0);
    for (int kk = 0; kk < nk; ++kk) {
        // the next stage goes into the buffer this wave finished reading in
        // the previous iteration; then wait for stage kk (10 loads per stage)
        if (kk + 1 < nk) {
            issue((kk + 1) & 1, kk + 1);
            wait_vmcnt<10>();
        } else {
            wait_vmcnt<0>();
        }
        const uint32_t so = (uint32_t)((kk & 1) * kWSt);
        const uint32_t b0 = aB[0] + so, b1 = aB[1] + so;
        // the five rows' U bits of this stage; byte 2 s + hl of row m is the
        // U fragment of sub-step s, read from the table
        uint2 ub[5];
        asm volatile(
            "ds_read_b64 %0, %5 offset:0\n\t"
            "ds_read_b64 %1, %5 offset:256\n\t"
            "ds_read_b64 %2, %5 offset:512\n\t"
            "ds_read_b64 %3, %5 offset:768\n\t"
            "ds_read_b64 %4, %5 offset:1024\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(ub[0]), "=&v"(ub[1]), "=&v"(ub[2]), "=&v"(ub[3]), "=&v"(ub[4])
            : "v"(ubit + so));
        uint32_t ua[4][5];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int m = 0; m < 5; ++m) {
                const uint32_t wd = s < 2 ? ub[m].x : ub[m].y;
                ua[s][m] = tbase + (((wd >> (16 * (s & 1) + 8 * hl)) & 0xffu) << 4);
            }
        // each sub-step's reads are in flight while the previous one's
        // products run
        SubOps x0, x1;
        read_sub<0>(ua[0], b0, b1, x0);
        read_sub_async<1>(ua[1], b0, b1, x1, x0);
        mma(x0);
        wait_ops(x1, x0);
        read_sub_async<2>(ua[2], b0, b1, x0, x1);
        mma(x1);
        wait_ops(x0, x1);
        read_sub_async<3>(ua[3], b0, b1, x1, x0);
        mma(x0);
        wait_ops(x1, x0);
        mma(x1);
    }

    // Output.  Accumulator (m, nt, r) is row 32 m + 8 (r / 4) + 4 hl + r % 4
    // of the wave's 160 and column 32 nt + l32 of its 64.  The H columns
    // (below d*d) go out in bf16 (nearest even) through the wave's own LDS
    // region (free now: no other wave reads it), so that the global stores
    // are whole 128-byte row pieces: rows of m-tiles 0-2, then 3-4.  The Z
    // columns (one column tile) go out in fp32 directly.
    if constexpr (F32) {
        float* of = reinterpret_cast<float*>(HZ) + (size_t)bh * Tq * nt * 128;
#pragma unroll
        for (int m = 0; m < 5; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qb = m0 + 32 * m + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (qb < Tq) of[(size_t)qb * nt * 128 + n0 + 32 * n + l32] = acc[m][n][r];
                }
        return;
    }
    char* out = HZ + (size_t)bh * Tq * kHzRowBytes;
    if (n0 >= 128 * 128) {
#pragma unroll
        for (int m = 0; m < 5; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int col = n0 + 32 * nt + l32;
                if (col >= kHzCols) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qb = m0 + 32 * m + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (qb < Tq)
                        reinterpret_cast<float*>(out + (size_t)qb * kHzRowBytes + 2 * 128 * 128)
                            [col - 128 * 128] = acc[m][nt][r];
                }
            }
        return;
    }
    __bf16* st = reinterpret_cast<__bf16*>(wbase);  // [rows][64] bf16
    auto flush = [&](int m_lo, int m_hi) {
#pragma unroll
        for (int m = m_lo; m < m_hi; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lr = 32 * (m - m_lo) + 8 * (r >> 2) + 4 * hl + (r & 3);
                    st[lr * 64 + 32 * nt + l32] = (__bf16)acc[m][nt][r];
                }
        wait_lgkm0();
        const int nrow = 32 * (m_hi - m_lo);
        for (int i = 0; i < nrow / 8; ++i) {
            const int lr = 8 * i + (lane >> 3);
            const int qb = m0 + 32 * m_lo + lr;
            const uint4 v = *reinterpret_cast<const uint4*>(wbase + lr * 128 + (lane & 7) * 16);
            if (qb < Tq)
                *reinterpret_cast<uint4*>(out + (size_t)qb * kHzRowBytes + n0 * 2 + (lane & 7) * 16) = v;
        }
        wait_lgkm0();  // the reads are done before the region is written again
    };
    flush(0, 3);
    flush(3, 5);
}

}  // namespace

hipError_t launch_unsel(const Dims& D, const int32_t* idx, const int32_t* negl, int kl,
                        const FwdWS& ws, hipStream_t s) {
    const int tp = tkv_pad(D);
    if (tp > kMaxTkvPad) return hipErrorInvalidValue;
    const int rows = ubit_rows(D);
    unsel_kernel<<<dim3((unsigned)(D.BH * rows)), 256, 0, s>>>(idx, D.k, negl, kl, ws.usel, D.Tq,
                                                               D.Tkv, tp, rows, 0);
    return hipGetLastError();
}

size_t sel_product_bits_bytes(const Dims& D) {
    const size_t a = (size_t)D.BH * (tkv_pad(D) / 64) * ubit_rows(D) * 8;
    const int tqp = (D.Tq + 63) & ~63;
    const int rt = (D.Tkv + kGemmM - 1) / kGemmM * kGemmM + 64;
    const size_t b = (size_t)D.BH * (tqp / 64) * rt * 8;
    return a > b ? a : b;
}

hipError_t launch_sel_product(const Dims& D, bool keys, const int32_t* idx, const int32_t* off,
                              const int32_t* list, uint8_t* bits, const uint16_t* B, float* out,
                              hipStream_t s) {
    // rows: query blocks (keys = false: the KV blocks each selects, B = per-
    // KV-block matrices) or KV blocks (keys = true: the query blocks selecting
    // each, B = per-query-block matrices); the k dimension is the other side
    const int nr = keys ? D.Tkv : D.Tq, nk = keys ? D.Tq : D.Tkv;
    const int nkp = (nk + 63) & ~63;
    if (nkp > kMaxTkvPad) return hipErrorInvalidValue;
    const int nM = (nr + kGemmM - 1) / kGemmM;
    const int rows = nM * kGemmM + 64;
    if (keys)
        csr_bits_kernel<<<dim3((unsigned)(D.BH * rows)), 256, 0, s>>>(off, list, D.k, bits, D.Tq,
                                                                    D.Tkv, nkp, rows);
    else
        unsel_kernel<<<dim3((unsigned)(D.BH * rows)), 256, 0, s>>>(idx, D.k, nullptr, 0, bits,
                                                                   D.Tq, D.Tkv, nkp, rows, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kNT32 = 128 * 128 / kGN;  // d x d matrices: 128 column tiles
    timing_before(s, K_BWD_LIN_PRODUCT);
    lin_gemm_kernel<true><<<dim3((unsigned)(D.BH * kNT32 * nM)), 256, 0, s>>>(
        bits, B, reinterpret_cast<char*>(out), nr, nk, nkp, nM, rows, kNT32, 128 * 128);
    timing_after(s, K_BWD_LIN_PRODUCT);
    return hipGetLastError();
}

hipError_t launch_lin_gemm(const Dims& D, const FwdWS& ws, hipStream_t s) {
    const int nM = (D.Tq + kGemmM - 1) / kGemmM;
    timing_before(s, K_LIN_GEMM);
    lin_gemm_kernel<false><<<dim3((unsigned)(D.BH * kNT * nM)), 256, 0, s>>>(
        ws.usel, ws.hz, ws.HZ, D.Tq, D.Tkv, tkv_pad(D), nM, ubit_rows(D), kNT, kHzPitch);
    timing_after(s, K_LIN_GEMM);
    return hipGetLastError();
}

}  // namespace sla2
