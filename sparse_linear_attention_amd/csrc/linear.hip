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
// the negligible ones, which leave the linear branch as well).  lin_gemm_kernel multiplies it with the per-block
// summaries written by the block-summaries pass (bf16 rows of h_j^T, then
// z_j) on the bf16 matrix cores (32x32x16, fp32 accumulation) into fp32
// rows of H_i^T and Z_i that the fused kernel's epilogue reads.
//
// Product tiles: 320 query blocks x 128 columns per work-group of 4 waves
// (2 x 2: each wave 5 x 2 tiles of 32 x 32), 64 KV blocks per LDS stage (one
// barrier per 40 products of a wave), both operands staged by direct-to-LDS
// loads three stages ahead, four stages; 80 KB of LDS, so that two
// work-groups share a compute unit and one's barrier gaps are filled by the
// other's products.  LDS layouts:
//   U bits   [320 rows][8 B]    bit b of byte g: KV block 8 g + b of the stage
//   hz tile  [64 rows][256 B]   64-byte unit u of row r at u ^ (r & 3)
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

constexpr int kMaxTkvPad = 7680;
constexpr int kGN = 128;                 // columns per tile
constexpr int kGK = 64;                  // KV blocks per stage
constexpr int kNT = kHzPitch / kGN;      // column tiles (130)
constexpr int kUB = 3072;                // U bits per stage: 320 rows x 8 bytes, loaded
                                         // as three 1 KB pieces (the last one partly unused)
constexpr int kBB = kGK * kGN * 2;       // summaries stage bytes (16 KB)
constexpr int kSt = kUB + kBB;
constexpr int kNS = 4;                   // stages
constexpr int kTbl = 4096;               // byte -> 8 bf16 0/1 values
static_assert(kGemmM == 320, "tile shape");
static_assert(kNS * kSt + kTbl <= 80 * 1024, "LDS budget: two work-groups per CU");

// One work-group per row of U: query block i of head bh (rows past T_q, up to
// the padded row count, are all zero).  Bit b of byte g of the row is KV
// block 8 g + b.  Stored k-step major, [BH][Tkvp / 64][rows][8 bytes], so
// that a product tile's 320 rows of one k-step are contiguous.
__global__ __launch_bounds__(256) void unsel_kernel(const int32_t* __restrict__ idx, int k,
                                                    const int32_t* __restrict__ negl, int kl,
                                                    uint8_t* __restrict__ U, int Tq, int Tkv,
                                                    int Tkvp, int rows) {
    __shared__ uint32_t row[kMaxTkvPad / 32];
    const int t = threadIdx.x;
    const long bh = blockIdx.x / rows;
    const int i = blockIdx.x % rows;
    const int nw = Tkvp / 32;
    for (int x = t; x < nw; x += 256) {
        const int lo = 32 * x;
        uint32_t v = 0;
        if (i < Tq) v = Tkv >= lo + 32 ? 0xffffffffu : (Tkv > lo ? (1u << (Tkv - lo)) - 1u : 0u);
        row[x] = v;
    }
    __syncthreads();
    if (i < Tq) {
        const size_t r = (size_t)bh * Tq + i;
        for (int x = t; x < k; x += 256) {
            const int j = idx[r * k + x];
            if ((unsigned)j < (unsigned)Tkv) atomicAnd(&row[j >> 5], ~(1u << (j & 31)));
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
          "i"(4096 * S), "i"(4096 * S + 1024));
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
          "i"(4096 * S), "i"(4096 * S + 1024));
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

// wait until at most `ahead` later stages (L loads each) are in flight
template <int L>
__device__ inline void wait_stages(int ahead) {
    if (ahead >= 2) wait_vmcnt<2 * L>();
    else if (ahead == 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
}

__global__ __launch_bounds__(256, 2) void lin_gemm_kernel(const uint8_t* __restrict__ U,
                                                         const uint16_t* __restrict__ hz,
                                                         float* __restrict__ HZ, int Tq, int Tkv,
                                                         int Tkvp, int nM, int rows) {
    __shared__ __attribute__((aligned(1024))) char lds[kNS * kSt + kTbl];
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    int g = blockIdx.x;
    const int mi = g % nM;
    g /= nM;
    const int ni = g % kNT;
    const long bh = g / kNT;
    const int m0 = mi * kGemmM, n0 = ni * kGN;
    const int nk = Tkvp / kGK;
    const rsrc_t ru = head_rsrc(U + (size_t)bh * nk * rows * 8);
    const rsrc_t rh = head_rsrc(hz + (size_t)bh * Tkv * kHzPitch);

    // byte table: entry v holds the 8 bf16 values bit e of v (0 or 1)
    char* const tbl = lds + kNS * kSt;
    if (t < 256) {
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d[e] = (((t >> (2 * e)) & 1) ? 0x3F80u : 0u) | (((t >> (2 * e + 1)) & 1) ? 0x3F800000u : 0u);
        *reinterpret_cast<uint4*>(tbl + 16 * t) = make_uint4(d[0], d[1], d[2], d[3]);
    }
    wait_lgkm0();  // visible to every wave after the first barrier of the loop

    // U bits of a stage: rows m0 .. m0 + 319 of k-step kk (2560 contiguous
    // bytes), loaded as pieces 0..2 of 1 KB by waves 0..2 (the tail of piece
    // 2 holds the next rows or the padding, unused)
    const uint32_t uoff = (uint32_t)(m0 * 8 + 16 * lane);
    // summaries pieces q = w + 4 i (16 of 4 rows x 256 B): this lane fills
    // position lane & 15 of row 4 q + lane / 16; rows past T_kv repeat row
    // T_kv - 1, whose U bits are 0
    int brow[4], bcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        brow[i] = 4 * (w + 4 * i) + (lane >> 4);
        const int u = ((lane & 15) >> 2) ^ (brow[i] & 3);
        bcol[i] = n0 + 32 * u + 8 * (lane & 3);
    }
    auto issue = [&](int stage, int kk) {
        char* A = lds + stage * kSt;
        char* B = A + kUB;
        if (w < 3) load_lds16(ru, uoff + 1024 * w, (uint32_t)kk * rows * 8, A + 1024 * w);
        const int j0 = kk * kGK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int jr = min(j0 + brow[i], Tkv - 1);
            load_lds16(rh, (uint32_t)(jr * kHzPitch + bcol[i]) * 2, 0, B + (w + 4 * i) * 1024);
        }
    };

    // per-lane LDS addresses (stage 0): this lane's U bits (row 160 wm + 32 m
    // + l32, 8 bytes) and the summaries operand of column tile nt
    // (transposed reads; sub-step and half rows as immediates)
    const uint32_t base = lds_addr(lds), tbase = lds_addr(tbl);
    const uint32_t ubit = base + (uint32_t)((160 * wm + l32) * 8);
    const int r16 = lane & 15, G = lane >> 4;
    uint32_t aB[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
        aB[nt] = base + kUB +
                 (uint32_t)((8 * (G >> 1) + (r16 >> 2)) * 256 + (((2 * wn + nt) ^ (r16 >> 2)) << 6) +
                            32 * (G & 1) + 8 * (r16 & 3));

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

#pragma unroll
    for (int q = 0; q < kNS - 1; ++q)
        if (q < nk) issue(q, q);
    for (int kk = 0; kk < nk; ++kk) {
        // stage kk has landed for this wave (waves 0-2 issue 5 loads per
        // stage, the others 4) ...
        const int ahead = min(kNS - 2, nk - 1 - kk);
        if (w < 3) wait_stages<5>(ahead);
        else wait_stages<4>(ahead);
        wg_barrier();  // ... and for every wave; all are done with stage kk - 1
        if (kk + kNS - 1 < nk) issue((kk + kNS - 1) % kNS, kk + kNS - 1);
        const uint32_t so = (uint32_t)((kk % kNS) * kSt);
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

    // rows (query blocks) 8 (r / 4) + 4 hl + r % 4 of each 32 x 32 tile,
    // column l32: 32 consecutive floats per row and half-wave
    float* out = HZ + (size_t)bh * Tq * kHzCols;
#pragma unroll
    for (int m = 0; m < 5; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int col = n0 + 64 * wn + 32 * nt + l32;
            if (col >= kHzCols) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qb = m0 + 160 * wm + 32 * m + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (qb < Tq) out[(size_t)qb * kHzCols + col] = acc[m][nt][r];
            }
        }
}

}  // namespace

hipError_t launch_unsel(const Dims& D, const int32_t* idx, const int32_t* negl, int kl,
                        const FwdWS& ws, hipStream_t s) {
    const int tp = tkv_pad(D);
    if (tp > kMaxTkvPad) return hipErrorInvalidValue;
    const int rows = ubit_rows(D);
    unsel_kernel<<<dim3((unsigned)(D.BH * rows)), 256, 0, s>>>(idx, D.k, negl, kl, ws.usel, D.Tq,
                                                               D.Tkv, tp, rows);
    return hipGetLastError();
}

hipError_t launch_lin_gemm(const Dims& D, const FwdWS& ws, hipStream_t s) {
    const int nM = (D.Tq + kGemmM - 1) / kGemmM;
    timing_before(s, K_LIN_GEMM);
    lin_gemm_kernel<<<dim3((unsigned)(D.BH * kNT * nM)), 256, 0, s>>>(
        ws.usel, ws.hz, ws.HZ, D.Tq, D.Tkv, tkv_pad(D), nM, ubit_rows(D));
    timing_after(s, K_LIN_GEMM);
    return hipGetLastError();
}

}  // namespace sla2
