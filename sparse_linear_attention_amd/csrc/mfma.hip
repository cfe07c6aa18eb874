// bf16 forward path on the CDNA4 matrix cores: block summaries, and the
// fused kernel for d = 64 (d = 128 has its own kernel, fused128.hip).
//
// 1) summaries_mfma: one pass over K and V.  Per KV block j of 64 tokens it
//    writes V_j^T and phi(K_j)^T in fp16, block-transposed ([d][64]) with the
//    token order permuted inside each group of 16 (positions = token index
//    with bits 2 and 3 swapped), and the per-block z_j = colsum phi(K_j); it
//    accumulates h = sum_j phi(K_j)^T V_j and z = sum_j z_j on the matrix
//    cores into per-chunk partials (reduced in a fixed order afterwards).
//    phi is elu + 1, or (phi_sm) the softmax of each K row over its D
//    channels in fp32 (the SLA notes' feature map), max-subtracted.
//    Linear-branch block summaries: SLA notes, key design 4 (h_j =
//    phi(K_j)^T V_j, z_j).
// 2) fused_mfma (d = 64): per (head, query block of 128) a work-group of 4
//    waves; wave w owns queries 32w..32w+31.  For every selected KV block
//    (ascending):
//      S^T = K_j Q^T            (bf16 MFMA 32x32x16, fp32 accumulate)
//      online softmax on S^T    (each lane holds one query's column)
//      O^T += V_j^T P^T         (fp16 MFMA; P rounded to fp16)
//      G^T += V_j^T phi(K_j)    (fp16 MFMA; the selected part of h)
//    Epilogue: H^T = h_tot^T - G^T, Z = z_tot - sum z_j, O_l^T = H^T phi(Q)^T
//    (fp16 MFMA) / (phi(Q) . Z), O = alpha O_s + (1 - alpha) O_l.
//    Sparse branch: "SLA2 深度解读" 04 and 08 (only mask-hit blocks run QK
//    and PV); linear branch: SLA notes key design 3 (H_i, Z_i, O_l);
//    combine: "SLA2 深度解读" 04.
//
// Only the C layout of the matrix instructions is relied on for meaning
// (P^T is fed straight from the S^T accumulators); the k order inside an
// instruction only has to agree between A and B, which holds because both
// operands are loaded with the same position rule.
#include <algorithm>

#include "cdna4.h"
#include "sla2_internal.h"

namespace sla2 {
namespace {
using namespace cdna4;

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
// two floats as bf16 (nearest even), a in the low half
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Cross-lane steps of the fp64 column sums (pooled keys).  Half-exchange:
// the lanes whose partner bit is clear keep x (their value of the lower half
// of a channel set), the others keep y (upper half); each gets its kept
// value plus the partner's value of the same half.  Partner lane ^ 32 and
// ^ 16 by the gfx950 lane swaps (x' = x's lower lanes with y's lower lanes
// moved up, y' = the rest; the kept sum is x' + y' in every lane), ^ 8 by a
// rotation of each 16-lane row.
__device__ inline double f64_of(unsigned lo, unsigned hi) {
    return __hiloint2double((int)hi, (int)lo);
}
__device__ inline double half_xchg32(double x, double y) {
    const auto l = __builtin_amdgcn_permlane32_swap((unsigned)__double2loint(x),
                                                    (unsigned)__double2loint(y), false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((unsigned)__double2hiint(x),
                                                    (unsigned)__double2hiint(y), false, false);
    return f64_of(l[0], h[0]) + f64_of(l[1], h[1]);
}
__device__ inline double half_xchg16(double x, double y) {
    const auto l = __builtin_amdgcn_permlane16_swap((unsigned)__double2loint(x),
                                                    (unsigned)__double2loint(y), false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((unsigned)__double2hiint(x),
                                                    (unsigned)__double2hiint(y), false, false);
    return f64_of(l[0], h[0]) + f64_of(l[1], h[1]);
}
template <int CTRL>
__device__ inline double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ inline double half_xchg8(double x, double y, bool up) {
    return (up ? y : x) + dpp_f64<0x128>(up ? x : y);  // row_ror:8 = lane ^ 8 in a row
}
// sum over the 8 lanes of each aligned group: lane ^ 1, ^ 2 (quad
// permutations), then the mirror inside the 8 (lane i <-> 7 - i)
__device__ inline double sum8_f64(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    return v;
}

// token u of a 64-block -> its position in the transposed layouts
__device__ inline int perm_pos(int u) {
    return (u & ~12) | ((u >> 1) & 4) | ((u << 1) & 8);
}

// ---------------------------------------------------------------------------
// block summaries
// ---------------------------------------------------------------------------
constexpr int kTPitch = 64 * 2 + 16;  // bytes per row of a [d][64] fp16 tile in LDS

// HZ: instead of phi(K)^T tiles, z_j and chunk partials, write every block's
// summaries for the linear-branch product (linear.hip): row j of hz holds
// h_j^T (V channel e, phi channel c; 16-byte units in the order hz_unit
// gives) and then z_j, in bf16; V^T tiles only if vt is not null.  With xk not null the pass
// also writes the router's pooled keys ("SLA2 深度解读" 03: the mean of each
// KV block, [BH][Tkv][D] fp64), from the K rows it holds anyway: each wave
// sums its channels over the 64 tokens (one per lane) in fp64 by a
// reduce-scatter across the lanes, 8 channels at a time; with kblk not null
// the sums themselves as well ([BH][Tkv][D] fp64: the low-bit path's K mean
// is taken from them).  The sums of bf16 values are exact in fp64
// unless a block's values span more than about 2^39 in magnitude, so they
// equal those of the router's own pooling pass.
template <int D, bool HZ>
__global__ __launch_bounds__(256, 4) void summaries_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, uint16_t* __restrict__ vt,
    uint16_t* __restrict__ pkt, float* __restrict__ zb, float* __restrict__ hpart,
    float* __restrict__ zpart, uint16_t* __restrict__ hz, int N, int Tkv, int nch, int H,
    Strides st, int phi_sm, double* __restrict__ xk, double* __restrict__ kblk, int bpc) {
    static_assert(!HZ || D == 128, "per-block summaries: d = 128");
    constexpr int NT = D / 32;
    constexpr int TPW = NT * NT / 4;  // h^T tiles per wave
    __shared__ __attribute__((aligned(16))) char sV[D * kTPitch];
    __shared__ __attribute__((aligned(16))) char sP[D * kTPitch];
    __shared__ float sRed[2][4][64];  // softmax phi: per-wave row max / sum
    // wave index as a scalar: conditions on it must be wave-uniform branches
    // (matrix instructions ignore EXEC, so they may never sit under a lane mask)
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int chunk = blockIdx.x;
    const long bh = blockIdx.y;
    const int j0 = chunk * bpc;
    const int j1 = min(Tkv, j0 + bpc);
    const uint16_t* Kh = K + head_base(st, bh, H);
    const uint16_t* Vh = V + head_base(st, bh, H);
    const int nt_w = w % NT;       // this wave's n-tile (phi(K) channels)
    const int mt_w0 = w / NT;      // first m-tile (V channels)
    constexpr int MT_STEP = 4 / NT;

    f32x16 acc[TPW];
#pragma unroll
    for (int s = 0; s < TPW; ++s) acc[s] = zero16();
    float zacc = 0.0f;  // thread t < D: channel t

    for (int j = j0; j < j1; ++j) {
        __syncthreads();
        // load 64 tokens x D channels; lane -> token, wave + pass -> channel group
        constexpr int CG = D / 8;
        constexpr int NP = CG / 4;
        const int u = lane;
        const int tok = j * 64 + u;
        const bool ok = tok < N;
        uint4 kvs[NP], vvs[NP];
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int cg = w + 4 * pass;
            kvs[pass] = make_uint4(0, 0, 0, 0);
            vvs[pass] = make_uint4(0, 0, 0, 0);
            if (ok) {
                kvs[pass] = *reinterpret_cast<const uint4*>(Kh + (size_t)tok * st.t + cg * 8);
                vvs[pass] = *reinterpret_cast<const uint4*>(Vh + (size_t)tok * st.t + cg * 8);
            }
        }
        // softmax phi: row max and 1 / sum exp over the D channels of token u
        // (this wave holds NP groups of 8; the four waves are combined in LDS)
        float rmax = 0.0f, rinv = 1.0f;
        if (phi_sm) {
            float m = -INFINITY;
#pragma unroll
            for (int pass = 0; pass < NP; ++pass) {
                const unsigned kw[4] = {kvs[pass].x, kvs[pass].y, kvs[pass].z, kvs[pass].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(bf16_lo(kw[e]), bf16_hi(kw[e])));
            }
            sRed[0][w][u] = m;
            __syncthreads();
            rmax = fmaxf(fmaxf(sRed[0][0][u], sRed[0][1][u]), fmaxf(sRed[0][2][u], sRed[0][3][u]));
            float sum = 0.0f;
#pragma unroll
            for (int pass = 0; pass < NP; ++pass) {
                const unsigned kw[4] = {kvs[pass].x, kvs[pass].y, kvs[pass].z, kvs[pass].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sum += __expf(bf16_lo(kw[e]) - rmax) + __expf(bf16_hi(kw[e]) - rmax);
            }
            sRed[1][w][u] = sum;
            __syncthreads();
            rinv = 1.0f / ((sRed[1][0][u] + sRed[1][1][u]) + (sRed[1][2][u] + sRed[1][3][u]));
        }
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int cg = w + 4 * pass;
            const unsigned kw[4] = {kvs[pass].x, kvs[pass].y, kvs[pass].z, kvs[pass].w};
            const unsigned vw[4] = {vvs[pass].x, vvs[pass].y, vvs[pass].z, vvs[pass].w};
            const int pos = perm_pos(u);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kf = (e & 1) ? bf16_hi(kw[e >> 1]) : bf16_lo(kw[e >> 1]);
                const float vf = (e & 1) ? bf16_hi(vw[e >> 1]) : bf16_lo(vw[e >> 1]);
                const float pf = phi_sm ? __expf(kf - rmax) * rinv : phi_fast(kf);
                const _Float16 ph = ok ? (_Float16)pf : (_Float16)0.0f;
                const _Float16 vh = ok ? (_Float16)vf : (_Float16)0.0f;
                const int c = cg * 8 + e;
                *reinterpret_cast<_Float16*>(sP + c * kTPitch + pos * 2) = ph;
                *reinterpret_cast<_Float16*>(sV + c * kTPitch + pos * 2) = vh;
            }
        }
        if constexpr (HZ) {
          if (xk) {
            // block mean of K, per group of 8 channels (w + 4 pass): v[i] is
            // channel 8 (w + 4 pass) + i of this lane's token; halve the set
            // per step, keeping the lower or upper half by a lane bit and
            // adding the partner's copy of it, then add across the remaining
            // lane bits: lane l ends with channel l / 8 of the group summed
            // over all 64 tokens
            const int n = min(64, N - j * 64);
#pragma unroll
            for (int pass = 0; pass < NP; ++pass) {
                const unsigned kw[4] = {kvs[pass].x, kvs[pass].y, kvs[pass].z, kvs[pass].w};
                double v[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = (double)bf16_lo(kw[e]);
                    v[2 * e + 1] = (double)bf16_hi(kw[e]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = half_xchg32(v[i], v[i + 4]);
#pragma unroll
                for (int i = 0; i < 2; ++i) v[i] = half_xchg16(v[i], v[i + 2]);
                v[0] = sum8_f64(half_xchg8(v[0], v[1], (lane & 8) != 0));
                if ((lane & 7) == 0) {
                    const size_t o = ((size_t)bh * Tkv + j) * D + (w + 4 * pass) * 8 + (lane >> 3);
                    xk[o] = v[0] / (double)n;
                    if (kblk) kblk[o] = v[0];
                }
            }
          }
        }
        __syncthreads();
        // write the transposed tiles (contiguous D*64 fp16 each) and z_j
        if (!HZ || vt) {
            uint16_t* gv = vt + ((size_t)bh * Tkv + j) * D * 64;
            for (int x = t; x < D * 8; x += 256) {
                const int row = x >> 3, c16 = x & 7;
                *reinterpret_cast<uint4*>(gv + row * 64 + c16 * 8) =
                    *reinterpret_cast<const uint4*>(sV + row * kTPitch + c16 * 16);
                if (!HZ) {
                    uint16_t* gp = pkt + ((size_t)bh * Tkv + j) * D * 64;
                    *reinterpret_cast<uint4*>(gp + row * 64 + c16 * 8) =
                        *reinterpret_cast<const uint4*>(sP + row * kTPitch + c16 * 16);
                }
            }
        }
        if (HZ && !hz) continue;  // no linear branch: V^T only
        uint16_t* hzj = HZ ? hz + ((size_t)bh * Tkv + j) * kHzPitch : nullptr;
        if (t < D) {
            float z = 0.0f;
            const _Float16* rowp = reinterpret_cast<const _Float16*>(sP + t * kTPitch);
            for (int p = 0; p < 64; ++p) z += (float)rowp[p];
            if (HZ) {
                hzj[D * D + t] = __builtin_bit_cast(uint16_t, (__bf16)z);
            } else {
                zb[((size_t)bh * Tkv + j) * D + t] = z;
                zacc += z;
            }
        }
        if constexpr (HZ) {
            // h_j (phi channels c x V channels e) = phi(K_j)^T V_j; lane holds
            // column e and four consecutive rows c per group of its tiles
            f32x16 hj[TPW];
#pragma unroll
            for (int s = 0; s < TPW; ++s) hj[s] = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f16x8 b = *reinterpret_cast<const f16x8*>(sV + (32 * nt_w + l32) * kTPitch +
                                                                (16 * ks + 8 * hl) * 2);
#pragma unroll
                for (int s = 0; s < TPW; ++s) {
                    const int mt = mt_w0 + s * MT_STEP;
                    const f16x8 a = *reinterpret_cast<const f16x8*>(
                        sP + (32 * mt + l32) * kTPitch + (16 * ks + 8 * hl) * 2);
                    hj[s] = mfma_f16(a, b, hj[s]);
                }
            }
            // bf16 (nearest even), then units of 8 consecutive c: the lane
            // pair (l32, l32 + 32) holds c = 8 g + 0..3 and 8 g + 4..7 of
            // group g; one lane-half swap gives the lower lane group 2 q
            // whole and the upper lane group 2 q + 1.  With D = 128 wave w
            // holds e = 32 w + l32 and tile s rows c = 32 s + .., so its
            // unit is (e, 4 s + 2 q + hl), at hz_unit = ((w * 4 + s) * 2 +
            // q) * 64 + lane: each store is 1 KB of the row, contiguous
            static_assert(!HZ || (NT == 4 && MT_STEP == 1), "unit order: D = 128");
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                uint32_t dw[4][2];
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    dw[g4][0] = pack_bf16x2(hj[s][4 * g4], hj[s][4 * g4 + 1]);
                    dw[g4][1] = pack_bf16x2(hj[s][4 * g4 + 2], hj[s][4 * g4 + 3]);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    uint32_t r[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const uint32_t send = hl ? dw[2 * q][h2] : dw[2 * q + 1][h2];
                        const auto x = __builtin_amdgcn_permlane32_swap(send, send, false, false);
                        r[h2] = hl ? x[0] : x[1];
                    }
                    const uint4 u = hl ? make_uint4(r[0], r[1], dw[2 * q + 1][0], dw[2 * q + 1][1])
                                       : make_uint4(dw[2 * q][0], dw[2 * q][1], r[0], r[1]);
                    *reinterpret_cast<uint4*>(hzj + (((w * TPW + s) * 2 + q) * 64 + lane) * 8) = u;
                }
            }
            continue;
        }
        // h^T (V channels x phi(K) channels) += V_j^T phi(K_j)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f16x8 b = *reinterpret_cast<const f16x8*>(sP + (32 * nt_w + l32) * kTPitch +
                                                            (16 * ks + 8 * hl) * 2);
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                const int mt = mt_w0 + s * MT_STEP;
                const f16x8 a = *reinterpret_cast<const f16x8*>(sV + (32 * mt + l32) * kTPitch +
                                                                (16 * ks + 8 * hl) * 2);
                acc[s] = mfma_f16(a, b, acc[s]);
            }
        }
    }
    if (HZ) return;
    // partial h[c][e]: c = phi(K) channel (C column), e = V channel (C row)
    float* hp = hpart + ((size_t)bh * nch + chunk) * D * D;
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        const int mt = mt_w0 + s * MT_STEP;
        const int c = 32 * nt_w + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = 32 * mt + 8 * (r >> 2) + 4 * hl + (r & 3);
            hp[(size_t)c * D + e] = acc[s][r];
        }
    }
    if (t < D) zpart[((size_t)bh * nch + chunk) * D + t] = zacc;
}

// ---------------------------------------------------------------------------
// fused sparse + linear + combine
// ---------------------------------------------------------------------------
template <int D>
struct FusedSmem {
    static constexpr int kKPitch = D * 2 + 16;              // K tile row (bf16)
    static constexpr int kK = 64 * kKPitch;                 // K tile
    static constexpr int kT = D * kTPitch;                  // V^T or phi(K)^T tile
    static constexpr int kHPitch = D * 2 + 16;              // H^T row (fp16)
    static constexpr int kTiles = kK + 2 * kT;
    static constexpr int kEpi = D * kHPitch + D * 4;        // H^T + Z
    static constexpr int kBytes = kTiles > kEpi ? kTiles : kEpi;
};

// lazy-rescale threshold (log2 units): P~ stays <= 2^8 between rescales
constexpr float kRescaleThr = 8.0f;

template <int D>
__global__ __launch_bounds__(256, 2) void fused_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ vt, const uint16_t* __restrict__ pkt,
    const float* __restrict__ zb, const int32_t* __restrict__ idx,
    const float* __restrict__ alpha, const float* __restrict__ htot,
    const float* __restrict__ ztot, void* __restrict__ O, int N, int Tq, int Tkv, int k,
    int H, Strides st, int alpha_qblock, int out_bf16) {
    using SM = FusedSmem<D>;
    constexpr int NT = D / 32;       // 32-wide tiles along d
    constexpr int KS = D / 16;       // k-steps of Q K^T
    __shared__ __attribute__((aligned(16))) char smem[SM::kBytes];
    char* sK = smem;
    char* sV = smem + SM::kK;
    char* sP = sV + SM::kT;

    // wave index as a scalar: conditions on it must be wave-uniform branches
    // (matrix instructions ignore EXEC, so they may never sit under a lane mask)
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    long bh;
    int qb;
    if (!head_major_map(blockIdx.x, Tq, &bh, &qb)) return;
    const int tq = qb * 128 + 32 * w + l32;  // this lane's query
    const bool valid_q = tq < N;
    const bool need_lin = k < Tkv;
    // G^T tiles: wave w accumulates every m-tile (V channels) of n-tile
    // w % NT (phi(K) channels); with D = 64 two waves share an n-tile.
    const int nt_w = w % NT;
    const float c_log2 = 1.4426950408889634f / sqrtf((float)D);

    // Q^T fragments (B operand): lane holds Q[tq][16ks + 8hl .. +8]
    bf16x8 qf[KS];
    {
        const uint16_t* qrow = Q + head_base(st, bh, H) + (size_t)(valid_q ? tq : 0) * st.t;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid_q) v = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    f32x16 o[NT], g[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        o[i] = zero16();
        g[i] = zero16();
    }
    float m_ref = -INFINITY;  // log2-domain reference max of this query
    float l_part = 0.0f;      // row sum over this lane's half of the tokens
    float zsel0 = 0.0f, zsel1 = 0.0f;

    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;
    const uint16_t* Kh = K + head_base(st, bh, H);

    for (int r = 0; r < k; ++r) {
        const int j = sel[r];
        __syncthreads();
        // ---- stage K_j (bf16 rows), V_j^T and phi(K_j)^T (fp16) in LDS
        constexpr int KCH = 64 * D / 8;  // 16-byte chunks of the K tile
#pragma unroll
        for (int x = t; x < KCH; x += 256) {
            const int row = x / (D / 8), cg = x % (D / 8);
            const int tok = j * 64 + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tok < N) v = *reinterpret_cast<const uint4*>(Kh + (size_t)tok * st.t + cg * 8);
            *reinterpret_cast<uint4*>(sK + row * SM::kKPitch + cg * 16) = v;
        }
        const uint16_t* gv = vt + ((size_t)bh * Tkv + j) * D * 64;
        const uint16_t* gp = pkt + ((size_t)bh * Tkv + j) * D * 64;
#pragma unroll
        for (int x = t; x < D * 8; x += 256) {
            const int row = x >> 3, c16 = x & 7;
            *reinterpret_cast<uint4*>(sV + row * kTPitch + c16 * 16) =
                *reinterpret_cast<const uint4*>(gv + row * 64 + c16 * 8);
            if (need_lin)
                *reinterpret_cast<uint4*>(sP + row * kTPitch + c16 * 16) =
                    *reinterpret_cast<const uint4*>(gp + row * 64 + c16 * 8);
        }
        if (need_lin && w == 0) {
            const float* z = zb + ((size_t)bh * Tkv + j) * D;
            if (D == 128) {
                const float2 zz = *reinterpret_cast<const float2*>(z + 2 * lane);
                zsel0 += zz.x;
                zsel1 += zz.y;
            } else {
                zsel0 += z[lane];
            }
        }
        __syncthreads();

        // ---- S^T = K_j Q^T (two 32-row tiles of KV)
        f32x16 s[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    sK + (32 * mt + l32) * SM::kKPitch + (16 * ks + 8 * hl) * 2);
                s[mt] = mfma_bf16(a, qf[ks], s[mt]);
            }
        }
        // ragged last KV block: tokens >= N get no logit
        if (j * 64 + 64 > N) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kvi = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
                    if (j * 64 + kvi >= N) s[mt][i] = -INFINITY;
                }
        }
        // ---- online softmax (log2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float xmax = mx * c_log2;
        const bool need = xmax > m_ref + kRescaleThr;
        if (__ballot(need)) {
            const float nref = need ? xmax : m_ref;
            const float f = __builtin_amdgcn_exp2f(m_ref - nref);
            l_part *= f;
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[i][e] *= f;
            m_ref = nref;
        }
        f16x8 pf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = s[q >> 1][8 * (q & 1) + e];
                pf[q][e] = (_Float16)__builtin_amdgcn_exp2f(fmaf(x, c_log2, -m_ref));
            }
        }
        // row sum over the fp16-rounded values (what P V actually uses)
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const f16x2 pr = {pf[q][e], pf[q][e + 1]};
                l_part = __builtin_amdgcn_fdot2(pr, ones, l_part, false);
            }
        // ---- O^T += V^T P^T and G^T += V^T phi(K)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f16x8 bk;
            if (need_lin)
                bk = *reinterpret_cast<const f16x8*>(sP + (32 * nt_w + l32) * kTPitch +
                                                     (16 * q + 8 * hl) * 2);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                const f16x8 a = *reinterpret_cast<const f16x8*>(sV + (32 * mt + l32) * kTPitch +
                                                                (16 * q + 8 * hl) * 2);
                o[mt] = mfma_f16(a, pf[q], o[mt]);
                if (need_lin) g[mt] = mfma_f16(a, bk, g[mt]);
            }
        }
    }

    // ---- epilogue
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    const float inv_l = (k > 0) ? 1.0f / l_tot : 0.0f;
    const float a_h = alpha_of(alpha, bh, H, qb, Tq, alpha_qblock);
    f32x16 ol[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) ol[i] = zero16();
    float inv_den = 0.0f;
    if (need_lin) {
        __syncthreads();
        char* sH = smem;                               // [D][kHPitch] fp16, H^T[e][c]
        float* sZ = reinterpret_cast<float*>(smem + D * SM::kHPitch);
        float* sM = sZ + D;                            // per-wave max |H| entry
        static_assert(SM::kEpi + 16 <= SM::kBytes, "epilogue LDS");
        const float* hT = htot + (size_t)bh * D * D;   // h[c][e]
        // H^T = h_tot^T - G^T goes to fp16 scaled by a power of two that puts
        // its largest entry in [2^13, 2^14): |H| grows with the number of
        // tokens left out and with the mean of V, past the fp16 range at
        // long sequences; the scale is undone after the product (exactly)
        if (w < NT) {
            const int c = 32 * nt_w + l32;
            float hmax = 0.0f;
#pragma unroll
            for (int mt = 0; mt < NT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
                    hmax = fmaxf(hmax, fabsf(hT[(size_t)c * D + e] - g[mt][i]));
                }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
            if (lane == 0) sM[w] = hmax;
        }
        __syncthreads();
        float hmx = sM[0];
#pragma unroll
        for (int i = 1; i < NT; ++i) hmx = fmaxf(hmx, sM[i]);
        int hex = 0;
        (void)frexpf(hmx, &hex);  // hmx = f 2^hex, f in [0.5, 1)
        const int sexp = hmx > 0.0f ? min(max(14 - hex, -100), 100) : 0;
        const float hs = ldexpf(1.0f, sexp), his = ldexpf(1.0f, -sexp);
        if (w < NT) {
            const int c = 32 * nt_w + l32;
#pragma unroll
            for (int mt = 0; mt < NT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
                    const float hv = (hT[(size_t)c * D + e] - g[mt][i]) * hs;
                    *reinterpret_cast<_Float16*>(sH + e * SM::kHPitch + c * 2) = (_Float16)hv;
                }
        }
        if (w == 0) {
            const float* zT = ztot + (size_t)bh * D;
            if (D == 128) {
                sZ[2 * lane] = zT[2 * lane] - zsel0;
                sZ[2 * lane + 1] = zT[2 * lane + 1] - zsel1;
            } else {
                sZ[lane] = zT[lane] - zsel0;
            }
        }
        __syncthreads();
        // phi(Q)^T fragments and the denominator phi(q) . Z
        f16x8 pq[KS];
        float den = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (float)qf[ks][e];
                const float p = x > 0.0f ? x + 1.0f : __expf(x);
                pq[ks][e] = (_Float16)p;
                den = fmaf(p, sZ[16 * ks + 8 * hl + e], den);
            }
        }
        den += __shfl_xor(den, 32);
        inv_den = (1.0f / den) * his;
        // O_l^T = H^T phi(Q)^T
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f16x8 a = *reinterpret_cast<const f16x8*>(
                    sH + (32 * mt + l32) * SM::kHPitch + (16 * ks + 8 * hl) * 2);
                ol[mt] = mfma_f16(a, pq[ks], ol[mt]);
            }
    }
    if (valid_q) {
        const size_t orow = head_base(st, bh, H) + (size_t)tq * st.t;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int e = 32 * mt + 8 * i4 + 4 * hl;
                float v[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    v[c] = a_h * (o[mt][4 * i4 + c] * inv_l) +
                           (1.0f - a_h) * (ol[mt][4 * i4 + c] * inv_den);
                store_out4(O, orow + e, v[0], v[1], v[2], v[3], out_bf16);
            }
    }
}


}  // namespace

hipError_t launch_summaries_mfma(const Dims& D, const void* K, const void* V,
                                 const FwdWS& ws, hipStream_t s, double* xk, double* kblk) {
    if (!hz_path(D) && D.d != 64) return hipErrorInvalidValue;  // d = 128 takes hz_path
    const int nch = summ_chunks(D);
    dim3 g(nch, (unsigned)D.BH);
    timing_before(s, K_SUMM_MFMA);
    if (hz_path(D)) {
        // (stage switches: no V^T without the sparse branch, no h_j, z_j
        // without the linear one).  Blocks per work-group: up to 8 (at the
        // 14B shape 5,920 work-groups, about six rounds of the 1,024 that are
        // resident at once, against three with 16: a shorter last round),
        // fewer when that leaves under 2048 work-groups (short sequences or
        // few heads), so that the pass still fills the GPU
        constexpr long kMaxBlocksPerGroup = 8;
        const long blocks = (long)D.Tkv * D.BH;
        const int bpc = (int)std::max(1L, std::min(kMaxBlocksPerGroup, blocks / 2048));
        dim3 gh((D.Tkv + bpc - 1) / bpc, (unsigned)D.BH);
        summaries_mfma_kernel<128, true><<<gh, 256, 0, s>>>(
            (const uint16_t*)K, (const uint16_t*)V, D.skip_sparse ? nullptr : ws.vt, nullptr,
            nullptr, nullptr, nullptr, D.skip_lin ? nullptr : ws.hz, D.N, D.Tkv, nch, D.H, D.st,
            D.phi_sm, xk, kblk, bpc);
    } else
        summaries_mfma_kernel<64, false><<<g, 256, 0, s>>>(
            (const uint16_t*)K, (const uint16_t*)V, ws.vt, ws.pkt, ws.zb, ws.hpart, ws.zpart,
            nullptr, D.N, D.Tkv, nch, D.H, D.st, D.phi_sm, nullptr, nullptr,
            kSummBlocksPerChunk);
    timing_after(s, K_SUMM_MFMA);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || hz_path(D)) return e;
    return launch_summaries_reduce(D, ws, s);
}

hipError_t launch_fused_mfma(const Dims& D, const void* Q, const void* K, const int32_t* idx,
                             const float* alpha, void* O, const FwdWS& ws, hipStream_t s) {
    if (D.d == 128) return launch_fused128(D, Q, K, idx, alpha, O, ws, false, s);
    // one work-group per (head, query block), Tq padded to a multiple of 8
    dim3 g((unsigned)(((D.Tq + 7) / 8) * 8 * D.BH), 1);
    timing_before(s, K_FUSED_MFMA);
    fused_mfma_kernel<64><<<g, 256, 0, s>>>((const uint16_t*)Q, (const uint16_t*)K, ws.vt,
                                             ws.pkt, ws.zb, idx, alpha, ws.htot, ws.ztot, O, D.N,
                                             D.Tq, D.Tkv, D.k, D.H, D.st, D.alpha_qblock,
                                             D.out_bf16);
    timing_after(s, K_FUSED_MFMA);
    return hipGetLastError();
}

}  // namespace sla2
