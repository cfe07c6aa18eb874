// bf16 forward path on the CDNA4 matrix cores.
//
// 1) summaries_mfma: one pass over K and V.  Per KV block j of 64 tokens it
//    writes V_j^T and phi(K_j)^T in fp16, block-transposed ([d][64]) with the
//    token order permuted inside each group of 16 (positions = token index
//    with bits 2 and 3 swapped), the per-block z_j = colsum phi(K_j), and
//    accumulates h = sum_j phi(K_j)^T V_j on the matrix cores into per-chunk
//    partials (reduced in a fixed order afterwards).  Linear-branch block
//    summaries: SLA notes, key design 4 (h_j = phi(K_j)^T V_j, z_j).
// 2) fused_mfma: per (head, query block of 128) a work-group of 4 waves; wave
//    w owns queries 32w..32w+31.  For every selected KV block (ascending):
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
// Operand layouts of v_mfma_f32_32x32x16_{bf16,f16}: A (32 x 16) lane l holds
// row l%32 and k = 8*(l/32)+[0..7]; B (16 x 32) lane l holds column l%32 and
// the same k; C (32 x 32) lane l holds column l%32 and rows
// 8*(r/4) + 4*(l/32) + r%4, r = 0..15.  Only the C layout is relied on for
// meaning (P^T is fed straight from the S^T accumulators); the k order inside
// an instruction only has to agree between A and B, which holds because both
// operands are loaded with the same position rule.
#include "sla2_internal.h"

namespace sla2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline float phi_fast(float x) { return x > 0.0f ? x + 1.0f : __expf(x); }

// token u of a 64-block -> its position in the transposed layouts
__device__ inline int perm_pos(int u) {
    return (u & ~12) | ((u >> 1) & 4) | ((u << 1) & 8);
}

// Work-groups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  The grid is laid out as heads x (8 ranges of ceil(Tq/8) query
// blocks); dispatch index g runs on XCD g % 8, which this map gives query
// blocks x*R .. x*R+R-1 of one head at a time: all XCDs work on the same head
// together (its gathered KV tiles stay in the shared last-level cache) and
// each XCD walks a contiguous range (neighbouring query blocks share some of
// their selected KV blocks in its L2).  Returns false for the padding slots.
__device__ inline bool head_major_map(int g, int Tq, long* bh, int* qb) {
    const int R = (Tq + 7) >> 3;   // query blocks per XCD and head
    const int x = g & 7, s = g >> 3;
    *bh = s / R;
    *qb = x * R + s % R;
    return *qb < Tq;
}

__device__ inline f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// ---------------------------------------------------------------------------
// block summaries
// ---------------------------------------------------------------------------
constexpr int kTPitch = 64 * 2 + 16;  // bytes per row of a [d][64] fp16 tile in LDS

template <int D>
__global__ __launch_bounds__(256) void summaries_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, uint16_t* __restrict__ vt,
    uint16_t* __restrict__ pkt, float* __restrict__ zb, float* __restrict__ hpart,
    float* __restrict__ zpart, int N, int Tkv, int nch) {
    constexpr int NT = D / 32;
    constexpr int TPW = NT * NT / 4;  // h^T tiles per wave
    __shared__ __attribute__((aligned(16))) char sV[D * kTPitch];
    __shared__ __attribute__((aligned(16))) char sP[D * kTPitch];
    // wave index as a scalar: conditions on it must be wave-uniform branches
    // (matrix instructions ignore EXEC, so they may never sit under a lane mask)
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int chunk = blockIdx.x;
    const long bh = blockIdx.y;
    const int j0 = chunk * kSummBlocksPerChunk;
    const int j1 = min(Tkv, j0 + kSummBlocksPerChunk);
    const uint16_t* Kh = K + (size_t)bh * N * D;
    const uint16_t* Vh = V + (size_t)bh * N * D;
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
#pragma unroll
        for (int pass = 0; pass < CG / 4; ++pass) {
            const int cg = w + 4 * pass;
            const int u = lane;
            const int tok = j * 64 + u;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            const bool ok = tok < N;
            if (ok) {
                kv = *reinterpret_cast<const uint4*>(Kh + (size_t)tok * D + cg * 8);
                vv = *reinterpret_cast<const uint4*>(Vh + (size_t)tok * D + cg * 8);
            }
            const unsigned kw[4] = {kv.x, kv.y, kv.z, kv.w};
            const unsigned vw[4] = {vv.x, vv.y, vv.z, vv.w};
            const int pos = perm_pos(u);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kf = (e & 1) ? bf16_hi(kw[e >> 1]) : bf16_lo(kw[e >> 1]);
                const float vf = (e & 1) ? bf16_hi(vw[e >> 1]) : bf16_lo(vw[e >> 1]);
                const _Float16 ph = ok ? (_Float16)phi_fast(kf) : (_Float16)0.0f;
                const _Float16 vh = ok ? (_Float16)vf : (_Float16)0.0f;
                const int c = cg * 8 + e;
                *reinterpret_cast<_Float16*>(sP + c * kTPitch + pos * 2) = ph;
                *reinterpret_cast<_Float16*>(sV + c * kTPitch + pos * 2) = vh;
            }
        }
        __syncthreads();
        // write the transposed tiles (contiguous D*64 fp16 each) and z_j
        uint16_t* gv = vt + ((size_t)bh * Tkv + j) * D * 64;
        uint16_t* gp = pkt + ((size_t)bh * Tkv + j) * D * 64;
        for (int x = t; x < D * 8; x += 256) {
            const int row = x >> 3, c16 = x & 7;
            *reinterpret_cast<uint4*>(gv + row * 64 + c16 * 8) =
                *reinterpret_cast<const uint4*>(sV + row * kTPitch + c16 * 16);
            *reinterpret_cast<uint4*>(gp + row * 64 + c16 * 8) =
                *reinterpret_cast<const uint4*>(sP + row * kTPitch + c16 * 16);
        }
        if (t < D) {
            float z = 0.0f;
            const _Float16* rowp = reinterpret_cast<const _Float16*>(sP + t * kTPitch);
            for (int p = 0; p < 64; ++p) z += (float)rowp[p];
            zb[((size_t)bh * Tkv + j) * D + t] = z;
            zacc += z;
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
    const float* __restrict__ ztot, float* __restrict__ O, int N, int Tq, int Tkv, int k,
    int H) {
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
        const uint16_t* qrow = Q + ((size_t)bh * N + (valid_q ? tq : 0)) * D;
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
    const uint16_t* Kh = K + (size_t)bh * N * D;

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
            if (tok < N) v = *reinterpret_cast<const uint4*>(Kh + (size_t)tok * D + cg * 8);
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
    const float a_h = alpha[bh % H];
    f32x16 ol[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) ol[i] = zero16();
    float inv_den = 0.0f;
    if (need_lin) {
        __syncthreads();
        char* sH = smem;                               // [D][kHPitch] fp16, H^T[e][c]
        float* sZ = reinterpret_cast<float*>(smem + D * SM::kHPitch);
        const float* hT = htot + (size_t)bh * D * D;   // h[c][e]
        if (w < NT) {
            const int c = 32 * nt_w + l32;
#pragma unroll
            for (int mt = 0; mt < NT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
                    const float hv = hT[(size_t)c * D + e] - g[mt][i];
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
        inv_den = 1.0f / den;
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
        float* orow = O + ((size_t)bh * N + tq) * D;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int e = 32 * mt + 8 * i4 + 4 * hl;
                float4 v;
                v.x = a_h * (o[mt][4 * i4 + 0] * inv_l) + (1.0f - a_h) * (ol[mt][4 * i4 + 0] * inv_den);
                v.y = a_h * (o[mt][4 * i4 + 1] * inv_l) + (1.0f - a_h) * (ol[mt][4 * i4 + 1] * inv_den);
                v.z = a_h * (o[mt][4 * i4 + 2] * inv_l) + (1.0f - a_h) * (ol[mt][4 * i4 + 2] * inv_den);
                v.w = a_h * (o[mt][4 * i4 + 3] * inv_l) + (1.0f - a_h) * (ol[mt][4 * i4 + 3] * inv_den);
                *reinterpret_cast<float4*>(orow + e) = v;
            }
    }
}


// ---------------------------------------------------------------------------
// fused kernel, d = 128: 8 waves = 4 query groups x 2 KV halves
// ---------------------------------------------------------------------------
// Wave w handles queries 32*(w%4) .. +31 of the block and KV rows
// 32*(w/4) .. +31 of every selected tile, with its own online-softmax state;
// the two KV halves are merged once at the end.  KV tiles arrive in three
// LDS stages through asynchronous direct-to-LDS loads issued two tiles
// ahead.  Stage layout (48 KB): K tile [64][256 B] with 16-byte chunk c of
// row r stored at chunk c ^ (r & 15); V^T and phi(K)^T tiles [128][128 B]
// with chunk c of row r at chunk c ^ ((r >> 1) & 7).  Both swizzles make the
// 32-row fragment reads bank-conflict free.
constexpr int kStageBytes = 49152;
__shared__ __attribute__((aligned(16))) char g_st0[kStageBytes];
__shared__ __attribute__((aligned(16))) char g_st1[kStageBytes];
__shared__ __attribute__((aligned(16))) char g_st2[kStageBytes];

template <int S>
__device__ inline char* stage_ptr() {
    return S == 0 ? g_st0 : (S == 1 ? g_st1 : g_st2);
}

#define SLA2_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ inline void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
}

// s_barrier without the memory fence of __syncthreads (which would also
// wait for the prefetch in flight); the empty asm keeps the compiler from
// moving memory accesses across it.  LDS writes that other waves read after
// it must be complete first (wait_lgkm0).
__device__ inline void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

typedef int i32x8 __attribute__((ext_vector_type(8)));

// e4m3 x e4m3 -> fp32 matrix product (32x32x64); E8M0 scale 127 = 1.0
__device__ inline f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Issues the direct-to-LDS loads of KV tile j into stage S: K (bf16: 2 per
// lane) or Khat (e4m3: 1), V^T (2) and, with the linear branch, phi(K)^T (2).
// The Khat tile uses rows of 128 B with the V^T swizzle.
template <int S, bool LIN, bool LOWBIT>
__device__ inline void issue_tile(const void* __restrict__ Kh, const uint16_t* __restrict__ vt_h,
                                  const uint16_t* __restrict__ pkt_h, int j, int N, int w,
                                  int lane) {
    char* st = stage_ptr<S>();
    if (LOWBIT) {
        const int row = 8 * w + (lane >> 3);
        const int lc = (lane & 7) ^ ((row >> 1) & 7);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const uint8_t*>(Kh) + ((size_t)j * 64 + row) * 128 + lc * 16,
            SLA2_LDS(st + w * 1024), 16, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = 2 * w + i;                 // 1 KB piece of the tile
            const int row = 4 * u + (lane >> 4);     // K: 4 rows per piece
            const int lc = (lane & 15) ^ (row & 15);
            const int tok = min(j * 64 + row, N - 1);
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const uint16_t*>(Kh) + (size_t)tok * 128 + lc * 8,
                SLA2_LDS(st + u * 1024), 16, 0, 0);
        }
    }
    const size_t tbase = (size_t)j * 128 * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = 2 * w + i;
        const int row = 8 * u + (lane >> 3);     // V^T: 8 rows per piece
        const int lc = (lane & 7) ^ ((row >> 1) & 7);
        __builtin_amdgcn_global_load_lds(vt_h + tbase + row * 64 + lc * 8,
                                         SLA2_LDS(st + 16384 + u * 1024), 16, 0, 0);
        if (LIN)
            __builtin_amdgcn_global_load_lds(pkt_h + tbase + row * 64 + lc * 8,
                                             SLA2_LDS(st + 32768 + u * 1024), 16, 0, 0);
    }
}

struct WaveState {
    f32x16 o[4];   // O^T tiles (d rows 32mt.., this wave's 32 queries)
    f32x16 g[4];   // G^T tiles (V channels 32mt.., phi(K) channels 32*qg..)
    float m_ref;   // log2-domain reference max of this lane's query
    float l_part;  // row-sum over this lane's rows of this KV half
    float zsel;    // lanes 0..15: sum of z_j[16*w + lane] over the selected tiles
    float zp[3];   // z_j of the tiles in flight, one per LDS stage
};

// Q operand of Q K^T for this lane: bf16 (8 k-steps of 16) or e4m3 (2 of 64)
template <bool LOWBIT> struct QOperand;
template <> struct QOperand<false> { bf16x8 f[8]; };
template <> struct QOperand<true> { i32x8 f[2]; };

// One KV tile from stage S for wave (qg, kh).  c_tile converts a raw
// product to log2 units (1/sqrt(d) log2(e), times s_Q s_K for the low bit).
template <int S, bool LIN, bool LOWBIT>
__device__ inline void tile_compute(WaveState& W, const QOperand<LOWBIT>& Qo, int j, int N,
                                    int w, int kh, int qg, int lane, int l32, int hl,
                                    float c_tile) {
    char* st = stage_ptr<S>();
    f32x16 s = zero16();
    const int krow = 32 * kh + l32;
    if (LOWBIT) {  // S^T = Khat_half Qhat^T on the fp8 matrix cores
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c0 = 4 * ks + 2 * hl, sw = (krow >> 1) & 7;
            const uint4 lo = *reinterpret_cast<const uint4*>(st + krow * 128 + ((c0) ^ sw) * 16);
            const uint4 hi = *reinterpret_cast<const uint4*>(st + krow * 128 + ((c0 + 1) ^ sw) * 16);
            i32x8 a;
            a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
            a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
            s = mfma_fp8(a, reinterpret_cast<const i32x8*>(Qo.f)[ks], s);
        }
    } else {  // S^T = K_half Q^T
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int pc = (2 * ks + hl) ^ (krow & 15);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + krow * 256 + pc * 16);
            s = mfma_bf16(a, reinterpret_cast<const bf16x8*>(Qo.f)[ks], s);
        }
    }
    if (j * 64 + 64 > N) {  // ragged last block (uniform branch)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kvi = 32 * kh + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (j * 64 + kvi >= N) s[i] = -INFINITY;
        }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (LOWBIT) {
        // P is quantised against the running maximum over whole tiles: the
        // two KV halves of a query group exchange their maxima
        float* xt = reinterpret_cast<float*>(st + 8192);  // [8 waves][64 lanes]
        xt[w * 64 + lane] = mx;
        wait_lgkm0();
        wg_barrier();
        mx = fmaxf(mx, xt[((w + 4) & 7) * 64 + lane]);
    }
    const float xmax = mx * c_tile;
    const bool need = LOWBIT ? (xmax > W.m_ref) : (xmax > W.m_ref + kRescaleThr);
    if (__ballot(need)) {
        const float nref = need ? xmax : W.m_ref;
        const float f = __builtin_amdgcn_exp2f(W.m_ref - nref);
        W.l_part *= f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) W.o[i][e] *= f;
        W.m_ref = nref;
    }
    // a KV half whose rows are all padding has no reference yet: P = 0
    const float mref = W.m_ref == -INFINITY ? 0.0f : W.m_ref;
    f16x8 pf[2];
    if (LOWBIT) {
        // 256 P~ rounded onto the e4m3 grid (P~ <= 1), carried exactly in fp16
        const float bias = 8.0f - mref;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * q + e], c_tile, bias));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * q + e + 1], c_tile, bias));
                const int code = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(p0, 448.0f),
                                                                 fminf(p1, 448.0f), 0, false);
                const auto back = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
                pf[q][e] = (_Float16)back[0];
                pf[q][e + 1] = (_Float16)back[1];
            }
    } else {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pf[q][e] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[8 * q + e], c_tile, -mref));
    }
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const f16x2 pr = {pf[q][e], pf[q][e + 1]};
            W.l_part = __builtin_amdgcn_fdot2(pr, ones, W.l_part, false);
        }
    // O^T += V^T P^T ; G^T += V^T phi(K)
    const char* sv = st + 16384;
    const char* sp = st + 32768;
    const int crow = 32 * qg + l32;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c2 = 4 * kh + 2 * q + hl;  // 16-byte chunk of the positions
        f16x8 bk;
        if (LIN)
            bk = *reinterpret_cast<const f16x8*>(sp + crow * 128 + (c2 ^ ((crow >> 1) & 7)) * 16);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int erow = 32 * mt + l32;
            const f16x8 a = *reinterpret_cast<const f16x8*>(sv + erow * 128 +
                                                            (c2 ^ ((erow >> 1) & 7)) * 16);
            W.o[mt] = mfma_f16(a, pf[q], W.o[mt]);
            if (LIN) W.g[mt] = mfma_f16(a, bk, W.g[mt]);
        }
    }
}

template <int S, int SN, bool LIN, bool LOWBIT>
__device__ inline void tile_step(WaveState& W, const QOperand<LOWBIT>& Qo, const int32_t* sel,
                                 int r, int k, const void* Kh, const uint16_t* vt_h,
                                 const uint16_t* pkt_h, const float* zb_h, const float* sk_h,
                                 int N, int w, int lane, int kh, int qg, int l32, int hl,
                                 float c_base) {
    // vector-memory operations per lane and tile, issued as one group: with
    // the linear branch one z_j load, then the direct-to-LDS loads (K: 2 or
    // Khat: 1, V^T: 2 [, phi(K)^T: 2]).  Only tile r+1's group was issued
    // after tile r's.
    constexpr int PER_TILE = (LOWBIT ? 1 : 2) + 2 + (LIN ? 3 : 0);
    if (r + 1 < k) wait_vmcnt<PER_TILE>();
    else wait_vmcnt<0>();
    wg_barrier();  // every wave's part of tile r is in LDS
    if (LIN) W.zsel += W.zp[S];    // z_j of tile r (older than tile r's loads)
    if (r + 2 < k) {
        const int jn = sel[r + 2];
        if (LIN) W.zp[SN] = (lane < 16) ? zb_h[(size_t)jn * 128 + 16 * w + lane] : 0.0f;
        issue_tile<SN, LIN, LOWBIT>(Kh, vt_h, pkt_h, jn, N, w, lane);
    }
    const int j = sel[r];
    const float c_tile = LOWBIT ? c_base * sk_h[j] : c_base;
    tile_compute<S, LIN, LOWBIT>(W, Qo, j, N, w, kh, qg, lane, l32, hl, c_tile);
}

template <bool LIN, bool LOWBIT>
__global__ __launch_bounds__(512) void fused_mfma_d128_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ vt, const uint16_t* __restrict__ pkt,
    const float* __restrict__ zb, const int32_t* __restrict__ idx,
    const float* __restrict__ alpha, const float* __restrict__ hfrag,
    const float* __restrict__ ztot, const uint8_t* __restrict__ qhat,
    const uint8_t* __restrict__ khat, const float* __restrict__ sq,
    const float* __restrict__ sk, float* __restrict__ O, int N, int Tq, int Tkv, int k,
    int H) {
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int qg = w & 3, kh = w >> 2;
    long bh;
    int qb;
    if (!head_major_map(blockIdx.x, Tq, &bh, &qb)) return;
    const int tq = qb * 128 + 32 * qg + l32;
    const bool valid_q = tq < N;
    const float c_log2 = 1.4426950408889634f / sqrtf(128.0f);

    // Q operand: lane holds row tq, k-chunk 8*hl.. of every 16 (bf16) or
    // 32*hl.. of every 64 (e4m3)
    QOperand<LOWBIT> Qo;
    float c_base = c_log2;
    if (LOWBIT) {
        const uint8_t* qrow = qhat + ((size_t)bh * Tq * 128 + (size_t)qb * 128 + 32 * qg + l32) * 128;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 lo = *reinterpret_cast<const uint4*>(qrow + 64 * ks + 32 * hl);
            const uint4 hi = *reinterpret_cast<const uint4*>(qrow + 64 * ks + 32 * hl + 16);
            i32x8 v;
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
            reinterpret_cast<i32x8*>(Qo.f)[ks] = v;
        }
        c_base = c_log2 * sq[bh * Tq + qb];
    } else {
        const uint16_t* qrow = Q + ((size_t)bh * N + (valid_q ? tq : 0)) * 128;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid_q) v = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
            reinterpret_cast<bf16x8*>(Qo.f)[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    WaveState W;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        W.o[i] = zero16();
        W.g[i] = zero16();
    }
    W.m_ref = -INFINITY;
    W.l_part = 0.0f;
    W.zsel = 0.0f;

    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;
    const float* zb_h = zb + (size_t)bh * Tkv * 128;
    const float* sk_h = LOWBIT ? sk + (size_t)bh * Tkv : nullptr;
    const void* Kh = LOWBIT ? (const void*)(khat + (size_t)bh * Tkv * 64 * 128)
                            : (const void*)(K + (size_t)bh * N * 128);
    const uint16_t* vt_h = vt + (size_t)bh * Tkv * 128 * 64;
    const uint16_t* pkt_h = pkt + (size_t)bh * Tkv * 128 * 64;

    W.zp[0] = W.zp[1] = W.zp[2] = 0.0f;
    for (int r = 0; r < 2 && r < k; ++r) {  // the first two tile groups
        if (LIN) W.zp[r] = (lane < 16) ? zb_h[(size_t)sel[r] * 128 + 16 * w + lane] : 0.0f;
        if (r == 0) issue_tile<0, LIN, LOWBIT>(Kh, vt_h, pkt_h, sel[0], N, w, lane);
        else issue_tile<1, LIN, LOWBIT>(Kh, vt_h, pkt_h, sel[1], N, w, lane);
    }
    for (int r = 0; r < k; r += 3) {
        tile_step<0, 2, LIN, LOWBIT>(W, Qo, sel, r, k, Kh, vt_h, pkt_h, zb_h, sk_h, N, w, lane,
                                     kh, qg, l32, hl, c_base);
        if (r + 1 < k)
            tile_step<1, 0, LIN, LOWBIT>(W, Qo, sel, r + 1, k, Kh, vt_h, pkt_h, zb_h, sk_h, N, w,
                                         lane, kh, qg, l32, hl, c_base);
        if (r + 2 < k)
            tile_step<2, 1, LIN, LOWBIT>(W, Qo, sel, r + 2, k, Kh, vt_h, pkt_h, zb_h, sk_h, N, w,
                                         lane, kh, qg, l32, hl, c_base);
    }
    wait_vmcnt<0>();
    __syncthreads();
    // ---- merge the two KV halves of (O, m, l): wave (qg, kh) finishes the
    // d rows 64*kh .. 64*kh+63 (m-tiles 2kh, 2kh+1) of its queries
    const float l_half = W.l_part + __shfl_xor(W.l_part, 32);
    float* xo = reinterpret_cast<float*>((w < 4 ? g_st0 : g_st1) + (w & 3) * 8192);
    float* xm = reinterpret_cast<float*>(g_st2);  // [8 waves][64 lanes][2]
    const int other = 1 - kh;
    const int partner = qg + 4 * other;
    // partner's rows out
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 16; ++i) xo[(s2 * 16 + i) * 64 + lane] = W.o[2 * other + s2][i];
    xm[(w * 64 + lane) * 2 + 0] = W.m_ref;
    xm[(w * 64 + lane) * 2 + 1] = l_half;
    __syncthreads();
    const float* po = reinterpret_cast<const float*>((partner < 4 ? g_st0 : g_st1) + (partner & 3) * 8192);
    const float m_p = xm[(partner * 64 + lane) * 2 + 0];
    const float l_p = xm[(partner * 64 + lane) * 2 + 1];
    const float m_s = W.m_ref;
    const float m_new = fmaxf(m_s, m_p);
    const float f_s = m_s == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_s - m_new);
    const float f_p = m_p == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_p - m_new);
    const float l_all = l_half * f_s + l_p * f_p;
    const float inv_l = (k > 0 && l_all > 0.0f) ? 1.0f / l_all : 0.0f;
    f32x16 os[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            os[s2][i] = (W.o[2 * kh + s2][i] * f_s + po[(s2 * 16 + i) * 64 + lane] * f_p) * inv_l;

    f32x16 ol[2] = {zero16(), zero16()};
    float inv_den = 0.0f;
    if (LIN) {
        // ---- G halves: H^T[e][c] = h_tot[c][e] - G^T[e][c] for e in my rows,
        // c in the n-tile of my query group
        __syncthreads();
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 16; ++i) xo[(s2 * 16 + i) * 64 + lane] = W.g[2 * other + s2][i];
        __syncthreads();
        f32x16 gs[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                gs[s2][i] = W.g[2 * kh + s2][i] + po[(s2 * 16 + i) * 64 + lane];
        __syncthreads();
        // H^T as fp16 in g_st0, row e, 16-byte chunk c' at c' ^ (e & 15)
        char* sH = g_st0;
        float* sZ = reinterpret_cast<float*>(g_st1);
        // this lane's 32 values of h_tot, stored contiguously in epilogue order
        const float4* hf = reinterpret_cast<const float4*>(
            hfrag + (size_t)bh * 128 * 128 + ((size_t)w * 64 + lane) * 32);
        const int c = 32 * qg + l32;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const float4 h4 = hf[s2 * 4 + i4];
                const float hv[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * i4 + j;
                    const int e = 32 * (2 * kh + s2) + 8 * i4 + 4 * hl + j;
                    const int chunk = (c >> 3) ^ (e & 15);
                    *reinterpret_cast<_Float16*>(sH + e * 256 + chunk * 16 + (c & 7) * 2) =
                        (_Float16)(hv[j] - gs[s2][i]);
                }
            }
        // Z = z_tot - sum of the selected blocks' z_j (wave w holds channels 16w..)
        if (lane < 16) sZ[16 * w + lane] = ztot[(size_t)bh * 128 + 16 * w + lane] - W.zsel;
        __syncthreads();
        // phi(Q)^T operand from the raw bf16 Q (registers on the bf16 path)
        bf16x8 qraw[8];
        if (LOWBIT) {
            const uint16_t* qrow = Q + ((size_t)bh * N + (valid_q ? tq : 0)) * 128;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (valid_q) v = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
                qraw[ks] = __builtin_bit_cast(bf16x8, v);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) qraw[ks] = reinterpret_cast<const bf16x8*>(Qo.f)[ks];
        }
        f16x8 pq[8];
        float den = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (float)qraw[ks][e];
                const float p = x > 0.0f ? x + 1.0f : __expf(x);
                pq[ks][e] = (_Float16)p;
                den = fmaf(p, sZ[16 * ks + 8 * hl + e], den);
            }
        den += __shfl_xor(den, 32);
        inv_den = 1.0f / den;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int erow = 32 * (2 * kh + s2) + l32;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int pc = (2 * ks + hl) ^ (erow & 15);
                const f16x8 a = *reinterpret_cast<const f16x8*>(sH + erow * 256 + pc * 16);
                ol[s2] = mfma_f16(a, pq[ks], ol[s2]);
            }
        }
    }
    // ---- output: stage the 128 x 128 fp32 tile in LDS (rows padded to 528 B;
    // query rows 0..63 in stage 0, 64..127 in stage 1), then store whole rows
    __syncthreads();  // all reads of the epilogue's LDS data are done
    {
        const float a_h = alpha[bh % H];
        const int qrow = 32 * qg + l32;
        char* sO = (qrow < 64 ? g_st0 : g_st1) + (qrow & 63) * 528;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int e = 32 * (2 * kh + s2) + 8 * i4 + 4 * hl;
                float4 v;
                v.x = a_h * os[s2][4 * i4 + 0] + (1.0f - a_h) * (ol[s2][4 * i4 + 0] * inv_den);
                v.y = a_h * os[s2][4 * i4 + 1] + (1.0f - a_h) * (ol[s2][4 * i4 + 1] * inv_den);
                v.z = a_h * os[s2][4 * i4 + 2] + (1.0f - a_h) * (ol[s2][4 * i4 + 2] * inv_den);
                v.w = a_h * os[s2][4 * i4 + 3] + (1.0f - a_h) * (ol[s2][4 * i4 + 3] * inv_den);
                *reinterpret_cast<float4*>(sO + e * 4) = v;
            }
    }
    __syncthreads();
    {
        const int nvalid = min(128, N - qb * 128);
        float* obase = O + ((size_t)bh * N + (size_t)qb * 128) * 128;
        // 512 threads: 16 rows of 32 x 16 B per pass; a wave stores 2 whole rows
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
            const int row = pass * 16 + (t >> 5), c4 = t & 31;
            if (row < nvalid) {
                const char* src = (row < 64 ? g_st0 : g_st1) + (row & 63) * 528 + c4 * 16;
                typedef float f32x4 __attribute__((ext_vector_type(4)));
                const f32x4 v = *reinterpret_cast<const f32x4*>(src);
                f32x4* dst = reinterpret_cast<f32x4*>(obase + (size_t)row * 128 + c4 * 4);
                __builtin_nontemporal_store(v, dst);
            }
        }
    }
}

}  // namespace

hipError_t launch_summaries_mfma(const Dims& D, const void* K, const void* V,
                                 const FwdWS& ws, hipStream_t s) {
    const int nch = summ_chunks(D);
    dim3 g(nch, (unsigned)D.BH);
    timing_before(s, K_SUMM_MFMA);
    if (D.d == 128)
        summaries_mfma_kernel<128><<<g, 256, 0, s>>>((const uint16_t*)K, (const uint16_t*)V,
                                                     ws.vt, ws.pkt, ws.zb, ws.hpart, ws.zpart,
                                                     D.N, D.Tkv, nch);
    else
        summaries_mfma_kernel<64><<<g, 256, 0, s>>>((const uint16_t*)K, (const uint16_t*)V,
                                                    ws.vt, ws.pkt, ws.zb, ws.hpart, ws.zpart,
                                                    D.N, D.Tkv, nch);
    timing_after(s, K_SUMM_MFMA);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_summaries_reduce(D, ws, s);
}

hipError_t launch_fused_mfma(const Dims& D, const void* Q, const void* K, const int32_t* idx,
                             const float* alpha, float* O, const FwdWS& ws, hipStream_t s) {
    // one work-group per (head, query block), Tq padded to a multiple of 8
    dim3 g((unsigned)(((D.Tq + 7) / 8) * 8 * D.BH), 1);
    if (D.d == 128) return launch_fused128(D, Q, K, idx, alpha, O, ws, false, s);
    timing_before(s, K_FUSED_MFMA);
    if (D.d == 128 && D.k < D.Tkv)
        fused_mfma_d128_kernel<true, false><<<g, 512, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, ws.vt, ws.pkt, ws.zb, idx, alpha, ws.hfrag,
            ws.ztot, nullptr, nullptr, nullptr, nullptr, O, D.N, D.Tq, D.Tkv, D.k, D.H);
    else if (D.d == 128)
        fused_mfma_d128_kernel<false, false><<<g, 512, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, ws.vt, ws.pkt, ws.zb, idx, alpha, ws.hfrag,
            ws.ztot, nullptr, nullptr, nullptr, nullptr, O, D.N, D.Tq, D.Tkv, D.k, D.H);
    else
        fused_mfma_kernel<64><<<g, 256, 0, s>>>(
            (const uint16_t*)Q, (const uint16_t*)K, ws.vt, ws.pkt, ws.zb, idx, alpha, ws.htot,
            ws.ztot, O, D.N, D.Tq, D.Tkv, D.k, D.H);
    timing_after(s, K_FUSED_MFMA);
    return hipGetLastError();
}

}  // namespace sla2

namespace sla2 {
hipError_t launch_fused_fp8(const Dims& D, const void* Q, const int32_t* idx, const float* alpha,
                            float* O, const FwdWS& ws, hipStream_t s) {
    dim3 g((unsigned)(((D.Tq + 7) / 8) * 8 * D.BH), 1);
    timing_before(s, K_FUSED_FP8);
    if (D.k < D.Tkv)
        fused_mfma_d128_kernel<true, true><<<g, 512, 0, s>>>(
            (const uint16_t*)Q, nullptr, ws.vt, ws.pkt, ws.zb, idx, alpha, ws.hfrag, ws.ztot,
            ws.qhat, ws.khat, ws.sq, ws.sk, O, D.N, D.Tq, D.Tkv, D.k, D.H);
    else
        fused_mfma_d128_kernel<false, true><<<g, 512, 0, s>>>(
            (const uint16_t*)Q, nullptr, ws.vt, ws.pkt, ws.zb, idx, alpha, ws.hfrag, ws.ztot,
            ws.qhat, ws.khat, ws.sq, ws.sk, O, D.N, D.Tq, D.Tkv, D.k, D.H);
    timing_after(s, K_FUSED_FP8);
    return hipGetLastError();
}
}  // namespace sla2
