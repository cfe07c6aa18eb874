// Fused sparse + linear + combine kernel for d = 128, b_q = 128, b_kv = 64
// (bf16 inputs; in the low-bit forms the Q K^T products run on the e4m3 or
// the int8 matrix cores).
//
// One work-group of 4 waves per (head, query block); wave w owns queries
// 32w .. 32w+31 of the block and all 64 keys of every selected KV tile, so
// each wave carries a complete online-softmax state and no partial results
// are merged across waves.  80 KB of LDS per work-group lets two work-groups
// share a compute unit: one group's prologue and epilogue overlap the
// other's tile loop.
//
// Per selected KV block j, in ascending order ("SLA2 深度解读" 04, 07, 08:
// only mask-hit blocks run Q K^T and P V, online softmax over them):
//   S^T = K_j Q^T                       bf16 MFMA (low bit: Khat Qhat^T on
//                                       e4m3 or int8 codes, times s_Q s_K)
//   online softmax on S^T               one query per lane column
//   O^T += V_j^T P^T                    fp16 MFMA (LOWBIT: P on the e4m3 grid)
// The linear branch's sums over the blocks the query block leaves out,
// H_i = sum h_j and Z_i = sum z_j (SLA notes, key designs 3 and 4), come
// ready from the dense product of linear.hip (one row per query block: H_i
// in bf16, Z_i in fp32).  Epilogue: O_l^T = H_i^T phi(Q)^T (bf16 matrix
// cores, phi(Q) rounded to bf16) / (phi(Q) . Z_i in fp32), O = alpha O_s +
// (1 - alpha) O_l ("SLA2 深度解读" 04).
//
// PHISM: phi is the softmax of each row over its 128 channels (the block
// summaries pass applies the same map to K).  V1 (SLA v1, "SLA: Beyond
// Sparsity ..." notes, key designs 2 and 3): the selected blocks are the
// critical ones, the linear branch covers the marginal blocks only (the
// product leaves the negligible ones out as well), and O = O_s + O_l W_p,
// the projection on the fp16 matrix cores with O_l split into a high fp16
// part and the fp16 rest.
//
// K (or Khat) and V^T tiles arrive by direct-to-LDS loads, K two tiles
// ahead (three stages), V^T one tile ahead (two stages).  LDS layouts:
//   K    [64 keys][256 B]   16-byte chunk c of row r at chunk c ^ (r & 15)
//   Khat [64 keys][128 B]   chunk c of row r at chunk c ^ ((r >> 1) & 7)
//   V^T  [128 ch][128 B]    chunk c of row r at chunk c ^ ((r >> 1) & 7)
// V^T comes from the block summaries pass in fp16 with the keys of each
// group of 16 stored at positions with bits 2 and 3 swapped, which makes the
// k order of P^T (taken straight from the S^T accumulators) line up with it;
// phi(K)^T is stored the same way.
#include <type_traits>

#include "cdna4.h"
#include "sla2_internal.h"

namespace sla2 {
namespace {
using namespace cdna4;

constexpr int kLdsBytes = 80 * 1024;
constexpr int kKRaw = 16384;  // K tile, bf16
constexpr int kKHat = 8192;   // Khat tile, e4m3
constexpr int kVT = 16384;    // V^T tile, fp16
constexpr int kV8 = 8192;     // Vhat^T tile, e4m3 (fully low-bit P V)
constexpr float kRescaleThr = 8.0f;

__shared__ __attribute__((aligned(1024))) char s_lds[kLdsBytes];

template <bool LOWBIT, bool LOWV>
struct Plan {
    static constexpr int kStage = LOWBIT ? kKHat : kKRaw;
    static constexpr int kStages = 3;
    static constexpr int vOff = kStages * kStage;
    static constexpr int v8Off = vOff + 2 * kVT;  // Vhat^T stages (LOWV)
    static constexpr int nK = LOWBIT ? 2 : 4;     // loads per lane, K tile
    static_assert(vOff + 2 * kVT + (LOWV ? 2 * kV8 : 0) <= kLdsBytes, "LDS budget");
    static_assert(32768 + 512 <= kLdsBytes, "epilogue LDS");
};

template <bool LOWBIT> struct QOp;
template <> struct QOp<false> { bf16x8 f[8]; };  // 8 k-steps of 16 channels
template <> struct QOp<true> { i32x8 f[2]; };    // 2 k-steps of 64 channels

// Tile loads.  A tile is moved in 1 KB pieces, piece u = 4i + w going to
// byte u * 1024 of its LDS stage; the lane's 16 bytes of piece u sit at the
// same per-lane byte offset (plus a fixed step per i) in every tile.  The
// loads are buffer loads on a per-head resource: the tile's offset is a
// scalar and each lane keeps a single 32-bit offset (the host limits every
// per-head span to 2^31 bytes).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t head_rsrc(const void* base) {
    // raw buffer (stride 0), no range limit, 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
__device__ inline void load_lds16(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SLA2_LDS(dst), 16, voff, soff, 0, 0);
}

// per-lane offsets: K rows are 256 B apart in LDS (16-byte chunk c of row r
// at c ^ (r & 15)) and rp bytes apart in global memory (256 for [B,H,N,d],
// 256 H for [B,N,H,d]); Khat and V^T rows are 128 B (chunk c of row r at
// c ^ ((r >> 1) & 7))
__device__ inline uint32_t k_lane_off(int w, int lane, uint32_t rp) {
    const int row = 4 * w + (lane >> 4);
    return (uint32_t)row * rp + ((uint32_t)((lane & 15) ^ (row & 15)) << 4);
}
__device__ inline uint32_t t_lane_off(int w, int lane) {
    const int row = 8 * w + (lane >> 3);
    return (uint32_t)(row * 128 + (((lane & 7) ^ ((row >> 1) & 7)) << 4));
}

// K (or Khat) tile j into one K stage
template <bool LOWBIT>
__device__ inline void issue_k(char* kst, rsrc_t rk, int j, int N, int w, int lane,
                               uint32_t koff, uint32_t toff, uint32_t rp) {
    if (LOWBIT) {  // Khat rows past N are stored (as zeros)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            load_lds16(rk, toff, (uint32_t)j * 8192 + 4096 * i, kst + (4 * i + w) * 1024);
    } else if (j * 64 + 64 <= N) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            load_lds16(rk, koff, (uint32_t)j * 64 * rp + 16 * rp * i, kst + (4 * i + w) * 1024);
    } else {  // ragged last block: padding rows read row N-1 (their logits are masked)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * i + 4 * w + (lane >> 4);
            const int tok = min(j * 64 + row, N - 1);
            const uint32_t off = (uint32_t)tok * rp + ((uint32_t)((lane & 15) ^ (row & 15)) << 4);
            load_lds16(rk, off, 0, kst + (4 * i + w) * 1024);
        }
    }
}

// V^T tile j into one V stage
__device__ inline void issue_v(char* vst, rsrc_t rv, int j, int w, uint32_t toff) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        load_lds16(rv, toff, (uint32_t)j * 16384 + 4096 * i, vst + (4 * i + w) * 1024);
}

// Vhat^T tile j (8 KB: [128 channels][64 B]) into one stage; LDS row r holds
// 16-byte chunk q at chunk q ^ ((r >> 2) & 3) (conflict-free reads of 32 B
// per lane); two 1 KB pieces per wave.
__device__ inline uint32_t v8_lane_off(int lane) {
    return (uint32_t)((lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4));
}
__device__ inline void issue_v8(char* v8st, rsrc_t rv8, int j, int w, uint32_t v8off) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = 4 * i + w;
        load_lds16(rv8, v8off, (uint32_t)j * kV8 + u * 1024, v8st + u * 1024);
    }
}

// QK: 0 = bf16 Q K^T, 1 = e4m3 codes, 2 = int8 codes
template <bool LIN, int QK, bool LOWV, bool PHISM, bool V1>
__global__ __launch_bounds__(256, 2) void fused128_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ vt, const int32_t* __restrict__ idx,
    const float* __restrict__ alpha, const char* __restrict__ HZ,
    const uint8_t* __restrict__ qhat, const uint8_t* __restrict__ khat,
    const float* __restrict__ sq, const float* __restrict__ sk,
    const uint8_t* __restrict__ vhat, const float* __restrict__ sv, void* __restrict__ O,
    int N, int Tq, int Tkv, int k, int H, Strides st, int alpha_qblock, int out_bf16,
    const uint16_t* __restrict__ wpf, int w_heads) {
    constexpr bool LOWBIT = QK != 0;
    static_assert(!(PHISM || V1) || (QK == 0 && !LOWV), "softmax phi and v1: bf16 path only");
    static_assert(LOWBIT || !LOWV, "quantised V only with the low-bit Q K^T");
    // V^T in fp16 feeds P V (unless P V runs on the e4m3 codes)
    constexpr bool kV16 = !LOWV;
    using P = Plan<LOWBIT, LOWV>;
    const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hl = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    long bh;
    int qb;
    if (!head_major_map(blockIdx.x, Tq, &bh, &qb)) return;
    const int tq = qb * 128 + 32 * w + l32;
    const bool valid_q = tq < N;
    const float c_log2 = 1.4426950408889634f / sqrtf(128.0f);

    // ---- Q operand (B of S^T = K Q^T): lane holds query tq
    QOp<LOWBIT> Qo;
    float c_base = c_log2;
    if (LOWBIT) {
        const uint8_t* qrow =
            qhat + ((size_t)bh * Tq * 128 + (size_t)qb * 128 + 32 * w + l32) * 128;
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
        const uint16_t* qrow = Q + head_base(st, bh, H) + (size_t)(valid_q ? tq : 0) * st.t;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid_q) v = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
            reinterpret_cast<bf16x8*>(Qo.f)[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- accumulators: O^T (d rows 32mt.., my queries)
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = zero16();
    float m_ref = -INFINITY, l_part = 0.0f;
    // LOWV: the row sums of 256 P^ come from the e4m3 matrix cores, as the
    // product of a row of ones (e4m3 1.0 = 0x38) with the P codes: every row
    // of lacc holds the sum over the tile's 64 keys for the lane's query
    f32x16 lacc = zero16();

    const int32_t* sel = idx + ((size_t)bh * Tq + qb) * k;
    const uint32_t rp = (uint32_t)st.t * 2;  // bytes between consecutive K rows
    const rsrc_t rk = LOWBIT ? head_rsrc(khat + (size_t)bh * Tkv * 64 * 128)
                             : head_rsrc(K + head_base(st, bh, H));
    const rsrc_t rv = head_rsrc(vt + (size_t)bh * Tkv * 128 * 64);
    const uint32_t koff = k_lane_off(w, lane, rp), toff = t_lane_off(w, lane);
    const float* sk_h = LOWBIT ? sk + (size_t)bh * Tkv : nullptr;
    char* const kbase = s_lds;
    char* const vbase = s_lds + P::vOff;
    char* const v8base = s_lds + P::v8Off;
    const rsrc_t rv8 = head_rsrc(LOWV ? vhat + (size_t)bh * Tkv * kV8 : vhat);
    const uint32_t v8off = v8_lane_off(lane);

    constexpr int nV = (kV16 ? 4 : 0) + (LOWV ? 2 : 0);  // loads per lane, V tile
    // S^T = K Q^T over the whole tile in K stage kst (two m-tiles of 32 keys)
    auto compute_s = [&](const char* kst, f32x16 (&s)[2]) {
        s[0] = zero16();
        s[1] = zero16();
        if (QK == 2) {
            // int8 codes: the 32 bytes of a lane's 64-channel step go to two
            // int8 MFMAs (16 each; A and B split alike, so each sums a
            // matching half of the channels); the int32 sums are exact and
            // converted once per tile
            i32x16 si[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) si[mt][i] = 0;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int kr = 32 * mt + l32, sw = (kr >> 1) & 7, c0 = 4 * ks + 2 * hl;
                    const uint4 lo = *reinterpret_cast<const uint4*>(kst + kr * 128 + ((c0 ^ sw) << 4));
                    const uint4 hi =
                        *reinterpret_cast<const uint4*>(kst + kr * 128 + (((c0 + 1) ^ sw) << 4));
                    const i32x8 q8 = reinterpret_cast<const i32x8*>(Qo.f)[ks];
                    const i32x4 qlo = {q8[0], q8[1], q8[2], q8[3]};
                    const i32x4 qhi = {q8[4], q8[5], q8[6], q8[7]};
                    si[mt] = mfma_i8(i32x4{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w}, qlo, si[mt]);
                    si[mt] = mfma_i8(i32x4{(int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w}, qhi, si[mt]);
                }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[mt][i] = (float)si[mt][i];
        } else if (LOWBIT) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int kr = 32 * mt + l32, sw = (kr >> 1) & 7, c0 = 4 * ks + 2 * hl;
                    const uint4 lo = *reinterpret_cast<const uint4*>(kst + kr * 128 + ((c0 ^ sw) << 4));
                    const uint4 hi =
                        *reinterpret_cast<const uint4*>(kst + kr * 128 + (((c0 + 1) ^ sw) << 4));
                    i32x8 a;
                    a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
                    a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
                    s[mt] = mfma_fp8(a, reinterpret_cast<const i32x8*>(Qo.f)[ks], s[mt]);
                }
        } else {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int kr = 32 * mt + l32;
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        kst + kr * 256 + (((2 * ks + hl) ^ (kr & 15)) << 4));
                    s[mt] = mfma_bf16(a, reinterpret_cast<const bf16x8*>(Qo.f)[ks], s[mt]);
                }
        }
    };

    // new running reference after a tile of logits whose maximum (over this
    // wave's column, both lane halves) is mx, with logit scale ct; rescales
    // O and l.  Returns the reference the tile's P is taken against.
    auto update_ref = [&](float mx, float ct) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float xmax = mx * ct;
        const bool need = LOWBIT ? (xmax > m_ref) : (xmax > m_ref + kRescaleThr);
        if (__ballot(need)) {
            const float nref = need ? xmax : m_ref;
            const float f = __builtin_amdgcn_exp2f(m_ref - nref);
            l_part *= f;
            if (LOWV) lacc[0] *= f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[i][e] *= f;
            m_ref = nref;
        }
        return m_ref == -INFINITY ? 0.0f : m_ref;
    };
    // a tile's S is complete: mask the keys past N, then the running
    // reference.  Only KV block T_kv - 1 is ragged, and the selection is
    // ascending (a documented precondition), so only the last selected tile
    // can be (may_ragged).
    auto finish_s = [&](f32x16 (&s)[2], int jx, float ct, auto may_ragged_c) {
        constexpr bool MAY_RAGGED = decltype(may_ragged_c)::value;
        if (MAY_RAGGED && jx * 64 + 64 > N) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (jx * 64 + 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3) >= N)
                        s[mt][i] = -INFINITY;
        }
        // pairwise maxima of the two m-tiles (one v_med3 each), then four
        // chains over them, whose links of two become three-input maxima (the
        // med3 results need no canonicalising); no NaN reaches here
        float m[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) m[i] = max2f(s[0][i], s[1][i]);
        float c4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c4[j] = fmaxf(fmaxf(fmaxf(m[j], m[j + 4]), m[j + 8]), m[j + 12]);
        return update_ref(fmaxf(fmaxf(fmaxf(c4[0], c4[1]), c4[2]), c4[3]), ct);
    };
    auto ctile = [&](int jx) { return LOWBIT ? c_base * sk_h[jx] : c_base; };
    // the query block's row of the linear-branch product into LDS by
    // direct loads: H_i^T (bf16) as [128 e rows][256 B] with chunk c' (c =
    // 8 c' ..) of row e at c' ^ (e & 15) (the K tile layout, 8 pieces of 1 KB
    // per wave), Z_i (fp32) after it.  The row holds the chunk at hz_unit(e,
    // c'); for the rows e = 16 i + r of piece i that unit is 512 (i / 2) +
    // 16 (i % 2) plus a part that depends on (r, c') only, so the lane's
    // offset is set once and the piece adds a uniform one.  Issued at the
    // start of the last tile step, into the K stages (free from then on; 32.5
    // KB of the 48), so that the loads run under the last P V (bf16 path).
    constexpr bool kEarlyH = LIN && !LOWBIT;
    auto issue_h = [&]() {
        const rsrc_t rh = head_rsrc(HZ + (size_t)bh * Tq * kHzRowBytes);
        const int hr = 4 * w + (lane >> 4), hc = (lane & 15) ^ hr;
        const uint32_t hoff = 16u * (uint32_t)hz_unit(hr, hc);
        const uint32_t row0 = (uint32_t)qb * kHzRowBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            load_lds16(rh, hoff, row0 + 8192 * (i >> 1) + 256 * (i & 1),
                       s_lds + (4 * i + w) * 1024);
        if (w < 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, SLA2_LDS(s_lds + 32768 + 256 * w), 4,
                                                     (uint32_t)lane * 4,
                                                     row0 + 32768 + 256 * w, 0, 0);
    };

    // ---- prologue: K_0, K_1, V_0, K_2 (in this order), then S_0 and its
    // reference
    f32x16 sc[2];
    float cur_ref = 0.0f, cur_ct = c_base;
    if (k > 0) {
        issue_k<LOWBIT>(kbase, rk, sel[0], N, w, lane, koff, toff, rp);
        if (k > 1) issue_k<LOWBIT>(kbase + P::kStage, rk, sel[1], N, w, lane, koff, toff, rp);
        if (kV16) issue_v(vbase, rv, sel[0], w, toff);
        if (LOWV) issue_v8(v8base, rv8, sel[0], w, v8off);
        if (k > 2) issue_k<LOWBIT>(kbase + 2 * P::kStage, rk, sel[2], N, w, lane, koff, toff, rp);
        // K_0 has landed (issued after it: K_1, V_0, K_2)
        if (k > 2) wait_vmcnt<2 * P::nK + nV>();
        else if (k > 1) wait_vmcnt<P::nK + nV>();
        else wait_vmcnt<nV>();
        wg_barrier();
        compute_s(kbase, sc);
        cur_ct = ctile(sel[0]);
        if (k == 1) cur_ref = finish_s(sc, sel[0], cur_ct, std::true_type{});
        else cur_ref = finish_s(sc, sel[0], cur_ct, std::false_type{});
    }

    // One tile step r, with S of tile r in sc and its reference cur_ref.
    // MORE1 / MORE2 / MORE3: tiles r+1 / r+2 / r+3 exist.  The products of
    // tile r+1's S do not depend on tile r, so they sit in one branch-free
    // block with tile r's P (vector ALU) and P V: the matrix cores work
    // while the exponentials are evaluated.  Tile r+1's maximum and the
    // rescale follow once its S is complete.  K tile x sits in stage x % 3,
    // V tile x in stage x % 2.  The last three steps are peeled off the loop,
    // so that inside it every load is unconditional.
    auto step = [&](int r, int ks_r, f32x16 (&sc)[2], f32x16 (&sn)[2], auto more1_c,
                    auto more2_c, auto more3_c, auto copy_c) {
        constexpr bool MORE1 = decltype(more1_c)::value;
        constexpr bool MORE2 = decltype(more2_c)::value;
        constexpr bool MORE3 = decltype(more3_c)::value;
        // K_{r+1} and V_r have landed for this wave (issued after V_r: K_{r+2}) ...
        if (MORE2) wait_vmcnt<P::nK>();
        else wait_vmcnt<0>();
        wg_barrier();  // ... and for every wave; all waves are done with K_r and V_{r-1}
        if (MORE1) {
            if (kV16) issue_v(vbase + ((r + 1) & 1) * kVT, rv, sel[r + 1], w, toff);
            if (LOWV) issue_v8(v8base + ((r + 1) & 1) * kV8, rv8, sel[r + 1], w, v8off);
        }
        if (MORE3)
            issue_k<LOWBIT>(kbase + ks_r * P::kStage, rk, sel[r + 3], N, w, lane, koff, toff, rp);
        if constexpr (kEarlyH && !MORE1) issue_h();
        if (MORE1) compute_s(kbase + (ks_r == 2 ? 0 : ks_r + 1) * P::kStage, sn);
        const char* vst = vbase + (r & 1) * kVT;
        const char* v8st = v8base + (r & 1) * kV8;
        const float c_tile = cur_ct, mref = cur_ref;
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        // O^T += V^T P^T for k-step kq (16 keys)
        auto pv_step = [&](int kq, const f16x8& pfk) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int erow = 32 * mt + l32;
                const f16x8 a = *reinterpret_cast<const f16x8*>(
                    vst + erow * 128 + (((2 * kq + hl) ^ ((erow >> 1) & 7)) << 4));
                o[mt] = mfma_f16(a, pfk, o[mt]);
            }
        };
        if (LOWV) {
            // codes of 256 P~ as the k operand of the e4m3 P V product: byte
            // 16 mt + i of this lane is the code of sc[mt][i]; the row sum is
            // taken over the decoded values.  The low-bit reference moves on
            // every new maximum (update_ref), so 256 P~ <= 256 (at most half
            // an ulp of the logit above it) and needs no clamp to e4m3's 448
            const float bias = 8.0f - mref;
            i32x8 pc;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float p4[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        p4[c] = __builtin_amdgcn_exp2f(fmaf(sc[mt][4 * q + c], c_tile, bias));
                    // the low half first, into any live register (the high
                    // half is written next): no zeroed word per code group
                    int wv = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], __float_as_int(p4[0]),
                                                             false);
                    wv = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], wv, true);
                    pc[4 * mt + q] = wv;
                }
            {
                i32x8 ones;
#pragma unroll
                for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;
                lacc = mfma_fp8(ones, pc, lacc);
            }
            // O^T += Vhat^T (256 P^)^T on the e4m3 matrix cores (one k-step of
            // 64 keys per d-tile); the channel scales s_V apply at the end
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int vrow = 32 * mt + l32, sw = (vrow >> 2) & 3;
                const uint4 lo = *reinterpret_cast<const uint4*>(v8st + vrow * 64 + (((2 * hl) ^ sw) << 4));
                const uint4 hi =
                    *reinterpret_cast<const uint4*>(v8st + vrow * 64 + (((2 * hl + 1) ^ sw) << 4));
                i32x8 a;
                a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
                a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
                o[mt] = mfma_fp8(a, pc, o[mt]);
            }
        } else {
            // P^T as the B operand of k-step kq (16 keys) takes rows 8(kq&1)..
            // 8(kq&1)+7 of m-tile kq>>1
    #pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                f16x8 pf;
                if (LOWBIT) {  // 256 P~ rounded onto the e4m3 grid, carried exactly in fp16
                    const float bias = 8.0f - mref;
    #pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kq >> 1][8 * (kq & 1) + e], c_tile, bias));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kq >> 1][8 * (kq & 1) + e + 1], c_tile, bias));
                        // only the low half is decoded: the high half's
                        // source is any live register.  Decoded straight to
                        // fp16 (scale 1; every e4m3 value is an fp16 value)
                        const int code =
                            __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
                        const f16x2 back = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, false);
                        pf[e] = back[0];
                        pf[e + 1] = back[1];
                    }
                } else {
    #pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pf[e] = (_Float16)__builtin_amdgcn_exp2f(
                            fmaf(sc[kq >> 1][8 * (kq & 1) + e], c_tile, -mref));
                }
    #pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const f16x2 pr = {pf[e], pf[e + 1]};
                    l_part = __builtin_amdgcn_fdot2(pr, ones, l_part, false);
                }
                pv_step(kq, pf);
            }
        }
        if (MORE1) {
            const int jn = sel[r + 1];
            cur_ct = ctile(jn);
            cur_ref = finish_s(sn, jn, cur_ct, std::integral_constant<bool, !MORE2>{});
            if constexpr (decltype(copy_c)::value) {
                sc[0] = sn[0];
                sc[1] = sn[1];
            }
        }
    };
    // Tile steps in pairs, the next tile's S alternating between sc and sn
    // (no register copies); the steps after the pairs keep the current S in
    // sc.
    f32x16 sn[2];
    const std::true_type T{};
    const std::false_type F{};
    auto adv = [](int x) { return x == 2 ? 0 : x + 1; };
    int r = 0, ks = 0;
    for (; r + 4 < k; r += 2) {
        step(r, ks, sc, sn, T, T, T, F);
        ks = adv(ks);
        step(r + 1, ks, sn, sc, T, T, T, F);
        ks = adv(ks);
    }
    if (r + 3 < k) {
        step(r++, ks, sc, sn, T, T, T, T);
        ks = adv(ks);
    }
    if (r + 2 < k) {
        step(r++, ks, sc, sn, T, T, F, T);
        ks = adv(ks);
    }
    if (r + 1 < k) {
        step(r++, ks, sc, sn, T, F, F, T);
        ks = adv(ks);
    }
    if (r < k) step(r, ks, sc, sn, F, F, F, T);

    // ---- epilogue
    const float l_all = LOWV ? lacc[0] : l_part + __shfl_xor(l_part, 32);
    const float inv_l = (k > 0 && l_all > 0.0f) ? 1.0f / l_all : 0.0f;
    f32x16 ol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ol[i] = zero16();
    float inv_den = 0.0f;
    if (LIN) {
        // H_i^T (bf16 row of the product, units at hz_unit) in LDS as
        // [128 d rows][256 B], chunk c' of row e at c' ^ (e & 15); Z_i fp32
        char* sH = s_lds;
        float* sZ = reinterpret_cast<float*>(s_lds + 32768);
        if constexpr (kEarlyH) {
            if (k == 0) issue_h();  // (no tile step issued it)
            wait_vmcnt<0>();
            wg_barrier();  // every wave's pieces have landed
        } else {
            wg_barrier();  // every wave is done with the tile stages
            const char* hrow = HZ + ((size_t)bh * Tq + qb) * kHzRowBytes;
            const int he = t >> 1, hc = 8 * (t & 1);  // row e, 16-byte chunks hc .. hc + 7
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(hrow + 16 * hz_unit(he, hc + i));
                *reinterpret_cast<uint4*>(sH + he * 256 + (((hc + i) ^ (he & 15)) << 4)) = v;
            }
            if (t < 128) sZ[t] = reinterpret_cast<const float*>(hrow + 2 * 128 * 128)[t];
            wait_lgkm0();
            wg_barrier();
        }
        // phi(Q)^T operand from the raw bf16 Q (registers on the bf16 path)
        bf16x8 qraw[8];
        if (LOWBIT) {
            const uint16_t* qrow = Q + head_base(st, bh, H) + (size_t)(valid_q ? tq : 0) * st.t;
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
        bf16x8 pq[8];
        float den = 0.0f;
        // softmax phi: max and 1 / sum exp over the query's 128 channels (64
        // in this lane, 64 in its partner lane ^ 32)
        float qmax = 0.0f, qinv = 1.0f;
        if (PHISM) {
            qmax = -INFINITY;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, (float)qraw[ks][e]);
            qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
            float qs = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) qs += __expf((float)qraw[ks][e] - qmax);
            qinv = 1.0f / (qs + __shfl_xor(qs, 32));
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const float4 z0 = *reinterpret_cast<const float4*>(sZ + 16 * ks + 8 * hl);
            const float4 z1 = *reinterpret_cast<const float4*>(sZ + 16 * ks + 8 * hl + 4);
            const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = PHISM ? __expf((float)qraw[ks][e] - qmax) * qinv
                                      : phi_fast((float)qraw[ks][e]);
                pq[ks][e] = (__bf16)p;
                // the same rounded phi in the denominator: O_l stays a
                // weighted mean of the value rows
                den = fmaf((float)pq[ks][e], zz[e], den);
            }
        }
        den += __shfl_xor(den, 32);
        inv_den = 1.0f / den;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int erow = 32 * mt + l32;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    sH + erow * 256 + (((2 * ks + hl) ^ (erow & 15)) << 4));
                ol[mt] = mfma_bf16(a, pq[ks], ol[mt]);
            }
        }
    }
    if constexpr (V1) {
        // O = O_s + O_l W_p: out^T (128 channels x 32 queries) = W_p^T O_l^T,
        // B = O_l^T from the accumulators (k-step 2 mt + h takes entries
        // 8h .. 8h+7 of m-tile mt; the fragments of W_p^T follow the same
        // k order), O_l as fp16 high part + fp16 rest
        f16x8 bhi[8], blo[8];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = LIN ? ol[mt][8 * h + e] * inv_den : 0.0f;
                    const _Float16 hi = (_Float16)x;
                    bhi[2 * mt + h][e] = hi;
                    blo[2 * mt + h][e] = (_Float16)(x - (float)hi);
                }
        const uint16_t* wf = wpf + (w_heads == 1 ? 0 : (size_t)(bh % H) * 128 * 128);
        const size_t orow = head_base(st, bh, H) + (size_t)(valid_q ? tq : 0) * st.t;
#pragma unroll
        for (int mo = 0; mo < 4; ++mo) {
            f32x16 pr = zero16();
            if (LIN) {
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const f16x8 a = *reinterpret_cast<const f16x8*>(
                        wf + ((size_t)(mo * 8 + ks) * 64 + lane) * 8);
                    pr = mfma_f16(a, bhi[ks], pr);
                    pr = mfma_f16(a, blo[ks], pr);
                }
            }
            if (valid_q) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    float v[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = o[mo][4 * i4 + c] * inv_l + pr[4 * i4 + c];
                    store_out4(O, orow + 32 * mo + 8 * i4 + 4 * hl, v[0], v[1], v[2], v[3],
                               out_bf16);
                }
            }
        }
        return;
    }
    if (valid_q) {
        const float a_h = alpha_of(alpha, bh, H, qb, Tq, alpha_qblock);
        const size_t orow = head_base(st, bh, H) + (size_t)tq * st.t;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                // O^T row e = 32 mt + 8 i4 + 4 hl + c; with LOWV scaled by s_V(e)
                float vs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                if (LOWV) {
                    const float4 s4 = *reinterpret_cast<const float4*>(
                        sv + bh * 128 + 32 * mt + 8 * i4 + 4 * hl);
                    vs[0] = s4.x;
                    vs[1] = s4.y;
                    vs[2] = s4.z;
                    vs[3] = s4.w;
                }
                float v[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    v[c] = a_h * (o[mt][4 * i4 + c] * vs[c] * inv_l) +
                           (1.0f - a_h) * (ol[mt][4 * i4 + c] * inv_den);
                store_out4(O, orow + 32 * mt + 8 * i4 + 4 * hl, v[0], v[1], v[2], v[3], out_bf16);
            }
    }
}

__global__ __launch_bounds__(256) void wp_frag_kernel(const float* __restrict__ Wp,
                                                     uint16_t* __restrict__ wpf) {
    // fragment (m-tile mo, k-step ks, lane, e) = W_p[dd][m]: m = 32 mo +
    // lane % 32, dd = 32 (ks / 2) + 16 (ks % 2) + 8 (e / 4) + 4 (lane / 32) + e % 4
    const float* W = Wp + (size_t)blockIdx.x * 128 * 128;
    uint16_t* out = wpf + (size_t)blockIdx.x * 128 * 128;
    for (int x = threadIdx.x; x < 128 * 128; x += 256) {
        const int e = x & 7, ln = (x >> 3) & 63, ks = (x >> 9) & 7, mo = x >> 12;
        const int m = 32 * mo + (ln & 31);
        const int dd = 32 * (ks >> 1) + 16 * (ks & 1) + 8 * (e >> 2) + 4 * (ln >> 5) + (e & 3);
        const _Float16 h = (_Float16)W[(size_t)dd * 128 + m];
        out[x] = __builtin_bit_cast(uint16_t, h);
    }
}

// Diagnostic of the e4m3 matrix-core dot product of the low-bit logits:
// C[t] = A[t] B[t]^T for tiles of 32 rows x 128 codes, as two chained
// 32x32x64 scaled products (scales 1.0) with the operand layout of the Q K^T
// above (lane l: row l % 32, codes 64 ks + 32 (l / 32) .. + 31).  One wave
// per tile; C row-major [32][32] fp32.
__global__ __launch_bounds__(64) void fp8_dot_kernel(const uint8_t* __restrict__ A,
                                                     const uint8_t* __restrict__ B,
                                                     float* __restrict__ C) {
    const size_t tile = blockIdx.x;
    const int l = threadIdx.x, row = l & 31, half = l >> 5;
    const uint8_t* a = A + (tile * 32 + row) * 128 + 32 * half;
    const uint8_t* b = B + (tile * 32 + row) * 128 + 32 * half;
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const i32x8 av = *reinterpret_cast<const i32x8*>(a + 64 * ks);
        const i32x8 bv = *reinterpret_cast<const i32x8*>(b + 64 * ks);
        acc = mfma_fp8(av, bv, acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
        C[tile * 1024 + (size_t)(8 * (r >> 2) + 4 * half + (r & 3)) * 32 + row] = acc[r];
}

}  // namespace

hipError_t launch_fp8_dot(const uint8_t* A, const uint8_t* B, float* C, int ntiles,
                          hipStream_t s) {
    fp8_dot_kernel<<<dim3((unsigned)ntiles), 64, 0, s>>>(A, B, C);
    return hipGetLastError();
}

hipError_t launch_wp_frag(const Dims& D, const float* Wp, const FwdWS& ws, hipStream_t s) {
    wp_frag_kernel<<<dim3((unsigned)D.w_heads), 256, 0, s>>>(Wp, ws.wpf);
    return hipGetLastError();
}

hipError_t launch_fused128(const Dims& D, const void* Q, const void* K, const int32_t* idx,
                           const float* alpha, void* O, const FwdWS& ws, bool lowbit,
                           hipStream_t s) {
    // one work-group per (head, query block), Tq padded to a multiple of 8
    const dim3 g((unsigned)(((D.Tq + 7) / 8) * 8 * D.BH), 1);
    const bool lin = D.k + (D.v1 ? D.kl : 0) < D.Tkv && !D.skip_lin;
    const int kloop = D.skip_sparse ? 0 : D.k;  // selected tiles the sparse branch visits
    // the dense linear-branch product has filled ws.HZ (linear.hip)
    const uint16_t* q = (const uint16_t*)Q;
    const uint16_t* kk = (const uint16_t*)K;
    const uint8_t* qh = lowbit ? ws.qhat : nullptr;
    const uint8_t* kh = lowbit ? ws.khat : nullptr;
    const float* sq = lowbit ? ws.sq : nullptr;
    const float* sk = lowbit ? ws.sk : nullptr;
    const bool lowv = lowbit && D.lowbit_v;
    const bool i8 = lowbit && D.int8_qk;
#define F128(L, Q, V) fused128_kernel<L, Q, V, false, false>
    auto kern = !lowbit ? (lin ? F128(true, 0, false) : F128(false, 0, false))
                : i8 ? (!lowv ? (lin ? F128(true, 2, false) : F128(false, 2, false))
                              : (lin ? F128(true, 2, true) : F128(false, 2, true)))
                : !lowv ? (lin ? F128(true, 1, false) : F128(false, 1, false))
                        : (lin ? F128(true, 1, true) : F128(false, 1, true));
#undef F128
    if (!lowbit && (D.phi_sm || D.v1)) {
        const bool sm = D.phi_sm, v1 = D.v1;
        kern = lin ? (sm ? (v1 ? fused128_kernel<true, 0, false, true, true>
                               : fused128_kernel<true, 0, false, true, false>)
                         : (v1 ? fused128_kernel<true, 0, false, false, true>
                               : fused128_kernel<true, 0, false, false, false>))
                   : (sm ? (v1 ? fused128_kernel<false, 0, false, true, true>
                               : fused128_kernel<false, 0, false, true, false>)
                         : (v1 ? fused128_kernel<false, 0, false, false, true>
                               : fused128_kernel<false, 0, false, false, false>));
    }
    const KernelKind kind = D.v1 ? K_FUSED_SLA1
                            : !lowbit ? K_FUSED_MFMA : i8 ? K_FUSED_I8 : K_FUSED_FP8;
    timing_before(s, kind);
    kern<<<g, 256, 0, s>>>(q, kk, ws.vt, idx, alpha, ws.HZ, qh, kh, sq, sk,
                           lowv ? ws.vhat : nullptr, lowv ? ws.sv : nullptr, O, D.N, D.Tq, D.Tkv,
                           kloop, D.H, D.st, D.alpha_qblock, D.out_bf16,
                           D.v1 ? ws.wpf : nullptr, D.w_heads);
    timing_after(s, kind);
    return hipGetLastError();
}

}  // namespace sla2
