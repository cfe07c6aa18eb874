// The C ABI's host-side logic (problem checks, block and top-k counts,
// workspace layouts, argument validation of every entry point) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every call either only
// queries sizes or fails validation, so nothing reaches the GPU.  Built and
// run by tests/test_sanitizers.py against a copy of the library whose host
// code is instrumented; exits non-zero on a wrong result (a sanitizer report
// aborts the process before that).
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "sla2.h"

static int fails = 0;
#define EXPECT(x)                                                     \
    do {                                                              \
        if (!(x)) {                                                   \
            fprintf(stderr, "failed: %s (line %d)\n", #x, __LINE__);  \
            ++fails;                                                  \
        }                                                             \
    } while (0)

static sla2_problem prob(int B, int H, int N, int d, int bq, float frac, int dtype) {
    sla2_problem p = {};
    p.B = B;
    p.H = H;
    p.N = N;
    p.d = d;
    p.bq = bq;
    p.bkv = 64;
    p.topk_frac = frac;
    p.w_heads = 1;
    p.phi = SLA2_PHI_ELU1;
    p.dtype = dtype;
    p.layout = SLA2_LAYOUT_BHND;
    p.alpha_mode = SLA2_ALPHA_PER_HEAD;
    p.out_dtype = SLA2_F32;
    p.lowbit = SLA2_LOWBIT_QK;
    p.flags = 0;
    return p;
}

int main() {
    // sizes over a spread of shapes, every op, both dtypes, both phi
    const int Ns[] = {1, 63, 64, 65, 700, 4100, 32760, 75600, 491520};
    for (int N : Ns)
        for (int d : {64, 128})
            for (int bq : {64, 128})
                for (int dt : {SLA2_F32, SLA2_BF16})
                    for (int phi : {SLA2_PHI_ELU1, SLA2_PHI_SOFTMAX})
                        for (float frac : {0.0f, 0.03f, 0.5f, 1.0f}) {
                            sla2_problem p = prob(1, 3, N, d, bq, frac, dt);
                            p.phi = phi;
                            const int tq = sla2_num_q_blocks(&p), tkv = sla2_num_kv_blocks(&p);
                            EXPECT(tq == (N + bq - 1) / bq && tkv == (N + 63) / 64);
                            const int k = sla2_topk(&p);
                            EXPECT(k >= 0 && k <= tkv);
                            for (int op = SLA2_OP_ROUTE; op <= SLA2_OP_ATTENTION_FP8; ++op) {
                                const sla2_status st = sla2_check(&p, op);
                                const size_t ws = sla2_workspace_bytes(&p, op);
                                EXPECT((st == SLA2_OK) == (ws > 0) || tkv > 7680);
                                (void)sla2_status_str(st);
                            }
                            EXPECT(sla1_num_negligible(&p, 0.1f) >= 0 || tkv > 7680);
                        }
    // invalid problems: no size, no check
    sla2_problem bad = prob(1, 2, 1000, 96, 128, 0.1f, SLA2_BF16);
    EXPECT(sla2_check(&bad, SLA2_OP_ROUTE) == SLA2_EUNSUPPORTED);
    EXPECT(sla2_workspace_bytes(&bad, SLA2_OP_FORWARD) == 0);
    bad = prob(0, 2, 1000, 128, 128, 0.1f, SLA2_BF16);
    EXPECT(sla2_check(&bad, SLA2_OP_ROUTE) == SLA2_EINVAL && sla2_topk(&bad) == -1);
    bad = prob(1, 2, 1000, 128, 128, 1.5f, SLA2_BF16);
    EXPECT(sla2_check(&bad, SLA2_OP_ROUTE) == SLA2_EINVAL);
    EXPECT(sla2_check(nullptr, SLA2_OP_ROUTE) == SLA2_EINVAL);
    EXPECT(sla2_check(&bad, 99) == SLA2_EINVAL);

    // argument validation of every entry point: null or misaligned pointers
    // and short workspaces are refused before any launch
    sla2_problem p = prob(1, 2, 1000, 128, 128, 0.1f, SLA2_BF16);
    void* g = (void*)(uintptr_t)(1 << 20);
    void* mis = (void*)(uintptr_t)((1 << 20) + 8);
    float* gf = (float*)g;
    int32_t* gi = (int32_t*)g;
    uint8_t* gb = (uint8_t*)g;
    const size_t wr = sla2_workspace_bytes(&p, SLA2_OP_ROUTE);
    const size_t wf = sla2_workspace_bytes(&p, SLA2_OP_FORWARD);
    const size_t wa = sla2_workspace_bytes(&p, SLA2_OP_ATTENTION);
    const size_t w8 = sla2_workspace_bytes(&p, SLA2_OP_FORWARD_FP8);
    const size_t wa8 = sla2_workspace_bytes(&p, SLA2_OP_ATTENTION_FP8);
    const size_t wb = sla2_workspace_bytes(&p, SLA2_OP_BACKWARD);
    const size_t wg = sla2_workspace_bytes(&p, SLA2_OP_ROUTE_GRAD);
    const size_t w1 = sla2_workspace_bytes(&p, SLA2_OP_SLA1_FORWARD);
    EXPECT(sla2_route(&p, nullptr, g, gf, gf, gi, nullptr, g, wr, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_route(&p, g, g, gf, gf, gi, nullptr, g, wr - 1, nullptr) == SLA2_EWORKSPACE);
    EXPECT(sla2_route(&p, mis, g, gf, gf, gi, nullptr, g, wr, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_forward(&p, g, g, g, gi, gf, nullptr, g, wf, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_forward(&p, g, g, g, gi, gf, g, g, wf - 256, nullptr) == SLA2_EWORKSPACE);
    EXPECT(sla2_attention(&p, g, g, g, gf, gf, gf, gi, g, g, wa - 1, nullptr) ==
           SLA2_EWORKSPACE);
    EXPECT(sla2_attention(&p, g, g, nullptr, gf, gf, gf, gi, g, g, wa, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_forward_fp8(&p, g, g, g, gi, gf, g, g, w8 - 1, nullptr) == SLA2_EWORKSPACE);
    EXPECT(sla2_attention_fp8(&p, g, g, g, gf, gf, gf, nullptr, g, g, wa8, nullptr) ==
           SLA2_EINVAL);
    EXPECT(sla2_quantize_fp8(&p, g, g, nullptr, gb, gf, gf, gf, g, w8, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_backward(&p, g, g, g, gi, gf, nullptr, gf, gf, gf, gf, g, wb, nullptr) ==
           SLA2_EINVAL);
    EXPECT(sla2_backward(&p, g, g, g, gi, gf, gf, gf, gf, gf, gf, g, wb - 256, nullptr) ==
           SLA2_EWORKSPACE);
    EXPECT(sla2_route_grad(&p, g, g, gf, gf, nullptr, gf, gf, g, wg, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_soft_topk(&p, g, g, gf, gf, 0.0f, gf, nullptr, g, wr, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_soft_topk_grad(&p, gf, gf, -1.0f, gf, nullptr) == SLA2_EINVAL);
    EXPECT(sla1_route(&p, g, g, 1.5f, gi, gi, nullptr, g, wr, nullptr) == SLA2_EINVAL);
    EXPECT(sla1_forward(&p, g, g, g, gi, gi, 0.1f, nullptr, g, g, w1, nullptr) == SLA2_EINVAL);
    EXPECT(sla1_forward(&p, g, g, g, gi, gi, 0.1f, gf, g, g, w1 - 1, nullptr) ==
           SLA2_EWORKSPACE);
    EXPECT(sla2_fp8_dot_tiles(gb, gb, gf, 0, nullptr) == SLA2_EINVAL);
    EXPECT(sla2_mfma_rate_probe(4, 1, 1, gf, nullptr) == SLA2_EINVAL);
    // past the no-allocation entry point's fixed array
    sla2_problem big = prob(1, 40, 75600, 128, 128, 0.03f, SLA2_BF16);
    EXPECT(sla2_attention_noalloc(&big, g, g, g, gf, gf, gf, gi, g, nullptr) ==
           SLA2_EWORKSPACE);
    EXPECT(sla2_noalloc_scratch_bytes() > 0);
    EXPECT(sla2_kernel_kinds() > 0 && sla2_kernel_name(0) != nullptr);
    EXPECT(sla2_kernel_name(-1)[0] == 0);
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
