// Accuracy of the gfx950 fp8 (OCP e4m3) matrix-core dot product, the one the
// low-bit logits use: 32x32 tiles of length-128 dot products computed with
// two chained 32x32x64 scaled MFMAs (scales 1.0), compared with the exact
// sums.  Prints the largest |computed - exact| / sum|a b| and the share of
// results that are exact.  The parity tests of the low-bit forward take their
// accumulation-error constant from this figure.
//
//   hipcc --offload-arch=gfx950 -O2 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o fp8_mfma_accuracy tests/probes/fp8_mfma_accuracy.hip
//   ./fp8_mfma_accuracy 0    absmax-scaled Gaussian rows
//   ./fp8_mfma_accuracy 1    correlated rows (large dot products)
//   ./fp8_mfma_accuracy 2    uniformly random codes over all exponents
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                              \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            return 1;                                                         \
        }                                                                     \
    } while (0)

// one wave per tile; lane l holds A[row l%32][k 64ks+32(l/32)..+32] and
// B[k ...][col l%32]; C lane l holds column l%32, rows 8(r/4)+4(l/32)+r%4
__global__ void dot_tiles(const i32x8* a, const i32x8* b, f32x16* c, int ntiles) {
    const int tile = blockIdx.x, l = threadIdx.x;
    if (tile >= ntiles) return;
    f32x16 acc = {};
    for (int ks = 0; ks < 2; ++ks)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a[(tile * 2 + ks) * 64 + l], b[(tile * 2 + ks) * 64 + l], acc, 0, 0, 0, 127, 0, 127);
    c[tile * 64 + l] = acc;
}

static double e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    const double v = e == 0 ? ldexp(m, -9) : ldexp(8 + m, e - 10);
    return s ? -v : v;
}

// nearest e4m3 code, ties to the even code (|x| <= 448)
static uint8_t e4m3_code(double x) {
    uint8_t best = 0;
    double bd = 1e300;
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7f) == 0x7f) continue;
        const double d = fabs(e4m3_value((uint8_t)c) - x);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = (uint8_t)c;
        }
    }
    return best;
}

int main(int argc, char** argv) {
    const int ntiles = 512, mode = argc > 1 ? atoi(argv[1]) : 0;
    std::mt19937_64 g(1234 + mode);
    std::normal_distribution<double> n01;
    std::vector<uint8_t> A((size_t)ntiles * 32 * 128), B((size_t)ntiles * 128 * 32);
    for (int t = 0; t < ntiles; ++t) {
        std::vector<double> common(128), ra(32 * 128), rb(32 * 128);
        for (auto& c : common) c = n01(g);
        double ma = 0, mb = 0;
        for (int i = 0; i < 32 * 128; ++i) {
            const double base = mode == 1 ? common[i % 128] : 0.0;
            ra[i] = base + n01(g);
            rb[i] = base + n01(g);
            ma = fmax(ma, fabs(ra[i]));
            mb = fmax(mb, fabs(rb[i]));
        }
        for (int r = 0; r < 32; ++r)
            for (int k = 0; k < 128; ++k) {
                uint8_t ca, cb;
                if (mode == 2) {
                    ca = (uint8_t)(g() & 0xff);
                    cb = (uint8_t)(g() & 0xff);
                    if ((ca & 0x7f) == 0x7f) ca = 0;
                    if ((cb & 0x7f) == 0x7f) cb = 0;
                } else {
                    ca = e4m3_code(ra[r * 128 + k] / ma * 448);
                    cb = e4m3_code(rb[r * 128 + k] / mb * 448);
                }
                A[((size_t)t * 32 + r) * 128 + k] = ca;
                B[((size_t)t * 128 + k) * 32 + r] = cb;
            }
    }
    std::vector<i32x8> pa((size_t)ntiles * 128), pb((size_t)ntiles * 128);
    for (int t = 0; t < ntiles; ++t)
        for (int ks = 0; ks < 2; ++ks)
            for (int l = 0; l < 64; ++l) {
                uint8_t ba[32], bb[32];
                for (int b = 0; b < 32; ++b) {
                    const int k = 64 * ks + 32 * (l / 32) + b;
                    ba[b] = A[((size_t)t * 32 + l % 32) * 128 + k];
                    bb[b] = B[((size_t)t * 128 + k) * 32 + l % 32];
                }
                memcpy(&pa[((size_t)t * 2 + ks) * 64 + l], ba, 32);
                memcpy(&pb[((size_t)t * 2 + ks) * 64 + l], bb, 32);
            }
    i32x8 *da = nullptr, *db = nullptr;
    f32x16* dc = nullptr;
    CHECK(hipMalloc(&da, pa.size() * sizeof(i32x8)));
    CHECK(hipMalloc(&db, pb.size() * sizeof(i32x8)));
    CHECK(hipMalloc(&dc, (size_t)ntiles * 64 * sizeof(f32x16)));
    CHECK(hipMemcpy(da, pa.data(), pa.size() * sizeof(i32x8), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, pb.data(), pb.size() * sizeof(i32x8), hipMemcpyHostToDevice));
    dot_tiles<<<ntiles, 64>>>(da, db, dc, ntiles);
    CHECK(hipGetLastError());
    std::vector<f32x16> C((size_t)ntiles * 64);
    CHECK(hipMemcpy(C.data(), dc, C.size() * sizeof(f32x16), hipMemcpyDeviceToHost));
    double worst = 0, mean = 0;
    long n = 0, exact = 0;
    for (int t = 0; t < ntiles; ++t)
        for (int l = 0; l < 64; ++l)
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r / 4) + 4 * (l / 32) + r % 4, col = l % 32;
                double s = 0, sa = 0;
                for (int k = 0; k < 128; ++k) {
                    const double p = e4m3_value(A[((size_t)t * 32 + row) * 128 + k]) *
                                     e4m3_value(B[((size_t)t * 128 + k) * 32 + col]);
                    s += p;
                    sa += fabs(p);
                }
                const double d = fabs((double)C[(size_t)t * 64 + l][r] - s);
                exact += d == 0;
                if (sa > 0) {
                    worst = fmax(worst, d / sa);
                    mean += d / sa;
                }
                ++n;
            }
    printf("mode %d: %ld dot products, exact %.4f, max |err|/sum|ab| %.3e (2^%.2f), mean %.3e\n",
           mode, n, (double)exact / n, worst, log2(worst), mean / n);
    CHECK(hipFree(da));
    CHECK(hipFree(db));
    CHECK(hipFree(dc));
    return 0;
}
