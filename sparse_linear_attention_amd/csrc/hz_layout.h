// Order of the d x d part of a linear-branch summaries row (d = 128): shared
// by the block-summaries pass that writes it, the product that sums such
// rows and the fused kernel that reads the sums.
#pragma once

#include <hip/hip_runtime.h>

namespace sla2 {

// The h_j^T part of a summaries row (and the H_i^T part of a product row)
// is stored in the order in which the block-summaries pass's matrix
// accumulators hold it, so that every store there is a contiguous 1 KB: the
// 16-byte unit of entries (e, 8 u .. 8 u + 7) (V channel e, phi channels c =
// 8 u ..) is unit ((e / 32 * 4 + u / 4) * 2 + (u / 2) % 2) * 64 + e % 32 +
// 32 (u % 2) of the row.  The product is indifferent to the column order;
// the fused kernel fetches each unit from here.
__host__ __device__ inline int hz_unit(int e, int u) {
    return (((e >> 5) * 4 + (u >> 2)) * 2 + ((u >> 1) & 1)) * 64 + (e & 31) + 32 * (u & 1);
}

}  // namespace sla2
