// Low-bit sparse branch (placeholder until the fp8 kernels land).
#include "sla2_internal.h"

namespace sla2 {

hipError_t launch_quantize_fp8(const Dims&, const void*, const void*, const FwdWS&, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_fused_fp8(const Dims&, const void*, const int32_t*, const float*, float*,
                            const FwdWS&, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace sla2
