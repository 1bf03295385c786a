// bf16 grouped expert GEMMs (placeholder until the MFMA bf16 kernels land).
#include "moe_internal.hpp"

namespace moe {

hipError_t launch_fwd_gemm_bf16(const uint16_t*, const uint16_t*, const float*, uint16_t*, const int32_t*,
                                const int32_t*, int64_t, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_dx_gemm_bf16(const uint16_t*, const uint16_t*, uint16_t*, int, const int32_t*, const int32_t*,
                               int64_t, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_dw_gemm_bf16(const uint16_t*, const uint16_t*, float*, float*, const int32_t*, const int32_t*,
                               int, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
