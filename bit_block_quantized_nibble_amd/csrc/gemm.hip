// MXFP4 GEMM (placeholder until the MFMA kernel lands).
#include "qbn_launch.h"
namespace qbn {
hipError_t launch_gemm(const qbn_tensor &, int64_t, const void *, int64_t, void *, int64_t, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace qbn
