// int4 layout repacks (placeholder until the tiled kernels land).
#include "qbn_launch.h"
namespace qbn {
hipError_t launch_repack(const qbn_tensor &, int, int, void *, void *, void *, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace qbn
