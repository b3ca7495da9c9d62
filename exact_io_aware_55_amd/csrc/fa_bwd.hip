// Backward pass placeholder (replaced by the recomputation kernels).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const void*,
                           const float*, void*, void*, void*, int, int, int, int, float, bool,
                           float*, float*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace fa
