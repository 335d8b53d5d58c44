// fused3d_bf16.hip - placeholder until the bf16 matrix-core kernel lands.
#include "ct_internal.h"

namespace ct {

hipError_t launch_fused3d_bf16(const uint16_t *, const uint16_t *, const float *, const float *,
                               float, float, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                               float *, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace ct
