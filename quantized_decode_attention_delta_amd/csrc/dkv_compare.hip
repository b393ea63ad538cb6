// In-run comparison caches: plain Q4_0 of absolute values and F16.
#include "dkv_common.h"

namespace dkv {

hipError_t launch_q40_encode(const dkv_config &, void *, const uint16_t *, const uint16_t *, const int32_t *, int,
                             hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_q40_export(const dkv_config &, const void *, const int32_t *, int, uint8_t *, uint16_t *,
                             hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_attn_q40(const dkv_config &, const void *, const float *, const int32_t *, float, float *, int,
                           int, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_attn_f16(const dkv_config &, const uint16_t *, const uint16_t *, int, const float *,
                           const int32_t *, float, float *, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace dkv
