// Matrix-core fused decode attention over the Delta-KV cache (gfx950).
#include "dkv_common.h"

namespace dkv {

bool fused_supported(const dkv_config &) { return false; }

hipError_t launch_attn_fused(const dkv_config &, const void *, const int32_t *, const float *, const int32_t *,
                             float, float *, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace dkv
