// kd_bwd.hip -- gate-aware chunkwise backward (placeholder until the kernel lands).
#include "kd_device.h"

namespace kd {

size_t bwd_workspace_bytes(int bf16, int d, int B, int T, int H) {
    (void)bf16;
    const size_t nc = (size_t)(T + CH - 1) / CH;
    return (size_t)B * H * nc * d * d * sizeof(float);
}

hipError_t launch_bwd(int, int, const void*, const void*, const void*, const void*, const float*,
                      const float*, const float*, const void*, const float*, void*, void*, void*,
                      void*, float*, float*, float*, void*, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace kd
