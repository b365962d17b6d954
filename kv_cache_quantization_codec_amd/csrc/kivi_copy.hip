// Host <-> device copies of the compact cache image (the payload that
// CacheSeek PR #4 "Feature(quantization): add KIVI KV-cache quantization for
// exact-prefix reuse" moves between devices and host storage).  Only the
// HIP runtime's asynchronous 2-D copy is used: one call per array packs or
// unpacks the slices' used prefix against the device arrays' capacity
// pitch, so the image carries no padding.

#include <hip/hip_runtime.h>

#include "kivi_launch.h"

namespace kivi {

int launch_copy_2d(void* dst, size_t dst_pitch, const void* src, size_t src_pitch, size_t width,
                   size_t height, void* stream) {
    if (width == 0 || height == 0) return 0;
    return (int)hipMemcpy2DAsync(dst, dst_pitch, src, src_pitch, width, height, hipMemcpyDefault,
                                 static_cast<hipStream_t>(stream));
}

}  // namespace kivi
