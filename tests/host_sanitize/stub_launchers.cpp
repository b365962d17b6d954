// Launchers that enqueue nothing, for building libkivi's host-side entry
// points (kivi_api.cpp) on the CPU with address and undefined-behaviour
// sanitizers.  Every stub reports success and touches no memory, so an
// argument set that passes validation ends here instead of in a kernel.
// Test infrastructure only: the product library is built from the HIP
// launchers.
#include "../../kv_cache_quantization_codec_amd/csrc/kivi_launch.h"

namespace kivi {

int launch_encode_k(const EncodeArgs&, void*) { return 0; }
int launch_encode_v(const EncodeArgs&, void*) { return 0; }
int launch_decode_k(const DecodeArgs&, void*) { return 0; }
int launch_decode_v(const DecodeArgs&, void*) { return 0; }
int launch_append_flush(const StepArgs&, void*) { return 0; }
int launch_ring_fill(const RingFillArgs&, void*) { return 0; }
int launch_attention(const AttnArgs&, void*) { return 0; }
int launch_fp8_encode(const Fp8Args&, void*) { return 0; }
int launch_fp8_decode(const Fp8Args&, void*) { return 0; }
int launch_copy_2d(void*, size_t, const void*, size_t, size_t, size_t, void*) { return 0; }

int attention_scratch(void*, void** ptr) {
    static float stand_in[4];       // never dereferenced: the attention stub launches nothing
    *ptr = stand_in;
    return 0;
}

}  // namespace kivi
