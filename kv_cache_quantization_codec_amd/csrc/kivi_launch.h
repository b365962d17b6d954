// Internal interface between the host-side entry points (kivi_api.cpp, plain
// C++) and the HIP launchers (kivi_kernels.hip).  Arguments arrive here
// already validated; every launcher returns a hipError_t value as int
// (0 = success) and enqueues work on `stream` only.
#pragma once

#include <stdint.h>

namespace kivi {

struct EncodeArgs {
    const uint16_t* in;      // fp16 [n_slices][in_stride]
    int64_t in_stride;       // elements between slices
    int64_t n_slices;
    int32_t n_tokens;        // tokens (keys) or rows (values) to quantize per slice
    int32_t cap_tokens;      // capacity that sets the output slice strides
    int32_t head_dim;
    int32_t group_size;
    int32_t bits;
    uint32_t* codes;
    uint16_t* scale;
    uint16_t* zero;
};

struct DecodeArgs {
    const uint32_t* codes;
    const uint16_t* scale;
    const uint16_t* zero;
    int64_t n_slices;
    int32_t n_tokens;
    int32_t cap_tokens;
    int32_t head_dim;
    int32_t group_size;
    int32_t bits;
    uint16_t* out;           // fp16 [n_slices][out_stride]
    int64_t out_stride;
};

struct StepArgs {
    const uint16_t* k_new;   // fp16 [n_slices][D]
    const uint16_t* v_new;
    uint16_t* k_ring;        // fp16 [n_slices][ring_slots][D]
    uint16_t* v_ring;
    uint32_t* k_codes;
    uint16_t* k_scale;
    uint16_t* k_zero;
    uint32_t* v_codes;
    uint16_t* v_scale;
    uint16_t* v_zero;
    int64_t n_slices;
    int32_t cap_tokens;
    int32_t head_dim;
    int32_t group_size;
    int32_t k_bits;
    int32_t v_bits;
    int32_t ring_slots;      // R + G
    int32_t ring_head;       // slot of the oldest residual token before the step
    int32_t ring_count;      // residual tokens before the step
    int32_t flush;           // 1: quantize the oldest G residual tokens
    int32_t n_quant;         // tokens quantized before the step (group index * G)
};

struct RingFillArgs {
    const uint16_t* k_in;    // fp16 [n_slices][in_stride]
    const uint16_t* v_in;
    int64_t in_stride;
    int64_t n_slices;
    int32_t first_token;     // token of the input that becomes ring slot 0
    int32_t n_tokens;        // tokens copied (slots 0 .. n_tokens-1)
    int32_t head_dim;
    int32_t ring_slots;
    uint16_t* k_ring;
    uint16_t* v_ring;
};

int launch_encode_k(const EncodeArgs& a, void* stream);
int launch_encode_v(const EncodeArgs& a, void* stream);
int launch_decode_k(const DecodeArgs& a, void* stream);
int launch_decode_v(const DecodeArgs& a, void* stream);
int launch_append_flush(const StepArgs& a, void* stream);
int launch_ring_fill(const RingFillArgs& a, void* stream);

}  // namespace kivi
