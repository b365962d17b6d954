// Internal interface between the host-side entry points (kivi_api.cpp, plain
// C++) and the HIP launchers (kivi_kernels.hip).  Arguments arrive here
// already validated; every launcher returns a hipError_t value as int
// (0 = success) and enqueues work on `stream` only.
#pragma once

#include <stddef.h>
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

// Work split of decode attention, shared by the workspace-size query and the
// launcher.  The quantized prefix is walked in blocks of 32 tokens; each
// slice gets n_qsplit workgroups over consecutive block ranges, plus one
// workgroup for the fp16 residual when there is one.  With a single split
// the attention kernel normalises and writes the output itself; otherwise
// it writes partial softmax sums and a second kernel merges them.
struct AttnPlan {
    int32_t n_blocks;          // 32-token blocks of the quantized prefix
    int32_t blocks_per_split;
    int32_t n_qsplit;          // workgroups per slice over the quantized prefix
    int32_t has_res;           // 1: one more workgroup per slice for the residual
    int32_t n_splits;          // n_qsplit + has_res
};

inline AttnPlan attn_plan(int64_t n_slices, int64_t n_quant, int64_t res_count) {
    const int64_t kTargetGroups = 32768;   // several waves of resident workgroups (short tail)
    const int64_t kMinBlocks = 4;          // keep partial-sum traffic below ~5%
    AttnPlan p{};
    p.n_blocks = (int32_t)((n_quant + 31) / 32);
    p.has_res = res_count > 0 ? 1 : 0;
    if (p.n_blocks > 0) {
        // workgroups per slice (at least 1; no overflow for any slice count)
        int64_t want = n_slices >= kTargetGroups ? 1 : n_slices > 0 ? (kTargetGroups + n_slices - 1) / n_slices : 1;
        int64_t cap = (p.n_blocks + kMinBlocks - 1) / kMinBlocks;
        if (want > cap) want = cap;
        if (want < 1) want = 1;
        p.blocks_per_split = (int32_t)((p.n_blocks + want - 1) / want);
        p.n_qsplit = (p.n_blocks + p.blocks_per_split - 1) / p.blocks_per_split;
    }
    p.n_splits = p.n_qsplit + p.has_res;
    return p;
}

struct AttnArgs {
    const uint32_t* k_codes;  // key layouts for cap_tokens tokens per slice
    const uint16_t* k_scale;
    const uint16_t* k_zero;
    const uint32_t* v_codes;  // value layouts for cap_tokens rows per slice
    const uint16_t* v_scale;
    const uint16_t* v_zero;
    const uint16_t* res_k;    // fp16 residual rings
    const uint16_t* res_v;
    const int32_t* n_quant_s; // per-slice counts (ragged batch) or nullptr
    const int32_t* res_count_s;
    const uint16_t* q;        // fp16 [n_slices][q_per_kv][D]
    uint16_t* out;            // fp16 [n_slices][q_per_kv][D]
    float* ws_ml;             // [n_slices][n_splits][q_per_kv][2] (max, sum), when split
    float* ws_o;              // [n_slices][n_splits][q_per_kv][D] unnormalised outputs
    int64_t n_slices;
    int64_t res_stride;       // elements between slices of res_k / res_v
    int32_t cap_tokens;
    int32_t n_quant;
    int32_t res_slots;
    int32_t res_head;
    int32_t res_count;
    int32_t head_dim;         // multiple of 32, <= 128
    int32_t group_size;
    int32_t k_bits;
    int32_t v_bits;
    int32_t q_per_kv;         // 1 .. 8
    float logit_scale;        // sm_scale * log2(e)
    AttnPlan plan;
};

// FP8 key cast: in/out element strides between slices (fp16 elements or
// code bytes); token rows of head_dim elements.
struct Fp8Args {
    const void* in;
    int64_t in_stride;
    void* out;
    int64_t out_stride;
    int64_t n_slices;
    int32_t n_tokens;
    int32_t head_dim;
};

int launch_encode_k(const EncodeArgs& a, void* stream);
int launch_encode_v(const EncodeArgs& a, void* stream);
int launch_decode_k(const DecodeArgs& a, void* stream);
int launch_decode_v(const DecodeArgs& a, void* stream);
int launch_append_flush(const StepArgs& a, void* stream);
int launch_ring_fill(const RingFillArgs& a, void* stream);
int launch_attention(const AttnArgs& a, void* stream);
// Device address of the static attention scratch (KIVI_ATTENTION_SCRATCH_BYTES
// bytes) on the device that `stream` belongs to (the current device for a
// null stream), looked up once per device; returns a hipError_t value.
int attention_scratch(void* stream, void** ptr);
int launch_fp8_encode(const Fp8Args& a, void* stream);
int launch_fp8_decode(const Fp8Args& a, void* stream);
// height rows of width bytes, between any mix of host and device memory
int launch_copy_2d(void* dst, size_t dst_pitch, const void* src, size_t src_pitch, size_t width,
                   size_t height, void* stream);

}  // namespace kivi
