// Host-side entry points of libkivi: argument validation, sizing and the
// streaming counters.  Plain C++ with no HIP header, so every check here runs
// (and is tested) without a GPU; work is handed to the launchers declared in
// kivi_launch.h only after all checks passed.
//
// Sizes follow the layouts of include/kivi.h (CacheSeek PR #4 "Feature
// (quantization): add KIVI KV-cache quantization for exact-prefix reuse":
// int32-packed codes plus scale/offset sidecars, sized by the manager).

#include "../../include/kivi.h"
#include "kivi_launch.h"

#include <stdint.h>

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxTokens = (int64_t(1) << 30);   // per slice, fits int32 math in kernels
// ring slots (R + G) of a stream: the key flush addresses the rings of up to
// 2*256/D slices of one block with 32-bit byte offsets (1 KB per slot)
constexpr int64_t kMaxRingSlots = (int64_t(1) << 21);

bool valid_bits(int32_t b) { return b == 2 || b == 4 || b == 8; }
bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

int check_config(const kivi_config* c) {
    if (!c) return KIVI_E_NULL;
    if (!valid_bits(c->k_bits) || !valid_bits(c->v_bits)) return KIVI_E_BITS;
    if (!valid_group(c->group_size)) return KIVI_E_GROUP;
    if (c->head_dim < 8 || c->head_dim > 256 || c->head_dim % 8 != 0) return KIVI_E_HEAD_DIM;
    if (c->residual_length < 0) return KIVI_E_RESIDUAL;
    return KIVI_OK;
}

// per-slice sizes; n >= 0 and a valid config assumed
int64_t k_words(const kivi_config* c, int64_t n) {
    return ceil_div(n, c->group_size) * (c->group_size * c->k_bits / 32) * c->head_dim;
}
int64_t k_stats(const kivi_config* c, int64_t n) { return ceil_div(n, c->group_size) * c->head_dim; }
int64_t v_groups(const kivi_config* c) { return ceil_div(c->head_dim, c->group_size); }
int64_t v_words(const kivi_config* c, int64_t n) {
    return n * v_groups(c) * (c->group_size * c->v_bits / 32);
}
int64_t v_stats(const kivi_config* c, int64_t n) { return n * v_groups(c); }

int record(int hip_err) {
    if (hip_err != 0) {
        g_last_hip_error = hip_err;
        return KIVI_E_HIP;
    }
    return KIVI_OK;
}

// Checks shared by encode and decode: counts, strides and the total size of
// every array addressed (so that no index overflows int64).
int check_common(const kivi_config* c, int64_t n_slices, int64_t n_tokens, int64_t cap_tokens,
                 int64_t fp16_stride, bool keys) {
    if (n_slices < 0 || n_tokens < 0 || cap_tokens < n_tokens) return KIVI_E_SHAPE;
    if (n_tokens > kMaxTokens || cap_tokens > kMaxTokens) return KIVI_E_SHAPE;
    if (fp16_stride % 8 != 0) return KIVI_E_ALIGN;
    int64_t need = 0;
    if (!mul_ok(n_tokens, c->head_dim, &need) || fp16_stride < need) return KIVI_E_SHAPE;
    int64_t total = 0;
    if (!mul_ok(n_slices, fp16_stride, &total) || !mul_ok(total, 2, &total)) return KIVI_E_SHAPE;
    const int64_t words = keys ? k_words(c, cap_tokens) : v_words(c, cap_tokens);
    if (!mul_ok(n_slices, words, &total) || !mul_ok(total, 4, &total)) return KIVI_E_SHAPE;
    return KIVI_OK;
}

int encode(bool keys, const kivi_config* cfg, const void* in, int64_t n_slices, int64_t n_tokens,
           int64_t in_stride, int64_t cap_tokens, int32_t* codes, void* scale, void* zero,
           void* stream) {
    int st = check_config(cfg);
    if (st) return st;
    if (n_slices == 0 || n_tokens == 0) {
        if (n_slices < 0 || n_tokens < 0) return KIVI_E_SHAPE;
        return KIVI_OK;
    }
    st = check_common(cfg, n_slices, n_tokens, cap_tokens, in_stride, keys);
    if (st) return st;
    if (!in || !codes || !scale || !zero) return KIVI_E_NULL;
    if (!aligned16(in) || !aligned16(codes) || !aligned16(scale) || !aligned16(zero)) return KIVI_E_ALIGN;
    kivi::EncodeArgs a;
    a.in = static_cast<const uint16_t*>(in);
    a.in_stride = in_stride;
    a.n_slices = n_slices;
    a.n_tokens = static_cast<int32_t>(n_tokens);
    a.cap_tokens = static_cast<int32_t>(cap_tokens);
    a.head_dim = cfg->head_dim;
    a.group_size = cfg->group_size;
    a.bits = keys ? cfg->k_bits : cfg->v_bits;
    a.codes = reinterpret_cast<uint32_t*>(codes);
    a.scale = static_cast<uint16_t*>(scale);
    a.zero = static_cast<uint16_t*>(zero);
    return record(keys ? kivi::launch_encode_k(a, stream) : kivi::launch_encode_v(a, stream));
}

int decode(bool keys, const kivi_config* cfg, const int32_t* codes, const void* scale, const void* zero,
           int64_t n_slices, int64_t n_tokens, int64_t cap_tokens, void* out, int64_t out_stride,
           void* stream) {
    int st = check_config(cfg);
    if (st) return st;
    if (n_slices == 0 || n_tokens == 0) {
        if (n_slices < 0 || n_tokens < 0) return KIVI_E_SHAPE;
        return KIVI_OK;
    }
    st = check_common(cfg, n_slices, n_tokens, cap_tokens, out_stride, keys);
    if (st) return st;
    if (!codes || !scale || !zero || !out) return KIVI_E_NULL;
    if (!aligned16(codes) || !aligned16(scale) || !aligned16(zero) || !aligned16(out)) return KIVI_E_ALIGN;
    kivi::DecodeArgs a;
    a.codes = reinterpret_cast<const uint32_t*>(codes);
    a.scale = static_cast<const uint16_t*>(scale);
    a.zero = static_cast<const uint16_t*>(zero);
    a.n_slices = n_slices;
    a.n_tokens = static_cast<int32_t>(n_tokens);
    a.cap_tokens = static_cast<int32_t>(cap_tokens);
    a.head_dim = cfg->head_dim;
    a.group_size = cfg->group_size;
    a.bits = keys ? cfg->k_bits : cfg->v_bits;
    a.out = static_cast<uint16_t*>(out);
    a.out_stride = out_stride;
    return record(keys ? kivi::launch_decode_k(a, stream) : kivi::launch_decode_v(a, stream));
}

// Pointers, capacity and counters of a stream (counters are checked only when
// `counters` is set: the prefill overwrites them).
int check_stream(const kivi_config* c, const kivi_stream* s, bool counters) {
    if (!s) return KIVI_E_NULL;
    if (s->n_slices < 0) return KIVI_E_SHAPE;
    const int64_t G = c->group_size;
    const int64_t slots = int64_t(c->residual_length) + G;
    if (s->cap_tokens < 0 || s->cap_tokens > kMaxTokens || s->cap_tokens % G != 0) return KIVI_E_STATE;
    if (slots > kMaxRingSlots) return KIVI_E_SHAPE;
    if (counters) {
        if (s->n_quant < 0 || s->n_quant % G != 0 || s->n_quant > s->cap_tokens) return KIVI_E_STATE;
        if (s->ring_head < 0 || s->ring_head >= slots) return KIVI_E_STATE;
        if (s->ring_count < 0 || s->ring_count > slots - 1) return KIVI_E_STATE;
    }
    if (s->n_slices == 0) return KIVI_OK;
    int64_t total = 0;
    if (!mul_ok(s->n_slices, slots * c->head_dim, &total)) return KIVI_E_SHAPE;
    if (!mul_ok(s->n_slices, k_words(c, s->cap_tokens) + v_words(c, s->cap_tokens), &total) ||
        !mul_ok(total, 4, &total))
        return KIVI_E_SHAPE;
    if (!s->k_codes || !s->v_codes || !s->k_scale || !s->k_zero || !s->v_scale || !s->v_zero ||
        !s->k_ring || !s->v_ring)
        return KIVI_E_NULL;
    if (!aligned16(s->k_codes) || !aligned16(s->v_codes) || !aligned16(s->k_scale) ||
        !aligned16(s->k_zero) || !aligned16(s->v_scale) || !aligned16(s->v_zero) ||
        !aligned16(s->k_ring) || !aligned16(s->v_ring))
        return KIVI_E_ALIGN;
    return KIVI_OK;
}

bool flush_due(int64_t count, int64_t residual, int64_t group) {
    return count > residual && count >= group;
}

// The compact image of a streaming cache: eight arrays, each with the
// used prefix of every slice packed back to back.  `dev_pitch` is a slice's
// size in the device arrays (capacity cap), `width` the bytes of n_quant
// tokens per slice; rings are copied whole (height 1).
struct ImagePart {
    int64_t width;
    int64_t dev_pitch;
    int64_t height;
};

bool image_parts(const kivi_config* c, int64_t n_slices, int64_t n_quant, int64_t cap,
                 ImagePart parts[8], int64_t* total) {
    const int64_t ring = (int64_t(c->residual_length) + c->group_size) * c->head_dim * 2;
    const int64_t kcw = k_words(c, n_quant) * 4, kcp = k_words(c, cap) * 4;
    const int64_t ksw = k_stats(c, n_quant) * 2, ksp = k_stats(c, cap) * 2;
    const int64_t vcw = v_words(c, n_quant) * 4, vcp = v_words(c, cap) * 4;
    const int64_t vsw = v_stats(c, n_quant) * 2, vsp = v_stats(c, cap) * 2;
    int64_t ring_all = 0;
    if (!mul_ok(n_slices, ring, &ring_all)) return false;
    const ImagePart p[8] = {{kcw, kcp, n_slices}, {ksw, ksp, n_slices}, {ksw, ksp, n_slices},
                            {vcw, vcp, n_slices}, {vsw, vsp, n_slices}, {vsw, vsp, n_slices},
                            {ring_all, ring_all, 1},  {ring_all, ring_all, 1}};
    int64_t sum = 0;
    for (int i = 0; i < 8; ++i) {
        int64_t bytes = 0;
        if (!mul_ok(p[i].width, p[i].height, &bytes) || __builtin_add_overflow(sum, bytes, &sum))
            return false;
        parts[i] = p[i];
    }
    *total = sum;
    return true;
}

// Decode attention: configuration limits of the attention kernels and the
// workspace they need (partial softmax sums when a slice is split).
int check_attention_config(const kivi_config* c, int32_t q_per_kv) {
    int s = check_config(c);
    if (s) return s;
    if (c->head_dim % 32 != 0 || c->head_dim > 128) return KIVI_E_HEAD_DIM;
    if (q_per_kv < 1 || q_per_kv > 8) return KIVI_E_SHAPE;
    return KIVI_OK;
}

// Bytes of workspace for a plan, or -1 on overflow.
int64_t attention_ws_bytes(const kivi_config* c, int64_t n_slices, int32_t q_per_kv,
                           const kivi::AttnPlan& p) {
    if (p.n_splits <= 1) return 0;
    int64_t per = 0, total = 0;
    if (!mul_ok(n_slices, (int64_t)p.n_splits * q_per_kv, &per)) return -1;
    if (!mul_ok(per, (int64_t)(c->head_dim + 2) * 4, &total)) return -1;
    return total;
}

// Decode attention, with the caller's workspace or (static_scratch) the
// library's per-device static buffer for the split partials.  Every check
// runs before the first HIP call; the static buffer's address is looked up
// only when the call needs it.
int attention_call(const kivi_config* cfg, const kivi_attn_cache* cache, int64_t n_slices,
                   int32_t q_per_kv, const void* q, float sm_scale, void* out, void* workspace,
                   int64_t workspace_bytes, bool static_scratch, void* stream) {
    int s = check_attention_config(cfg, q_per_kv);
    if (s) return s;
    if (!cache) return KIVI_E_NULL;
    const kivi_attn_cache& c = *cache;
    const int64_t D = cfg->head_dim;
    if (n_slices < 0) return KIVI_E_SHAPE;
    if (c.cap_tokens < 0 || c.cap_tokens > kMaxTokens || c.n_quant < 0 || c.n_quant > c.cap_tokens)
        return KIVI_E_SHAPE;
    if (c.res_count < 0 || c.res_slots < c.res_count || c.res_slots > kMaxTokens) return KIVI_E_SHAPE;
    if (c.res_count > 0 && (c.res_head < 0 || c.res_head >= c.res_slots)) return KIVI_E_SHAPE;
    if (!__builtin_isfinite(sm_scale)) return KIVI_E_SHAPE;
    if (n_slices == 0) return KIVI_OK;
    if (c.n_quant + c.res_count < 1) return KIVI_E_SHAPE;
    if ((c.n_quant_per_slice && (reinterpret_cast<uintptr_t>(c.n_quant_per_slice) & 3u)) ||
        (c.res_count_per_slice && (reinterpret_cast<uintptr_t>(c.res_count_per_slice) & 3u)))
        return KIVI_E_ALIGN;
    const kivi::AttnPlan plan = kivi::attn_plan(n_slices, c.n_quant, c.res_count);
    int64_t groups = 0;
    if (!mul_ok(n_slices, plan.n_splits, &groups) || groups > INT32_MAX) return KIVI_E_SHAPE;
    int64_t tmp = 0;
    if (!mul_ok(n_slices, (int64_t)q_per_kv * D * 2, &tmp)) return KIVI_E_SHAPE;
    if (c.n_quant > 0) {
        if (!mul_ok(n_slices, k_words(cfg, c.cap_tokens) * 4, &tmp) ||
            !mul_ok(n_slices, v_words(cfg, c.cap_tokens) * 4, &tmp))
            return KIVI_E_SHAPE;
    }
    if (c.res_count > 0) {
        if (c.res_slice_stride % 8 != 0) return KIVI_E_ALIGN;
        if (!mul_ok(c.res_slots, D, &tmp) || c.res_slice_stride < tmp) return KIVI_E_SHAPE;
        if (!mul_ok(n_slices, c.res_slice_stride, &tmp)) return KIVI_E_SHAPE;
    }
    const int64_t need = attention_ws_bytes(cfg, n_slices, q_per_kv, plan);
    if (need < 0) return KIVI_E_SHAPE;
    if (static_scratch) {
        if (need > KIVI_ATTENTION_SCRATCH_BYTES) return KIVI_E_SCRATCH;
    } else if (workspace_bytes < need) {
        return KIVI_E_SHAPE;
    }
    if (!q || !out) return KIVI_E_NULL;
    if (c.n_quant > 0 && (!c.k_codes || !c.k_scale || !c.k_zero || !c.v_codes || !c.v_scale || !c.v_zero))
        return KIVI_E_NULL;
    if (c.res_count > 0 && (!c.res_k || !c.res_v)) return KIVI_E_NULL;
    if (!static_scratch && need > 0 && !workspace) return KIVI_E_NULL;
    if (!aligned16(q) || !aligned16(out) || (!static_scratch && need > 0 && !aligned16(workspace)))
        return KIVI_E_ALIGN;
    if (c.n_quant > 0 && (!aligned16(c.k_codes) || !aligned16(c.k_scale) || !aligned16(c.k_zero) ||
                          !aligned16(c.v_codes) || !aligned16(c.v_scale) || !aligned16(c.v_zero)))
        return KIVI_E_ALIGN;
    if (c.res_count > 0 && (!aligned16(c.res_k) || !aligned16(c.res_v))) return KIVI_E_ALIGN;
    if (static_scratch && need > 0) {
        // all checks passed: the first HIP call (the buffer of the stream's device)
        s = record(kivi::attention_scratch(stream, &workspace));
        if (s) return s;
    }

    kivi::AttnArgs a;
    a.k_codes = reinterpret_cast<const uint32_t*>(c.k_codes);
    a.k_scale = static_cast<const uint16_t*>(c.k_scale);
    a.k_zero = static_cast<const uint16_t*>(c.k_zero);
    a.v_codes = reinterpret_cast<const uint32_t*>(c.v_codes);
    a.v_scale = static_cast<const uint16_t*>(c.v_scale);
    a.v_zero = static_cast<const uint16_t*>(c.v_zero);
    a.res_k = static_cast<const uint16_t*>(c.res_k);
    a.res_v = static_cast<const uint16_t*>(c.res_v);
    a.n_quant_s = c.n_quant > 0 ? c.n_quant_per_slice : nullptr;
    a.res_count_s = c.res_count > 0 ? c.res_count_per_slice : nullptr;
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    a.ws_ml = need > 0 ? static_cast<float*>(workspace) : nullptr;
    a.ws_o = need > 0 ? static_cast<float*>(workspace) + n_slices * plan.n_splits * q_per_kv * 2 : nullptr;
    a.n_slices = n_slices;
    a.res_stride = c.res_slice_stride;
    a.cap_tokens = static_cast<int32_t>(c.cap_tokens);
    a.n_quant = static_cast<int32_t>(c.n_quant);
    a.res_slots = static_cast<int32_t>(c.res_slots);
    a.res_head = static_cast<int32_t>(c.res_count > 0 ? c.res_head : 0);
    a.res_count = static_cast<int32_t>(c.res_count);
    a.head_dim = cfg->head_dim;
    a.group_size = cfg->group_size;
    a.k_bits = cfg->k_bits;
    a.v_bits = cfg->v_bits;
    a.q_per_kv = q_per_kv;
    a.logit_scale = sm_scale * 1.4426950408889634f;
    a.plan = plan;
    return record(kivi::launch_attention(a, stream));
}

// ---- layer-wise coding of a model with per-layer configurations ----

uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }

// A host array of device pointers of any pointee type, read as void pointers.
const void* const* cv(const void* p) { return static_cast<const void* const*>(p); }

// Layers a and b can share one launch on this side of the codec.
bool same_side(const kivi_config& a, const kivi_config& b, bool keys) {
    return a.group_size == b.group_size && a.head_dim == b.head_dim &&
           (keys ? a.k_bits == b.k_bits : a.v_bits == b.v_bits);
}

// Bytes of one layer's codes and of one of its sidecars.
void layer_bytes(const kivi_config& c, bool keys, int64_t n_slices, int64_t cap, int64_t* code_b,
                 int64_t* stat_b) {
    *code_b = 4 * n_slices * (keys ? k_words(&c, cap) : v_words(&c, cap));
    *stat_b = 2 * n_slices * (keys ? k_stats(&c, cap) : v_stats(&c, cap));
}

// Checks every layer, then calls run(first, count) once per run of layers
// that one launch can code (same side configuration, fp16 layers and
// payload arrays back to back).  run is the single-layer entry point over
// count*n_slices slices.
template <class Run>
int coded_layers(bool keys, const kivi_config* cfgs, int64_t n_layers, const void* fp16,
                 int64_t layer_stride, int64_t n_slices, int64_t n_tokens, int64_t slice_stride,
                 int64_t cap, const void* const* codes, const void* const* scale,
                 const void* const* zero, Run run) {
    if (n_layers < 0) return KIVI_E_SHAPE;
    if (n_layers == 0) return KIVI_OK;
    if (!cfgs) return KIVI_E_NULL;
    for (int64_t l = 0; l < n_layers; ++l) {
        const int st = check_config(&cfgs[l]);
        if (st) return st;
        if (cfgs[l].head_dim != cfgs[0].head_dim) return KIVI_E_HEAD_DIM;
    }
    if (n_slices == 0 || n_tokens == 0) return (n_slices < 0 || n_tokens < 0) ? KIVI_E_SHAPE : KIVI_OK;
    for (int64_t l = 0; l < n_layers; ++l) {
        const int st = check_common(&cfgs[l], n_slices, n_tokens, cap, slice_stride, keys);
        if (st) return st;
    }
    int64_t layer_min = 0, span = 0;
    if (layer_stride % 8 != 0) return KIVI_E_ALIGN;
    if (!mul_ok(n_slices, slice_stride, &layer_min) || layer_stride < layer_min) return KIVI_E_SHAPE;
    if (!mul_ok(n_layers - 1, layer_stride, &span) || __builtin_add_overflow(span, layer_min, &span) ||
        !mul_ok(span, 2, &span))
        return KIVI_E_SHAPE;
    if (!fp16 || !codes || !scale || !zero) return KIVI_E_NULL;
    if (!aligned16(fp16)) return KIVI_E_ALIGN;
    for (int64_t l = 0; l < n_layers; ++l)
        if (!codes[l] || !scale[l] || !zero[l]) return KIVI_E_NULL;
    // end of the run that starts at layer a
    const bool fp16_packed = layer_stride == layer_min;
    auto run_end = [&](int64_t a) {
        int64_t b = a + 1, code_b = 0, stat_b = 0;
        layer_bytes(cfgs[a], keys, n_slices, cap, &code_b, &stat_b);
        while (b < n_layers && fp16_packed && same_side(cfgs[b], cfgs[a], keys) &&
               addr(codes[b]) == addr(codes[b - 1]) + code_b &&
               addr(scale[b]) == addr(scale[b - 1]) + stat_b &&
               addr(zero[b]) == addr(zero[b - 1]) + stat_b)
            ++b;
        return b;
    };
    // only a run's first layer needs aligned arrays: the launch addresses the
    // others from it, as slices of one array
    for (int64_t a = 0; a < n_layers; a = run_end(a))
        if (!aligned16(codes[a]) || !aligned16(scale[a]) || !aligned16(zero[a])) return KIVI_E_ALIGN;
    for (int64_t a = 0; a < n_layers;) {
        const int64_t b = run_end(a);
        const int st = run(a, b - a);
        if (st) return st;
        a = b;
    }
    return KIVI_OK;
}

}  // namespace

extern "C" {

const char* kivi_status_string(int status) {
    switch (status) {
        case KIVI_OK: return "KIVI_OK";
        case KIVI_E_NULL: return "KIVI_E_NULL: a required pointer is NULL";
        case KIVI_E_BITS: return "KIVI_E_BITS: k_bits and v_bits must be 2, 4 or 8";
        case KIVI_E_GROUP: return "KIVI_E_GROUP: group_size must be 32, 64 or 128";
        case KIVI_E_HEAD_DIM: return "KIVI_E_HEAD_DIM: head_dim must be a multiple of 8 in [8, 256]";
        case KIVI_E_RESIDUAL: return "KIVI_E_RESIDUAL: residual_length must be >= 0";
        case KIVI_E_SHAPE: return "KIVI_E_SHAPE: bad count, stride or capacity";
        case KIVI_E_ALIGN: return "KIVI_E_ALIGN: pointers must be 16-byte aligned, strides multiples of 8";
        case KIVI_E_CAPACITY: return "KIVI_E_CAPACITY: the quantized store is full";
        case KIVI_E_STATE: return "KIVI_E_STATE: inconsistent stream counters";
        case KIVI_E_HIP: return "KIVI_E_HIP: a HIP launch failed";
        case KIVI_E_SCRATCH:
            return "KIVI_E_SCRATCH: the call needs more than KIVI_ATTENTION_SCRATCH_BYTES of partial sums";
        default: return "unknown kivi status";
    }
}

int kivi_last_hip_error(void) { return g_last_hip_error; }

int kivi_validate_config(const kivi_config* cfg) { return check_config(cfg); }

int64_t kivi_k_code_words(const kivi_config* cfg, int64_t n) {
    return (check_config(cfg) || n < 0 || n > kMaxTokens) ? -1 : k_words(cfg, n);
}
int64_t kivi_k_stat_elems(const kivi_config* cfg, int64_t n) {
    return (check_config(cfg) || n < 0 || n > kMaxTokens) ? -1 : k_stats(cfg, n);
}
int64_t kivi_v_code_words(const kivi_config* cfg, int64_t n) {
    return (check_config(cfg) || n < 0 || n > kMaxTokens) ? -1 : v_words(cfg, n);
}
int64_t kivi_v_stat_elems(const kivi_config* cfg, int64_t n) {
    return (check_config(cfg) || n < 0 || n > kMaxTokens) ? -1 : v_stats(cfg, n);
}
int64_t kivi_ring_elems(const kivi_config* cfg) {
    return check_config(cfg) ? -1 : (int64_t(cfg->residual_length) + cfg->group_size) * cfg->head_dim;
}

int kivi_encode_k(const kivi_config* cfg, const void* k, int64_t n_slices, int64_t n_tokens,
                  int64_t in_stride, int64_t cap, int32_t* codes, void* scale, void* zero,
                  void* stream) {
    return encode(true, cfg, k, n_slices, n_tokens, in_stride, cap, codes, scale, zero, stream);
}

int kivi_encode_v(const kivi_config* cfg, const void* v, int64_t n_slices, int64_t n_tokens,
                  int64_t in_stride, int64_t cap, int32_t* codes, void* scale, void* zero,
                  void* stream) {
    return encode(false, cfg, v, n_slices, n_tokens, in_stride, cap, codes, scale, zero, stream);
}

int kivi_decode_k(const kivi_config* cfg, const int32_t* codes, const void* scale, const void* zero,
                  int64_t n_slices, int64_t n_tokens, int64_t cap, void* out, int64_t out_stride,
                  void* stream) {
    return decode(true, cfg, codes, scale, zero, n_slices, n_tokens, cap, out, out_stride, stream);
}

int kivi_decode_v(const kivi_config* cfg, const int32_t* codes, const void* scale, const void* zero,
                  int64_t n_slices, int64_t n_tokens, int64_t cap, void* out, int64_t out_stride,
                  void* stream) {
    return decode(false, cfg, codes, scale, zero, n_slices, n_tokens, cap, out, out_stride, stream);
}

int kivi_boundary_layers(int64_t n_layers, int64_t n, int32_t* flags) {
    if (n_layers < 0) return KIVI_E_SHAPE;
    if (n_layers == 0) return 0;
    if (!flags) return KIVI_E_NULL;
    const int64_t m = n <= 0 ? 0 : (n < n_layers / 2 ? n : n_layers / 2);
    int count = 0;
    for (int64_t l = 0; l < n_layers; ++l) {
        flags[l] = (l < m || n_layers - 1 - l < m) ? 1 : 0;
        count += flags[l];
    }
    return count;
}

int kivi_encode_k_layers(const kivi_config* cfgs, int64_t n_layers, const void* k, int64_t layer_stride,
                         int64_t n_slices, int64_t n_tokens, int64_t slice_stride, int64_t cap,
                         int32_t* const* codes, void* const* scale, void* const* zero, void* stream) {
    return coded_layers(true, cfgs, n_layers, k, layer_stride, n_slices, n_tokens, slice_stride, cap,
                        cv(codes), cv(scale), cv(zero), [&](int64_t a, int64_t count) {
                            return encode(true, &cfgs[a], static_cast<const uint16_t*>(k) + a * layer_stride,
                                          count * n_slices, n_tokens, slice_stride, cap, codes[a],
                                          scale[a], zero[a], stream);
                        });
}

int kivi_encode_v_layers(const kivi_config* cfgs, int64_t n_layers, const void* v, int64_t layer_stride,
                         int64_t n_slices, int64_t n_tokens, int64_t slice_stride, int64_t cap,
                         int32_t* const* codes, void* const* scale, void* const* zero, void* stream) {
    return coded_layers(false, cfgs, n_layers, v, layer_stride, n_slices, n_tokens, slice_stride, cap,
                        cv(codes), cv(scale), cv(zero), [&](int64_t a, int64_t count) {
                            return encode(false, &cfgs[a], static_cast<const uint16_t*>(v) + a * layer_stride,
                                          count * n_slices, n_tokens, slice_stride, cap, codes[a],
                                          scale[a], zero[a], stream);
                        });
}

int kivi_decode_k_layers(const kivi_config* cfgs, int64_t n_layers, const int32_t* const* codes,
                         const void* const* scale, const void* const* zero, int64_t n_slices,
                         int64_t n_tokens, int64_t cap, void* out, int64_t layer_stride,
                         int64_t slice_stride, void* stream) {
    return coded_layers(true, cfgs, n_layers, out, layer_stride, n_slices, n_tokens, slice_stride, cap,
                        cv(codes), scale, zero, [&](int64_t a, int64_t count) {
                            return decode(true, &cfgs[a], codes[a], scale[a], zero[a], count * n_slices,
                                          n_tokens, cap, static_cast<uint16_t*>(out) + a * layer_stride,
                                          slice_stride, stream);
                        });
}

int kivi_decode_v_layers(const kivi_config* cfgs, int64_t n_layers, const int32_t* const* codes,
                         const void* const* scale, const void* const* zero, int64_t n_slices,
                         int64_t n_tokens, int64_t cap, void* out, int64_t layer_stride,
                         int64_t slice_stride, void* stream) {
    return coded_layers(false, cfgs, n_layers, out, layer_stride, n_slices, n_tokens, slice_stride, cap,
                        cv(codes), scale, zero, [&](int64_t a, int64_t count) {
                            return decode(false, &cfgs[a], codes[a], scale[a], zero[a], count * n_slices,
                                          n_tokens, cap, static_cast<uint16_t*>(out) + a * layer_stride,
                                          slice_stride, stream);
                        });
}

int kivi_stream_prefill(const kivi_config* cfg, kivi_stream* st, const void* k, const void* v,
                        int64_t n_tokens, int64_t in_stride, void* stream) {
    int s = check_config(cfg);
    if (s) return s;
    s = check_stream(cfg, st, false);
    if (s) return s;
    if (n_tokens < 0 || n_tokens > kMaxTokens) return KIVI_E_SHAPE;
    const int64_t G = cfg->group_size, R = cfg->residual_length;
    const int64_t nq = (n_tokens > R ? (n_tokens - R) / G : 0) * G;
    const int64_t rest = n_tokens - nq;           // <= R + G - 1 by construction
    if (nq > st->cap_tokens) return KIVI_E_CAPACITY;
    if (st->n_slices > 0 && n_tokens > 0) {
        if (in_stride % 8 != 0) return KIVI_E_ALIGN;
        int64_t need = 0, total = 0;
        if (!mul_ok(n_tokens, cfg->head_dim, &need) || in_stride < need) return KIVI_E_SHAPE;
        if (!mul_ok(st->n_slices, in_stride, &total)) return KIVI_E_SHAPE;
        if (!k || !v) return KIVI_E_NULL;
        if (!aligned16(k) || !aligned16(v)) return KIVI_E_ALIGN;
        if (nq > 0) {
            s = kivi_encode_k(cfg, k, st->n_slices, nq, in_stride, st->cap_tokens, st->k_codes,
                              st->k_scale, st->k_zero, stream);
            if (s) return s;
        }
        // value rows are per token: the residual's rows are quantized now too
        // (up to the capacity), as kivi_append_flush does for each new token
        const int64_t nv = n_tokens < st->cap_tokens ? n_tokens : st->cap_tokens;
        if (nv > 0) {
            s = kivi_encode_v(cfg, v, st->n_slices, nv, in_stride, st->cap_tokens, st->v_codes,
                              st->v_scale, st->v_zero, stream);
            if (s) return s;
        }
        if (rest > 0) {
            kivi::RingFillArgs a;
            a.k_in = static_cast<const uint16_t*>(k);
            a.v_in = static_cast<const uint16_t*>(v);
            a.in_stride = in_stride;
            a.n_slices = st->n_slices;
            a.first_token = static_cast<int32_t>(nq);
            a.n_tokens = static_cast<int32_t>(rest);
            a.head_dim = cfg->head_dim;
            a.ring_slots = static_cast<int32_t>(R + G);
            a.k_ring = static_cast<uint16_t*>(st->k_ring);
            a.v_ring = static_cast<uint16_t*>(st->v_ring);
            s = record(kivi::launch_ring_fill(a, stream));
            if (s) return s;
        }
    }
    st->n_quant = nq;
    st->ring_head = 0;
    st->ring_count = rest;
    return KIVI_OK;
}

int kivi_append_flush(const kivi_config* cfg, kivi_stream* st, const void* k_new, const void* v_new,
                      void* stream) {
    int s = check_config(cfg);
    if (s) return s;
    s = check_stream(cfg, st, true);
    if (s) return s;
    const int64_t G = cfg->group_size, R = cfg->residual_length;
    const int64_t slots = R + G;
    const bool flush = flush_due(st->ring_count + 1, R, G);
    if (flush && st->n_quant + G > st->cap_tokens) return KIVI_E_CAPACITY;
    if (st->n_slices > 0) {
        if (!k_new || !v_new) return KIVI_E_NULL;
        if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_E_ALIGN;
        kivi::StepArgs a;
        a.k_new = static_cast<const uint16_t*>(k_new);
        a.v_new = static_cast<const uint16_t*>(v_new);
        a.k_ring = static_cast<uint16_t*>(st->k_ring);
        a.v_ring = static_cast<uint16_t*>(st->v_ring);
        a.k_codes = reinterpret_cast<uint32_t*>(st->k_codes);
        a.k_scale = static_cast<uint16_t*>(st->k_scale);
        a.k_zero = static_cast<uint16_t*>(st->k_zero);
        a.v_codes = reinterpret_cast<uint32_t*>(st->v_codes);
        a.v_scale = static_cast<uint16_t*>(st->v_scale);
        a.v_zero = static_cast<uint16_t*>(st->v_zero);
        a.n_slices = st->n_slices;
        a.cap_tokens = static_cast<int32_t>(st->cap_tokens);
        a.head_dim = cfg->head_dim;
        a.group_size = cfg->group_size;
        a.k_bits = cfg->k_bits;
        a.v_bits = cfg->v_bits;
        a.ring_slots = static_cast<int32_t>(slots);
        a.ring_head = static_cast<int32_t>(st->ring_head);
        a.ring_count = static_cast<int32_t>(st->ring_count);
        a.flush = flush ? 1 : 0;
        a.n_quant = static_cast<int32_t>(st->n_quant);
        s = record(kivi::launch_append_flush(a, stream));
        if (s) return s;
    }
    st->ring_count += 1;
    if (flush) {
        st->n_quant += G;
        st->ring_head = (st->ring_head + G) % slots;
        st->ring_count -= G;
    }
    return KIVI_OK;
}

int64_t kivi_attention_workspace_bytes(const kivi_config* cfg, int64_t n_slices, int32_t q_per_kv,
                                       int64_t n_quant, int64_t res_count) {
    if (check_attention_config(cfg, q_per_kv)) return -1;
    if (n_slices < 0 || n_quant < 0 || n_quant > kMaxTokens || res_count < 0 || res_count > kMaxTokens)
        return -1;
    return attention_ws_bytes(cfg, n_slices, q_per_kv, kivi::attn_plan(n_slices, n_quant, res_count));
}

int kivi_decode_attention(const kivi_config* cfg, const kivi_attn_cache* cache, int64_t n_slices,
                          int32_t q_per_kv, const void* q, float sm_scale, void* out,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    return attention_call(cfg, cache, n_slices, q_per_kv, q, sm_scale, out, workspace, workspace_bytes,
                          false, stream);
}

int kivi_decode_attention_noalloc(const kivi_config* cfg, const kivi_attn_cache* cache, int64_t n_slices,
                                  int32_t q_per_kv, const void* q, float sm_scale, void* out,
                                  void* stream) {
    return attention_call(cfg, cache, n_slices, q_per_kv, q, sm_scale, out, nullptr, 0, true, stream);
}

int64_t kivi_stream_image_bytes(const kivi_config* cfg, int64_t n_slices, int64_t n_quant) {
    if (check_config(cfg)) return -1;
    if (n_slices < 0 || n_quant < 0 || n_quant > kMaxTokens || n_quant % cfg->group_size != 0) return -1;
    ImagePart parts[8];
    int64_t total = 0;
    if (!image_parts(cfg, n_slices, n_quant, n_quant, parts, &total)) return -1;
    return total;
}

int kivi_stream_offload(const kivi_config* cfg, const kivi_stream* st, void* host, int64_t host_bytes,
                        void* stream) {
    int s = check_config(cfg);
    if (s) return s;
    s = check_stream(cfg, st, true);
    if (s) return s;
    if (st->n_slices == 0) return KIVI_OK;
    ImagePart parts[8];
    int64_t total = 0;
    if (!image_parts(cfg, st->n_slices, st->n_quant, st->cap_tokens, parts, &total)) return KIVI_E_SHAPE;
    if (host_bytes < total) return KIVI_E_SHAPE;
    if (!host) return KIVI_E_NULL;
    const void* src[8] = {st->k_codes, st->k_scale, st->k_zero, st->v_codes,
                          st->v_scale, st->v_zero,  st->k_ring, st->v_ring};
    char* dst = static_cast<char*>(host);
    for (int i = 0; i < 8; ++i) {
        s = record(kivi::launch_copy_2d(dst, parts[i].width, src[i], parts[i].dev_pitch, parts[i].width,
                                        parts[i].height, stream));
        if (s) return s;
        dst += parts[i].width * parts[i].height;
    }
    return KIVI_OK;
}

int kivi_stream_restore(const kivi_config* cfg, kivi_stream* st, const void* host, int64_t host_bytes,
                        int64_t n_quant, int64_t ring_head, int64_t ring_count, void* stream) {
    int s = check_config(cfg);
    if (s) return s;
    s = check_stream(cfg, st, false);
    if (s) return s;
    const int64_t G = cfg->group_size, slots = int64_t(cfg->residual_length) + G;
    if (n_quant < 0 || n_quant % G != 0) return KIVI_E_STATE;
    if (n_quant > st->cap_tokens) return KIVI_E_CAPACITY;
    if (ring_head < 0 || ring_head >= slots || ring_count < 0 || ring_count > slots - 1) return KIVI_E_STATE;
    if (st->n_slices > 0) {
        ImagePart parts[8];
        int64_t total = 0;
        if (!image_parts(cfg, st->n_slices, n_quant, st->cap_tokens, parts, &total)) return KIVI_E_SHAPE;
        if (host_bytes < total) return KIVI_E_SHAPE;
        if (!host) return KIVI_E_NULL;
        void* dst[8] = {st->k_codes, st->k_scale, st->k_zero, st->v_codes,
                        st->v_scale, st->v_zero,  st->k_ring, st->v_ring};
        const char* src = static_cast<const char*>(host);
        for (int i = 0; i < 8; ++i) {
            s = record(kivi::launch_copy_2d(dst[i], parts[i].dev_pitch, src, parts[i].width, parts[i].width,
                                            parts[i].height, stream));
            if (s) return s;
            src += parts[i].width * parts[i].height;
        }
        // value rows of the residual tokens, re-quantized from the ring in at
        // most two contiguous runs of slots (below the capacity only)
        const int64_t D = cfg->head_dim, ngv = v_groups(cfg);
        const int64_t wpt = ngv * (G * cfg->v_bits / 32);
        int64_t todo = ring_count < st->cap_tokens - n_quant ? ring_count : st->cap_tokens - n_quant;
        int64_t slot = ring_head, row = n_quant;
        while (todo > 0) {
            const int64_t run = todo < slots - slot ? todo : slots - slot;
            kivi::EncodeArgs a;
            a.in = static_cast<const uint16_t*>(st->v_ring) + slot * D;
            a.in_stride = slots * D;
            a.n_slices = st->n_slices;
            a.n_tokens = static_cast<int32_t>(run);
            a.cap_tokens = static_cast<int32_t>(st->cap_tokens);
            a.head_dim = cfg->head_dim;
            a.group_size = cfg->group_size;
            a.bits = cfg->v_bits;
            a.codes = reinterpret_cast<uint32_t*>(st->v_codes) + row * wpt;
            a.scale = static_cast<uint16_t*>(st->v_scale) + row * ngv;
            a.zero = static_cast<uint16_t*>(st->v_zero) + row * ngv;
            s = record(kivi::launch_encode_v(a, stream));
            if (s) return s;
            todo -= run;
            row += run;
            slot = 0;
        }
    }
    st->n_quant = n_quant;
    st->ring_head = ring_head;
    st->ring_count = ring_count;
    return KIVI_OK;
}

namespace {

int fp8_call(bool enc, const void* in, int64_t n_slices, int64_t n_tokens, int64_t D, int64_t in_stride,
             void* out, int64_t out_stride, void* stream) {
    if (D < 8 || D > 256 || D % 8 != 0) return KIVI_E_HEAD_DIM;
    if (n_slices < 0 || n_tokens < 0 || n_tokens > kMaxTokens) return KIVI_E_SHAPE;
    if (n_tokens * (D / 8) > (int64_t(1) << 30)) return KIVI_E_SHAPE;   // 32-bit chunk index per slice
    if (n_slices == 0 || n_tokens == 0) return KIVI_OK;
    if (in_stride % 16 != 0 || out_stride % 16 != 0) return KIVI_E_ALIGN;
    int64_t need = 0, total = 0;
    if (!mul_ok(n_tokens, D, &need) || in_stride < need || out_stride < need) return KIVI_E_SHAPE;
    // bytes of either array (fp16 on one side, one-byte codes on the other)
    const int64_t wider = in_stride > out_stride ? in_stride : out_stride;
    if (!mul_ok(n_slices, wider, &total) || !mul_ok(total, 2, &total)) return KIVI_E_SHAPE;
    if (!in || !out) return KIVI_E_NULL;
    if (!aligned16(in) || !aligned16(out)) return KIVI_E_ALIGN;
    kivi::Fp8Args a;
    a.in = in;
    a.in_stride = in_stride;
    a.out = out;
    a.out_stride = out_stride;
    a.n_slices = n_slices;
    a.n_tokens = static_cast<int32_t>(n_tokens);
    a.head_dim = static_cast<int32_t>(D);
    return record(enc ? kivi::launch_fp8_encode(a, stream) : kivi::launch_fp8_decode(a, stream));
}

}  // namespace

int kivi_fp8_encode(const void* in, int64_t n_slices, int64_t n_tokens, int64_t head_dim,
                    int64_t in_stride, uint8_t* out, int64_t out_stride, void* stream) {
    return fp8_call(true, in, n_slices, n_tokens, head_dim, in_stride, out, out_stride, stream);
}

int kivi_fp8_decode(const uint8_t* in, int64_t n_slices, int64_t n_tokens, int64_t head_dim,
                    int64_t in_stride, void* out, int64_t out_stride, void* stream) {
    return fp8_call(false, in, n_slices, n_tokens, head_dim, in_stride, out, out_stride, stream);
}

}  // extern "C"
