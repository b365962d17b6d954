/*
 * kivi.h -- C ABI of libkivi, the KIVI grouped KV-cache codec for AMD
 * MI355X (gfx950).
 *
 * Method.  CacheForge README, "How it works": keys are quantized per
 * channel, values per token, and the most recent tokens stay in higher
 * precision; its "Example" section names the four knobs k_bits, v_bits,
 * group_size and residual_length (the count of recent tokens kept fp16).
 * CacheSeek pull request #4 ("Feature(quantization): add KIVI KV-cache
 * quantization for exact-prefix reuse"), description: KIVI encode/decode
 * with grouped statistics, padding of partial groups, codes packed into
 * int32 words, and a compact qdata/scale/offset payload that is produced
 * on the tensor's own device.
 *
 * The pages print no formula; this library implements the reading
 *   per group:  mn, mx     = min, max of the group's valid fp16 elements
 *                            (a negative zero counts as +0)
 *               scale      = fp16( fp32( fp32(mx - mn) / (2^b - 1) ) )
 *               zero       = mn                              (exact in fp16)
 *   per element: q         = clamp( rint( fp32( fp32(x - zero) / scale ) ),
 *                                   0, 2^b - 1 )   (IEEE division, rint
 *                                                   = round half to even;
 *                                                   q = 0 when scale == 0)
 *   decode:     xhat       = fp16( fp32( q * scale + zero ) )
 * with every rounding to nearest, ties to even.  Code i of a 32-bit word
 * sits at bits [i*b, i*b + b); word w of a group holds the group's
 * elements w*(32/b) .. w*(32/b) + 32/b - 1.  Padding slots hold code 0.
 *
 * Terms used below.
 *   slice    one independent (layer, batch, head) sequence of a KV cache.
 *   D        head_dim.  G = group_size.  b = k_bits or v_bits.
 *   W        = G*b/32, int32 words per group.
 *   NG_k(n)  = ceil(n / G), key groups of n tokens (last one padded).
 *   NG_v     = ceil(D / G), value groups of one token (last one padded).
 *
 * Layouts (row-major, innermost last; fp16 data is passed as raw 16-bit
 * patterns through void pointers):
 *   K or V input   fp16  [n_slices][in_slice_stride]; token t of slice s
 *                        starts at element s*in_slice_stride + t*D.
 *   key codes      int32 [n_slices][NG_k(cap_tokens)*W][D]   (channel innermost)
 *   key scale/zero fp16  [n_slices][NG_k(cap_tokens)][D]
 *   value codes    int32 [n_slices][cap_tokens][NG_v*W]
 *   value scale/zero fp16 [n_slices][cap_tokens][NG_v]
 *   decoded K or V fp16  [n_slices][out_slice_stride]; token t of slice s
 *                        starts at element s*out_slice_stride + t*D.
 *
 * Ownership and execution.  The caller allocates and frees every buffer
 * (device memory for all array arguments; host memory for kivi_config and
 * kivi_stream).  The library never allocates, frees or synchronises: each
 * call only validates its arguments on the host and enqueues kernels on
 * hip_stream (a hipStream_t; NULL means the default stream), so outputs are
 * ready when that stream reaches the enqueued work.  Calls on different
 * streams are independent and re-entrant; the library's only global state
 * is the thread-local code of the last failed HIP launch, plus the static
 * device scratch of kivi_decode_attention_noalloc (and its address per
 * device), which only that entry point uses.
 *
 * Errors.  Every entry point returns KIVI_OK (0) or a negative KIVI_E_*
 * code.  Argument checks all run before any HIP call, so a non-zero return
 * other than KIVI_E_HIP means that nothing was enqueued and no output (and
 * no kivi_stream field) was touched.  Nothing aborts and no C++ exception
 * crosses the ABI.  Array pointers must be 16-byte aligned and slice
 * strides multiples of 8 elements.  Calls with n_slices == 0 or
 * n_tokens == 0 validate the configuration and return KIVI_OK without
 * touching any pointer.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Codec configuration (CacheForge README, "Example": k_bits, v_bits,
 * group_size, residual_length; vLLM turboquant/config.py, TurboQuantConfig:
 * head_dim, e.g. 64, 96, 128).
 *   k_bits, v_bits   2, 4 or 8, independently.
 *   group_size       32, 64 or 128; shared by keys (tokens per key group)
 *                    and values (channels per value group).
 *   residual_length  R >= 0: the most recent R tokens stay fp16.
 *   head_dim         D, a multiple of 8 in [8, 256]. */
typedef struct kivi_config {
    int32_t k_bits;
    int32_t v_bits;
    int32_t group_size;
    int32_t residual_length;
    int32_t head_dim;
} kivi_config;

enum {
    KIVI_OK = 0,
    KIVI_E_NULL = -1,       /* a required pointer is NULL */
    KIVI_E_BITS = -2,       /* k_bits or v_bits not in {2, 4, 8} */
    KIVI_E_GROUP = -3,      /* group_size not in {32, 64, 128} */
    KIVI_E_HEAD_DIM = -4,   /* head_dim not a multiple of 8 in [8, 256] */
    KIVI_E_RESIDUAL = -5,   /* residual_length < 0 */
    KIVI_E_SHAPE = -6,      /* negative count, stride < n_tokens*D, cap_tokens < n_tokens, size overflow */
    KIVI_E_ALIGN = -7,      /* pointer not 16-byte aligned or stride not a multiple of 8 */
    KIVI_E_CAPACITY = -8,   /* streaming flush would pass cap_tokens */
    KIVI_E_STATE = -9,      /* kivi_stream counters inconsistent */
    KIVI_E_HIP = -10,       /* a HIP launch failed; see kivi_last_hip_error() */
    KIVI_E_SCRATCH = -11    /* the call needs more than the library's static scratch */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* kivi_status_string(int status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int kivi_last_hip_error(void);

/* Checks a configuration; returns KIVI_OK or the matching KIVI_E_* code. */
int kivi_validate_config(const kivi_config* cfg);

/* Sizes per slice, for a capacity of n_tokens quantized tokens (CacheSeek
 * PR #4: the manager accounts the stored payload size itself).  Return -1
 * for an invalid configuration, n_tokens < 0 or n_tokens above 2^30 (the
 * per-slice token limit of every call).
 *   kivi_k_code_words  int32 words of key codes     = NG_k(n)*W_k*D
 *   kivi_k_stat_elems  fp16 elements of ONE key sidecar (scale or zero)
 *                                                   = NG_k(n)*D
 *   kivi_v_code_words  int32 words of value codes   = n*NG_v*W_v
 *   kivi_v_stat_elems  fp16 elements of ONE value sidecar = n*NG_v
 *   kivi_ring_elems    fp16 elements of one residual ring (keys or values)
 *                      of the streaming state       = (R + G)*D          */
int64_t kivi_k_code_words(const kivi_config* cfg, int64_t n_tokens);
int64_t kivi_k_stat_elems(const kivi_config* cfg, int64_t n_tokens);
int64_t kivi_v_code_words(const kivi_config* cfg, int64_t n_tokens);
int64_t kivi_v_stat_elems(const kivi_config* cfg, int64_t n_tokens);
int64_t kivi_ring_elems(const kivi_config* cfg);

/* Per-channel key quantization (CacheForge README, "How it works": keys
 * per channel; CacheSeek PR #4: grouped stats, padding, int32 packing).
 * Quantizes tokens [0, n_tokens) of every slice of k_fp16 in groups of G
 * tokens per channel; the last group of a slice may be partial, its
 * statistics use only the valid tokens and its pad slots get code 0.  The
 * caller passes n_tokens = T - R to keep the R most recent of T tokens in
 * fp16 (those are not read).  Writes, per slice, key groups [0, NG_k(n))
 * of codes/scale/zero, laid out for a capacity of cap_tokens >= n_tokens
 * tokens (pass cap_tokens = n_tokens for dense output); groups beyond
 * NG_k(n) are not touched. */
int kivi_encode_k(const kivi_config* cfg, const void* k_fp16,
                  int64_t n_slices, int64_t n_tokens, int64_t in_slice_stride,
                  int64_t cap_tokens, int32_t* codes,
                  void* scale_fp16, void* zero_fp16, void* hip_stream);

/* Per-token value quantization (CacheForge README, "How it works": values
 * per token).  Quantizes rows [0, n_tokens) of every slice in groups of G
 * channels; when D is not a multiple of G the last group is padded.  Writes
 * value rows [0, n_tokens) of the cap_tokens-row layouts. */
int kivi_encode_v(const kivi_config* cfg, const void* v_fp16,
                  int64_t n_slices, int64_t n_tokens, int64_t in_slice_stride,
                  int64_t cap_tokens, int32_t* codes,
                  void* scale_fp16, void* zero_fp16, void* hip_stream);

/* Unpack and dequantize keys (CacheSeek PR #4: decoding moves only the
 * compact qdata/scale/offset to the target device before dequantization).
 * Reads key groups [0, NG_k(n_tokens)) of a cap_tokens layout and writes
 * exactly n_tokens*D fp16 values per slice to out_fp16 (never a pad slot). */
int kivi_decode_k(const kivi_config* cfg, const int32_t* codes,
                  const void* scale_fp16, const void* zero_fp16,
                  int64_t n_slices, int64_t n_tokens, int64_t cap_tokens,
                  void* out_fp16, int64_t out_slice_stride, void* hip_stream);

/* Unpack and dequantize values; same contract as kivi_decode_k for value
 * rows [0, n_tokens). */
int kivi_decode_v(const kivi_config* cfg, const int32_t* codes,
                  const void* scale_fp16, const void* zero_fp16,
                  int64_t n_slices, int64_t n_tokens, int64_t cap_tokens,
                  void* out_fp16, int64_t out_slice_stride, void* hip_stream);

/* Per-layer bit mixes (vLLM turboquant/config.py, get_boundary_skip_layers:
 * "boundary protection" exempts the first n and the last n attention
 * layers of a dense model from an aggressive preset; n is capped at half the
 * layer count and the two sets are merged).  Here a protected layer takes a
 * configuration of its own (normally more bits) instead of no compression;
 * keeping those layers in fp16 is the caller's choice of not coding them.
 *
 * kivi_boundary_layers: for a model of n_layers layers, sets flags[l] = 1
 * for the protected layers and 0 for the others (flags: host int32
 * [n_layers]).  Returns the number of protected layers (>= 0),
 * KIVI_E_SHAPE for n_layers < 0, KIVI_E_NULL for flags == NULL with
 * n_layers > 0.  n <= 0 protects nothing.  Host only. */
int kivi_boundary_layers(int64_t n_layers, int64_t n, int32_t* flags);

/* Coding of a model cache whose layers may have different configurations.
 * cfgs: host array of n_layers configurations (all with one head_dim).
 * Every layer has n_slices slices and a capacity of cap_tokens tokens.
 * fp16 side: layer l starts at element l*layer_stride of the input (encode)
 * or output (decode) array, and within a layer the layout is the
 * single-layer one with slice_stride; layer_stride >= n_slices*slice_stride,
 * a multiple of 8.  Payload side: codes[l], scale[l], zero[l] are host
 * arrays of n_layers device pointers, layer l's key (or value) layouts, as
 * for the single-layer calls.
 * Results are those of one single-layer call per layer with cfgs[l].  A
 * run of consecutive layers is coded by ONE launch over all its slices when
 * the layers agree on the coded side's bits, group_size and head_dim, the
 * fp16 layers are back to back (layer_stride == n_slices*slice_stride) and
 * each payload array of a layer starts where the previous layer's ends
 * (which is how a caller lays out a mix in one allocation per run); other
 * layers get a launch each.  The 16-byte alignment rule applies to the
 * arrays of each run's first layer only: the other layers of a run are
 * addressed as slices of those arrays.  Every layer's arguments are checked
 * before the first launch, so an error other than KIVI_E_HIP enqueues
 * nothing. */
int kivi_encode_k_layers(const kivi_config* cfgs, int64_t n_layers, const void* k_fp16,
                         int64_t layer_stride, int64_t n_slices, int64_t n_tokens,
                         int64_t slice_stride, int64_t cap_tokens, int32_t* const* codes,
                         void* const* scale_fp16, void* const* zero_fp16, void* hip_stream);
int kivi_encode_v_layers(const kivi_config* cfgs, int64_t n_layers, const void* v_fp16,
                         int64_t layer_stride, int64_t n_slices, int64_t n_tokens,
                         int64_t slice_stride, int64_t cap_tokens, int32_t* const* codes,
                         void* const* scale_fp16, void* const* zero_fp16, void* hip_stream);
int kivi_decode_k_layers(const kivi_config* cfgs, int64_t n_layers, const int32_t* const* codes,
                         const void* const* scale_fp16, const void* const* zero_fp16,
                         int64_t n_slices, int64_t n_tokens, int64_t cap_tokens, void* out_fp16,
                         int64_t layer_stride, int64_t slice_stride, void* hip_stream);
int kivi_decode_v_layers(const kivi_config* cfgs, int64_t n_layers, const int32_t* const* codes,
                         const void* const* scale_fp16, const void* const* zero_fp16,
                         int64_t n_slices, int64_t n_tokens, int64_t cap_tokens, void* out_fp16,
                         int64_t layer_stride, int64_t slice_stride, void* hip_stream);

/* Streaming state of the decode phase (CacheForge README, "How it works"
 * and its figure on the quantization flow during prefill and decoding: the
 * recent tokens stay fp16 while older ones are quantized).  Device arrays:
 *   k_codes, k_scale, k_zero, v_codes, v_scale, v_zero
 *       the key/value layouts above for cap_tokens tokens per slice;
 *   k_ring, v_ring
 *       fp16 [n_slices][R + G][D]: the fp16 residual of each slice as a
 *       ring; residual token i (0 = oldest) sits in slot
 *       (ring_head + i) mod (R + G).
 * Value groups are per token, so a value row is quantized as soon as its
 * token arrives (by the prefill or by the step that appends it): store rows
 * n_quant .. n_quant + ring_count - 1 (those below cap_tokens) already hold
 * the codes of the residual tokens.  Only rows below n_quant are part of the
 * quantized prefix; readers take the residual from the fp16 ring.
 * Host counters (owned by the caller, updated by the library):
 *   n_slices    slices in every array.
 *   cap_tokens  quantized-token capacity, a multiple of G.
 *   n_quant     tokens quantized so far, a multiple of G, <= cap_tokens.
 *   ring_head   slot of the oldest residual token, in [0, R + G).
 *   ring_count  residual tokens, in [0, R + G - 1] between calls.
 * Every stream call rejects R + G above 2^21 ring slots with KIVI_E_SHAPE
 * (the kernels address a few slices' rings with 32-bit byte offsets). */
typedef struct kivi_stream {
    int32_t* k_codes;
    int32_t* v_codes;
    void* k_scale;
    void* k_zero;
    void* v_scale;
    void* v_zero;
    void* k_ring;
    void* v_ring;
    int64_t n_slices;
    int64_t cap_tokens;
    int64_t n_quant;
    int64_t ring_head;
    int64_t ring_count;
} kivi_stream;

/* Prefill: quantizes the first floor((n_tokens - R)/G)*G tokens of every
 * slice of k_fp16/v_fp16 (layout as for kivi_encode_k) into the stream's
 * arrays and copies the remaining tokens into the rings in age order; sets
 * n_quant to that token count, ring_head = 0 and ring_count to the rest.
 * The stream's array pointers, n_slices and cap_tokens must be set; its
 * counters are overwritten.  The rest is at most R + G - 1 tokens, so it
 * always fits the ring.  KIVI_E_CAPACITY when the quantized prefix exceeds
 * cap_tokens; KIVI_E_STATE when cap_tokens is not a multiple of G. */
int kivi_stream_prefill(const kivi_config* cfg, kivi_stream* st,
                        const void* k_fp16, const void* v_fp16,
                        int64_t n_tokens, int64_t in_slice_stride, void* hip_stream);

/* One decode step: appends k_new/v_new (fp16
 * [n_slices][D], contiguous) to the residual; if the residual then holds
 * more than R tokens and at least G, its oldest G tokens are quantized as
 * key group n_quant/G and value rows n_quant .. n_quant+G-1 of every slice,
 * and the counters advance (n_quant += G, ring_head += G mod R+G,
 * ring_count -= G).  One kernel launch either way.  KIVI_E_CAPACITY (and
 * nothing enqueued, counters unchanged) when that flush would pass
 * cap_tokens. */
int kivi_append_flush(const kivi_config* cfg, kivi_stream* st,
                      const void* k_new_fp16, const void* v_new_fp16, void* hip_stream);

/* FP8 keys of the k8v4 layout (vLLM turboquant/config.py: the
 * turboquant_k8v4 preset stores keys in 8 bits and values in 4; its
 * TurboQuantConfig docstring makes 8-bit keys FP8 with no rotation or
 * codebook, and key_packed_size counts one byte per element with no
 * overhead, i.e. a plain cast).  The values of that layout are
 * kivi_encode_v with group_size = head_dim (one scale and zero per value
 * vector, value_packed_size).  The page names neither the FP8 variant nor
 * its rounding; the library uses OCP E4M3 (bias 7, 3 mantissa bits,
 * subnormals, largest finite 448, NaN only at S.1111.111), round to nearest
 * with ties to the even code, saturation to +-448, sign kept.
 *   kivi_fp8_encode  fp16 [n_slices][in_slice_stride] -> codes uint8
 *                    [n_slices][out_slice_stride]; token t of a slice
 *                    occupies elements t*D .. t*D + D - 1 of both.
 *   kivi_fp8_decode  codes -> fp16 (exact; every E4M3 value is an fp16
 *                    value), same addressing.
 * head_dim: a multiple of 8 in [8, 256] (KIVI_E_HEAD_DIM); strides at least
 * n_tokens*D and multiples of 16 elements (KIVI_E_SHAPE / KIVI_E_ALIGN);
 * pointers 16-byte aligned.  NaN and infinite inputs are out of contract. */
int kivi_fp8_encode(const void* in_fp16, int64_t n_slices, int64_t n_tokens, int64_t head_dim,
                    int64_t in_slice_stride, uint8_t* out, int64_t out_slice_stride,
                    void* hip_stream);
int kivi_fp8_decode(const uint8_t* in, int64_t n_slices, int64_t n_tokens, int64_t head_dim,
                    int64_t in_slice_stride, void* out_fp16, int64_t out_slice_stride,
                    void* hip_stream);

/* Compact host image of a streaming cache (CacheSeek PR #4 "Feature
 * (quantization): add KIVI KV-cache quantization for exact-prefix reuse":
 * encoding runs on the source device, only the compact qdata/scale/offset
 * payload travels to host memory for storage, and decoding moves only that
 * payload to the target device before dequantizing).  The image holds, for
 * every slice, the quantized prefix of n_quant tokens and the fp16 residual
 * ring, as eight arrays one after another, each slice-major and packed
 * without the device arrays' unused capacity:
 *   key codes   [n_slices][NG_k(n_quant)*W_k][D]  int32
 *   key scale   [n_slices][NG_k(n_quant)][D]      fp16   (then key zero)
 *   value codes [n_slices][n_quant][NG_v*W_v]     int32
 *   value scale [n_slices][n_quant][NG_v]         fp16   (then value zero)
 *   key ring    [n_slices][R + G][D]              fp16   (then value ring)
 * Ring slots are copied as they are, so the image keeps ring_head and
 * ring_count meaningful; the caller stores those counters with it.
 * kivi_stream_image_bytes returns the image size (-1 on invalid input);
 * n_quant must be a multiple of G, as in every kivi_stream. */
int64_t kivi_stream_image_bytes(const kivi_config* cfg, int64_t n_slices, int64_t n_quant);

/* Enqueues the copies of st's image (at st->n_quant tokens) into host
 * memory `host` (host_bytes >= the image size; pinned memory makes the
 * copies asynchronous).  Device arrays and counters are not modified.
 * KIVI_E_SHAPE when host_bytes is too small, KIVI_E_STATE for inconsistent
 * counters. */
int kivi_stream_offload(const kivi_config* cfg, const kivi_stream* st, void* host,
                        int64_t host_bytes, void* hip_stream);

/* Enqueues the copies of an image of n_quant tokens from host memory into
 * st's device arrays (st->n_slices slices, capacity st->cap_tokens >=
 * n_quant) and sets st->n_quant, ring_head and ring_count to the given
 * values, which must satisfy the kivi_stream invariants (KIVI_E_STATE
 * otherwise; KIVI_E_CAPACITY when n_quant > cap_tokens).  The value rows
 * of the residual tokens (rows n_quant .. n_quant + ring_count - 1 below
 * capacity, which a kivi_stream quantizes on arrival) are not part of the
 * image: the restore re-quantizes them from the restored ring, so the
 * stream continues exactly as the one that was offloaded. */
int kivi_stream_restore(const kivi_config* cfg, kivi_stream* st, const void* host,
                        int64_t host_bytes, int64_t n_quant, int64_t ring_head,
                        int64_t ring_count, void* hip_stream);

/* Decode-phase attention over the quantized cache (CacheForge README,
 * "Contribution scope": the inherited KIVI code brings the model
 * integrations and the kernels that consume the quantized cache; "How it
 * works": keys quantized per channel, values per token, the newest tokens in
 * fp16).  The pages give no formula for this consumer; the library computes
 * ordinary softmax attention of one query token per query head,
 *     out[s][j] = sum_t softmax_t( sm_scale * q[s][j] . k_t ) * v_t,
 * over every cached token t of slice s: the n_quant quantized tokens,
 * dequantized as code * scale + zero (kept in fp32, not rounded to fp16),
 * then the res_count fp16 residual tokens.  q_per_kv consecutive query
 * heads share one KV slice (grouped-query attention; 1 = multi-head).
 *
 * Cache description (host struct owned by the caller; device arrays):
 *   k_codes .. v_zero  the key/value layouts above for cap_tokens tokens per
 *                      slice; key groups [0, NG_k(n_quant)) and value rows
 *                      [0, n_quant) are read, nothing else.
 *   n_quant            quantized tokens per slice, in [0, cap_tokens]; any
 *                      count (the last key group may be partial).
 *   res_k, res_v       fp16 residual tokens: token i (0 = oldest) of slice s
 *                      is the D elements at s*res_slice_stride +
 *                      ((res_head + i) mod res_slots)*D, i < res_count.
 *                      A kivi_stream maps to res_slots = R + G, res_slice_stride
 *                      = (R + G)*D, res_head = ring_head, res_count =
 *                      ring_count; a full-cache encode of T tokens maps to
 *                      res_k = k + n_quant*D with the input's slice stride
 *                      and res_slots = res_count = T - n_quant, res_head = 0.
 *                      May be NULL when res_count == 0.
 *   n_quant_per_slice, res_count_per_slice
 *                      optional device arrays of n_slices int32 (NULL: every
 *                      slice has n_quant quantized and res_count residual
 *                      tokens).  Given, slice s has n_quant_per_slice[s]
 *                      quantized and res_count_per_slice[s] residual tokens
 *                      (a ragged batch); n_quant and res_count are then the
 *                      upper bounds that size the work and the workspace,
 *                      and the kernels clamp each value into [0, bound].  A
 *                      slice with no token at all gets an all-zero output. */
typedef struct kivi_attn_cache {
    const int32_t* k_codes;
    const void* k_scale;
    const void* k_zero;
    const int32_t* v_codes;
    const void* v_scale;
    const void* v_zero;
    int64_t cap_tokens;
    int64_t n_quant;
    const void* res_k;
    const void* res_v;
    int64_t res_slice_stride;
    int64_t res_slots;
    int64_t res_head;
    int64_t res_count;
    const int32_t* n_quant_per_slice;
    const int32_t* res_count_per_slice;
} kivi_attn_cache;

/* Bytes of device workspace that kivi_decode_attention needs for these
 * sizes (0 when every slice is done in one pass and no workspace is used).
 * The library splits long caches over several workgroups per slice and
 * merges their partial softmax sums in a second kernel; the workspace holds
 * those partials.  -1 on an invalid configuration or size. */
int64_t kivi_attention_workspace_bytes(const kivi_config* cfg, int64_t n_slices,
                                       int32_t q_per_kv, int64_t n_quant,
                                       int64_t res_count);

/* Attention of q_fp16 [n_slices][q_per_kv][D] (contiguous) over the cache,
 * written to out_fp16 [n_slices][q_per_kv][D] (rounded to nearest fp16).
 * Requirements beyond the codec's: head_dim a multiple of 32 and at most
 * 128 (KIVI_E_HEAD_DIM); q_per_kv in [1, 8], n_quant + res_count >= 1,
 * res_count <= res_slots, 0 <= res_head < res_slots, sm_scale finite and
 * workspace_bytes >= kivi_attention_workspace_bytes(...) (KIVI_E_SHAPE);
 * residual stride a multiple of 8 elements (KIVI_E_ALIGN).  workspace may
 * be NULL when that size is 0.  Async on hip_stream like the codec calls. */
int kivi_decode_attention(const kivi_config* cfg, const kivi_attn_cache* cache,
                          int64_t n_slices, int32_t q_per_kv, const void* q_fp16,
                          float sm_scale, void* out_fp16, void* workspace,
                          int64_t workspace_bytes, void* hip_stream);

/* Size in bytes of the static attention scratch that libkivi holds on each
 * device it runs kivi_decode_attention_noalloc on (from that device's first
 * such call until the process ends). */
#define KIVI_ATTENTION_SCRATCH_BYTES (128LL << 20)

/* kivi_decode_attention for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, kernels and results (bit for bit) as
 * kivi_decode_attention, without the workspace: when the call splits slices
 * (kivi_attention_workspace_bytes(...) > 0) its partial sums go to a
 * library-owned static device buffer of KIVI_ATTENTION_SCRATCH_BYTES bytes
 * per device, and a call that would need more returns KIVI_E_SCRATCH with
 * nothing enqueued (split the slices over several calls).  Nothing is
 * allocated or freed, by the library or by any routine it calls.  The device
 * is the one hip_stream belongs to (the current device for NULL); the first
 * call on a device looks up that device's buffer address once (no
 * allocation; make that first call outside graph capture).  Every call on
 * one device shares its buffer and leaves the last call's partials in it:
 * calls that overlap on one device (concurrent streams, or threads) race and
 * must be ordered by the caller.  The buffer needs no clearing: every
 * partial is written before it is read. */
int kivi_decode_attention_noalloc(const kivi_config* cfg, const kivi_attn_cache* cache,
                                  int64_t n_slices, int32_t q_per_kv, const void* q_fp16,
                                  float sm_scale, void* out_fp16, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */
