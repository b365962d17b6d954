// HIP kernels of libkivi for gfx950 (MI355X), and their launchers.
//
// The codec (CacheForge README, "How it works"; CacheSeek PR #4 "Feature
// (quantization): add KIVI KV-cache quantization for exact-prefix reuse"):
// keys are quantized per channel over groups of G tokens, values per token
// over groups of G channels, each group with an fp16 scale and zero taken
// from its min and max, codes of b bits packed LSB-first into 32-bit words,
// partial groups padded with code 0.  Arithmetic (the reading the pages
// leave open, stated once): scale = fp16(fp32(fp32(mx - mn) / (2^b - 1))),
// zero = mn, q = clamp(rint(fp32(fp32(x - zero) / scale)), 0, 2^b - 1) with
// round-half-even and IEEE division, q = 0 when scale == 0, and
// xhat = fp16(fp32(q * scale + zero)).
//
// Everything here is HBM-bandwidth bound (about 2.4-3.1 bytes moved per
// element each way), so there is no MFMA: the design goals are full-width
// (16-byte) coalesced global accesses, cheap cross-lane reductions, and as
// few VALU instructions per element as the exact arithmetic allows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_launch.h"

namespace kivi {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte access
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
constexpr int kMaxGrid = 1 << 22;

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float lo_f32(uint32_t u) {
    return (float)__builtin_bit_cast(f16, (uint16_t)(u & 0xFFFFu));
}
__device__ __forceinline__ float hi_f32(uint32_t u) {
    return (float)__builtin_bit_cast(f16, (uint16_t)(u >> 16));
}
__device__ __forceinline__ f16x2 pmin(f16x2 a, f16x2 b) { return __builtin_elementwise_min(a, b); }
__device__ __forceinline__ f16x2 pmax(f16x2 a, f16x2 b) { return __builtin_elementwise_max(a, b); }

// Exchange within the wave (all lanes active).  CTRL is a DPP control word:
// 0xB1 = quad_perm[1,0,3,2] (lane ^ 1), 0x4E = quad_perm[2,3,0,1] (lane ^ 2),
// 0x141 = row_half_mirror (within 8 lanes), 0x140 = row_mirror (within 16).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Per-group quantization parameters.
struct QParams {
    float zero;     // the group minimum, +0 for a zero of either sign
    float scale;    // fp16 scale widened to fp32
    float rcp;      // ~1/scale (within 1 ulp), 0 when scale == 0
    float nzr;      // -fp32(zero * rcp)
    bool fast;      // the fast path below is exact for this group
};

// Statistics -> parameters.  mn/mx are fp16 values held in fp32 (exact).
//   scale = fp16(fp32(fp32(mx - mn) / (2^b - 1)))
// The fp32 quotient is computed as fp32(fp64(rng) * fp64(1/(2^b-1))): for any
// fp32 rng the fp64 product is within 2^-52 (relative) of rng/(2^b-1), while
// rng/(2^b-1) for an odd divisor below 2^8 is never within 2^-41 of an fp32
// rounding midpoint, so the final rounding equals that of the exact quotient.
// The empty asm keeps the fp32 step: without it the compiler merges the two
// narrowing conversions into one fp64->fp16 rounding, a different result.
template <int BITS>
__device__ __forceinline__ QParams make_params(float mn, float mx, uint32_t& scale_bits,
                                               uint32_t& zero_bits) {
    constexpr double kInvLevels = 1.0 / (double)((1 << BITS) - 1);
    mn = mn + 0.0f;                       // -0 -> +0 (round-to-nearest)
    mx = mx + 0.0f;
    // Keep both canonical values: otherwise (-y + 0) - mn may be rewritten as
    // -y - mn, which yields -0 for an all-zero group.
    asm volatile("" : "+v"(mn), "+v"(mx));
    const float rng = mx - mn;
    float s32 = (float)((double)rng * kInvLevels);
    asm volatile("" : "+v"(s32));
    const f16 sh = (f16)s32;
    QParams p;
    p.scale = (float)sh;
    p.zero = mn;
    p.rcp = (p.scale == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(p.scale);
    const float zr = mn * p.rcp;
    p.nzr = -zr;
    p.fast = (p.scale >= 0x1p-14f) && (__builtin_fabsf(zr) <= 1024.0f);
    scale_bits = __builtin_bit_cast(uint16_t, sh);
    zero_bits = __builtin_bit_cast(uint16_t, (f16)mn);
    return p;
}

// Code of one element by the definition: IEEE fp32 division (correctly
// rounded: no fast-math), round half to even, clamp; 0 when scale == 0.
template <int BITS>
__device__ __forceinline__ uint32_t quant_exact(float x, const QParams& p) {
    constexpr float kTop = (float)((1 << BITS) - 1);
    const float d = x - p.zero;
    const float q = __builtin_fminf(__builtin_rintf(d / p.scale), kTop);
    return (p.scale == 0.0f) ? 0u : (uint32_t)q;
}

// Fast path for groups with p.fast: y = fp32(x * rcp - zr) in one fma (x is
// the fp16 input, widened inside the instruction).  Let q = (x - zero)/s be
// the exact quotient.  A normal fp16 scale s is within 2^-11 (relative) of
// (mx - mn)/(2^b - 1), so 0 <= q <= (2^b - 1)(1 + 2^-10) < 256.  Error terms:
// the final rounding of y, 2^-24|y| <= 2^-16; zr = fp32(zero*rcp) with
// |zr| <= 2^10, 2^-14; rcp within 1 ulp (2^-23 relative) of 1/s, 2^-23 q <=
// 2^-15.  The definition's Q = fp32(fp32(x - zero)/s) is within 2^-23 q of
// q.  So |y - Q| <= 0.57 * 2^-12: rint(y) == rint(Q) unless y lies within
// 2^-12 of a half-integer, where the exact path decides, and rint(y) never
// exceeds 2^b - 1, so no clamp is needed.
template <int BITS>
__device__ __forceinline__ uint32_t quant_fast(float x, const QParams& p) {
    const float y = __builtin_fmaf(x, p.rcp, p.nzr);
    const float r = __builtin_rintf(y);
    uint32_t q = (uint32_t)r;
    if (__builtin_fabsf(y - r) > 0.5f - 0x1p-12f) q = quant_exact<BITS>(x, p);
    return q;
}

// Codes of N elements x(i) of one group, as floats (exact small integers,
// ready for packing by fp32 accumulation).  Fast groups take a branch-free
// pass that also records the largest |y - rint(y)|; only when some element
// came within 2^-12 of a half-integer (rare) is the pass redone with the
// per-element check of quant_fast.
template <int BITS, int N, typename X>
__device__ __forceinline__ void quant_n(X x, const QParams& p, float* q) {
    if (p.fast) {
        float worst = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float y = __builtin_fmaf(x(i), p.rcp, p.nzr);
            const float r = __builtin_rintf(y);
            q[i] = r;
            worst = __builtin_fmaxf(worst, __builtin_fabsf(y - r));
        }
        if (worst > 0.5f - 0x1p-12f) {
#pragma unroll
            for (int i = 0; i < N; ++i) q[i] = (float)quant_fast<BITS>(x(i), p);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) q[i] = (float)quant_exact<BITS>(x(i), p);
    }
}

// fp16 of fp32(q * scale + zero); q * scale is exact in fp32, so the fma
// rounds once to fp32.  The empty asm keeps that fp32 result from being
// fused with the narrowing conversion into a single rounding to fp16.
__device__ __forceinline__ f16 dequant1(uint32_t q, float scale, float zero) {
    float y = __builtin_fmaf((float)q, scale, zero);
    asm volatile("" : "+v"(y));
    return (f16)y;
}

// ---------------------------------------------------------------------------
// keys: one channel pair of one key group (G tokens) per thread
// ---------------------------------------------------------------------------

// Quantizes channels 2p, 2p+1 of one key group, whose token t (as an fp16
// pair) `load(t)` returns, with `nv` valid tokens, and stores its W code words per
// channel and both sidecars.  `grp` is the group's index in the (slice,
// group) output arrays.  Both channels are quantized in one pass over the
// tokens and packed as they go, so only the staged values stay live; the
// pass is redone with per-element checks only when some element came within
// 2^-12 of a rounding tie (see quant_fast).
template <int BITS, int G, bool FULL, typename Load>
__device__ __forceinline__ void key_column(Load load, int nv, int D, int p, int64_t grp,
                                           uint32_t* __restrict__ codes,
                                           uint16_t* __restrict__ scale,
                                           uint16_t* __restrict__ zero) {
    constexpr int W = G * BITS / 32;
    constexpr int PER = 32 / BITS;
    uint32_t v[G];
#pragma unroll
    for (int t = 0; t < G; ++t) v[t] = load(FULL ? t : (t < nv ? t : nv - 1));
    f16x2 mn = as_h2(v[0]), mx = mn;
#pragma unroll
    for (int t = 1; t < G; ++t) {
        mn = pmin(mn, as_h2(v[t]));
        mx = pmax(mx, as_h2(v[t]));
    }
    uint32_t sb0, zb0, sb1, zb1;
    const QParams p0 = make_params<BITS>((float)mn.x, (float)mx.x, sb0, zb0);
    const QParams p1 = make_params<BITS>((float)mn.y, (float)mx.y, sb1, zb1);
    uint32_t w0[W], w1[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
        w0[w] = 0;
        w1[w] = 0;
    }
    if (p0.fast && p1.fast) {
        // Codes are packed as they are made: at b = 2 and 4 they accumulate
        // in fp32 as sum(code * 2^(b*k)) over 16-bit half words (exact),
        // one fma each instead of a conversion, a shift and an OR; at b = 8
        // each goes into its byte with v_cvt_pk_u8_f32.  Near-ties (see
        // quant_fast) are tracked per segment of 4 tokens, and only flagged
        // segments are checked again element by element: with 64 lanes x
        // 64 elements per wave, most waves hold some element within 2^-12 of
        // a tie, so a second pass over whole lanes would run in most waves.
        constexpr int TH = BITS == 8 ? 2 : 16 / BITS;     // tokens per 16-bit half word
        constexpr int SEG = 4;                            // tokens per near-tie segment
        constexpr float kNear = 0.5f - 0x1p-12f;
        float h0[2 * W], h1[2 * W];
#pragma unroll
        for (int k = 0; k < 2 * W; ++k) {
            h0[k] = 0.0f;
            h1[k] = 0.0f;
        }
        auto put = [&](int t, float c0, float c1) {
            if constexpr (BITS == 8) {
                w0[t / PER] = __builtin_amdgcn_cvt_pk_u8_f32(c0, t % PER, w0[t / PER]);
                w1[t / PER] = __builtin_amdgcn_cvt_pk_u8_f32(c1, t % PER, w1[t / PER]);
            } else {
                const float wt = (float)(1u << (BITS * (t % TH)));
                h0[t / TH] = __builtin_fmaf(c0, wt, h0[t / TH]);
                h1[t / TH] = __builtin_fmaf(c1, wt, h1[t / TH]);
            }
        };
#pragma unroll
        for (int sg = 0; sg < G / SEG; ++sg) {
            float worst = 0.0f;
#pragma unroll
            for (int t = SEG * sg; t < SEG * sg + SEG; ++t) {
                const float y0 = __builtin_fmaf(lo_f32(v[t]), p0.rcp, p0.nzr);
                const float y1 = __builtin_fmaf(hi_f32(v[t]), p1.rcp, p1.nzr);
                float r0 = __builtin_rintf(y0);
                float r1 = __builtin_rintf(y1);
                if (FULL || t < nv) {
                    worst = __builtin_fmaxf(worst, __builtin_fmaxf(__builtin_fabsf(y0 - r0),
                                                                   __builtin_fabsf(y1 - r1)));
                } else {
                    r0 = 0.0f;
                    r1 = 0.0f;
                }
                put(t, r0, r1);
            }
            if (__builtin_expect(worst > kNear, 0)) {
#pragma unroll
                for (int t = SEG * sg; t < SEG * sg + SEG; ++t) {
                    if (!FULL && t >= nv) continue;
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch) {
                        const QParams& q = ch ? p1 : p0;
                        const float x = ch ? hi_f32(v[t]) : lo_f32(v[t]);
                        const float y = __builtin_fmaf(x, q.rcp, q.nzr);
                        const float rr = __builtin_rintf(y);
                        if (__builtin_fabsf(y - rr) > kNear) {
                            const float c = (float)quant_exact<BITS>(x, q);
                            if constexpr (BITS == 8) {
                                uint32_t& wd = ch ? w1[t / PER] : w0[t / PER];
                                wd = __builtin_amdgcn_cvt_pk_u8_f32(c, t % PER, wd);
                            } else {
                                float& hk = ch ? h1[t / TH] : h0[t / TH];
                                hk = __builtin_fmaf(c - rr, (float)(1u << (BITS * (t % TH))), hk);
                            }
                        }
                    }
                }
            }
        }
        if constexpr (BITS != 8) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                w0[w] = (uint32_t)h0[2 * w] | ((uint32_t)h0[2 * w + 1] << 16);
                w1[w] = (uint32_t)h1[2 * w] | ((uint32_t)h1[2 * w + 1] << 16);
            }
        }
    } else {
        // a channel outside the fast path: every element by the definition
        // (or by quant_fast for the other channel)
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const float x0 = lo_f32(v[t]), x1 = hi_f32(v[t]);
            uint32_t c0 = p0.fast ? quant_fast<BITS>(x0, p0) : quant_exact<BITS>(x0, p0);
            uint32_t c1 = p1.fast ? quant_fast<BITS>(x1, p1) : quant_exact<BITS>(x1, p1);
            if (!FULL && t >= nv) {
                c0 = 0;
                c1 = 0;
            }
            w0[t / PER] |= c0 << ((t % PER) * BITS);
            w1[t / PER] |= c1 << ((t % PER) * BITS);
        }
    }
    // streaming stores: the payload is not read again by this launch
    uint32_t* cdst = codes + grp * (int64_t)(W * D) + 2 * p;
#pragma unroll
    for (int w = 0; w < W; ++w)
        __builtin_nontemporal_store(u32x2{w0[w], w1[w]}, reinterpret_cast<u32x2*>(cdst + w * D));
    __builtin_nontemporal_store(sb0 | (sb1 << 16),
                                reinterpret_cast<uint32_t*>(scale + grp * D + 2 * p));
    __builtin_nontemporal_store(zb0 | (zb1 << 16),
                                reinterpret_cast<uint32_t*>(zero + grp * D + 2 * p));
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, no stride).  Loads
// through it take the wave-uniform part of the address in scalar registers,
// so per-load address arithmetic costs no vector instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr int kNontemporal = 2;   // buffer-load cache policy: streaming, do not keep

// XCD-aware block order.  MI355X has 8 XCDs (each with its own L2), and the
// dispatcher hands workgroup i to XCD i mod 8, so with the identity order
// neighbouring work items (neighbouring stretches of HBM) go to eight
// different XCDs.  This returns the work item of this workgroup such that
// each XCD takes runs of RUN consecutive items: within every super-chunk of
// 8*RUN workgroups, XCD x gets items [x*RUN, x*RUN + RUN).  Workgroups past
// the last whole super-chunk keep their own index, so the map is a bijection
// of [0, gridDim.x) and a grid-stride loop over it still visits every item
// once.  (Key encode, Llama-2-7B shape: 1.76-1.80 -> 1.65-1.67 ms at RUN 16
// or 128; value encode 2-4% faster at RUN 128, value decode 1.5% at RUN 16;
// key decode gains nothing and keeps the identity order.)
template <int RUN>
__device__ __forceinline__ int64_t xcd_block() {
    constexpr int64_t kChunk = 8 * (int64_t)RUN;
    const int64_t b = blockIdx.x;
    if (b >= (int64_t)(gridDim.x / kChunk) * kChunk) return b;
    return (b / kChunk) * kChunk + (b % 8) * RUN + (b / 8) % RUN;
}

// Full-cache key encode, full groups.  Thread (ti, p) of a block owns channel
// pair p of key group g0 + ti of one slice, for all G tokens of the group:
// token t is one dword, and the lanes of a wave read whole token rows (D/2
// consecutive dwords, 256 bytes at D = 128), so every load is coalesced.  The
// G values stay in registers for the statistics and the codes.  (Staging the
// tile in LDS with 16-byte loads, or with direct-to-LDS loads, measured
// slower: each lane needs its whole column in registers anyway.)  The
// partial last group of each slice is left to encode_k_tail_kernel, so this
// loop has no bounds logic at all.
template <int BITS, int G>
__global__ void __launch_bounds__(kBlock)
encode_k_kernel(const uint16_t* __restrict__ in, int64_t in_stride, int D, int ng_full, int tpb,
                int batches_per_slice, int64_t n_batches, uint32_t* __restrict__ codes,
                uint16_t* __restrict__ scale, uint16_t* __restrict__ zero, int out_groups) {
    const int half_d = D >> 1;
    const int tid = threadIdx.x;
    const int ti = tid / half_d;
    const int p = tid - ti * half_d;
    if (ti >= tpb) return;
    const int voff = (ti * G * D + 2 * p) * 2;          // bytes from the batch base
    const int row_bytes = D * 2;
    for (int64_t batch = xcd_block<16>(); batch < n_batches; batch += gridDim.x) {
        const int64_t s = batch / batches_per_slice;
        const int g0 = (int)(batch - s * batches_per_slice) * tpb;
        const int g = g0 + ti;
        if (g >= ng_full) continue;
        const __amdgpu_buffer_rsrc_t rsrc =
            buffer_rsrc(in + s * in_stride + (int64_t)g0 * G * D, (uint32_t)(tpb * G * row_bytes));
        auto load = [&](int t) {
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, t * row_bytes,
                                                                   kNontemporal);
        };
        key_column<BITS, G, true>(load, G, D, p, s * out_groups + g, codes, scale, zero);
    }
}

// The partial last key group (n_tokens % G valid tokens) of every slice.
template <int BITS, int G>
__global__ void __launch_bounds__(kBlock)
encode_k_tail_kernel(const uint16_t* __restrict__ in, int64_t in_stride, int n_tokens, int D,
                     int64_t n_slices, uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
                     uint16_t* __restrict__ zero, int out_groups) {
    const int half_d = D >> 1;
    const int tpb = kBlock / half_d;
    const int ti = threadIdx.x / half_d;
    const int p = threadIdx.x - ti * half_d;
    const int64_t s = (int64_t)blockIdx.x * tpb + ti;
    if (ti >= tpb || s >= n_slices) return;
    const int g = n_tokens / G;
    const int nv = n_tokens - g * G;
    const uint32_t* col =
        reinterpret_cast<const uint32_t*>(in + s * in_stride + (int64_t)g * G * D) + p;
    auto load = [&](int t) { return col[t * half_d]; };
    key_column<BITS, G, false>(load, nv, D, p, s * out_groups + g, codes, scale, zero);
}

// ---------------------------------------------------------------------------
// values: one 8-channel chunk of one token row per lane
// ---------------------------------------------------------------------------

// Lane c of a token row (lanes-per-row a power of two >= G/8) holds channels
// 8c .. 8c+7 in `x`; lanes c >= D/8 are padding (`cvalid` false).  All lanes
// of the wave must call this together (DPP reductions inside).  Stores the
// row's code words and, from the first lane of each group, its sidecars,
// when `store` is set.
template <int BITS, int G, bool ALL = false>
__device__ __forceinline__ void value_chunk(const u32x4& x, bool cvalid, int c, bool store,
                                            uint32_t* __restrict__ row_codes,
                                            uint16_t* __restrict__ row_scale,
                                            uint16_t* __restrict__ row_zero) {
    constexpr int GL = G / 8;                 // lanes per value group
    const f16x2 a0 = as_h2(x.x), a1 = as_h2(x.y), a2 = as_h2(x.z), a3 = as_h2(x.w);
    const f16x2 mn2 = pmin(pmin(a0, a1), pmin(a2, a3));
    const f16x2 mx2 = pmax(pmax(a0, a1), pmax(a2, a3));
    f16 mn = mn2.x < mn2.y ? mn2.x : mn2.y;
    f16 mx = mx2.x > mx2.y ? mx2.x : mx2.y;
    if (!ALL && !cvalid) {
        mn = (f16)__builtin_inff();
        mx = (f16)(-__builtin_inff());
    }
    // reduce (min, -max) over the group's lanes with one packed min per step
    f16x2 pr;
    pr.x = mn;
    pr.y = -mx;
    uint32_t pu = as_u32(pr);
    if (GL >= 2) pu = as_u32(pmin(as_h2(pu), as_h2(dpp<0xB1>(pu))));
    if (GL >= 4) pu = as_u32(pmin(as_h2(pu), as_h2(dpp<0x4E>(pu))));
    if (GL >= 8) pu = as_u32(pmin(as_h2(pu), as_h2(dpp<0x141>(pu))));
    if (GL >= 16) pu = as_u32(pmin(as_h2(pu), as_h2(dpp<0x140>(pu))));
    pr = as_h2(pu);
    uint32_t sb, zb;
    const QParams prm = make_params<BITS>((float)pr.x, -(float)pr.y, sb, zb);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
    float q[8];
    quant_n<BITS, 8>([&](int i) { return (i & 1) ? hi_f32(xs[i >> 1]) : lo_f32(xs[i >> 1]); }, prm, q);
    if (!ALL && !cvalid) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = 0.0f;
    }
    // codes packed by fp32 accumulation over 16-bit half words (exact), or
    // into bytes with v_cvt_pk_u8_f32
    if (BITS == 4) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a0 = __builtin_fmaf(q[i], (float)(1u << (4 * i)), a0);
            a1 = __builtin_fmaf(q[4 + i], (float)(1u << (4 * i)), a1);
        }
        const uint32_t w = (uint32_t)a0 | ((uint32_t)a1 << 16);
        if (store) __builtin_nontemporal_store(w, row_codes + c);
    } else if (BITS == 8) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w0 = __builtin_amdgcn_cvt_pk_u8_f32(q[i], i, w0);
            w1 = __builtin_amdgcn_cvt_pk_u8_f32(q[4 + i], i, w1);
        }
        if (store)
            __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(row_codes + 2 * c));
    } else {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = __builtin_fmaf(q[i], (float)(1u << (2 * i)), a);
        const uint32_t h = (uint32_t)a;
        const uint32_t nb = dpp<0xB1>(h);
        if (store && (c & 1) == 0) __builtin_nontemporal_store(h | (nb << 16), row_codes + (c >> 1));
    }
    if (store && (c % GL) == 0) {
        row_scale[c / GL] = (uint16_t)sb;
        row_zero[c / GL] = (uint16_t)zb;
    }
}

// Full-cache value encode: a block covers `rows_per_block` token rows of one
// slice; 2^lpt_log2 lanes per row.
// ALL: every lane of a row holds 8 real channels that belong to a stored
// group (D/8 is the lane count and G divides D), so no padding logic.
template <int BITS, int G, bool ALL>
__global__ void __launch_bounds__(kBlock)
encode_v_kernel(const uint16_t* __restrict__ in, int64_t in_stride, int n_tokens, int D,
                int lpt_log2, int rows_per_block, int blocks_per_slice, int64_t n_blocks,
                uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
                uint16_t* __restrict__ zero, int cap, int ngv) {
    constexpr int GL = G / 8;
    const int lpt = 1 << lpt_log2;
    const int c = threadIdx.x & (lpt - 1);
    const int r0 = threadIdx.x >> lpt_log2;
    const int rstep = kBlock >> lpt_log2;
    const bool cvalid = ALL || c < (D >> 3);
    const bool in_group = ALL || (c / GL) < ngv;
    const int wpt = ngv * G * BITS / 32;
    for (int64_t blk = xcd_block<128>(); blk < n_blocks; blk += gridDim.x) {
        const int64_t s = blk / blocks_per_slice;
        const int tb = (int)(blk - s * blocks_per_slice) * rows_per_block;
        const uint16_t* src = in + s * in_stride;
        for (int r = r0; r < rows_per_block; r += rstep) {
            const int t = tb + r;
            const bool rvalid = t < n_tokens;
            u32x4 x = u32x4{0, 0, 0, 0};
            if (rvalid && cvalid)
                x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)t * D + 8 * c));
            const int64_t row = s * cap + t;
            value_chunk<BITS, G, ALL>(x, cvalid, c, rvalid && in_group, codes + row * wpt,
                                      scale + row * ngv, zero + row * ngv);
        }
    }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

__device__ __forceinline__ void widen8(const u32x4& h, float* f) {
    const uint32_t u[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo_f32(u[i]);
        f[2 * i + 1] = hi_f32(u[i]);
    }
}

__device__ __forceinline__ uint32_t pack2(f16 a, f16 b) {
    f16x2 h;
    h.x = a;
    h.y = b;
    return as_u32(h);
}

// Keys: lane c of a tile owns channels 8c..8c+7 of one group for all its
// tokens; per token it writes 16 bytes of the token-major output.  Full groups
// (all but a slice's last) take a path without conditions.
template <int BITS, int G, bool FULL>
__device__ __forceinline__ void decode_k_group(const uint32_t* __restrict__ src,
                                               const uint16_t* __restrict__ sc16,
                                               const uint16_t* __restrict__ zr16, int nv, int D,
                                               uint16_t* __restrict__ dst) {
    constexpr int W = G * BITS / 32;
    constexpr int PER = 32 / BITS;
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    float sf[8], zf[8];
    widen8(*reinterpret_cast<const u32x4*>(sc16), sf);
    widen8(*reinterpret_cast<const u32x4*>(zr16), zf);
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(src + w * D);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(src + w * D + 4);
        const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = w * PER + i;
            if (FULL || t < nv) {
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t q0 = (wd[2 * k] >> (i * BITS)) & kMask;
                    const uint32_t q1 = (wd[2 * k + 1] >> (i * BITS)) & kMask;
                    o[k] = pack2(dequant1(q0, sf[2 * k], zf[2 * k]),
                                 dequant1(q1, sf[2 * k + 1], zf[2 * k + 1]));
                }
                __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]},
                                            reinterpret_cast<u32x4*>(dst + (int64_t)t * D));
            }
        }
    }
}

template <int BITS, int G>
__global__ void __launch_bounds__(kBlock)
decode_k_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
                const uint16_t* __restrict__ zero, int n_tokens, int D, int ng, int out_groups,
                int tiles_per_block, int64_t n_tiles, int64_t n_blocks, uint16_t* __restrict__ out,
                int64_t out_stride) {
    constexpr int W = G * BITS / 32;
    const int cpr = D >> 3;
    const int ti = threadIdx.x / cpr;
    const int c = threadIdx.x - ti * cpr;
    if (ti >= tiles_per_block) return;
    for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
        const int64_t tile = blk * tiles_per_block + ti;
        if (tile >= n_tiles) continue;
        const int64_t s = tile / ng;
        const int g = (int)(tile - s * ng);
        const int nv = min(G, n_tokens - g * G);
        const int64_t grp = s * out_groups + g;
        const uint32_t* src = codes + grp * (int64_t)(W * D) + 8 * c;
        const uint16_t* sc = scale + grp * D + 8 * c;
        const uint16_t* zr = zero + grp * D + 8 * c;
        uint16_t* dst = out + s * out_stride + (int64_t)g * G * D + 8 * c;
        if (nv == G)
            decode_k_group<BITS, G, true>(src, sc, zr, nv, D, dst);
        else
            decode_k_group<BITS, G, false>(src, sc, zr, nv, D, dst);
    }
}

constexpr int kRowsPerThread = 4;

// Values: lane c of a token row owns channels 8c..8c+7; each thread loads the
// codes and sidecars of its kRowsPerThread rows before decoding them.  Blocks
// whose rows are all valid (all but the last block of a slice) run without
// any condition, so the scheduler can issue every load before the first use.
template <int BITS, int G, bool FULL>
__device__ __forceinline__ void decode_v_rows(const uint32_t* __restrict__ codes,
                                              const uint16_t* __restrict__ scale,
                                              const uint16_t* __restrict__ zero, int64_t s,
                                              int tb, int rstep, int n_tokens, int D, int c,
                                              int cap, int ngv, uint16_t* __restrict__ out,
                                              int64_t out_stride) {
    constexpr int GL = G / 8;
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    const int wpt = ngv * G * BITS / 32;
    const int gi = c / GL;
    u32x2 wd[kRowsPerThread];
    float sc[kRowsPerThread], zr[kRowsPerThread];
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
        // past the end, re-read the last row (not stored)
        const int t = FULL ? tb + j * rstep : min(tb + j * rstep, n_tokens - 1);
        const int64_t row = s * cap + t;
        const uint32_t* rc = codes + row * wpt;
        if (BITS == 8) {
            wd[j] = *reinterpret_cast<const u32x2*>(rc + 2 * c);
        } else {
            wd[j].x = (BITS == 4) ? rc[c] : (rc[c >> 1] >> ((c & 1) * 16));
            wd[j].y = 0;
        }
        sc[j] = (float)__builtin_bit_cast(f16, scale[row * ngv + gi]);
        zr[j] = (float)__builtin_bit_cast(f16, zero[row * ngv + gi]);
    }
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
        const int t = tb + j * rstep;
        uint32_t q[8];
        if (BITS == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                q[i] = (wd[j].x >> (8 * i)) & kMask;
                q[4 + i] = (wd[j].y >> (8 * i)) & kMask;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = (wd[j].x >> (BITS * i)) & kMask;
        }
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = pack2(dequant1(q[2 * k], sc[j], zr[j]), dequant1(q[2 * k + 1], sc[j], zr[j]));
        if (FULL || t < n_tokens)
            __builtin_nontemporal_store(
                u32x4{o[0], o[1], o[2], o[3]},
                reinterpret_cast<u32x4*>(out + s * out_stride + (int64_t)t * D + 8 * c));
    }
}

template <int BITS, int G>
__global__ void __launch_bounds__(kBlock)
decode_v_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
                const uint16_t* __restrict__ zero, int n_tokens, int D, int lpt_log2,
                int blocks_per_slice, int64_t n_blocks, int cap, int ngv,
                uint16_t* __restrict__ out, int64_t out_stride) {
    const int lpt = 1 << lpt_log2;
    const int c = threadIdx.x & (lpt - 1);
    const int r0 = threadIdx.x >> lpt_log2;
    const int rstep = kBlock >> lpt_log2;
    const int rows_per_block = kRowsPerThread * rstep;
    if (c >= (D >> 3)) return;
    for (int64_t blk = xcd_block<16>(); blk < n_blocks; blk += gridDim.x) {
        const int64_t s = blk / blocks_per_slice;
        const int row0 = (int)(blk - s * blocks_per_slice) * rows_per_block;
        if (row0 + rows_per_block <= n_tokens)
            decode_v_rows<BITS, G, true>(codes, scale, zero, s, row0 + r0, rstep, n_tokens, D, c,
                                         cap, ngv, out, out_stride);
        else
            decode_v_rows<BITS, G, false>(codes, scale, zero, s, row0 + r0, rstep, n_tokens, D, c,
                                          cap, ngv, out, out_stride);
    }
}

// Value encode at G = 32 when every lane of a row holds 8 channels of a
// stored group (D % 32 == 0, D/8 lanes per row): each lane takes 4 rows,
// r0 + k*rstep for k = 0..3.  A group is a quad of lanes, and after the
// quad's min/max reduction all four lanes know the statistics of all four
// rows' groups; lane e of the quad derives the parameters of row e's group
// only and the quad broadcasts them back (DPP), so each group's parameters
// cost one lane instead of four: the encoder is short of VALU issue
// slots, not of bandwidth.  Codes as in value_chunk; rows past n_tokens are
// coded from zeros and not stored.
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, K * 0x55, 0xF, 0xF, false);
}

template <int BITS>
__global__ void __launch_bounds__(kBlock)
encode_v_quad_kernel(const uint16_t* __restrict__ in, int64_t in_stride, int n_tokens, int D, int lpt_log2,
                     int blocks_per_slice, int64_t n_blocks, uint32_t* __restrict__ codes,
                     uint16_t* __restrict__ scale, uint16_t* __restrict__ zero, int cap) {
    constexpr int G = 32;
    const int lpt = 1 << lpt_log2;
    const int c = threadIdx.x & (lpt - 1);
    const int r0 = threadIdx.x >> lpt_log2;
    const int rstep = kBlock >> lpt_log2;
    const int rows_per_block = 4 * rstep;
    const int e = c & 3, gq = c >> 2;
    const int ngv = D / G;
    const int wpt = D * BITS / 32;
    for (int64_t blk = xcd_block<128>(); blk < n_blocks; blk += gridDim.x) {
        const int64_t s = blk / blocks_per_slice;
        const int tb = (int)(blk - s * blocks_per_slice) * rows_per_block + r0;
        const uint16_t* src = in + s * in_stride;
        u32x4 x[4];
        uint32_t pr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = tb + k * rstep;
            x[k] = u32x4{0, 0, 0, 0};
            if (t < n_tokens)
                x[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)t * D + 8 * c));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f16x2 a0 = as_h2(x[k].x), a1 = as_h2(x[k].y), a2 = as_h2(x[k].z), a3 = as_h2(x[k].w);
            const f16x2 mn2 = pmin(pmin(a0, a1), pmin(a2, a3));
            const f16x2 mx2 = pmax(pmax(a0, a1), pmax(a2, a3));
            f16x2 p2;
            p2.x = mn2.x < mn2.y ? mn2.x : mn2.y;
            p2.y = -(mx2.x > mx2.y ? mx2.x : mx2.y);
            uint32_t pu = as_u32(p2);
            pu = as_u32(pmin(as_h2(pu), as_h2(dpp<0xB1>(pu))));
            pr[k] = as_u32(pmin(as_h2(pu), as_h2(dpp<0x4E>(pu))));
        }
        // lane e: the parameters of row e's group
        const f16x2 pe = as_h2(e == 0 ? pr[0] : e == 1 ? pr[1] : e == 2 ? pr[2] : pr[3]);
        uint32_t sb, zb;
        const QParams prm = make_params<BITS>((float)pe.x, -(float)pe.y, sb, zb);
        // outside the fast path: 1/scale = 0, -zero/scale = 1/2, so that
        // every element takes the exact branch below
        const uint32_t rcp_e = __builtin_bit_cast(uint32_t, prm.fast ? prm.rcp : 0.0f);
        const uint32_t nzr_e = __builtin_bit_cast(uint32_t, prm.fast ? prm.nzr : 0.5f);
        const uint32_t sz_e = sb | (zb << 16);
        {
            const int te = tb + e * rstep;
            if (te < n_tokens) {
                const int64_t row = s * cap + te;
                scale[row * ngv + gq] = (uint16_t)sb;
                zero[row * ngv + gq] = (uint16_t)zb;
            }
        }
        auto code_row = [&](int k, uint32_t rcpb, uint32_t nzrb, uint32_t sz) {
            const float rcp = __builtin_bit_cast(float, rcpb), nzr = __builtin_bit_cast(float, nzrb);
            const uint32_t xs[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
            auto xv = [&](int i) { return (i & 1) ? hi_f32(xs[i >> 1]) : lo_f32(xs[i >> 1]); };
            float q[8];
            float worst = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float y = __builtin_fmaf(xv(i), rcp, nzr);
                q[i] = __builtin_rintf(y);
                worst = __builtin_fmaxf(worst, __builtin_fabsf(y - q[i]));
            }
            if (__builtin_expect(worst > 0.5f - 0x1p-12f, 0)) {
                QParams qp;
                qp.scale = (float)__builtin_bit_cast(f16, (uint16_t)(sz & 0xFFFFu));
                qp.zero = (float)__builtin_bit_cast(f16, (uint16_t)(sz >> 16));
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float y = __builtin_fmaf(xv(i), rcp, nzr);
                    if (__builtin_fabsf(y - q[i]) > 0.5f - 0x1p-12f) q[i] = (float)quant_exact<BITS>(xv(i), qp);
                }
            }
            const int t = tb + k * rstep;
            const bool store = t < n_tokens;
            uint32_t* row_codes = codes + (s * cap + t) * (int64_t)wpt;
            if (BITS == 4) {
                float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a0 = __builtin_fmaf(q[i], (float)(1u << (4 * i)), a0);
                    a1 = __builtin_fmaf(q[4 + i], (float)(1u << (4 * i)), a1);
                }
                if (store) __builtin_nontemporal_store((uint32_t)a0 | ((uint32_t)a1 << 16), row_codes + c);
            } else if (BITS == 8) {
                uint32_t w0 = 0, w1 = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    w0 = __builtin_amdgcn_cvt_pk_u8_f32(q[i], i, w0);
                    w1 = __builtin_amdgcn_cvt_pk_u8_f32(q[4 + i], i, w1);
                }
                if (store)
                    __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(row_codes + 2 * c));
            } else {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) a = __builtin_fmaf(q[i], (float)(1u << (2 * i)), a);
                const uint32_t h = (uint32_t)a;
                const uint32_t nb = dpp<0xB1>(h);
                if (store && (c & 1) == 0) __builtin_nontemporal_store(h | (nb << 16), row_codes + (c >> 1));
            }
        };
        code_row(0, quad_bcast<0>(rcp_e), quad_bcast<0>(nzr_e), quad_bcast<0>(sz_e));
        code_row(1, quad_bcast<1>(rcp_e), quad_bcast<1>(nzr_e), quad_bcast<1>(sz_e));
        code_row(2, quad_bcast<2>(rcp_e), quad_bcast<2>(nzr_e), quad_bcast<2>(sz_e));
        code_row(3, quad_bcast<3>(rcp_e), quad_bcast<3>(nzr_e), quad_bcast<3>(sz_e));
    }
}

// ---------------------------------------------------------------------------
// streaming: append one token per slice, optionally flush the oldest G
// ---------------------------------------------------------------------------

// Key flush: thread (ti, p) quantizes channel pair p of slice kblk*tpb + ti
// from the oldest G residual tokens.  The ring slot of residual token t is
// the same for every slice, so it is a scalar offset of a buffer load.
template <int BITS, int G>
__device__ __forceinline__ void flush_keys(const StepArgs& a, int tpb, int64_t kblk) {
    const int D = a.head_dim;
    const int half_d = D >> 1;
    const int tid = threadIdx.x;
    const int ti = tid / half_d;
    const int p = tid - ti * half_d;
    const int64_t s0 = kblk * tpb;
    const int64_t s = s0 + ti;
    if (ti >= tpb || s >= a.n_slices) return;
    const int row_bytes = D * 2;
    const int64_t nblk = (a.n_slices - s0 < tpb) ? a.n_slices - s0 : tpb;
    const __amdgpu_buffer_rsrc_t ring = buffer_rsrc(
        a.k_ring + s0 * a.ring_slots * (int64_t)D, (uint32_t)(nblk * a.ring_slots * row_bytes));
    const __amdgpu_buffer_rsrc_t fresh =
        buffer_rsrc(a.k_new + s0 * (int64_t)D, (uint32_t)(nblk * row_bytes));
    const int ring_off = (ti * a.ring_slots * D + 2 * p) * 2;
    const int new_off = (ti * D + 2 * p) * 2;
    auto load = [&](int t) {
        if (t == a.ring_count)      // the token appended by this same launch
            return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(fresh, new_off, 0, 0);
        int slot = a.ring_head + t;
        if (slot >= a.ring_slots) slot -= a.ring_slots;
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ring, ring_off, slot * row_bytes, 0);
    };
    const int out_groups = a.cap_tokens / G;
    key_column<BITS, G, true>(load, G, D, p, s * out_groups + a.n_quant / G, a.k_codes,
                              a.k_scale, a.k_zero);
}

// Key flush of the usual step (all G tokens already in the ring, and the
// group does not wrap around its end).  A tile is spb slices; lane (j, c)
// of a slice's (G/8) x (D/8) lanes holds channels 8c .. 8c+7 of tokens
// [8j, 8j + 8) of the group as 8 16-byte row chunks, so each load
// instruction of a wave reads whole rows.  The lanes of a channel chunk
// then (1) combine their partial min/max, (2) derive each channel pair's
// parameters once (lane j < 4 takes pair j) and share them, and (3) each
// code their own 8 x 8 elements; at b = 2 a lane's 8 tokens are half a
// code word, and each even lane ORs in its odd partner's upper halves.
// With D = 128 and G = 32 a slice is one wave whose four token octets are
// its four 16-lane rows, and all three exchanges stay inside the wave;
// other shapes exchange through LDS between workgroup barriers.  The
// 16-byte loads and the short dependency chain are what matter: 16,384
// slices (G = 32, D = 128) read their groups in 25 us with 16-byte loads
// against 33 us with the 4-byte loads of a lane-per-channel-pair layout,
// and coding through LDS took 38 us (caches cold).
constexpr int kFlushTokensPerLane = 8;

struct FlushParams {        // the 8 channels of one chunk
    float rcp[8];
    float nzr[8];
    uint32_t sbits[4];      // fp16 scale pairs
    uint32_t zbits[4];      // fp16 zero pairs
};

template <int NT>           // threads per block
struct FlushLds {
    union {
        struct {
            u32x4 mn[NT];   // partial minima, fp16 pairs of channels 8c .. 8c+7
            u32x4 mx[NT];
        } part;             // steps 1-2
        u32x4 w[2][NT];     // upper half code words of odd lanes (b = 2), step 3
    };
    FlushParams prm[NT / 4];    // one per chunk (G/8 >= 4 lanes each)
};

// Workgroup barrier over LDS: this wave's LDS accesses complete, then the
// barrier (global memory accesses are not waited for).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A lane's place in a flush tile.
template <int G>
struct FlushLane {
    static constexpr int J = G / kFlushTokensPerLane;   // lanes per channel chunk
    int cpr;        // chunks per row, D / 8
    int P;          // lanes per slice
    int si, j, c;   // slice in the tile, token octet, channel chunk
    int chunk;      // chunk index in the tile
    bool in_block;  // false for lanes past spb * P: they take part in the barriers only
    __device__ FlushLane(int D, int spb) {
        cpr = D >> 3;
        P = J * cpr;
        const int tid = threadIdx.x;
        si = tid / P;
        const int r = tid - si * P;
        j = r / cpr;
        c = r - j * cpr;
        chunk = si * cpr + c;
        in_block = si < spb;
    }
};

// Slice of this lane in tile kt (lanes of slices past the end read slice
// kt*spb, in bounds, and store nothing).
template <int G>
__device__ __forceinline__ int64_t flush_slice(const StepArgs& a, int spb, int64_t kt,
                                               const FlushLane<G>& ln, bool& live) {
    const int64_t s0 = kt * spb;
    live = ln.in_block && s0 + ln.si < a.n_slices;
    return s0 + (live ? ln.si : 0);
}

// Rows of tile kt through a buffer resource over the tile's slices: the
// tile base is scalar, each lane keeps one 32-bit offset and the row step
// is a scalar offset.
template <int G>
__device__ __forceinline__ void flush_load(const StepArgs& a, int spb, int64_t kt,
                                           const FlushLane<G>& ln, u32x4 (&x)[kFlushTokensPerLane]) {
    const int D = a.head_dim;
    const int row_bytes = 2 * D;
    const int64_t s0 = kt * spb;
    const int64_t nblk = (a.n_slices - s0 < spb) ? a.n_slices - s0 : spb;
    const __amdgpu_buffer_rsrc_t ring = buffer_rsrc(
        a.k_ring + s0 * a.ring_slots * (int64_t)D, (uint32_t)(nblk * a.ring_slots * row_bytes));
    const int si = (ln.in_block && ln.si < nblk) ? ln.si : 0;
    const int voff = (si * a.ring_slots + a.ring_head + kFlushTokensPerLane * ln.j) * row_bytes + 16 * ln.c;
#pragma unroll
    for (int i = 0; i < kFlushTokensPerLane; ++i)
        x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ring, voff, i * row_bytes,
                                                                               kNontemporal));
}

// Partial min/max of a lane's 8 channels (fp16 pairs) over its 8 tokens.
__device__ __forceinline__ void flush_minmax(const u32x4 (&x)[kFlushTokensPerLane], f16x2 (&mn)[4],
                                             f16x2 (&mx)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) mn[k] = mx[k] = as_h2(x[0][k]);
#pragma unroll
    for (int i = 1; i < kFlushTokensPerLane; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mn[k] = pmin(mn[k], as_h2(x[i][k]));
            mx[k] = pmax(mx[k], as_h2(x[i][k]));
        }
}

// Parameters of one channel pair from its fp16 min/max pair.  A channel
// outside the fast path gets 1/scale = 0, -zero/scale = 1/2: its y is then
// 1/2 for every element, which always takes the exact branch of
// flush_rows_code.
template <int BITS>
__device__ __forceinline__ void flush_pair_params(f16x2 mn, f16x2 mx, float& rcp0, float& rcp1,
                                                  float& nzr0, float& nzr1, uint32_t& sbits,
                                                  uint32_t& zbits) {
    uint32_t s0b, z0b, s1b, z1b;
    const QParams p0 = make_params<BITS>((float)mn.x, (float)mx.x, s0b, z0b);
    const QParams p1 = make_params<BITS>((float)mn.y, (float)mx.y, s1b, z1b);
    rcp0 = p0.fast ? p0.rcp : 0.0f;
    rcp1 = p1.fast ? p1.rcp : 0.0f;
    nzr0 = p0.fast ? p0.nzr : 0.5f;
    nzr1 = p1.fast ? p1.nzr : 0.5f;
    sbits = s0b | (s1b << 16);
    zbits = z0b | (z1b << 16);
}

// Codes of a lane's 8 tokens x 8 channels, packed as they are made: at
// b = 2 and 4 they accumulate in fp32 as sum(code * 2^(b*t)) over at most
// 16 bits, which is exact; at b = 8 each goes into its byte with
// v_cvt_pk_u8_f32.  Each row of 8 elements is coded branch-free and checked
// once (its largest |y - rint(y)|); a row with an element within 2^-12 of a
// rounding tie (see quant_fast), or of a channel outside the fast path, is
// checked again element by element, and each such element gets its code
// from the exact branch, which asks `bits(k)` for the fp16 scale and zero
// pairs of channel pair k.  On random data about one row in five per wave
// takes that branch.  w: b = 2, each channel's 16-bit half word in bits
// 0-15; b = 4, one word; b = 8, two.
template <int BITS, typename Bits>
__device__ __forceinline__ void flush_rows_code(const u32x4 (&x)[kFlushTokensPerLane], const float (&rcp)[8],
                                                const float (&nzr)[8], Bits bits,
                                                uint32_t (&w)[8][BITS == 8 ? 2 : 1]) {
    constexpr int NA = BITS == 4 ? 2 : 1;       // fp32 accumulators per channel (b = 2, 4)
    float acc[8][NA];
    uint32_t wb[8][2];                          // b = 8: code words of tokens 0-3, 4-7
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < NA; ++n) acc[m][n] = 0.0f;
        wb[m][0] = wb[m][1] = 0;
    }
    // weight of token i's code in its accumulator
    auto weight = [](int i) { return (float)(1u << (BITS == 8 ? 0 : BITS * (BITS == 4 ? (i & 3) : i))); };
#pragma unroll
    for (int i = 0; i < kFlushTokensPerLane; ++i) {
        float worst = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t xp = x[i][m >> 1];
            const float xm = (m & 1) ? hi_f32(xp) : lo_f32(xp);
            const float y = __builtin_fmaf(xm, rcp[m], nzr[m]);
            const float rr = __builtin_rintf(y);
            worst = __builtin_fmaxf(worst, __builtin_fabsf(y - rr));
            if constexpr (BITS == 8)
                wb[m][i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(rr, i & 3, wb[m][i >> 2]);
            else
                acc[m][BITS == 4 ? i >> 2 : 0] = __builtin_fmaf(rr, weight(i), acc[m][BITS == 4 ? i >> 2 : 0]);
        }
        if (__builtin_expect(worst > 0.5f - 0x1p-12f, 0)) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t xp = x[i][m >> 1];
                const float xm = (m & 1) ? hi_f32(xp) : lo_f32(xp);
                const float y = __builtin_fmaf(xm, rcp[m], nzr[m]);
                const float rr = __builtin_rintf(y);
                if (__builtin_fabsf(y - rr) > 0.5f - 0x1p-12f) {
                    uint32_t sb, zb;
                    bits(m >> 1, sb, zb);
                    QParams q;
                    q.scale = (float)__builtin_bit_cast(f16, (uint16_t)(sb >> (16 * (m & 1))));
                    q.zero = (float)__builtin_bit_cast(f16, (uint16_t)(zb >> (16 * (m & 1))));
                    const float cm = (float)quant_exact<BITS>(xm, q);
                    if constexpr (BITS == 8)
                        wb[m][i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(cm, i & 3, wb[m][i >> 2]);
                    else
                        acc[m][BITS == 4 ? i >> 2 : 0] =
                            __builtin_fmaf(cm - rr, weight(i), acc[m][BITS == 4 ? i >> 2 : 0]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if constexpr (BITS == 8) {
            w[m][0] = wb[m][0];
            w[m][1] = wb[m][1];
        } else if constexpr (BITS == 4) {
            w[m][0] = (uint32_t)acc[m][0] | ((uint32_t)acc[m][1] << 16);
        } else {
            w[m][0] = (uint32_t)acc[m][0];
        }
    }
}

// Stores a lane's code words (b = 4, 8: all lanes; b = 2: the even lanes,
// whose words already hold the odd partner's upper halves) and, from lane
// j = 0 of each chunk, the chunk's sidecars.
template <int BITS, int G>
__device__ __forceinline__ void flush_store(const StepArgs& a, int64_t s, int j, int c,
                                            const uint32_t (&w)[8][BITS == 8 ? 2 : 1],
                                            const uint32_t (&sbits)[4], const uint32_t (&zbits)[4],
                                            bool sidecars = true) {
    constexpr int TW = kFlushTokensPerLane * BITS / 32;   // whole words per channel and lane (0: half)
    constexpr int W = G * BITS / 32;
    const int D = a.head_dim;
    const int64_t grp = s * (a.cap_tokens / G) + a.n_quant / G;
    uint32_t* cdst = a.k_codes + grp * (int64_t)(W * D) + 8 * c;
    if constexpr (TW > 0) {
#pragma unroll
        for (int n = 0; n < TW; ++n) {
            u32x4* dst = reinterpret_cast<u32x4*>(cdst + (int64_t)(j * TW + n) * D);
            __builtin_nontemporal_store(u32x4{w[0][n], w[1][n], w[2][n], w[3][n]}, dst);
            __builtin_nontemporal_store(u32x4{w[4][n], w[5][n], w[6][n], w[7][n]}, dst + 1);
        }
    } else if (!(j & 1)) {
        u32x4* dst = reinterpret_cast<u32x4*>(cdst + (int64_t)(j >> 1) * D);
        __builtin_nontemporal_store(u32x4{w[0][0], w[1][0], w[2][0], w[3][0]}, dst);
        __builtin_nontemporal_store(u32x4{w[4][0], w[5][0], w[6][0], w[7][0]}, dst + 1);
    }
    if (sidecars && j == 0) {
        __builtin_nontemporal_store(u32x4{sbits[0], sbits[1], sbits[2], sbits[3]},
                                    reinterpret_cast<u32x4*>(a.k_scale + grp * D + 8 * c));
        __builtin_nontemporal_store(u32x4{zbits[0], zbits[1], zbits[2], zbits[3]},
                                    reinterpret_cast<u32x4*>(a.k_zero + grp * D + 8 * c));
    }
}

// LDS of one wave of the D = 128, G = 32 flush (16 channel chunks).
struct FlushWaveLds {
    u32x4 mn[64];           // partial min/max per lane; later the odd rows' half words
    u32x4 mx[64];
    float rcp[16][8];       // per chunk: its 8 channels' parameters
    float nzr[16][8];
    uint32_t sbits[16][4];
    uint32_t zbits[16][4];
};

// One slice per wave, D = 128 and G = 32: lane l holds chunk c = l & 15 of
// token octet j = l >> 4, so the chunk's four lanes are c + 16r.  The
// exchanges go through the wave's own LDS with no workgroup barrier: the
// LDS accesses of one wave execute in order, and wave_barrier keeps the
// compiler from moving them across the exchange points.  (Cross-lane
// permlane swaps did the same work at about 32 cycles each; LDS traffic
// also takes no VALU issue slots, which this kernel is short of.)
template <int BITS>
__device__ __forceinline__ void flush_keys_wave(const StepArgs& a, int64_t s, FlushWaveLds& L) {
    static_assert(kFlushTokensPerLane == 8, "four token octets per 32-token group");
    const int l = threadIdx.x & 63;
    const int j = l >> 4, c = l & 15;
    const bool live = s < a.n_slices;
    const int64_t sl = live ? s : 0;
    const int row_bytes = 256;
    const __amdgpu_buffer_rsrc_t ring =
        buffer_rsrc(a.k_ring + sl * a.ring_slots * (int64_t)128, (uint32_t)(a.ring_slots * row_bytes));
    const int voff = (a.ring_head + 8 * j) * row_bytes + 16 * c;
    u32x4 x[kFlushTokensPerLane];
#pragma unroll
    for (int i = 0; i < kFlushTokensPerLane; ++i)
        x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ring, voff, i * row_bytes,
                                                                               kNontemporal));
    {
        f16x2 mn[4], mx[4];
        flush_minmax(x, mn, mx);
        L.mn[l] = u32x4{as_u32(mn[0]), as_u32(mn[1]), as_u32(mn[2]), as_u32(mn[3])};
        L.mx[l] = u32x4{as_u32(mx[0]), as_u32(mx[1]), as_u32(mx[2]), as_u32(mx[3])};
    }
    __builtin_amdgcn_wave_barrier();
    {
        // lane j reduces channel pair j of its chunk over the four rows
        const uint32_t* pmn = reinterpret_cast<const uint32_t*>(L.mn);
        const uint32_t* pmx = reinterpret_cast<const uint32_t*>(L.mx);
        f16x2 mn = as_h2(pmn[4 * c + j]), mx = as_h2(pmx[4 * c + j]);
#pragma unroll
        for (int r = 1; r < 4; ++r) {
            mn = pmin(mn, as_h2(pmn[4 * (16 * r + c) + j]));
            mx = pmax(mx, as_h2(pmx[4 * (16 * r + c) + j]));
        }
        flush_pair_params<BITS>(mn, mx, L.rcp[c][2 * j], L.rcp[c][2 * j + 1], L.nzr[c][2 * j],
                                L.nzr[c][2 * j + 1], L.sbits[c][j], L.zbits[c][j]);
    }
    __builtin_amdgcn_wave_barrier();
    float rcp[8], nzr[8];
    uint32_t sbits[4], zbits[4];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        rcp[m] = L.rcp[c][m];
        nzr[m] = L.nzr[c][m];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        sbits[k] = L.sbits[c][k];
        zbits[k] = L.zbits[c][k];
    }
    uint32_t w[8][BITS == 8 ? 2 : 1];
    flush_rows_code<BITS>(x, rcp, nzr, [&](int k, uint32_t& sbk, uint32_t& zbk) {
        sbk = sbits[k];
        zbk = zbits[k];
    }, w);
    if constexpr (BITS == 2) {
        // odd rows post their half words as upper halves, in step 1's space
        // (its last reads came before the previous exchange point)
        if (j & 1) {
            L.mn[l] = u32x4{w[0][0], w[1][0], w[2][0], w[3][0]} << 16u;
            L.mx[l] = u32x4{w[4][0], w[5][0], w[6][0], w[7][0]} << 16u;
        }
        __builtin_amdgcn_wave_barrier();
        if (!(j & 1)) {
            const u32x4 h0 = L.mn[l + 16], h1 = L.mx[l + 16];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                w[k][0] |= h0[k];
                w[4 + k][0] |= h1[k];
            }
        }
    }
    if (live) {
        const int64_t grp = s * (a.cap_tokens / 32) + a.n_quant / 32;
        flush_store<BITS, 32>(a, s, j, c, w, sbits, zbits, false);
        // sidecars: row 0 the scales, row 1 the zeros, one instruction
        if (j < 2)
            __builtin_nontemporal_store(
                j ? u32x4{zbits[0], zbits[1], zbits[2], zbits[3]} : u32x4{sbits[0], sbits[1], sbits[2], sbits[3]},
                reinterpret_cast<u32x4*>((j ? a.k_zero : a.k_scale) + grp * 128 + 8 * c));
    }
}

// The general flush tile (spb slices, any D and G with (G/8) x (D/8) lanes
// per slice within the block): the exchanges go through LDS.
template <int BITS, int G, int NT>
__device__ __forceinline__ void flush_keys_rows(const StepArgs& a, int spb, int64_t kt, FlushLds<NT>& sm) {
    constexpr int J = FlushLane<G>::J;
    const FlushLane<G> ln(a.head_dim, spb);
    const int tid = threadIdx.x;
    bool live;
    const int64_t s = flush_slice<G>(a, spb, kt, ln, live);
    u32x4 x[kFlushTokensPerLane];
    flush_load<G>(a, spb, kt, ln, x);
    {
        f16x2 mn[4], mx[4];
        flush_minmax(x, mn, mx);
        if (ln.in_block) {
            sm.part.mn[tid] = u32x4{as_u32(mn[0]), as_u32(mn[1]), as_u32(mn[2]), as_u32(mn[3])};
            sm.part.mx[tid] = u32x4{as_u32(mx[0]), as_u32(mx[1]), as_u32(mx[2]), as_u32(mx[3])};
        }
    }
    lds_barrier();
    if (ln.in_block && ln.j < 4) {
        const int base = ln.si * ln.P + ln.c;
        const int j = ln.j;
        const uint32_t* pmn = reinterpret_cast<const uint32_t*>(sm.part.mn);
        const uint32_t* pmx = reinterpret_cast<const uint32_t*>(sm.part.mx);
        f16x2 mn = as_h2(pmn[4 * base + j]), mx = as_h2(pmx[4 * base + j]);
#pragma unroll 4
        for (int jj = 1; jj < J; ++jj) {
            mn = pmin(mn, as_h2(pmn[4 * (base + jj * ln.cpr) + j]));
            mx = pmax(mx, as_h2(pmx[4 * (base + jj * ln.cpr) + j]));
        }
        FlushParams& fp = sm.prm[ln.chunk];
        flush_pair_params<BITS>(mn, mx, fp.rcp[2 * j], fp.rcp[2 * j + 1], fp.nzr[2 * j], fp.nzr[2 * j + 1],
                                fp.sbits[j], fp.zbits[j]);
    }
    lds_barrier();
    const FlushParams& fp = sm.prm[ln.in_block ? ln.chunk : 0];
    float rcp[8], nzr[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        rcp[m] = fp.rcp[m];
        nzr[m] = fp.nzr[m];
    }
    uint32_t w[8][BITS == 8 ? 2 : 1];
    flush_rows_code<BITS>(x, rcp, nzr, [&](int k, uint32_t& sbk, uint32_t& zbk) {
        sbk = fp.sbits[k];
        zbk = fp.zbits[k];
    }, w);
    if constexpr (BITS == 2) {
        // step 1's space is free: every read of it came before the second barrier
        if (ln.in_block && (ln.j & 1)) {
            sm.w[0][tid] = u32x4{w[0][0], w[1][0], w[2][0], w[3][0]} << 16u;
            sm.w[1][tid] = u32x4{w[4][0], w[5][0], w[6][0], w[7][0]} << 16u;
        }
        lds_barrier();
        if (ln.in_block && !(ln.j & 1)) {
            const u32x4 h0 = sm.w[0][tid + ln.cpr];
            const u32x4 h1 = sm.w[1][tid + ln.cpr];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                w[k][0] |= h0[k];
                w[4 + k][0] |= h1[k];
            }
        }
    }
    uint32_t sbits[4], zbits[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        sbits[k] = fp.sbits[k];
        zbits[k] = fp.zbits[k];
    }
    if (live) flush_store<BITS, G>(a, s, ln.j, ln.c, w, sbits, zbits);
}

// Append of slice s (one token row, 2^lpt_log2 lanes of 8 channels): the new
// key and value rows go into ring slot (head + count) mod slots, and the
// value row is quantized at once into store row n_quant + count -- value
// groups are per token, so a row's codes never depend on later tokens.  The
// store therefore already holds the codes of every residual value row (rows
// past cap_tokens are skipped: they can never be flushed); only the key
// groups wait for a flush.
template <int BITS, int G, int NT = kBlock>
__device__ __forceinline__ void append_row(const StepArgs& a, int64_t ablk, int lpt_log2) {
    constexpr int GL = G / 8;
    const int D = a.head_dim;
    const int lpt = 1 << lpt_log2;
    const int c = threadIdx.x & (lpt - 1);
    const int64_t s0 = ablk * (NT >> lpt_log2) + (threadIdx.x >> lpt_log2);
    const bool svalid = s0 < a.n_slices;
    const int64_t s = svalid ? s0 : a.n_slices - 1;
    const bool cvalid = c < (D >> 3);
    const int cc = cvalid ? c : 0;
    int slot = a.ring_head + a.ring_count;
    if (slot >= a.ring_slots) slot -= a.ring_slots;
    const int64_t ring_row = (s * a.ring_slots + slot) * (int64_t)D;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(a.k_new + s * D + 8 * cc);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(a.v_new + s * D + 8 * cc);
    if (svalid && cvalid) {
        *reinterpret_cast<u32x4*>(a.k_ring + ring_row + 8 * c) = kx;
        *reinterpret_cast<u32x4*>(a.v_ring + ring_row + 8 * c) = vx;
    }
    const int ngv = (D + G - 1) / G;
    const bool in_group = (c / GL) < ngv;
    const int wpt = ngv * G * BITS / 32;
    const int32_t vrow = a.n_quant + a.ring_count;
    const int64_t row = s * a.cap_tokens + vrow;
    value_chunk<BITS, G>(vx, cvalid, c, svalid && in_group && vrow < a.cap_tokens,
                         a.v_codes + row * wpt, a.v_scale + row * ngv, a.v_zero + row * ngv);
}

// Block ranges: [0, nk) key flush tiles (nk = 0 on a step without flush),
// [nk, nk + na) appends.
template <int G>
__global__ void __launch_bounds__(kBlock)
append_flush_kernel(StepArgs a, int tpb, int lpt_log2, int64_t nk, int64_t na) {
    const int64_t b = blockIdx.x;
    if (b < nk) {
        switch (a.k_bits) {
            case 2: flush_keys<2, G>(a, tpb, b); break;
            case 4: flush_keys<4, G>(a, tpb, b); break;
            default: flush_keys<8, G>(a, tpb, b); break;
        }
        return;
    }
    switch (a.v_bits) {
        case 2: append_row<2, G>(a, b - nk, lpt_log2); break;
        case 4: append_row<4, G>(a, b - nk, lpt_log2); break;
        default: append_row<8, G>(a, b - nk, lpt_log2); break;
    }
}

// A flush step whose key group lies straight in the ring: block ranges
// [0, nt) key flush tiles of spb slices (WAVE: one slice per wave, D = 128,
// G = 32), [nt, nt + na) appends, NT threads per block.  Kernels of their
// own, one per key width, so that neither the one-lane-per-pair path's
// registers nor those of the other widths limit these waves.
template <int KB, int G, int NT, bool WAVE>
__global__ void __launch_bounds__(NT)
append_flush_rows_kernel(StepArgs a, int spb, int lpt_log2, int64_t nt) {
    const int64_t b = blockIdx.x;
    if (b < nt) {
        if constexpr (WAVE) {
            __shared__ FlushWaveLds sw[NT / 64];
            // the wave index is uniform over the wave; saying so keeps the
            // slice's buffer resource in scalar registers (otherwise every
            // load becomes a loop over the distinct resources of its lanes)
            const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
            flush_keys_wave<KB>(a, b * (NT / 64) + wave, sw[wave]);
        } else {
            __shared__ FlushLds<NT> sm;
            flush_keys_rows<KB, G, NT>(a, spb, b, sm);
        }
        return;
    }
    switch (a.v_bits) {
        case 2: append_row<2, G, NT>(a, b - nt, lpt_log2); break;
        case 4: append_row<4, G, NT>(a, b - nt, lpt_log2); break;
        default: append_row<8, G, NT>(a, b - nt, lpt_log2); break;
    }
}

// Prefill: copy tokens [first, first + n) of each slice into ring slots [0, n).
__global__ void __launch_bounds__(kBlock)
ring_fill_kernel(RingFillArgs a, int64_t per_tensor) {
    const int cpr = a.head_dim >> 3;
    for (int64_t chunk = (int64_t)blockIdx.x * kBlock + threadIdx.x; chunk < 2 * per_tensor;
         chunk += (int64_t)gridDim.x * kBlock) {
        const bool is_v = chunk >= per_tensor;
        int64_t cidx = is_v ? chunk - per_tensor : chunk;
        const int cc = (int)(cidx % cpr);
        cidx /= cpr;
        const int i = (int)(cidx % a.n_tokens);
        const int64_t s = cidx / a.n_tokens;
        const uint16_t* src = (is_v ? a.v_in : a.k_in) + s * a.in_stride +
                              (int64_t)(a.first_token + i) * a.head_dim + 8 * cc;
        uint16_t* dst = (is_v ? a.v_ring : a.k_ring) + (s * a.ring_slots + i) * (int64_t)a.head_dim + 8 * cc;
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
}

// ---------------------------------------------------------------------------
// launch geometry
// ---------------------------------------------------------------------------

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

unsigned grid_for(int64_t blocks) {
    return (unsigned)(blocks < kMaxGrid ? (blocks > 0 ? blocks : 1) : kMaxGrid);
}

// key groups per block: as many as keep 256 threads busy with one channel
// pair each
int key_tiles_per_block(int D) { return (2 * kBlock) / D; }

// lanes per token row for the value kernels: a power of two covering both the
// row's 8-channel chunks and one whole value group (G/8 lanes)
int value_lanes_log2(int G, int D) {
    int need = D / 8;
    if (G / 8 > need) need = G / 8;
    int l = 0;
    while ((1 << l) < need) ++l;
    return l;
}

constexpr int kValueRowsPerBlock = 64;

// Occupancy caps of the decoders.  They write 2 bytes per element and read
// about 0.4, and fewer resident workgroups (fewer concurrent write streams)
// run faster: at the Llama-2-7B shape key decode takes 1.59 ms with at most
// 3 workgroups per CU against 1.77 ms with the 8 its registers allow, value
// decode 1.55 ms with at most 5 against 1.71 ms with 12 (Mistral-7B shape
// 3.30 vs 3.59 and 3.56 vs 3.92 ms; outputs identical).  The launches
// reserve LDS that the kernels do not use, which is what caps them: 3
// workgroups of 53 KB, or 5 of 32 KB, fill the 160 KB of a CU.  The encoders
// are read-bound and run fastest at full occupancy.
constexpr size_t kDecodeKLdsCap = 53 * 1024;
constexpr size_t kDecodeVLdsCap = 32 * 1024;

template <int BITS, int G>
int run_encode_k(const EncodeArgs& a, hipStream_t st) {
    const int D = a.head_dim;
    const int ng_full = a.n_tokens / G;
    const int tpb = key_tiles_per_block(D);
    const int out_groups = (a.cap_tokens + G - 1) / G;
    if (ng_full > 0) {
        const int bps = (ng_full + tpb - 1) / tpb;
        const int64_t nb = a.n_slices * bps;
        hipLaunchKernelGGL((encode_k_kernel<BITS, G>), dim3(grid_for(nb)), dim3(kBlock), 0, st,
                           a.in, a.in_stride, D, ng_full, tpb, bps, nb, a.codes, a.scale, a.zero,
                           out_groups);
        const int err = (int)hipGetLastError();
        if (err) return err;
    }
    if (a.n_tokens % G) {
        const int64_t nb = ceil_div64(a.n_slices, tpb);
        if (nb > 0x7FFFFFFF) return (int)hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((encode_k_tail_kernel<BITS, G>), dim3((unsigned)nb), dim3(kBlock), 0,
                           st, a.in, a.in_stride, a.n_tokens, D, a.n_slices, a.codes, a.scale,
                           a.zero, out_groups);
    }
    return (int)hipGetLastError();
}

template <int BITS, int G>
int run_encode_v(const EncodeArgs& a, hipStream_t st) {
    const int D = a.head_dim;
    const int l2 = value_lanes_log2(G, D);
    const int bps = (a.n_tokens + kValueRowsPerBlock - 1) / kValueRowsPerBlock;
    const int64_t nb = a.n_slices * bps;
    const int ngv = (D + G - 1) / G;
    const bool all = (1 << l2) == D / 8 && D % G == 0;
    if (G == 32 && all) {
        const int rows_per_block = 4 * (kBlock >> l2);
        const int bpq = (a.n_tokens + rows_per_block - 1) / rows_per_block;
        const int64_t nq = a.n_slices * bpq;
        hipLaunchKernelGGL((encode_v_quad_kernel<BITS>), dim3(grid_for(nq)), dim3(kBlock), 0, st, a.in,
                           a.in_stride, a.n_tokens, D, l2, bpq, nq, a.codes, a.scale, a.zero, a.cap_tokens);
    } else if (all)
        hipLaunchKernelGGL((encode_v_kernel<BITS, G, true>), dim3(grid_for(nb)), dim3(kBlock), 0,
                           st, a.in, a.in_stride, a.n_tokens, D, l2, kValueRowsPerBlock, bps, nb,
                           a.codes, a.scale, a.zero, a.cap_tokens, ngv);
    else
        hipLaunchKernelGGL((encode_v_kernel<BITS, G, false>), dim3(grid_for(nb)), dim3(kBlock), 0,
                           st, a.in, a.in_stride, a.n_tokens, D, l2, kValueRowsPerBlock, bps, nb,
                           a.codes, a.scale, a.zero, a.cap_tokens, ngv);
    return (int)hipGetLastError();
}

template <int BITS, int G>
int run_decode_k(const DecodeArgs& a, hipStream_t st) {
    const int D = a.head_dim;
    const int ng = (a.n_tokens + G - 1) / G;
    const int tiles_pb = kBlock / (D / 8);
    const int64_t n_tiles = a.n_slices * ng;
    const int64_t nb = ceil_div64(n_tiles, tiles_pb);
    const int out_groups = (a.cap_tokens + G - 1) / G;
    hipLaunchKernelGGL((decode_k_kernel<BITS, G>), dim3(grid_for(nb)), dim3(kBlock), kDecodeKLdsCap, st, a.codes,
                       a.scale, a.zero, a.n_tokens, D, ng, out_groups, tiles_pb, n_tiles, nb, a.out,
                       a.out_stride);
    return (int)hipGetLastError();
}

template <int BITS, int G>
int run_decode_v(const DecodeArgs& a, hipStream_t st) {
    const int D = a.head_dim;
    const int l2 = value_lanes_log2(G, D);
    const int rpb = kRowsPerThread * (kBlock >> l2);
    const int bps = (a.n_tokens + rpb - 1) / rpb;
    const int64_t nb = a.n_slices * bps;
    const int ngv = (D + G - 1) / G;
    hipLaunchKernelGGL((decode_v_kernel<BITS, G>), dim3(grid_for(nb)), dim3(kBlock), kDecodeVLdsCap, st, a.codes,
                       a.scale, a.zero, a.n_tokens, D, l2, bps, nb, a.cap_tokens, ngv, a.out,
                       a.out_stride);
    return (int)hipGetLastError();
}

// Flush step from ring rows with NT threads per block.
template <int KB, int G, int NT, bool WAVE>
int launch_flush_rows(const StepArgs& a, int spb, int l2, int64_t nt, int64_t na, hipStream_t st) {
    if (na + nt > 0x7FFFFFFF) return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((append_flush_rows_kernel<KB, G, NT, WAVE>), dim3((unsigned)(nt + na)), dim3(NT), 0, st,
                       a, spb, l2, nt);
    return (int)hipGetLastError();
}

template <int G, int NT, bool WAVE>
int run_flush_rows(const StepArgs& a, int spb, hipStream_t st) {
    const int l2 = value_lanes_log2(G, a.head_dim);
    const int64_t nt = ceil_div64(a.n_slices, spb);
    const int64_t na = ceil_div64(a.n_slices, NT >> l2);
    if (a.k_bits == 2) return launch_flush_rows<2, G, NT, WAVE>(a, spb, l2, nt, na, st);
    if (a.k_bits == 4) return launch_flush_rows<4, G, NT, WAVE>(a, spb, l2, nt, na, st);
    return launch_flush_rows<8, G, NT, WAVE>(a, spb, l2, nt, na, st);
}

template <int G>
int run_append_flush(const StepArgs& a, hipStream_t st) {
    const int D = a.head_dim;
    const int l2 = value_lanes_log2(G, D);
    const int64_t na = ceil_div64(a.n_slices, kBlock >> l2);
    // the usual flush: all G tokens in the ring, not wrapping around its end,
    // and a slice's (G/8) x (D/8) lanes within one block (all but G = 128
    // with D > 128).  D = 128 with G = 32 takes the wave-local path; other
    // slices of at most one wave take one-wave workgroups, so that the waves
    // never wait for each other at the LDS steps' barriers.
    const int lanes = (G / kFlushTokensPerLane) * (D / 8);
    if (a.flush && a.ring_count >= G && a.ring_head + G <= a.ring_slots && lanes <= kBlock) {
        if constexpr (G == 32)
            if (D == 128) return run_flush_rows<G, kBlock, true>(a, kBlock / 64, st);
        return lanes <= 64 ? run_flush_rows<G, 64, false>(a, 64 / lanes, st)
                           : run_flush_rows<G, kBlock, false>(a, kBlock / lanes, st);
    }
    const int tpb = key_tiles_per_block(D);
    const int64_t nk = a.flush ? ceil_div64(a.n_slices, tpb) : 0;
    const int64_t total = nk + na;
    if (total > 0x7FFFFFFF) return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((append_flush_kernel<G>), dim3((unsigned)total), dim3(kBlock), 0, st, a, tpb,
                       l2, nk, na);
    return (int)hipGetLastError();
}

#define KIVI_DISPATCH(RUN)                                                   \
    switch (a.group_size) {                                                  \
        case 32:                                                             \
            return a.bits == 2 ? RUN<2, 32>(a, st)                           \
                   : a.bits == 4 ? RUN<4, 32>(a, st) : RUN<8, 32>(a, st);    \
        case 64:                                                             \
            return a.bits == 2 ? RUN<2, 64>(a, st)                           \
                   : a.bits == 4 ? RUN<4, 64>(a, st) : RUN<8, 64>(a, st);    \
        default:                                                             \
            return a.bits == 2 ? RUN<2, 128>(a, st)                          \
                   : a.bits == 4 ? RUN<4, 128>(a, st) : RUN<8, 128>(a, st);  \
    }

}  // namespace

int launch_encode_k(const EncodeArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    KIVI_DISPATCH(run_encode_k)
}

int launch_encode_v(const EncodeArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    KIVI_DISPATCH(run_encode_v)
}

int launch_decode_k(const DecodeArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    KIVI_DISPATCH(run_decode_k)
}

int launch_decode_v(const DecodeArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    KIVI_DISPATCH(run_decode_v)
}

int launch_append_flush(const StepArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (a.group_size) {
        case 32: return run_append_flush<32>(a, st);
        case 64: return run_append_flush<64>(a, st);
        default: return run_append_flush<128>(a, st);
    }
}

int launch_ring_fill(const RingFillArgs& a, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t per_tensor = a.n_slices * (int64_t)a.n_tokens * (a.head_dim / 8);
    const int64_t nb = ceil_div64(2 * per_tensor, kBlock);
    hipLaunchKernelGGL(ring_fill_kernel, dim3(grid_for(nb)), dim3(kBlock), 0, st, a, per_tensor);
    return (int)hipGetLastError();
}

}  // namespace kivi
