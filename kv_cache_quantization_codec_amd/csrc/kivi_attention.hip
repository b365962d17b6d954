// Decode-phase attention over the KIVI-quantized cache, for gfx950 (MI355X).
//
// One query token per query head attends to every cached token of its KV
// slice: the quantized prefix, dequantized as code * scale + zero with the
// stored fp16 statistics (keys per channel over groups of G tokens, values
// per token over groups of G channels: CacheForge README, "How it works"),
// then the fp16 residual of recent tokens.  The pages name the consumer of
// the cache (CacheForge README, "Contribution scope": the inherited model
// integrations and kernels) but print no formula; this is ordinary softmax
// attention with q_per_kv query heads sharing one KV slice.
//
// Design.  Both contractions run on the matrix cores
// (v_mfma_f32_16x16x32_f16), with the quantization folded out of the inner
// loop instead of dequantizing every element:
//   keys:   q . khat_t = sum_d (q_d * s_gd) * c_td + sum_d q_d * z_gd
//   values: sum_t p_t vhat_td = sum_t (p_t * s_tg) * c_td + sum_t p_t * z_tg
// * The scaled operand (q*s per key group, p*s per value group) is computed
//   once per group in fp32 and split into fp16 hi + lo parts that occupy two
//   MFMA rows of the same head (rows 2h and 2h+1), so the products carry
//   about 22 bits; the two rows are added after the MFMA.
// * A code c enters as the fp16 bit pattern c << sh, i.e. the subnormal (or
//   lowest-binade) value c * 2^(sh-24), exact because c << sh < 2^11; sh is
//   the code's bit offset inside its byte.  Extracting it costs one v_perm
//   (pick the byte of two words) and one AND per pair of codes; the column
//   factor 2^(24-sh) is applied to the fp32 result.
// * The zero-point terms are separate MFMAs: q against the group's zeros
//   (identical in every token column), and p against the rows' zeros, whose
//   16 output columns hold up to 16 value groups at once.
// * Online softmax in base 2 per 32-token block; heads live in MFMA rows, so
//   each lane holds two heads' scores of one token and the row reductions
//   are DPP moves inside a 16-lane row.
// One wave per workgroup; a workgroup walks a range of 32-token blocks of
// one slice (or that slice's residual) and either writes the normalised
// output or, when the slice is split, its partial (max, sum, output) for a
// merge kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_launch.h"

namespace kivi {
namespace {

typedef _Float16 f16;
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxD = 128;
constexpr int kAqStride = kMaxD + 8;      // halves per row of the q*s operand
constexpr int kTokStride = 32 + 8;        // halves per row of a 32-token operand
constexpr int kVcStride = 32 + 4;         // words per transposed value-code column
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f4 mfma(const h8& a, const h8& b, const f4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 2^e for integer e in the normal range, exactly.
__device__ __forceinline__ float pow2(int e) { return __builtin_bit_cast(float, (127 + e) << 23); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// max / sum over the 16 lanes of a DPP row (every lane gets the result):
// lane ^ 1, lane ^ 2, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    return v + dpp_f<0x140>(v);
}

// Where a lane's code sits: element m of a word (m = position along the
// packing axis) occupies bits [BITS*m, BITS*m + BITS): byte bi, shift sh.
template <int BITS>
struct CodePos {
    uint32_t sel;    // v_perm selector: byte bi of S1 -> byte 0, of S0 -> byte 2
    uint32_t mask;   // the code in both 16-bit halves
    float col;       // 2^(24 - sh), undoes the subnormal encoding
    __device__ explicit CodePos(int m) {
        const int bit = BITS * m;
        const int bi = bit >> 3, sh = bit & 7;
        sel = (uint32_t)bi | (0x0Cu << 8) | ((uint32_t)(4 + bi) << 16) | (0x0Cu << 24);
        mask = ((uint32_t)((1 << BITS) - 1) << sh) * 0x00010001u;
        col = pow2(24 - sh);
    }
};

// Eight codes (one per word, consecutive along the MFMA reduction axis) as
// fp16 operands: element e from word e.
template <int BITS>
__device__ __forceinline__ h8 codes8(const u32x4& lo, const u32x4& hi, const CodePos<BITS>& cp) {
    u32x4 r;
    r.x = __builtin_amdgcn_perm(lo.y, lo.x, cp.sel) & cp.mask;
    r.y = __builtin_amdgcn_perm(lo.w, lo.z, cp.sel) & cp.mask;
    r.z = __builtin_amdgcn_perm(hi.y, hi.x, cp.sel) & cp.mask;
    r.w = __builtin_amdgcn_perm(hi.w, hi.z, cp.sel) & cp.mask;
    return __builtin_bit_cast(h8, r);
}

__device__ __forceinline__ uint32_t pack_h2(f16 a, f16 b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// fp32 x as fp16 hi + lo with hi = fp16(x), lo = fp16(x - hi); x - hi is
// exact in fp32, so hi + lo is within 2^-22 |x| of x (|x| < 65504).
__device__ __forceinline__ void split_hl(float x, f16& hi, f16& lo) {
    hi = (f16)x;
    lo = (f16)(x - (float)hi);
}

template <int KB, int VB>
struct Smem {
    f16 aq[16][kAqStride];                 // q*s of the current key group, hi/lo rows
    f16 kz[kMaxD];                         // zeros of the current key group
    uint32_t kc[KB][kMaxD];                // key codes of a 32-token block
    uint32_t vc[VB * kMaxD / 32][kVcStride];  // value codes, [word column][row]
    f16 vz[4][kTokStride];                 // value zeros, [group][row]
    float vs[32][4];                       // value scales, [row][group]
    float pp[8][32];                       // softmax weights, [head][token]
    f16 ap[16][kTokStride];                // p*s of one value group, hi/lo rows
    f16 apz[16][kTokStride];               // p, hi/lo rows
};

// Per-wave running softmax state and output accumulators for the two heads
// this lane's MFMA rows hold (a = 2*kq, b = 2*kq + 1).
struct Acc {
    float m_a, m_b, l_a, l_b;
    f4 o[kMaxD / 16];   // MFMA output tiles of 16 channels
    f4 z;               // value zero-point term, columns = value groups
};

// Online-softmax update with scores x (log2 units) of two 16-token tiles;
// returns the block weights p in xa/xb and rescales the accumulators.
__device__ __forceinline__ void softmax_block(Acc& acc, float xa[2], float xb[2], int n_tiles16) {
    const float bm_a = row16_max(fmaxf(xa[0], xa[1]));
    const float bm_b = row16_max(fmaxf(xb[0], xb[1]));
    const float mn_a = fmaxf(acc.m_a, bm_a), mn_b = fmaxf(acc.m_b, bm_b);
    const float al_a = __builtin_amdgcn_exp2f(acc.m_a - mn_a);
    const float al_b = __builtin_amdgcn_exp2f(acc.m_b - mn_b);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        xa[tt] = __builtin_amdgcn_exp2f(xa[tt] - mn_a);
        xb[tt] = __builtin_amdgcn_exp2f(xb[tt] - mn_b);
    }
    acc.l_a = acc.l_a * al_a + row16_sum(xa[0] + xa[1]);
    acc.l_b = acc.l_b * al_b + row16_sum(xb[0] + xb[1]);
    acc.m_a = mn_a;
    acc.m_b = mn_b;
#pragma unroll
    for (int nt = 0; nt < kMaxD / 16; ++nt) {
        if (nt < n_tiles16) {
            acc.o[nt][0] *= al_a;
            acc.o[nt][1] *= al_a;
            acc.o[nt][2] *= al_b;
            acc.o[nt][3] *= al_b;
        }
    }
    acc.z[0] *= al_a;
    acc.z[1] *= al_a;
    acc.z[2] *= al_b;
    acc.z[3] *= al_b;
}

// Softmax weights of the block to LDS ([head][token]) and, as hi/lo fp16
// rows, to the operand apz ([2h / 2h+1][token]).
template <int KB, int VB>
__device__ __forceinline__ void weights_to_lds(Smem<KB, VB>& sm, const float pa[2], const float pb[2],
                                               int r) {
    const int L = threadIdx.x, j = L & 15, kq = L >> 4;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        sm.pp[2 * kq][16 * tt + j] = pa[tt];
        sm.pp[2 * kq + 1][16 * tt + j] = pb[tt];
    }
    __syncthreads();
    const int t = L & 31;
    for (int h = L >> 5; h < r; h += 2) {
        f16 hi, lo;
        split_hl(sm.pp[h][t], hi, lo);
        sm.apz[2 * h][t] = hi;
        sm.apz[2 * h + 1][t] = lo;
    }
    __syncthreads();
}

template <int KB, int VB>
__device__ __forceinline__ void write_result(const AttnArgs& a, const Acc& acc, int64_t s, int split,
                                             const float oa[], const float ob[]) {
    const int L = threadIdx.x, j = L & 15, kq = L >> 4;
    const int D = a.head_dim, r = a.q_per_kv, nt16 = D / 16;
    const int ha = 2 * kq, hb = 2 * kq + 1;
    if (a.plan.n_splits == 1) {
        const float ia = 1.0f / acc.l_a, ib = 1.0f / acc.l_b;
#pragma unroll
        for (int nt = 0; nt < kMaxD / 16; ++nt) {
            if (nt < nt16) {
                if (ha < r) a.out[(s * r + ha) * D + 16 * nt + j] = __builtin_bit_cast(uint16_t, (f16)(oa[nt] * ia));
                if (hb < r) a.out[(s * r + hb) * D + 16 * nt + j] = __builtin_bit_cast(uint16_t, (f16)(ob[nt] * ib));
            }
        }
        return;
    }
    const int64_t base = (s * a.plan.n_splits + split) * r;
#pragma unroll
    for (int nt = 0; nt < kMaxD / 16; ++nt) {
        if (nt < nt16) {
            if (ha < r) a.ws_o[(base + ha) * D + 16 * nt + j] = oa[nt];
            if (hb < r) a.ws_o[(base + hb) * D + 16 * nt + j] = ob[nt];
        }
    }
    if (j == 0) {
        if (ha < r) {
            a.ws_ml[(base + ha) * 2] = acc.m_a;
            a.ws_ml[(base + ha) * 2 + 1] = acc.l_a;
        }
        if (hb < r) {
            a.ws_ml[(base + hb) * 2] = acc.m_b;
            a.ws_ml[(base + hb) * 2 + 1] = acc.l_b;
        }
    }
}

// ---------------------------------------------------------------------------
// the attention kernel: blockIdx.x = slice * n_splits + split
// ---------------------------------------------------------------------------

template <int KB, int VB>
__global__ void __launch_bounds__(kWave) attention_kernel(const AttnArgs a) {
    __shared__ Smem<KB, VB> sm;
    const int L = threadIdx.x, j = L & 15, kq = L >> 4;
    const int D = a.head_dim, G = a.group_size, r = a.q_per_kv;
    const int nk32 = D / 32, nt16 = D / 16;
    const int64_t s = blockIdx.x / a.plan.n_splits;
    const int split = (int)(blockIdx.x - s * a.plan.n_splits);
    const bool residual = a.plan.has_res && split == a.plan.n_splits - 1;

    // operand rows that are never written stay zero
    for (int i = L; i < 16 * kAqStride; i += kWave) (&sm.aq[0][0])[i] = (f16)0;
    for (int i = L; i < 16 * kTokStride; i += kWave) {
        (&sm.ap[0][0])[i] = (f16)0;
        (&sm.apz[0][0])[i] = (f16)0;
    }

    // q as MFMA A operand, rows 2h = q_h and 2h+1 = 0: lane row j, channels
    // 32*kk + 8*kq .. +7
    h8 qa[kMaxD / 32];
    {
        const int h = j >> 1;
        const bool live = (j & 1) == 0 && h < r;
        const uint16_t* qrow = a.q + (s * r + (live ? h : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < kMaxD / 32; ++kk) {
            u32x4 w = u32x4{0, 0, 0, 0};
            if (live && kk < nk32) w = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * kq);
            qa[kk] = __builtin_bit_cast(h8, w);
        }
    }

    Acc acc;
    acc.m_a = acc.m_b = kNegInf;
    acc.l_a = acc.l_b = 0.0f;
#pragma unroll
    for (int nt = 0; nt < kMaxD / 16; ++nt) acc.o[nt] = f4{0, 0, 0, 0};
    acc.z = f4{0, 0, 0, 0};
    __syncthreads();

    float oa[kMaxD / 16], ob[kMaxD / 16];

    if (residual) {
        // ---- fp16 residual: plain fp16 operands ----
        const uint16_t* rk = a.res_k + s * a.res_stride;
        const uint16_t* rv = a.res_v + s * a.res_stride;
        for (int i0 = 0; i0 < a.res_count; i0 += 32) {
            float xa[2], xb[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int i = i0 + 16 * tt + j;
                const bool valid = i < a.res_count;
                int slot = a.res_head + (valid ? i : 0);
                if (slot >= a.res_slots) slot -= a.res_slots;
                const uint16_t* row = rk + (int64_t)slot * D;
                f4 sc = f4{0, 0, 0, 0};
#pragma unroll
                for (int kk = 0; kk < kMaxD / 32; ++kk) {
                    if (kk < nk32) {
                        u32x4 w = u32x4{0, 0, 0, 0};
                        if (valid) w = *reinterpret_cast<const u32x4*>(row + 32 * kk + 8 * kq);
                        sc = mfma(qa[kk], __builtin_bit_cast(h8, w), sc);
                    }
                }
                xa[tt] = valid ? (sc[0] + sc[1]) * a.logit_scale : kNegInf;
                xb[tt] = valid ? (sc[2] + sc[3]) * a.logit_scale : kNegInf;
            }
            softmax_block(acc, xa, xb, nt16);
            weights_to_lds(sm, xa, xb, r);
            // values: B[token 8kq+e][channel 16nt+j]
            const h8 pa8 = *reinterpret_cast<const h8*>(&sm.apz[j][8 * kq]);
            int slots[8];
            bool valid[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = i0 + 8 * kq + e;
                valid[e] = i < a.res_count;
                int slot = a.res_head + (valid[e] ? i : 0);
                if (slot >= a.res_slots) slot -= a.res_slots;
                slots[e] = slot;
            }
#pragma unroll
            for (int nt = 0; nt < kMaxD / 16; ++nt) {
                if (nt < nt16) {
                    h8 b;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint16_t x = valid[e] ? rv[(int64_t)slots[e] * D + 16 * nt + j] : (uint16_t)0;
                        b[e] = __builtin_bit_cast(f16, x);
                    }
                    acc.o[nt] = mfma(pa8, b, acc.o[nt]);
                }
            }
            __syncthreads();   // pp / apz are rewritten by the next block
        }
#pragma unroll
        for (int nt = 0; nt < kMaxD / 16; ++nt) {
            oa[nt] = acc.o[nt][0] + acc.o[nt][1];
            ob[nt] = acc.o[nt][2] + acc.o[nt][3];
        }
        write_result<KB, VB>(a, acc, s, split, oa, ob);
        return;
    }

    // ---- quantized prefix: blocks [b0, b1) of 32 tokens ----
    const int b0 = split * a.plan.blocks_per_split;
    const int b1 = min(b0 + a.plan.blocks_per_split, a.plan.n_blocks);
    const int n = a.n_quant;
    const int Wk = G * KB / 32;                           // key words per channel per group
    const int ngk_cap = (a.cap_tokens + G - 1) / G;
    const int ngv = (D + G - 1) / G;
    const int wpt = ngv * G * VB / 32;                    // value words per row
    const int vcols = D * VB / 32;                        // value words that hold real channels
    const uint32_t* kcs = a.k_codes + s * (int64_t)ngk_cap * Wk * D;
    const uint16_t* kss = a.k_scale + s * (int64_t)ngk_cap * D;
    const uint16_t* kzs = a.k_zero + s * (int64_t)ngk_cap * D;
    const uint32_t* vcs = a.v_codes + s * (int64_t)a.cap_tokens * wpt;
    const uint16_t* vss = a.v_scale + s * (int64_t)a.cap_tokens * ngv;
    const uint16_t* vzs = a.v_zero + s * (int64_t)a.cap_tokens * ngv;

    // q of channel pair (2L, 2L+1) for the q*s operand
    float qf[8][2];
    const bool pair_live = 2 * L < D;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        qf[h][0] = qf[h][1] = 0.0f;
        if (h < r && pair_live) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(a.q + (s * r + h) * D + 2 * L);
            qf[h][0] = (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xFFFF));
            qf[h][1] = (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16));
        }
    }

    const CodePos<KB> kpos(j % (32 / KB));
    const CodePos<VB> vpos(j % (32 / VB));
    f4 zk = f4{0, 0, 0, 0};
    int cur_group = -1;

    for (int blk = b0; blk < b1; ++blk) {
        const int t0 = 32 * blk;
        const int g = t0 / G;
        // key statistics of a new group: q*s operand rows and zeros
        if (g != cur_group) {
            cur_group = g;
            if (pair_live) {
                const uint32_t sw = *reinterpret_cast<const uint32_t*>(kss + (int64_t)g * D + 2 * L);
                const uint32_t zw = *reinterpret_cast<const uint32_t*>(kzs + (int64_t)g * D + 2 * L);
                const float s0 = (float)__builtin_bit_cast(f16, (uint16_t)(sw & 0xFFFF));
                const float s1 = (float)__builtin_bit_cast(f16, (uint16_t)(sw >> 16));
                *reinterpret_cast<uint32_t*>(&sm.kz[2 * L]) = zw;
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    if (h < r) {
                        f16 h0, l0, h1, l1;
                        split_hl(qf[h][0] * s0, h0, l0);
                        split_hl(qf[h][1] * s1, h1, l1);
                        *reinterpret_cast<uint32_t*>(&sm.aq[2 * h][2 * L]) = pack_h2(h0, h1);
                        *reinterpret_cast<uint32_t*>(&sm.aq[2 * h + 1][2 * L]) = pack_h2(l0, l1);
                    }
                }
            }
        }
        // stage the block: key codes (KB word rows of D words, contiguous)
        {
            const uint32_t* src = kcs + ((int64_t)g * Wk + ((t0 % G) / 32) * KB) * D;
            for (int v = L; v < KB * D / 4; v += kWave) {
                const int row = (4 * v) / D, col = (4 * v) % D;
                *reinterpret_cast<u32x4*>(&sm.kc[row][col]) = *reinterpret_cast<const u32x4*>(src + 4 * v);
            }
        }
        // value codes of rows t0 .. t0+31 (word columns < vcols), transposed;
        // rows past n_quant are zero (and never read from memory)
        for (int v = L; v < 32 * (vcols / 2); v += kWave) {
            const int row = v / (vcols / 2), c2 = 2 * (v % (vcols / 2));
            const int t = t0 + row;
            uint32_t w0 = 0, w1 = 0;
            if (t < n) {
                const uint32_t* src = vcs + (int64_t)t * wpt + c2;
                w0 = src[0];
                w1 = src[1];
            }
            sm.vc[c2][row] = w0;
            sm.vc[c2 + 1][row] = w1;
        }
        // value statistics of the 32 rows
        for (int v = L; v < 32 * ngv; v += kWave) {
            const int row = v / ngv, gv = v % ngv;
            const int t = t0 + row;
            uint16_t sb = 0, zb = 0;
            if (t < n) {
                sb = vss[(int64_t)t * ngv + gv];
                zb = vzs[(int64_t)t * ngv + gv];
            }
            sm.vs[row][gv] = (float)__builtin_bit_cast(f16, sb);
            sm.vz[gv][row] = __builtin_bit_cast(f16, zb);
        }
        __syncthreads();

        // keys: scores of two 16-token tiles, and the zero-point term
        if (t0 % G == 0 || blk == b0) {
            zk = f4{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < kMaxD / 32; ++kk)
                if (kk < nk32) zk = mfma(qa[kk], *reinterpret_cast<const h8*>(&sm.kz[32 * kk + 8 * kq]), zk);
        }
        f4 sc[2] = {f4{0, 0, 0, 0}, f4{0, 0, 0, 0}};
#pragma unroll
        for (int kk = 0; kk < kMaxD / 32; ++kk) {
            if (kk < nk32) {
                const h8 aop = *reinterpret_cast<const h8*>(&sm.aq[j][32 * kk + 8 * kq]);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int wi = (16 * tt + j) / (32 / KB);
                    const uint32_t* wp = &sm.kc[wi][32 * kk + 8 * kq];
                    const h8 bop = codes8<KB>(*reinterpret_cast<const u32x4*>(wp),
                                              *reinterpret_cast<const u32x4*>(wp + 4), kpos);
                    sc[tt] = mfma(aop, bop, sc[tt]);
                }
            }
        }
        float xa[2], xb[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const bool valid = t0 + 16 * tt + j < n;
            xa[tt] = valid ? ((sc[tt][0] + sc[tt][1]) * kpos.col + zk[0]) * a.logit_scale : kNegInf;
            xb[tt] = valid ? ((sc[tt][2] + sc[tt][3]) * kpos.col + zk[2]) * a.logit_scale : kNegInf;
        }
        softmax_block(acc, xa, xb, nt16);
        weights_to_lds(sm, xa, xb, r);

        // values: zero-point term over all groups at once (columns = groups)
        {
            const h8 pz = *reinterpret_cast<const h8*>(&sm.apz[j][8 * kq]);
            h8 bz = __builtin_bit_cast(h8, u32x4{0, 0, 0, 0});
            if (j < ngv) bz = *reinterpret_cast<const h8*>(&sm.vz[j][8 * kq]);
            acc.z = mfma(pz, bz, acc.z);
        }
        // values: p*s operand per value group, then the code tiles of that group
        int cur_vg = -1;
        const int t = L & 31;
#pragma unroll
        for (int nt = 0; nt < kMaxD / 16; ++nt) {
            if (nt < nt16) {
                const int gv = (16 * nt) / G;
                if (gv != cur_vg) {
                    cur_vg = gv;
                    if (nt > 0) __syncthreads();
                    const float sv = sm.vs[t][gv];
                    for (int h = L >> 5; h < r; h += 2) {
                        f16 hi, lo;
                        split_hl(sm.pp[h][t] * sv, hi, lo);
                        sm.ap[2 * h][t] = hi;
                        sm.ap[2 * h + 1][t] = lo;
                    }
                    __syncthreads();
                }
                const h8 aop = *reinterpret_cast<const h8*>(&sm.ap[j][8 * kq]);
                const int col = (16 * nt + j) / (32 / VB);
                const uint32_t* wp = &sm.vc[col][8 * kq];
                const h8 bop = codes8<VB>(*reinterpret_cast<const u32x4*>(wp),
                                          *reinterpret_cast<const u32x4*>(wp + 4), vpos);
                acc.o[nt] = mfma(aop, bop, acc.o[nt]);
            }
        }
        __syncthreads();   // the staging buffers are rewritten by the next block
    }

    // output = code term * column factor + zero term of the channel's group;
    // the zero term of group gv sits in column gv of the same 16-lane row
    const float za = acc.z[0] + acc.z[1], zb = acc.z[2] + acc.z[3];
#pragma unroll
    for (int nt = 0; nt < kMaxD / 16; ++nt) {
        const int gv = (16 * nt) / G;
        const float zra = __shfl(za, 16 * kq + gv, kWave);
        const float zrb = __shfl(zb, 16 * kq + gv, kWave);
        oa[nt] = (acc.o[nt][0] + acc.o[nt][1]) * vpos.col + zra;
        ob[nt] = (acc.o[nt][2] + acc.o[nt][3]) * vpos.col + zrb;
    }
    write_result<KB, VB>(a, acc, s, split, oa, ob);
}

// Merge of the partial results of a split slice: one workgroup per (slice,
// query head), lanes over channels.
__global__ void __launch_bounds__(kWave) attention_merge_kernel(const AttnArgs a) {
    const int r = a.q_per_kv, D = a.head_dim, ns = a.plan.n_splits;
    const int64_t s = blockIdx.x / r;
    const int h = (int)(blockIdx.x - s * r);
    const int L = threadIdx.x;
    float mx = kNegInf;
    for (int i = 0; i < ns; ++i) mx = fmaxf(mx, a.ws_ml[((s * ns + i) * r + h) * 2]);
    float lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int i = 0; i < ns; ++i) {
        const int64_t base = (s * ns + i) * r + h;
        const float w = __builtin_amdgcn_exp2f(a.ws_ml[base * 2] - mx);
        lsum += w * a.ws_ml[base * 2 + 1];
        if (L < D) o0 += w * a.ws_o[base * D + L];
        if (L + kWave < D) o1 += w * a.ws_o[base * D + L + kWave];
    }
    const float inv = 1.0f / lsum;
    uint16_t* dst = a.out + (s * r + h) * D;
    if (L < D) dst[L] = __builtin_bit_cast(uint16_t, (f16)(o0 * inv));
    if (L + kWave < D) dst[L + kWave] = __builtin_bit_cast(uint16_t, (f16)(o1 * inv));
}

template <int KB, int VB>
int run_attention(const AttnArgs& a, hipStream_t st) {
    const int64_t groups = a.n_slices * a.plan.n_splits;
    hipLaunchKernelGGL((attention_kernel<KB, VB>), dim3((unsigned)groups), dim3(kWave), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    if (a.plan.n_splits > 1) {
        hipLaunchKernelGGL(attention_merge_kernel, dim3((unsigned)(a.n_slices * a.q_per_kv)), dim3(kWave), 0,
                           st, a);
        e = hipGetLastError();
    }
    return (int)e;
}

}  // namespace

int launch_attention(const AttnArgs& a, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (a.n_slices == 0) return 0;
#define KIVI_ATTN(KB, VB) \
    if (a.k_bits == KB && a.v_bits == VB) return run_attention<KB, VB>(a, st);
    KIVI_ATTN(2, 2) KIVI_ATTN(2, 4) KIVI_ATTN(2, 8)
    KIVI_ATTN(4, 2) KIVI_ATTN(4, 4) KIVI_ATTN(4, 8)
    KIVI_ATTN(8, 2) KIVI_ATTN(8, 4) KIVI_ATTN(8, 8)
#undef KIVI_ATTN
    return (int)hipErrorInvalidValue;
}

}  // namespace kivi
