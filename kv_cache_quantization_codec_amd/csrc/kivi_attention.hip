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
//   the code's bit offset inside its byte.  Codes are staged in LDS
//   byte-transposed (see bytes_t4), so a lane's eight codes for one operand
//   sit in two dwords and come out with one AND, or a shift and an AND, per
//   pair; the column factor 2^(24-sh) is applied to the fp32 result.
// * The value zero-point term is a separate MFMA: p against the rows'
//   zeros, whose 16 output columns hold up to 16 value groups at once.  The
//   key zero-point term (identical in every token column of a group) is an
//   MFMA of q against the group's zeros when a KV slice serves 3-8 query
//   heads, and an fp32 dot product reduced over the wave for 1-2.
// * Value codes are loaded so that the lanes of one load instruction read
//   whole consecutive token rows (a code unit is one word column of tokens
//   p, p + 16, p + 8, p + 24); the value product's token order follows the
//   units (vslot), and the weight operands are written in that order.
// * Four kernel variants by the bound on query heads per KV slice (1, 2,
//   4, 8) size the LDS operand rows and drop the second head of a lane row
//   where there is none.  Lane rows of the value-weight step that hold no
//   head take a share of the value groups; the key-score operand rows
//   repeat in every group of four (1-2 heads) or eight (3-4 heads) MFMA
//   rows, so every lane row has the weights it needs without a cross-lane
//   copy.  A slice's full 32-token blocks run without per-token bounds;
//   only its last block can be partial.
// * The logit scale is folded into the pre-scaled query (1-2 heads) or the
//   column factor and key zero term (3-8 heads).
// * Online softmax in base 2 per 32-token block; heads live in MFMA rows, so
//   each lane holds two heads' scores of one token and the row reductions
//   are DPP moves inside a 16-lane row.  A block whose scores all stay at or
//   below the running maxima (most blocks of a long cache) skips the
//   reductions and the rescale; the sums are per lane until the end.
// One wave per workgroup; a workgroup walks a range of 32-token blocks of
// one slice (or that slice's residual) and either writes the normalised
// output or, when the slice is split, its partial (max, sum, output) for a
// merge kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "../../include/kivi.h"
#include "kivi_launch.h"

namespace kivi {
namespace {

typedef _Float16 f16;
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTokStride = 32 + 8;        // halves per row of a 32-token operand
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

// Sum over the whole wave (every lane gets the total): row sums, then the
// four rows' totals read out as uniform values.
__device__ __forceinline__ float wave_sum(float v) {
    const int b = __builtin_bit_cast(int, row16_sum(v));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// base + a 32-bit byte offset: with a wave-uniform base the load can take
// the scalar-base form, and the lane's address arithmetic stays 32-bit.
template <class T>
__device__ __forceinline__ const T* at_byte(const T* base, uint32_t off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

__device__ __forceinline__ float lo_f(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xFFFF)); }
__device__ __forceinline__ float hi_f(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16)); }

// Codes are staged in LDS byte-transposed: four words w0..w3 (four channels
// of one key word row, or one value word column of four consecutive tokens)
// become four dwords, dword b holding byte b of each word in the order
// (w0, w2, w1, w3).  A lane's eight codes for one MFMA operand (eight
// consecutive channels, or tokens, at one code position) then sit in two
// dwords instead of eight words, which cuts the operand's LDS reads
// fourfold, and the order lets a single AND pick out two of the codes.
__device__ __forceinline__ u32x4 bytes_t4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    const uint32_t p = __builtin_amdgcn_perm(w2, w0, 0x05010400u);   // w0.0 w2.0 w0.1 w2.1
    const uint32_t q = __builtin_amdgcn_perm(w2, w0, 0x07030602u);   // w0.2 w2.2 w0.3 w2.3
    const uint32_t r = __builtin_amdgcn_perm(w3, w1, 0x05010400u);   // w1.0 w3.0 w1.1 w3.1
    const uint32_t u = __builtin_amdgcn_perm(w3, w1, 0x07030602u);   // w1.2 w3.2 w1.3 w3.3
    return u32x4{__builtin_amdgcn_perm(r, p, 0x05040100u),           // w0.0 w2.0 w1.0 w3.0
                 __builtin_amdgcn_perm(r, p, 0x07060302u),           // w0.1 w2.1 w1.1 w3.1
                 __builtin_amdgcn_perm(u, q, 0x05040100u),           // w0.2 w2.2 w1.2 w3.2
                 __builtin_amdgcn_perm(u, q, 0x07060302u)};          // w0.3 w2.3 w1.3 w3.3
}

// Where a lane's code sits: element m of a word (m = position along the
// packing axis) occupies bits [BITS*m, BITS*m + BITS): byte bi, shift sh.
template <int BITS>
struct CodePos {
    int bi;          // byte of the word, i.e. dword of a transposed group of four
    uint32_t mask;   // the code in both 16-bit halves
    float col;       // 2^(24 - sh), undoes the subnormal encoding
    __device__ explicit CodePos(int m) {
        const int bit = BITS * m;
        const int sh = bit & 7;
        bi = bit >> 3;
        mask = ((uint32_t)((1 << BITS) - 1) << sh) * 0x00010001u;
        col = pow2(24 - sh);
    }
};

// Eight codes as fp16 operands from two transposed dwords d0 (elements
// 0..3) and d1 (4..7): code c at shift sh becomes the fp16 bit pattern
// c << sh, the exact subnormal c * 2^(sh - 24).
__device__ __forceinline__ h8 codes8(uint32_t d0, uint32_t d1, uint32_t mask) {
    return __builtin_bit_cast(h8, u32x4{d0 & mask, (d0 >> 8) & mask, d1 & mask, (d1 >> 8) & mask});
}

// A wave's LDS instructions execute in program order, so one wave sharing
// data through LDS needs no s_barrier (nor the fence of __syncthreads, which
// would also wait for the global loads kept in flight across a block); this
// only stops the compiler from moving LDS accesses across the point.
__device__ __forceinline__ void lds_order() { __asm__ __volatile__("" ::: "memory"); }

// Operand slot of value-product token t in [0, 16) (token t + 16 takes the
// next slot): a lane's eight slots 8kq .. 8kq + 7 hold the tokens of code
// units p = 2kq and 2kq + 1, each unit being tokens p, p + 16, p + 8, p + 24.
__device__ __forceinline__ int vslot(int t) { return 8 * ((t & 7) >> 1) + 4 * (t & 1) + 2 * (t >> 3); }

// 16-byte LDS read as an MFMA operand.
__device__ __forceinline__ h8 lds_h8(const void* p) {
    return __builtin_bit_cast(h8, *reinterpret_cast<const u32x4*>(p));
}

// fp32 x as fp16 hi + lo with hi = fp16(x), lo = fp16(x - hi); x - hi is
// exact in fp32, so hi + lo is within 2^-22 |x| of x (|x| < 65504).
__device__ __forceinline__ void split_hl(float x, f16& hi, f16& lo) {
    hi = (f16)x;
    lo = (f16)(x - (float)hi);
}

// Two products x_i = a_i * b_i (exact, fused) split as packed pairs
// hi = (fp16(x0), fp16(x1)) and lo = (fp16(x0 - hi0), fp16(x1 - hi1)): the
// mixed-precision FMAs write one 16-bit half each and read hi's halves
// directly, four instructions in all.  hi + lo is within 2^-22 |x_i| of x_i.
__device__ __forceinline__ void split_prod2(float a0, float b0, float a1, float b1, uint32_t& hi,
                                            uint32_t& lo) {
    __asm__("v_fma_mixlo_f16 %0, %2, %3, 0\n\t"
            "v_fma_mixhi_f16 %0, %4, %5, 0\n\t"
            "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel_hi:[0,0,1]\n\t"
            "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
            : "=&v"(hi), "=&v"(lo)
            : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}

// LDS of one wave (D = head_dim, at most RMAX query heads per KV slice, so
// 2*RMAX live MFMA rows).  When that leaves MFMA rows dead (2*RMAX < 16),
// each A-operand array has one more row that is always zero: lanes of the
// dead rows read it (one address, a broadcast), so operand reads need no
// exec masking.  Row strides are padded by 16 bytes so that the rows an
// MFMA operand read touches fall in different banks.  The head bound RMAX
// is 2, 4 or 8 (the smallest that covers q_per_kv): sizing the rows by it
// keeps LDS from limiting the resident waves (multi-head 7.4 KB, 4 heads
// 11.6 KB, 8 heads 17.4 KB per wave at head_dim 128).
template <int RMAX>
constexpr int operand_rows() { return 2 * RMAX < 16 ? 2 * RMAX + 1 : 2 * RMAX; }

template <int KB, int VB, int D, int RMAX>
struct alignas(16) Smem {
    f16 q[RMAX + 1][D + 8];                // the slice's queries, one row per head
    f16 aq[operand_rows<RMAX>()][D + 8];   // q*s of the current key group, hi/lo rows
    f16 kz[D];                             // zeros of the current key group
    uint32_t kt[KB][D];                    // key codes of a 32-token block: [word row][channel/4][byte]
    uint32_t vt[VB * D / 32][32 + 4];      // value codes: [word column][token unit][byte] (padded)
    f16 vz[5][kTokStride];                 // value zeros, [group][operand slot of the row]; row 4 zero
    float vs[4][32 + 4];                   // value scales, [group][row]
    f16 ap[4][operand_rows<RMAX>()][kTokStride];   // p*s per value group, hi/lo rows
    f16 apz[operand_rows<RMAX>()][kTokStride];     // p, hi/lo rows
};

// Per-wave running softmax state and output accumulators for the two heads
// this lane's MFMA rows hold (a = 2*kq, b = 2*kq + 1).  The running maxima
// are uniform over a 16-lane row; the sums l are this lane's share (its two
// tokens of every block), summed over the row once at the end.
template <int D>
struct Acc {
    float m_a, m_b, l_a, l_b;
    f4 o[D / 16];       // MFMA output tiles of 16 channels
    f4 z;               // value zero-point term, columns = value groups
};

// Online-softmax update with scores x (log2 units) of two 16-token tiles;
// returns the block weights p in xa/xb and rescales the accumulators.
// Where no score of the block exceeds its head's running maximum (all but a
// few blocks of a long cache), the maximum stays and every rescale factor
// is exactly 1, so the row reductions and the rescale are skipped; the
// weights are the same either way.
// HB: a lane row's second head can exist (at most one head per KV slice
// leaves head b, and its weights, untouched).
template <int D, bool HB>
__device__ __forceinline__ void softmax_block(Acc<D>& acc, float xa[2], float xb[2]) {
    const float ma = fmaxf(xa[0], xa[1]), mb = HB ? fmaxf(xb[0], xb[1]) : kNegInf;
    if (__ballot(ma > acc.m_a || (HB && mb > acc.m_b)) != 0) {
        const float mn_a = fmaxf(acc.m_a, row16_max(ma));
        const float al_a = __builtin_amdgcn_exp2f(acc.m_a - mn_a);
        acc.m_a = mn_a;
        acc.l_a *= al_a;
        float al_b = 1.0f;
        if constexpr (HB) {
            const float mn_b = fmaxf(acc.m_b, row16_max(mb));
            al_b = __builtin_amdgcn_exp2f(acc.m_b - mn_b);
            acc.m_b = mn_b;
            acc.l_b *= al_b;
        }
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) {
            acc.o[nt][0] *= al_a;
            acc.o[nt][1] *= al_a;
            if constexpr (HB) {
                acc.o[nt][2] *= al_b;
                acc.o[nt][3] *= al_b;
            }
        }
        acc.z[0] *= al_a;
        acc.z[1] *= al_a;
        if constexpr (HB) {
            acc.z[2] *= al_b;
            acc.z[3] *= al_b;
        }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        xa[tt] = __builtin_amdgcn_exp2f(xa[tt] - acc.m_a);
        if constexpr (HB) xb[tt] = __builtin_amdgcn_exp2f(xb[tt] - acc.m_b);
    }
    acc.l_a += xa[0] + xa[1];
    if constexpr (HB) acc.l_b += xb[0] + xb[1];
}

// The residual block's softmax weights (this lane: tokens 16tt + j of heads
// 2kq and 2kq+1) as hi/lo fp16 rows of the value operand apz ([2h / 2h+1]
// [token]); the residual's value product runs in token order.
template <class SM>
__device__ __forceinline__ void weights_to_lds(SM& sm, const float pa[2], const float pb[2], int r) {
    const int L = threadIdx.x, j = L & 15, kq = L >> 4;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int h = 2 * kq + hh;
        if (h < r) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f16 hi, lo;
                split_hl(hh ? pb[tt] : pa[tt], hi, lo);
                sm.apz[2 * h][16 * tt + j] = hi;
                sm.apz[2 * h + 1][16 * tt + j] = lo;
            }
        }
    }
    lds_order();
}

template <int D>
__device__ __forceinline__ void write_result(const AttnArgs& a, const Acc<D>& acc, int64_t s, int split,
                                             const float oa[], const float ob[]) {
    const int L = threadIdx.x, j = L & 15, kq = L >> 4;
    const int r = a.q_per_kv;
    const int ha = 2 * kq, hb = 2 * kq + 1;
    // the row totals of the lanes' partial sums
    const float l_a = row16_sum(acc.l_a), l_b = row16_sum(acc.l_b);
    if (a.plan.n_splits == 1) {
        // a slice with no token at all (ragged batch) has l = 0: output 0
        const float ia = l_a > 0.0f ? 1.0f / l_a : 0.0f;
        const float ib = l_b > 0.0f ? 1.0f / l_b : 0.0f;
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) {
            if (ha < r) a.out[(s * r + ha) * D + 16 * nt + j] = __builtin_bit_cast(uint16_t, (f16)(oa[nt] * ia));
            if (hb < r) a.out[(s * r + hb) * D + 16 * nt + j] = __builtin_bit_cast(uint16_t, (f16)(ob[nt] * ib));
        }
        return;
    }
    const int64_t base = (s * a.plan.n_splits + split) * r;
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
        if (ha < r) a.ws_o[(base + ha) * D + 16 * nt + j] = oa[nt];
        if (hb < r) a.ws_o[(base + hb) * D + 16 * nt + j] = ob[nt];
    }
    if (j == 0) {
        if (ha < r) {
            a.ws_ml[(base + ha) * 2] = acc.m_a;
            a.ws_ml[(base + ha) * 2 + 1] = l_a;
        }
        if (hb < r) {
            a.ws_ml[(base + hb) * 2] = acc.m_b;
            a.ws_ml[(base + hb) * 2 + 1] = l_b;
        }
    }
}

// ---------------------------------------------------------------------------
// the attention kernel: blockIdx.x = slice * n_splits + split
// ---------------------------------------------------------------------------

// Register budget: 4 waves per SIMD (128 VGPRs) for the one-head variant
// with codes of at most 4 bits and the two-head one with 2-bit values,
// which fit it without spilling; 3 waves for the rest where the compiler
// can meet it (measured 5% faster than 2 at head_dim 128, 2/2-bit); the
// wider code types stay at 2, which the compiler reports and this file
// accepts.
template <int KB, int VB, int RMAX>
constexpr int min_waves() {
    return (RMAX == 1 && KB <= 4 && VB <= 4) || (RMAX == 2 && KB <= 4 && VB == 2) ? 4 : 3;
}
#pragma clang diagnostic ignored "-Wpass-failed"
template <int KB, int VB, int D, int G, int RMAX>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(min_waves<KB, VB, RMAX>(), 8))) attention_kernel(const AttnArgs a) {
    constexpr int NK32 = D / 32, NT16 = D / 16, ROWS = 2 * RMAX, OROWS = operand_rows<RMAX>();
    constexpr bool HB = RMAX > 1;                         // a lane row can hold a second head
    constexpr bool FEW = RMAX <= 2;                       // at most two heads: MFMA rows 0-3
    __shared__ Smem<KB, VB, D, RMAX> sm;
    const int L = threadIdx.x, j = L & 15, kq = L >> 4;
    const int r = a.q_per_kv;
    const int64_t s = blockIdx.x / a.plan.n_splits;
    const int split = (int)(blockIdx.x - s * a.plan.n_splits);
    const bool residual = a.plan.has_res && split == a.plan.n_splits - 1;
    // this slice's token counts: uniform, or per slice (ragged) clamped to
    // the bounds that sized the work
    const int n_quant_s = a.n_quant_s ? min(max(a.n_quant_s[s], 0), a.n_quant) : a.n_quant;
    const int res_count_s = a.res_count_s ? min(max(a.res_count_s[s], 0), a.res_count) : a.res_count;

    // LDS set-up: operand rows that are never written (and the zero rows)
    // stay zero; the queries, where the kernel reads them from LDS (rows of
    // heads >= r and the zero row are zero).  One wave per workgroup: its
    // LDS accesses execute in order, so a compiler barrier orders them (a
    // __syncthreads fence would also wait for every load in flight).
    auto setup_lds = [&](bool with_q) {
        for (int i = L; i < OROWS * (D + 8); i += kWave) (&sm.aq[0][0])[i] = (f16)0;
        for (int i = L; i < 4 * OROWS * kTokStride; i += kWave) (&sm.ap[0][0][0])[i] = (f16)0;
        for (int i = L; i < OROWS * kTokStride; i += kWave) (&sm.apz[0][0])[i] = (f16)0;
        if (L < kTokStride) sm.vz[4][L] = (f16)0;
        if (with_q)
            for (int i = L; i < (RMAX + 1) * D / 8; i += kWave) {
                const int h = i / (D / 8), c = 8 * (i - h * (D / 8));
                u32x4 w = u32x4{0, 0, 0, 0};
                if (h < r && h < RMAX) w = *reinterpret_cast<const u32x4*>(a.q + (s * r + h) * D + c);
                *reinterpret_cast<u32x4*>(&sm.q[h][c]) = w;
            }
        lds_order();
    };
    // A-operand rows: lane row j; lanes of rows >= ROWS read the zero row
    // (there are none when ROWS = 16)
    const int jr = j < ROWS ? j : OROWS - 1;
    // key-score A rows: with at most 2 (4) heads their rows repeat in every
    // group of 4 (8) MFMA rows, so every lane row gets the scores of the
    // heads whose weights it works on
    constexpr int PER = FEW ? 4 : RMAX == 4 ? 8 : 16;
    const int jp = j % PER;
    const int jk = jp < ROWS ? jp : OROWS - 1;
    // q as MFMA A operand, rows 2h = q_h and 2h+1 = 0 (repeating like the
    // key-score rows): lane row j, channels 32*kk + 8*kq .. +7
    const int qr = ((jp & 1) == 0 && (jp >> 1) < RMAX) ? jp >> 1 : RMAX;
    auto qa = [&](int kk) { return lds_h8(&sm.q[qr][32 * kk + 8 * kq]); };

    Acc<D> acc;
    acc.m_a = acc.m_b = kNegInf;
    acc.l_a = acc.l_b = 0.0f;
#pragma unroll
    for (int nt = 0; nt < NT16; ++nt) acc.o[nt] = f4{0, 0, 0, 0};
    acc.z = f4{0, 0, 0, 0};

    float oa[NT16], ob[NT16];

    if (residual) {
        // ---- fp16 residual: plain fp16 operands ----
        setup_lds(true);
        const uint16_t* rk = a.res_k + s * a.res_stride;
        const uint16_t* rv = a.res_v + s * a.res_stride;
        for (int i0 = 0; i0 < res_count_s; i0 += 32) {
            float xa[2], xb[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int i = i0 + 16 * tt + j;
                const bool valid = i < res_count_s;
                int slot = a.res_head + (valid ? i : 0);
                if (slot >= a.res_slots) slot -= a.res_slots;
                const uint16_t* row = rk + (int64_t)slot * D;
                u32x4 w[NK32];
#pragma unroll
                for (int kk = 0; kk < NK32; ++kk) {
                    w[kk] = *reinterpret_cast<const u32x4*>(row + 32 * kk + 8 * kq);
                    if (!valid) w[kk] = u32x4{0, 0, 0, 0};
                }
                f4 sc = f4{0, 0, 0, 0};
#pragma unroll
                for (int kk = 0; kk < NK32; ++kk) sc = mfma(qa(kk), __builtin_bit_cast(h8, w[kk]), sc);
                xa[tt] = valid ? (sc[0] + sc[1]) * a.logit_scale : kNegInf;
                xb[tt] = HB && valid ? (sc[2] + sc[3]) * a.logit_scale : kNegInf;
            }
            softmax_block<D, HB>(acc, xa, xb);
            weights_to_lds(sm, xa, xb, r);
            // values: B[token 8kq+e][channel 16nt+j]
            const h8 pa8 = lds_h8(&sm.apz[jr][8 * kq]);
            const uint16_t* vrow[8];
            bool valid[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = i0 + 8 * kq + e;
                valid[e] = i < res_count_s;
                int slot = a.res_head + (valid[e] ? i : 0);
                if (slot >= a.res_slots) slot -= a.res_slots;
                vrow[e] = rv + (int64_t)slot * D + j;
            }
#pragma unroll
            for (int nt = 0; nt < NT16; ++nt) {
                h8 b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t x = vrow[e][16 * nt];
                    b[e] = __builtin_bit_cast(f16, valid[e] ? x : (uint16_t)0);
                }
                acc.o[nt] = mfma(pa8, b, acc.o[nt]);
            }
            lds_order();       // pp / apz are rewritten by the next block
        }
#pragma unroll
        for (int nt = 0; nt < NT16; ++nt) {
            oa[nt] = acc.o[nt][0] + acc.o[nt][1];
            ob[nt] = acc.o[nt][2] + acc.o[nt][3];
        }
        write_result<D>(a, acc, s, split, oa, ob);
        return;
    }

    // ---- quantized prefix: blocks [b0, b1) of 32 tokens ----
    const int b0 = split * a.plan.blocks_per_split;
    const int n = n_quant_s;
    const int b1 = min(b0 + a.plan.blocks_per_split, (n + 31) / 32);
    constexpr int Wk = G * KB / 32;                       // key words per channel per group
    constexpr int NGV = (D + G - 1) / G;                  // value groups per row
    constexpr int WPT = NGV * G * VB / 32;                // value words per row
    const int ngk_cap = (a.cap_tokens + G - 1) / G;
    const int ngv = NGV, wpt = WPT;
    constexpr int RW = D * VB / 32;                       // value words per row that hold real channels
    const uint32_t* kcs = a.k_codes + s * (int64_t)ngk_cap * Wk * D;
    const uint16_t* kss = a.k_scale + s * (int64_t)ngk_cap * D;
    const uint16_t* kzs = a.k_zero + s * (int64_t)ngk_cap * D;
    const uint32_t* vcs = a.v_codes + s * (int64_t)a.cap_tokens * wpt;
    const uint16_t* vss = a.v_scale + s * (int64_t)a.cap_tokens * ngv;
    const uint16_t* vzs = a.v_zero + s * (int64_t)a.cap_tokens * ngv;
    const bool pair_live = 2 * L < D;                     // this lane's channel pair (2L, 2L+1) exists
    // At most two heads: this lane's query channels (2L, 2L+1) of heads 0
    // and 1 stay in registers (0 where absent), and a key group's zero-point
    // term sum_d q_d z_d is a dot product over the wave (fp32, as the MFMA
    // would accumulate it) instead of four MFMAs and their LDS operands.
    float qreg[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
    float zg0 = 0.0f, zg1 = 0.0f;                         // zero terms of heads 0 and 1
    if constexpr (FEW) {
#pragma unroll
        for (int h = 0; h < RMAX; ++h)
            if (h < r && pair_live) {
                const uint32_t qw = *reinterpret_cast<const uint32_t*>(a.q + (s * r + h) * D + 2 * L);
                qreg[h][0] = lo_f(qw) * a.logit_scale;
                qreg[h][1] = hi_f(qw) * a.logit_scale;
            }
    }
    // Three or four heads: their query channels (2L, 2L+1) stay in
    // registers too (unscaled), for the q*s operand rows of each key group.
    float q4[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
    if constexpr (RMAX == 4) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
            if (h < r && pair_live) {
                const uint32_t qw = *reinterpret_cast<const uint32_t*>(a.q + (s * r + h) * D + 2 * L);
                q4[h][0] = lo_f(qw);
                q4[h][1] = hi_f(qw);
            }
    }

    // One block's global data, held in registers from the previous block's
    // compute until it is written to LDS (so its load latency is hidden).
    constexpr int KCH = KB * D / 4;                       // 16-byte key-code chunks per block
    constexpr int KV = (KCH + kWave - 1) / kWave;
    constexpr int VU = 8 * RW;                            // value units: one word column of 4 tokens
    constexpr int VV = (VU + kWave - 1) / kWave;
    // value scales and zeros of a block: 32 rows of NGV halves, staged as
    // pairs of one row (a dword) when NGV is even, else one half per load
    constexpr int SPL = NGV % 2 == 0 ? 2 : 1;             // halves per staged load
    constexpr int NSE = 32 * NGV / SPL;                   // staged loads per block
    constexpr int NSW = (NSE + kWave - 1) / kWave;
    struct Stage {
        u32x4 k[KV];
        uint32_t v[VV][4];
        uint32_t vsb[NSW], vzb[NSW];
        uint32_t ks, kz;
    };
    // Addresses: wave-uniform bases of the block (64-bit, scalar) plus lane
    // byte offsets below 2^32 (at most 32 rows of one block).
    auto load = [&](int blk, Stage& st, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;  // all 32 rows of the block are valid
        const int t0 = 32 * blk, g = t0 / G;
        const int last = n - 1 - t0;                      // rows past n read row n-1 (weights 0)
        auto clamp = [&](int row) { return FULL ? row : min(row, last); };
        const uint32_t* srck = kcs + ((int64_t)g * Wk + ((t0 % G) / 32) * KB) * D;
        const uint32_t* vrow = vcs + (int64_t)t0 * WPT;
        const uint16_t* srow = vss + (int64_t)t0 * NGV;
        const uint16_t* zrow = vzs + (int64_t)t0 * NGV;
#pragma unroll
        for (int i = 0; i < KV; ++i) {
            const int v = L + kWave * i;
            if (KCH % kWave == 0 || v < KCH)
                st.k[i] = __builtin_nontemporal_load(at_byte(reinterpret_cast<const u32x4*>(srck), 16u * v));
        }
#pragma unroll
        for (int i = 0; i < VV; ++i) {
            const int u = L + kWave * i;
            if (VU % kWave == 0 || u < VU) {
                // word column c2, tokens p, p + 16, p + 8, p + 24 (the value
                // product's token order, see below); the lanes of one load
                // instruction cover whole consecutive token rows
                const int c2 = u % RW, p = u / RW;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = clamp(p + 16 * (e & 1) + 8 * (e >> 1));
                    st.v[i][e] = __builtin_nontemporal_load(at_byte(vrow, 4u * (uint32_t)(row * WPT + c2)));
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int e = SPL * (L + kWave * i);
            if (NSE % kWave == 0 || e < 32 * NGV) {
                const int row = e / NGV, gv = e - row * NGV;
                const uint32_t off = 2u * (uint32_t)(clamp(row) * NGV + gv);   // masked below
                if constexpr (SPL == 2) {    // 4-byte aligned: even NGV and gv
                    st.vsb[i] = *at_byte(reinterpret_cast<const uint32_t*>(srow), off);
                    st.vzb[i] = *at_byte(reinterpret_cast<const uint32_t*>(zrow), off);
                } else {
                    st.vsb[i] = *at_byte(srow, off);
                    st.vzb[i] = *at_byte(zrow, off);
                }
            }
        }
        if ((t0 % G == 0 || blk == b0) && pair_live) {
            st.ks = *at_byte(reinterpret_cast<const uint32_t*>(kss + (int64_t)g * D), 4u * L);
            st.kz = *at_byte(reinterpret_cast<const uint32_t*>(kzs + (int64_t)g * D), 4u * L);
        }
    };
    auto commit = [&](int blk, const Stage& st, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int t0 = 32 * blk;
#pragma unroll
        for (int i = 0; i < KV; ++i) {
            const int v = L + kWave * i;
            if (KCH % kWave == 0 || v < KCH) {
                const int row = (4 * v) / D, col = (4 * v) % D;
                const u32x4& w = st.k[i];
                *reinterpret_cast<u32x4*>(&sm.kt[row][col]) = bytes_t4(w.x, w.y, w.z, w.w);
            }
        }
#pragma unroll
        for (int i = 0; i < VV; ++i) {
            const int u = L + kWave * i;
            if (VU % kWave == 0 || u < VU) {
                const uint32_t* w = st.v[i];
                *reinterpret_cast<u32x4*>(&sm.vt[u % RW][4 * (u / RW)]) = bytes_t4(w[0], w[1], w[2], w[3]);
            }
        }
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int e = SPL * (L + kWave * i);
            if (NSE % kWave == 0 || e < 32 * NGV) {
                const int row = e / NGV, gv = e - row * NGV;
                const bool live = FULL || t0 + row < n;
                const int zs = vslot(row & 15) + (row >> 4);
#pragma unroll
                for (int u = 0; u < SPL; ++u) {
                    const uint16_t sb = (uint16_t)(st.vsb[i] >> (16 * u)), zb = (uint16_t)(st.vzb[i] >> (16 * u));
                    sm.vs[gv + u][row] = live ? (float)__builtin_bit_cast(f16, sb) : 0.0f;
                    sm.vz[gv + u][zs] = __builtin_bit_cast(f16, live ? zb : (uint16_t)0);
                }
            }
        }
        // a new key group: q*s operand rows (fp32 product split hi/lo) and zeros
        if constexpr (FEW) {
            if (t0 % G == 0 || blk == b0) {
                const float z0 = pair_live ? lo_f(st.kz) : 0.0f, z1 = pair_live ? hi_f(st.kz) : 0.0f;
                zg0 = wave_sum(__builtin_fmaf(qreg[0][1], z1, qreg[0][0] * z0));
                if constexpr (HB) zg1 = r > 1 ? wave_sum(__builtin_fmaf(qreg[1][1], z1, qreg[1][0] * z0)) : 0.0f;
                if (pair_live) {
                    const float s0 = lo_f(st.ks), s1 = hi_f(st.ks);
#pragma unroll
                    for (int h = 0; h < RMAX; ++h) {
                        if (h < r) {
                            uint32_t hi, lo;
                            split_prod2(qreg[h][0], s0, qreg[h][1], s1, hi, lo);
                            *reinterpret_cast<uint32_t*>(&sm.aq[2 * h][2 * L]) = hi;
                            *reinterpret_cast<uint32_t*>(&sm.aq[2 * h + 1][2 * L]) = lo;
                        }
                    }
                }
            }
        } else if ((t0 % G == 0 || blk == b0) && pair_live) {
            const float s0 = lo_f(st.ks), s1 = hi_f(st.ks);
            *reinterpret_cast<uint32_t*>(&sm.kz[2 * L]) = st.kz;
            if constexpr (RMAX == 4) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    if (h < r) {
                        uint32_t hi, lo;
                        split_prod2(q4[h][0], s0, q4[h][1], s1, hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.aq[2 * h][2 * L]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.aq[2 * h + 1][2 * L]) = lo;
                    }
                }
            } else {
                for (int h = 0; h < r; ++h) {
                    const uint32_t qw = *reinterpret_cast<const uint32_t*>(&sm.q[h][2 * L]);
                    uint32_t hi, lo;
                    split_prod2(lo_f(qw), s0, hi_f(qw), s1, hi, lo);
                    *reinterpret_cast<uint32_t*>(&sm.aq[2 * h][2 * L]) = hi;
                    *reinterpret_cast<uint32_t*>(&sm.aq[2 * h + 1][2 * L]) = lo;
                }
            }
        }
    };

    const int js = vslot(j);                              // operand slots of tokens j, j + 16
    const CodePos<KB> kpos(j % (32 / KB));
    const CodePos<VB> vpos(j % (32 / VB));
    // the logit scale rides on the column factor where q is not pre-scaled
    const float kcol = FEW ? kpos.col : kpos.col * a.logit_scale;
    const int zrow = j < ngv ? j : 4;                     // value-zero operand row (4: zeros)
    f4 zk = f4{0, 0, 0, 0};
    Stage stage;
    // blocks [b0, bf) hold 32 valid tokens each; only the slice's last block
    // may be partial and needs the per-token bounds
    const int bf = min(b1, n / 32);
    // with 1-2 heads the quantized prefix reads no query from LDS (the
    // query registers above serve it), so its LDS set-up follows the first
    // block's loads; with 3-8 heads the query rows go first
    if constexpr (!FEW) setup_lds(true);
    if (b0 < bf) load(b0, stage, std::true_type{});
    else if (b0 < b1) load(b0, stage, std::false_type{});
    if constexpr (FEW) setup_lds(false);

    auto block = [&](int blk, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int t0 = 32 * blk;
        commit(blk, stage, full_tag);
        lds_order();
        if (blk + 1 < bf) load(blk + 1, stage, std::true_type{});
        else if (blk + 1 < b1) load(blk + 1, stage, std::false_type{});

        // keys: the zero-point term of a new group, then the scores of two
        // 16-token tiles
        if (!FEW && (t0 % G == 0 || blk == b0)) {
            zk = f4{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < NK32; ++kk) zk = mfma(qa(kk), lds_h8(&sm.kz[32 * kk + 8 * kq]), zk);
        }
        f4 sc[2] = {f4{0, 0, 0, 0}, f4{0, 0, 0, 0}};
#pragma unroll
        for (int kk = 0; kk < NK32; ++kk) {
            const h8 aop = lds_h8(&sm.aq[jk][32 * kk + 8 * kq]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int wi = (16 * tt + j) / (32 / KB);
                const uint32_t* dp = &sm.kt[wi][32 * kk + 8 * kq + kpos.bi];
                const h8 bop = codes8(dp[0], dp[4], kpos.mask);
                sc[tt] = mfma(aop, bop, sc[tt]);
            }
        }
        float xa[2], xb[2];
        const float za = FEW ? zg0 : zk[0] * a.logit_scale, zb = FEW ? zg1 : zk[2] * a.logit_scale;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const bool valid = FULL || t0 + 16 * tt + j < n;
            xa[tt] = valid ? (sc[tt][0] + sc[tt][1]) * kcol + za : kNegInf;
            xb[tt] = HB && valid ? (sc[tt][2] + sc[tt][3]) * kcol + zb : kNegInf;
        }
        softmax_block<D, HB>(acc, xa, xb);

        // values: the product runs over the block's tokens in the slot
        // order of vslot (tokens t and t + 16 in adjacent slots), so the two
        // weights a lane holds (tokens j and 16 + j of heads 2kq and 2kq+1)
        // fill one dword of each hi/lo operand row: p itself, and p*s for
        // every value group.  Lane rows that hold no head take a share of
        // the groups, with the weights copied from the lanes that hold them.
        if constexpr (RMAX == 4 && NGV >= 2) {
            // heads live in lane rows kq = 0, 1; rows 2, 3 repeat them (the
            // key-score rows repeat) and take the upper half of the value
            // groups
            const bool upper = kq >= 2;
            constexpr int HG = NGV / 2;                    // groups of the lower rows
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int h = 2 * (kq & 1) + hh;
                if (h < r) {
                    const float p0 = hh ? xb[0] : xa[0], p1 = hh ? xb[1] : xa[1];
                    uint32_t hi, lo;
                    if (!upper) {
                        split_prod2(p0, 1.0f, p1, 1.0f, hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.apz[2 * h][js]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.apz[2 * h + 1][js]) = lo;
                    }
#pragma unroll
                    for (int g2 = 0; g2 < NGV - HG; ++g2) {
                        const int gv = upper ? HG + g2 : g2;
                        if (upper || g2 < HG) {
                            split_prod2(p0, sm.vs[gv][j], p1, sm.vs[gv][16 + j], hi, lo);
                            *reinterpret_cast<uint32_t*>(&sm.ap[gv][2 * h][js]) = hi;
                            *reinterpret_cast<uint32_t*>(&sm.ap[gv][2 * h + 1][js]) = lo;
                        }
                    }
                }
            }
        } else if constexpr (FEW && NGV >= 2) {
            // every lane row holds the weights of both heads (the key-score
            // rows repeat); row kq takes value groups kq, kq + 4, ...
#pragma unroll
            for (int hh = 0; hh < RMAX; ++hh) {
                if (hh < r) {
                    const float p0 = hh ? xb[0] : xa[0], p1 = hh ? xb[1] : xa[1];
                    uint32_t hi, lo;
                    if (kq == 0) {
                        split_prod2(p0, 1.0f, p1, 1.0f, hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.apz[2 * hh][js]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.apz[2 * hh + 1][js]) = lo;
                    }
#pragma unroll
                    for (int g4 = 0; g4 < (NGV + 3) / 4; ++g4) {
                        const int gv = 4 * g4 + kq;
                        if (gv < NGV) {
                            split_prod2(p0, sm.vs[gv][j], p1, sm.vs[gv][16 + j], hi, lo);
                            *reinterpret_cast<uint32_t*>(&sm.ap[gv][2 * hh][js]) = hi;
                            *reinterpret_cast<uint32_t*>(&sm.ap[gv][2 * hh + 1][js]) = lo;
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int hh = 0; hh < (HB ? 2 : 1); ++hh) {
                const int h = 2 * kq + hh;
                if (h < r) {
                    const float p0 = hh ? xb[0] : xa[0], p1 = hh ? xb[1] : xa[1];
                    uint32_t hi, lo;
                    split_prod2(p0, 1.0f, p1, 1.0f, hi, lo);
                    *reinterpret_cast<uint32_t*>(&sm.apz[2 * h][js]) = hi;
                    *reinterpret_cast<uint32_t*>(&sm.apz[2 * h + 1][js]) = lo;
    #pragma unroll
                    for (int gv = 0; gv < NGV; ++gv) {
                        split_prod2(p0, sm.vs[gv][j], p1, sm.vs[gv][16 + j], hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.ap[gv][2 * h][js]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.ap[gv][2 * h + 1][js]) = lo;
                    }
                }
            }
        }
        lds_order();
        // values: zero-point term over all groups at once (columns = groups)
        {
            const h8 pz = lds_h8(&sm.apz[jr][8 * kq]);
            const h8 bz = lds_h8(&sm.vz[zrow][8 * kq]);
            acc.z = mfma(pz, bz, acc.z);
        }
#pragma unroll
        for (int nt = 0; nt < NT16; ++nt) {
            const int gv = (16 * nt) / G;
            const h8 aop = lds_h8(&sm.ap[gv][jr][8 * kq]);
            const int col = (16 * nt + j) / (32 / VB);
            const uint32_t* dp = &sm.vt[col][8 * kq + vpos.bi];
            const h8 bop = codes8(dp[0], dp[4], vpos.mask);
            acc.o[nt] = mfma(aop, bop, acc.o[nt]);
        }
        lds_order();   // the next block's commit overwrites what this one read
    };
    int blk = b0;
    for (; blk < bf; ++blk) block(blk, std::true_type{});
    for (; blk < b1; ++blk) block(blk, std::false_type{});

    // output = code term * column factor + zero term of the channel's group;
    // the zero term of group gv sits in column gv of the same 16-lane row
    const float za = acc.z[0] + acc.z[1], zb = acc.z[2] + acc.z[3];
#pragma unroll
    for (int nt = 0; nt < NT16; ++nt) {
        const int gv = (16 * nt) / G;
        const float zra = __shfl(za, 16 * kq + gv, kWave);
        const float zrb = __shfl(zb, 16 * kq + gv, kWave);
        oa[nt] = (acc.o[nt][0] + acc.o[nt][1]) * vpos.col + zra;
        ob[nt] = (acc.o[nt][2] + acc.o[nt][3]) * vpos.col + zrb;
    }
    write_result<D>(a, acc, s, split, oa, ob);
}

// Merge of the partial results of a split slice: one wave per (slice,
// query head), four of them per workgroup, lanes over channels.  The
// splits' loads go out four at a time; the sums run over the splits in
// order.
constexpr int kMergeWaves = 4;
__global__ void __launch_bounds__(kMergeWaves * kWave) attention_merge_kernel(const AttnArgs a) {
    const int r = a.q_per_kv, D = a.head_dim, ns = a.plan.n_splits;
    const int64_t pair = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
    if (pair >= a.n_slices * r) return;
    const int64_t s = pair / r;
    const int h = (int)(pair - s * r);
    const int L = threadIdx.x & (kWave - 1);
    const bool c0 = L < D, c1 = L + kWave < D;
    const int64_t base0 = s * ns * r + h;                 // partial of split i: base0 + i * r
    float mx = kNegInf;
    for (int i0 = 0; i0 < ns; i0 += 4) {
        float m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) m[u] = i0 + u < ns ? a.ws_ml[(base0 + (int64_t)(i0 + u) * r) * 2] : kNegInf;
#pragma unroll
        for (int u = 0; u < 4; ++u) mx = fmaxf(mx, m[u]);
    }
    uint16_t* dst = a.out + (s * r + h) * D;
    if (mx == kNegInf) {                       // a slice with no token at all: output 0
        if (c0) dst[L] = 0;
        if (c1) dst[L + kWave] = 0;
        return;
    }
    float lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int i0 = 0; i0 < ns; i0 += 4) {
        float mm[4], ll[4], x0[4], x1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool in = i0 + u < ns;
            const int64_t b = base0 + (int64_t)(in ? i0 + u : 0) * r;
            mm[u] = a.ws_ml[b * 2];
            ll[u] = a.ws_ml[b * 2 + 1];
            x0[u] = c0 ? a.ws_o[b * D + L] : 0.0f;
            x1[u] = c1 ? a.ws_o[b * D + L + kWave] : 0.0f;
            if (!in) mm[u] = kNegInf;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (i0 + u < ns) {
                const float w = __builtin_amdgcn_exp2f(mm[u] - mx);
                lsum += w * ll[u];
                o0 += w * x0[u];
                o1 += w * x1[u];
            }
        }
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;   // a slice with no token: 0
    if (c0) dst[L] = __builtin_bit_cast(uint16_t, (f16)(o0 * inv));
    if (c1) dst[L + kWave] = __builtin_bit_cast(uint16_t, (f16)(o1 * inv));
}

template <int KB, int VB, int D, int G>
int run_attention(const AttnArgs& a, hipStream_t st) {
    const int64_t groups = a.n_slices * a.plan.n_splits;
    if (a.q_per_kv <= 1)
        hipLaunchKernelGGL((attention_kernel<KB, VB, D, G, 1>), dim3((unsigned)groups), dim3(kWave), 0, st, a);
    else if (a.q_per_kv <= 2)
        hipLaunchKernelGGL((attention_kernel<KB, VB, D, G, 2>), dim3((unsigned)groups), dim3(kWave), 0, st, a);
    else if (a.q_per_kv <= 4)
        hipLaunchKernelGGL((attention_kernel<KB, VB, D, G, 4>), dim3((unsigned)groups), dim3(kWave), 0, st, a);
    else
        hipLaunchKernelGGL((attention_kernel<KB, VB, D, G, 8>), dim3((unsigned)groups), dim3(kWave), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    if (a.plan.n_splits > 1) {
        const int64_t pairs = a.n_slices * a.q_per_kv;
        hipLaunchKernelGGL(attention_merge_kernel, dim3((unsigned)((pairs + kMergeWaves - 1) / kMergeWaves)),
                           dim3(kMergeWaves * kWave), 0, st, a);
        e = hipGetLastError();
    }
    return (int)e;
}

// The split partials of kivi_decode_attention_noalloc: a static buffer of
// each device (held until the process ends), so that entry point allocates
// nothing.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels get the per-device address from attention_scratch.
__device__ __align__(256) float scratch[KIVI_ATTENTION_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

int attention_scratch(void* stream, void** ptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return (int)e;
    int dev = cur;
    if (stream) {
        e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev);
        if (e != hipSuccess) return (int)e;
    }
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            // once per device, with that device current
            if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return (int)e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (dev != cur) {
                const hipError_t back = hipSetDevice(cur);
                if (e == hipSuccess) e = back;
            }
            if (e != hipSuccess || !p) return (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return (int)hipSuccess;
}

int launch_attention(const AttnArgs& a, void* stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (a.n_slices == 0) return 0;
#define KIVI_ATTN_G(KB, VB, D)                                                         \
    switch (a.group_size) {                                                            \
        case 32: return run_attention<KB, VB, D, 32>(a, st);                           \
        case 64: return run_attention<KB, VB, D, 64>(a, st);                           \
        case 128: return run_attention<KB, VB, D, 128>(a, st);                         \
        default: return (int)hipErrorInvalidValue;                                     \
    }
#define KIVI_ATTN(KB, VB)                                                              \
    if (a.k_bits == KB && a.v_bits == VB) {                                            \
        switch (a.head_dim) {                                                          \
            case 32: KIVI_ATTN_G(KB, VB, 32)                                           \
            case 64: KIVI_ATTN_G(KB, VB, 64)                                           \
            case 96: KIVI_ATTN_G(KB, VB, 96)                                           \
            case 128: KIVI_ATTN_G(KB, VB, 128)                                         \
            default: return (int)hipErrorInvalidValue;                                 \
        }                                                                              \
    }
    KIVI_ATTN(2, 2) KIVI_ATTN(2, 4) KIVI_ATTN(2, 8)
    KIVI_ATTN(4, 2) KIVI_ATTN(4, 4) KIVI_ATTN(4, 8)
    KIVI_ATTN(8, 2) KIVI_ATTN(8, 4) KIVI_ATTN(8, 8)
#undef KIVI_ATTN
#undef KIVI_ATTN_G
    return (int)hipErrorInvalidValue;
}

}  // namespace kivi
