// FP8 keys of the k8v4 cache layout, for gfx950 (MI355X).
//
// vLLM turboquant/config.py: the turboquant_k8v4 preset keeps keys in 8 bits
// and values in 4; 8-bit keys are FP8 with no rotation or codebook, and
// key_packed_size counts one byte per element with no scale -- a plain
// cast.  (The values of that layout are the KIVI value codec with one group
// per head, which the codec kernels already provide.)
//
// Format and rounding (the page names neither): OCP E4M3 (1 sign, 4
// exponent bits with bias 7, 3 mantissa bits, subnormals, NaN only at
// S.1111.111, largest finite 448); round to nearest, ties to the even code;
// magnitudes of 448 and more saturate to 448; the sign is kept.  The
// conversion is integer arithmetic on the fp16 bit pattern, so it does not
// depend on the hardware conversion's rounding or overflow behaviour.
//
// Both directions are elementwise and HBM-bound (3 bytes per element); a
// thread handles 8 consecutive elements of a token row: one 16-byte fp16
// access and one 8-byte code access.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_launch.h"

namespace kivi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;

// fp16 bits (finite) -> E4M3 code.
__device__ __forceinline__ uint32_t f16_to_e4m3(uint32_t h) {
    const uint32_t sign = (h >> 8) & 0x80u;
    const uint32_t mag = h & 0x7FFFu;
    if (mag >= 0x5F00u) return sign | 0x7Eu;            // |x| >= 448 (fp16 0x5F00)
    const uint32_t e = mag >> 10;                         // fp16 biased exponent
    uint32_t code;
    if (e >= 9) {
        // |x| >= 2^-6: an E4M3 normal with biased exponent e - 8; keep 3 of
        // the 10 mantissa bits, round half to even (a carry moves into the
        // exponent field, which is the right result)
        const uint32_t m = mag & 0x3FFu;
        const uint32_t rem = m & 0x7Fu;
        code = ((e - 8) << 3) | (m >> 7);
        code += (rem > 0x40u) || (rem == 0x40u && (code & 1u));
    } else {
        // |x| < 2^-6: subnormal code q = rint(|x| * 2^9), from 0 to 8 (8 is
        // the smallest normal, 0x08).  |x| * 2^9 = v * 2^-k with
        // v = 1024 + m, k = 16 - e for a normal fp16 and v = m, k = 15 for a
        // subnormal one; k is in [8, 15].
        const uint32_t v = e ? (0x400u | (mag & 0x3FFu)) : (mag & 0x3FFu);
        const uint32_t k = e ? 16u - e : 15u;
        const uint32_t q = v >> k;
        const uint32_t rem = v & ((1u << k) - 1u), half = 1u << (k - 1u);
        code = q + ((rem > half) || (rem == half && (q & 1u)));
    }
    return sign | code;
}

// E4M3 code -> fp16 bits (exact; S.1111.111 -> NaN).
__device__ __forceinline__ uint32_t e4m3_to_f16(uint32_t c) {
    const uint32_t sign = (c & 0x80u) << 8;
    const uint32_t E = (c >> 3) & 0xFu, m = c & 7u;
    if (E == 0xFu && m == 7u) return sign | 0x7E00u;
    if (E != 0) return sign | ((E + 8u) << 10) | (m << 7);   // (1 + m/8) 2^(E-7)
    if (m == 0) return sign;
    // m * 2^-9 with m in 1..7: an fp16 normal 2^(lz-9) * (m / 2^lz)
    const uint32_t lz = m >= 4 ? 2u : (m >= 2 ? 1u : 0u);
    return sign | ((6u + lz) << 10) | ((m << (10u - lz)) & 0x3FFu);
}

// blockIdx.y strides over slices; threads of x cover the slice's 8-element
// chunks (n_tokens * D / 8 of them).
__global__ void __launch_bounds__(kBlock)
fp8_encode_kernel(const uint16_t* __restrict__ in, int64_t in_stride, int n_tokens, int D,
                  int64_t n_slices, uint8_t* __restrict__ out, int64_t out_stride) {
    const int cpr = D / 8;
    const int chunks = n_tokens * cpr;
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= chunks) return;
    const int t = i / cpr, c = i - t * cpr;
    for (int64_t s = blockIdx.y; s < n_slices; s += gridDim.y) {
        const u32x4 x = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(in + s * in_stride + (int64_t)t * D + 8 * c));
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        uint32_t b[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            b[2 * k] = f16_to_e4m3(w[k] & 0xFFFFu);
            b[2 * k + 1] = f16_to_e4m3(w[k] >> 16);
        }
        const u32x2 o = {b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                         b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out + s * out_stride + (int64_t)t * D + 8 * c));
    }
}

__global__ void __launch_bounds__(kBlock)
fp8_decode_kernel(const uint8_t* __restrict__ in, int64_t in_stride, int n_tokens, int D,
                  int64_t n_slices, uint16_t* __restrict__ out, int64_t out_stride) {
    const int cpr = D / 8;
    const int chunks = n_tokens * cpr;
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= chunks) return;
    const int t = i / cpr, c = i - t * cpr;
    for (int64_t s = blockIdx.y; s < n_slices; s += gridDim.y) {
        const u32x2 x = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(in + s * in_stride + (int64_t)t * D + 8 * c));
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            h[k] = e4m3_to_f16((x.x >> (8 * k)) & 0xFFu);
            h[4 + k] = e4m3_to_f16((x.y >> (8 * k)) & 0xFFu);
        }
        const u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + s * out_stride + (int64_t)t * D + 8 * c));
    }
}

dim3 fp8_grid(const Fp8Args& a) {
    const int64_t chunks = (int64_t)a.n_tokens * (a.head_dim / 8);
    const int64_t gy = a.n_slices < 65535 ? a.n_slices : 65535;
    return dim3((unsigned)((chunks + kBlock - 1) / kBlock), (unsigned)gy);
}

}  // namespace

int launch_fp8_encode(const Fp8Args& a, void* stream) {
    if (a.n_slices == 0 || a.n_tokens == 0) return 0;
    hipLaunchKernelGGL(fp8_encode_kernel, fp8_grid(a), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(a.in), a.in_stride, a.n_tokens, a.head_dim, a.n_slices,
                       static_cast<uint8_t*>(a.out), a.out_stride);
    return (int)hipGetLastError();
}

int launch_fp8_decode(const Fp8Args& a, void* stream) {
    if (a.n_slices == 0 || a.n_tokens == 0) return 0;
    hipLaunchKernelGGL(fp8_decode_kernel, fp8_grid(a), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(a.in), a.in_stride, a.n_tokens, a.head_dim, a.n_slices,
                       static_cast<uint16_t*>(a.out), a.out_stride);
    return (int)hipGetLastError();
}

}  // namespace kivi
