// fp4q_device.h -- scalar building blocks of the libfp4q kernels (gfx950).
//
// Every function here is __host__ __device__ so that a CPU test can run the
// very same code over all relevant inputs; the kernels inline them.
//
// Pages cited (titles as printed):
//   [Fusion] "Format-Aware Fusion: The Engineering Practice That Doubles FP4
//            Pretraining Throughput"
//   [Stack]  "FP4 Is No Longer Just a Hardware Feature -- The NVFP4 Software
//            Stack Is Taking Shape"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define FP4Q_HD __host__ __device__ __forceinline__

namespace fp4q {

FP4Q_HD float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
FP4Q_HD uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two bf16 values packed in a u32 (element 0 in the low half); widening to
// binary32 is exact.
FP4Q_HD float bf16_lo(uint32_t u) { return u2f(u << 16); }
FP4Q_HD float bf16_hi(uint32_t u) { return u2f(u & 0xFFFF0000u); }

// binary32 -> bf16 bits, round to nearest even (finite values).
FP4Q_HD uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = f2u(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// SiLU(x) = x / (1 + e^-x) (SwiGLU's gate activation; Shazeer, "GLU Variants
// Improve Transformer") in binary32 as one fixed sequence of IEEE operations,
// so that every implementation of the sequence returns the same bits (the
// activation feeds the MX producer of H, whose codes must be reproducible);
// fused multiply-adds are explicit (one rounding each), nothing else is
// contracted (the library is built with contraction off).
//   e^t, t in [-20, 80]: Cody-Waite reduction k = rint(t log2 e) (half to
//   even), r = fma(-k, ln2_hi, t) (exact: ln2_hi has 15 significant bits),
//   r = fma(-k, ln2_lo, r); the degree-7 Taylor polynomial of e^r by Horner
//   with fma; times 2^k (exact).
//   SiLU: t = min(max(-x, -20), 80) (NaN -> -20); d = 1 + e^t; y = the bit
//   pattern 0x7EF311C3 - bits(d) (within 5.1 % of 1/d), three Newton steps
//   q = fma(-d, y, 1), y = fma(y, q, y); SiLU = x * y.  So SiLU(x) = x
//   exactly above 20, x / (1 + e^80) below -80, NaN stays NaN.
FP4Q_HD float exp_seq_f32(float t)
{
    const float k = __builtin_rintf(t * 0x1.715476p+0f);
    float r = __builtin_fmaf(-k, 0x1.62e4p-1f, t);
    r = __builtin_fmaf(-k, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;                   // 1/5040
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);   // 1/720
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);    // 1/120
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);    // 1/24
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);    // 1/6
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)k);
}

FP4Q_HD float silu_f32(float x)
{
    const float t = __builtin_fminf(__builtin_fmaxf(-x, -20.0f), 80.0f);
    const float d = 1.0f + exp_seq_f32(t);
    float y = u2f(0x7EF311C3u - f2u(d));
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const float q = __builtin_fmaf(-d, y, 1.0f);
        y = __builtin_fmaf(y, q, y);
    }
    return x * y;
}

// E2M1 stochastic rounding ([Fusion] section "Two Key Numerical Techniques":
// up or down with probability proportional to the distance).  The grid step
// is g = 0.5 below 2, 1 in [2, 4), 2 in [4, 6); with t = |y| / g, f its
// fractional part (the distance to the lower neighbour in steps), the value
// rounds up iff f * 2^16 > r16.  |y| >= 6 saturates.  r16 is uniform on
// [0, 65535].  Evaluated branch-free and exactly, on the code axis in fixed
// point (X = code * 2^22 + 2^22 f, codes 0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6):
//  - |y| >= 1: X = bits(|y|) - bits(0.5) (one binade holds two codes);
//  - |y| < 1: the grid is linear, X = 2^23 |y| (exact); for integer m,
//    f 2^22 > m iff ceil(f 2^22) > m, so X = ceil(2^23 |y|) serves;
//  - both at once: X = max(bits(|y|) - bits(0.5) saturated at 0,
//    ceil(2^23 min(|y|, 1))); below 1 the second term is the larger (equal
//    or above within [0.5, 1), the first is 0 below 0.5), from 1 on the first;
// then adding 2^22 - 1 - 64 r16 carries into the code iff 2^22 f > 64 r16
// (64 r16 < 2^22 - 1, so a ceiling that reaches the next code still rounds
// up).  Saturation is min(code, 7): the code is at least 7 for every
// |y| >= 6 (Inf and NaN included, no 32-bit wrap) and at most 7 below.  The
// selects stay selects: no divergent branch per element.
FP4Q_HD uint32_t e2m1_sr(float y, uint32_t r16)
{
    const uint32_t b = f2u(y);
    const uint32_t u = b & 0x7FFFFFFFu;
    const uint32_t s = (b >> 28) & 8u;
    const uint32_t ul = u < 0x3F800000u ? u : 0x3F800000u;  // |y| clamped to 1: in range of the conversion
    const uint32_t xl = (uint32_t)__builtin_ceilf(u2f(ul) * 8388608.0f);
    const uint32_t xh = u > 0x3F000000u ? u - 0x3F000000u : 0u;
    const uint32_t X = xh > xl ? xh : xl;
    const uint32_t c = (X + 0x3FFFFFu - (r16 << 6)) >> 22;
    return s | (c < 7u ? c : 7u);
}

// OCP MX shared exponent byte (E8M0) of a block whose amax has binary32 bits
// amax_bits: E = floor(log2 amax) - 2 clamped at -127 (zero and tiny blocks),
// byte = E + 127 = max(biased exponent field - 2, 0).
FP4Q_HD uint32_t mx_scale_byte(uint32_t amax_bits) { return (amax_bits >> 23) > 2u ? (amax_bits >> 23) - 2u : 0u; }

// 2^-E for scale byte E + 127: a normal binary32 for every byte the rule
// above produces (biased exponent 254 - byte in [2, 254]).
FP4Q_HD float mx_inv_scale(uint32_t byte) { return u2f((254u - byte) << 23); }

// OCP FP8 E4M3 value of a code 0x00..0x7E (bias 7, 3 mantissa bits,
// subnormal step 2^-9).
FP4Q_HD float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0) return (float)m * 0x1p-9f;
    return u2f(((e + 120u) << 23) | (m << 20));
}

// E4M3 round-to-nearest-even with saturation to 448 (0x7E), z >= 0 finite.
// Below 2^-6 the E4M3 step is 2^-9, so the code is rint(z * 512) (this also
// yields 0x08 when z rounds up to 2^-6); above, the 23-bit mantissa is
// rounded to 3 bits at bit 20 with the carry flowing into the exponent.
FP4Q_HD uint32_t e4m3_rne_satfinite(float z)
{
    if (z >= 448.0f) return 0x7Eu;
    const uint32_t b = f2u(z);
    if (b < 0x3C800000u) {  // z < 2^-6
        return (uint32_t)rintf(z * 512.0f);
    }
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t eb = (r >> 23) - 120u;  // E4M3 biased exponent (fp32 bias 127, E4M3 bias 7)
    const uint32_t code = (eb << 3) | ((r >> 20) & 7u);
    return code < 0x7Eu ? code : 0x7Eu;
}

// NVFP4 block scale byte and its reciprocal decode scale for block amax b in
// a domain with tensor scale S ([Stack] section "NVFP4 is more than a 4-bit
// value"; the clamp of section "The third change": the block scale never
// becomes zero).  Two correctly rounded divisions in this order, then
// d = e4m3(sb) * S and one reciprocal.
FP4Q_HD uint32_t nv_block_scale(float b, float S)
{
    const float sbf = (b / 6.0f) / S;
    const uint32_t sb = e4m3_rne_satfinite(sbf);
    return sb == 0u ? 1u : sb;
}
FP4Q_HD float nv_inv_decode(uint32_t sb, float S) { return 1.0f / (e4m3_value(sb) * S); }

// FP32 tensor-level scale of a domain with amax A (A = 0 gives 1): the
// domain's largest block then maps onto E4M3 448 x E2M1 6 = 2688.
FP4Q_HD float nv_tensor_scale(float A) { return A == 0.0f ? 1.0f : A / 2688.0f; }

// a ^ b ^ c: one v_bitop3_b32 (truth table 0x96) on gfx950.
FP4Q_HD uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
    return a ^ b ^ c;
#endif
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// -> 64-bit multiplies with the published multipliers and Weyl key increments.
FP4Q_HD void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1,
                           uint32_t out[4])
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// 16 random bits of element j (0..7) of the 8-element group whose Philox
// words are w[4]: word j/2, high half for odd j.
FP4Q_HD uint32_t r16_of(const uint32_t w[4], int j) { return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu); }

// Device-only helpers shared by the producers and the GEMM epilogue that
// quantizes its output.
// 2^E as binary32 for E8M0 byte E + 127 (byte 0 -> the subnormal 2^-127).
__device__ __forceinline__ float mx_scale_f32(uint32_t byte) { return byte ? u2f(byte << 23) : u2f(0x00400000u); }

// E2M1 round-to-nearest-even of x / scale for 8 values, by gfx950's scaled
// FP4 convert (2 values per instruction, element 2j in the low nibble of byte
// j); scale an exact power of two (see cvt8_bf16 in quant.hip for how the
// instruction was checked against the library's RNE rule).
__device__ __forceinline__ uint32_t cvt8_f32(const float f[8], float scale)
{
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[0], f[1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[2], f[3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[4], f[5], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, f[6], f[7], scale, 3);
    return r;
}


}  // namespace fp4q
