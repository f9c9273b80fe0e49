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
// Improve Transformer") in binary32, division-free, as a fixed sequence of
// IEEE operations (fused multiply-adds explicit, nothing else contracted:
// the library is built with contraction off), so that its error over every
// input the kernels feed it -- all finite bf16 values -- is measured once
// on the host and holds on the GPU.
//   e = e^t with t = -min(|x|, 112) (below e^-112 nothing changes): Cody-
//   Waite reduction k = rint(t log2 e) (half to even), r = fma(-k, ln2_hi,
//   t) (exact: ln2_hi has 15 significant bits), r = fma(-k, ln2_lo, r); the
//   degree-7 Taylor polynomial p of e^r by Horner with fma; e = p 2^k.
//   d = 1 + e lies in (1, 2]; its reciprocal y takes three Newton steps
//   q = fma(-d, y, 1), y = fma(y, q, y) from the bit-pattern seed
//   0x7EF311C3 - bits(d) (within 5.1 % of 1/d).
//   x >= 0: SiLU = x y.  x < 0: SiLU = x e^x / (1 + e^x) = (x p y) 2^k, the
//   power of two applied last so that a result in the subnormal range is
//   rounded once (x is clamped at -112 there: below, the result rounds to
//   -0).  NaN stays NaN.
FP4Q_HD float silu_f32(float x)
{
    const float a = __builtin_fminf(__builtin_fabsf(x), 112.0f);
    const float t = -a;
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
    const int ki = (int)k;
    const float d = 1.0f + __builtin_ldexpf(p, ki);
    float y = u2f(0x7EF311C3u - f2u(d));
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const float q = __builtin_fmaf(-d, y, 1.0f);
        y = __builtin_fmaf(y, q, y);
    }
    const float neg = __builtin_ldexpf((-a * p) * y, ki);
    return x < 0.0f ? neg : x * y;
}

// E2M1 stochastic rounding ([Fusion] section "Two Key Numerical Techniques":
// up or down with probability proportional to the distance), eight values at
// a time: the codes of y[0..7] packed into one word (code j in bits 4j..4j+3),
// value j drawing r16 = r16_of(w, j).  The grid step is g = 0.5 below 2, 1 in
// [2, 4), 2 in [4, 6); with t = |y| / g and f its fractional part (the
// distance to the lower neighbour in steps), a value rounds up iff
// f * 2^16 > r16; |y| >= 6 saturates.  r16 is uniform on [0, 65535].
// Evaluated branch-free and exactly, on the code axis in fixed point
// (X = code * 2^22 + 2^22 f, codes 0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6):
//  - a = min(|y|, 6) first (Inf and NaN give 6): saturation happens before
//    the rounding, and every X below stays at most 7 * 2^22;
//  - a >= 1: X = bits(a) - bits(0.5) (one binade holds two codes);
//  - a < 1: the grid is linear, X = 2^23 a (exact); for integer m,
//    f 2^22 > m iff ceil(f 2^22) > m, so X = ceil(2^23 a) serves.  It is
//    read off the bits of 0.5 a + 0.5 rounded toward +infinity (on [0.5, 1]
//    binary32 steps are 2^-24, so those bits are bits(0.5) + ceil(2^23 a));
//  - both at once: X + bits(0.5) = max(that, bits(a), bits(0.5)): below 1
//    the first term is the larger, from 1 on the second (0.5 a + 0.5 <= a);
// then adding 2^22 - 1 - 64 r16 carries into the code iff 2^22 f > 64 r16
// (64 r16 < 2^22 - 1, so a ceiling that reaches the next code still rounds
// up).  The sign bit is kept for values that round to zero.  On the GPU the
// eight rounded-up FMAs run in one inline-assembly block that switches the
// wave's binary32 rounding mode (MODE bits 1:0) to +infinity and back, so no
// other floating-point instruction can be scheduled inside it; on the host
// the rounding up is done exactly through binary64.
FP4Q_HD uint32_t e2m1_sr8(const float y[8], const uint32_t w[4])
{
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __builtin_fminf(__builtin_fabsf(y[j]), 6.0f);
    uint32_t h[8];
#if defined(__HIP_DEVICE_COMPILE__)
    float r[8];
    asm volatile(
        "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 1\n\t"
        "s_nop 1\n\t"
        "v_fma_f32 %0, %8, 0.5, 0.5\n\t"
        "v_fma_f32 %1, %9, 0.5, 0.5\n\t"
        "v_fma_f32 %2, %10, 0.5, 0.5\n\t"
        "v_fma_f32 %3, %11, 0.5, 0.5\n\t"
        "v_fma_f32 %4, %12, 0.5, 0.5\n\t"
        "v_fma_f32 %5, %13, 0.5, 0.5\n\t"
        "v_fma_f32 %6, %14, 0.5, 0.5\n\t"
        "v_fma_f32 %7, %15, 0.5, 0.5\n\t"
        "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
        "s_nop 1"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = f2u(r[j]);
#else
    for (int j = 0; j < 8; ++j) {
        // the smallest binary32 f >= 0.5 a + 0.5, i.e. with 2 f - 1 >= a
        // (exact in binary64: f lies in [0.5, 3.5])
        float f = (float)(0.5 * (double)a[j] + 0.5);
        while (2.0 * (double)f - 1.0 < (double)a[j]) f = u2f(f2u(f) + 1u);
        h[j] = f2u(f);
    }
#endif
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t m = h[j] > f2u(a[j]) ? h[j] : f2u(a[j]);
        const uint32_t x = m > 0x3F000000u ? m : 0x3F000000u;  // X + bits(0.5)
        const uint32_t r16 = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
        // t = X + 2^22 - 1 - 64 r16 = x - 64 r16 - 0x3EC00001 (mod 2^32): on the
        // GPU -64 r16 is one 24-bit multiply that reads its half of the random
        // word directly, and the sum one three-operand add
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t n64;  // -64 times half (j & 1) of w[j >> 1], zero-extended
        if (j & 1)
            asm("v_mul_i32_i24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
                : "=v"(n64) : "v"(-64), "v"(w[j >> 1]));
        else
            asm("v_mul_i32_i24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
                : "=v"(n64) : "v"(-64), "v"(w[j >> 1]));
#else
        const uint32_t n64 = 0u - (r16 << 6);
#endif
        const uint32_t t = x + n64 + (0u - 0x3EC00001u);
        out |= ((t >> 22) | ((f2u(y[j]) >> 28) & 8u)) << (4 * j);
    }
    return out;
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

// E4M3 round-to-nearest-even with saturation to 448 (0x7E), z >= 0.
// Below 2^-6 the E4M3 step is 2^-9, so the code is rint(z * 512) (this also
// yields 0x08 when z rounds up to 2^-6); above, the 23-bit mantissa is
// rounded to 3 bits at bit 20 with the carry flowing into the exponent, and
// every z >= 448 (Inf and NaN included) comes out at least 0x7E, so one min
// saturates.  Both forms are computed and one is selected (no branch).
FP4Q_HD uint32_t e4m3_rne_satfinite(float z)
{
    const uint32_t b = f2u(z);
    const uint32_t sub = (uint32_t)rintf(fminf(z * 512.0f, 8.0f));  // z < 2^-6 (the min keeps the cast defined)
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);  // E4M3 bias 7, binary32 bias 127
    return b < 0x3C800000u ? sub : (code < 0x7Eu ? code : 0x7Eu);
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

// a / d rounded to nearest from y = RN(1/d) by one correction step
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Dev. 34(1), 1990): q0 = RN(a y) lies
// within one ulp of a / d, r = a - d q0 is exact (one FMA), and
// RN(q0 + r y) = RN(a / d), provided nothing overflows and neither q0 nor r
// leaves the normal range.
FP4Q_HD float div_by_recip(float a, float d, float y)
{
    const float q0 = a * y;
    const float r = __builtin_fmaf(-q0, d, a);
    return __builtin_fmaf(r, y, q0);
}

// A scale domain's constants for nv_block_scale_fast: S, RN(1/S), and
// whether the correction-step form is exact for every block of the domain.
// With 2^-92 <= S <= 2^116 (S = A / 2688 for a finite amax A of at least
// about 2^-80.6) both quotients b / 6 and (b / 6) / S, and their remainders,
// stay normal wherever the E4M3 code depends on them: a block scale below
// 2^-10 gives code 1 in either case (0 is clamped to 1), and that needs
// b / 6 >= 2^-102.  Outside the range (tiny, Inf or NaN S) the plain
// divisions run.
struct NvDomain {
    float S, rS;
    bool fast;
};
FP4Q_HD NvDomain nv_domain(float S)
{
    NvDomain t;
    t.S = S;
    t.rS = 1.0f / S;
    t.fast = S >= 0x1p-92f && S <= 0x1p116f;
    return t;
}

// nv_block_scale(b, S) with the two divisions done by correction steps
// from RN(1/6) and RN(1/S): the same value of (b / 6) / S, bit for bit,
// in a domain whose `fast` holds (checked on the host against the
// divisions for every bf16 block amax b <= A and every bf16 domain amax A).
FP4Q_HD uint32_t nv_block_scale_fast(float b, const NvDomain &t)
{
    float sbf;
    if (t.fast)
        sbf = div_by_recip(div_by_recip(b, 6.0f, 0x1.555556p-3f), t.S, t.rS);
    else
        sbf = (b / 6.0f) / t.S;
    const uint32_t sb = e4m3_rne_satfinite(sbf);
    return sb == 0u ? 1u : sb;
}

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

// The grid-stride walk of a partial-maximum pass: the thread starting at
// chunk `start` visits start, start + stride, ... below n, four per step
// (visit4(c) covers c, c + stride, c + 2 stride, c + 3 stride) while four
// fit, then one per step (visit1).  The counter is 64-bit: n may lie within
// a stride of 2^32, where a 32-bit counter would wrap back below n and never
// exit; every index handed to a visitor is below n, so it fits in 32 bits.
template <class F4, class F1>
FP4Q_HD void grid_stride_chunks(uint32_t start, uint32_t stride, uint32_t n, F4 &&visit4, F1 &&visit1)
{
    uint64_t c = start;
    for (; c + 3ull * stride < n; c += 4ull * stride) visit4((uint32_t)c);
    for (; c < n; c += stride) visit1((uint32_t)c);
}

// Division of 32-bit numerators by a divisor d fixed for a launch, as a
// multiply-high and shifts (Granlund and Montgomery, "Division by Invariant
// Integers using Multiplication", PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> 1)) >> (l - 1)
// for t = mulhi(m, n) and l >= 1 (d = 1: n itself).  Exact for every
// 32-bit n.
struct FastDiv {
    uint32_t m, l;
};
inline FastDiv fast_div_for(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint32_t m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    return FastDiv{m, l};
}
FP4Q_HD uint32_t fast_div(uint32_t n, FastDiv f)
{
    if (f.l == 0) return n;
    const uint32_t t = (uint32_t)(((uint64_t)f.m * n) >> 32);
    return (t + ((n - t) >> 1)) >> (f.l - 1);
}

// NVFP4 operand addresses (K % 16 == 0; tiled needs K % 128 == 0).  Linear:
// codes [R][K/2], scales [R][K/16].  Tiled (the NV GEMM's consumer layout):
// step-major row blocks, codes [Rp/32][K/128][32][64] and scales
// [Rp/32][K/128][32][8] (Rp = R rounded up to 32), so that one 128-wide K
// step of a 32-row group is 2 KiB of codes and 256 bytes of scales, each
// contiguous.  Byte offset of the 4 code bytes of 8-element chunk c8 of row
// r, and of the scale byte of 16-element block j of row r:
FP4Q_HD uint64_t nv_code_off(uint32_t r, uint32_t c8, uint32_t K, bool tiled)
{
    if (!tiled) return (uint64_t)r * (K >> 1) + (uint64_t)c8 * 4u;
    return (((uint64_t)(r >> 5) * (K >> 7) + (c8 >> 4)) * 32u + (r & 31u)) * 64u + (c8 & 15u) * 4u;
}
FP4Q_HD uint64_t nv_scale_off(uint32_t r, uint32_t j, uint32_t K, bool tiled)
{
    if (!tiled) return (uint64_t)r * (K >> 4) + j;
    return (((uint64_t)(r >> 5) * (K >> 7) + (j >> 3)) * 32u + (r & 31u)) * 8u + (j & 7u);
}

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
