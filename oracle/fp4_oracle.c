/*
 * fp4_oracle.c -- plain, slow, scalar CPU reference for the FP4 block-scaled
 * quantizer and the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the GPU
 * path.  Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off (no fast-math,
 * no FMA contraction, so every float operation below is one IEEE-754 binary32
 * operation rounded to nearest-even, in the order written).
 *
 * Pages cited (titles as printed):
 *   [Fusion]  "Format-Aware Fusion: The Engineering Practice That Doubles FP4
 *              Pretraining Throughput"
 *   [Stack]   "FP4 Is No Longer Just a Hardware Feature -- The NVFP4 Software
 *              Stack Is Taking Shape"
 *   [OnGPUs]  "4-Bit Floating Point (FP4) on GPUs: How It Works and When It
 *              Pays Off"
 * Outside definitions used where the pages name a format without defining it:
 *   OCP Microscaling Formats (MX) v1.0 (E8M0 shared scale, 32-element blocks,
 *   shared exponent = floor(log2(amax)) - emax_elem with emax_elem = 2 for E2M1);
 *   OCP 8-bit Floating Point (E4M3, the no-infinity variant, max 448);
 *   Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 *   (SC'11) for Philox4x32-10.
 *
 * Pipeline order, per block, as the pages state it ([Stack], section "The first
 * change: PyTorch is bringing FP4 packing into compiler fusion"): block amax ->
 * scale calculation -> divide by the scale -> convert to E2M1 -> pack two values
 * per byte.  The oracle runs those steps one after another, per block, with no
 * fusion or reordering.
 *
 * Parity status: every exported function is pinned by the CPU tests (closed
 * forms, exhaustive enumeration, a second formulation, brute force, or rocRAND
 * for Philox).  None is "parity unpinned".
 */
#include <assert.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of a binary32; widening is exact. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* E2M1 magnitudes by 3-bit code: 1 sign, 2 exponent, 1 mantissa bit, largest
 * value 6, no infinity or NaN ([OnGPUs], section "How Does 4-Bit Floating Point
 * Work in Practice?"; [Stack], section "NVFP4 is more than a 4-bit value"). */
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oc_e2m1_value(uint8_t code)
{
    double m = kE2M1Mag[code & 7];
    return (code & 8) ? -m : m;
}

/* index of the largest magnitude not above m (m finite, 0 <= m < 6) */
static int e2m1_floor_index(double m)
{
    int k0 = 0;
    for (int i = 0; i < 8; ++i)
        if (kE2M1Mag[i] <= m) k0 = i;
    return k0;
}

/* E2M1 round-to-nearest, ties to the even code; |y| >= 6 saturates to 6; the
 * sign bit is kept (so -0.0 and small negatives encode as 0x8).  Nearest is
 * decided by an exact fp64 comparison of 2|y| with lo+hi. */
uint8_t oc_e2m1_rne(float y)
{
    assert(isfinite(y));
    int s = signbit(y) ? 1 : 0;
    double m = fabs((double)y);
    int k;
    if (m >= 6.0) {
        k = 7;
    } else {
        int k0 = e2m1_floor_index(m);
        double lo = kE2M1Mag[k0], hi = kE2M1Mag[k0 + 1];
        double twice = 2.0 * m, mid = lo + hi;
        if (twice > mid) k = k0 + 1;
        else if (twice < mid) k = k0;
        else k = (k0 % 2 == 0) ? k0 : k0 + 1;
    }
    return (uint8_t)((s << 3) | k);
}

/* E2M1 stochastic rounding ([Fusion], section "Two Key Numerical Techniques":
 * round up or down with probability proportional to the distance).  With
 * lo <= |y| < hi the two neighbours and f = (|y| - lo)/(hi - lo) the fractional
 * distance, round up iff r16 < f * 65536, r16 uniform on [0, 65535].  Both the
 * subtraction and the division are exact in fp64 (and in fp32). */
uint8_t oc_e2m1_sr(float y, uint32_t r16)
{
    assert(isfinite(y));
    assert(r16 < 65536u);
    int s = signbit(y) ? 1 : 0;
    double m = fabs((double)y);
    int k;
    if (m >= 6.0) {
        k = 7;
    } else {
        int k0 = e2m1_floor_index(m);
        double lo = kE2M1Mag[k0], hi = kE2M1Mag[k0 + 1];
        double f = (m - lo) / (hi - lo);
        k = ((double)r16 < f * 65536.0) ? k0 + 1 : k0;
    }
    return (uint8_t)((s << 3) | k);
}

/* OCP FP8 E4M3 (no infinities; 0x7F is NaN): bias 7, 3 mantissa bits,
 * largest finite 0x7E = 448, smallest subnormal 0x01 = 2^-9. */
double oc_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 0xF, m = code & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -v : v;
}

/* E4M3 round-to-nearest-even with saturation to the largest finite value,
 * for z >= 0: anything at or above 448 saturates to 0x7E; below that, a
 * brute-force search over the 127 non-negative finite codes with exact fp64
 * distances (all operands are below 2^10, so the differences are exact), ties
 * to the code with even last bit. */
uint8_t oc_e4m3_rne_satfinite(float z)
{
    assert(isfinite(z) && z >= 0.0f);
    double zd = (double)z;
    if (zd >= 448.0) return 0x7E;
    int best = 0;
    double bestd = fabs(oc_e4m3_value(0) - zd);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(oc_e4m3_value((uint8_t)c) - zd);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11) and the stochastic-rounding    */
/* bit stream                                                          */
/* ------------------------------------------------------------------ */

void oc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16 random bits for element (row, col) of the logical [R x K] operand being
 * quantized: one Philox call covers 8 consecutive K positions.
 *   counter = {col / 8, row, stream, 0}, key = {seed low word, seed high word}
 *   word    = out[(col / 2) mod 4];  bits = odd col ? word >> 16 : word & 0xffff
 * The bits depend only on logical coordinates, never on how work is split. */
uint32_t oc_r16(uint64_t seed, uint32_t stream, uint32_t row, uint32_t col)
{
    uint32_t ctr[4] = {col >> 3, row, stream, 0u};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oc_philox4x32_10(ctr, key, w);
    uint32_t word = w[(col >> 1) & 3];
    return (col & 1) ? (word >> 16) : (word & 0xffffu);
}

/* ------------------------------------------------------------------ */
/* MXFP4: 32-element blocks, E8M0 scale                                */
/* ------------------------------------------------------------------ */

/* OCP MX shared exponent for E2M1 elements: floor(log2(amax)) - 2, clamped to
 * the E8M0 range [-127, 127]; an all-zero block takes the smallest scale, in
 * line with "epsilon of the scale dtype <= scale" ([Stack], section "The third
 * change: oneDNN is defining a safe numerical range for FP4 scales").
 * floor(log2) is taken exactly with frexp (valid for subnormals too). */
int oc_mx_shared_exponent(float amax)
{
    assert(isfinite(amax) && amax >= 0.0f);
    if (amax == 0.0f) return -127;
    int e2;
    (void)frexp((double)amax, &e2); /* amax = f * 2^e2, f in [0.5, 1) */
    int e = (e2 - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Quantize one 32-element block v[] (fp32 values, element i at K index 32j+i
 * of logical row r).  Writes 16 code bytes (element 2t in the low nibble,
 * 2t+1 in the high nibble: [Stack] pairs even and odd elements in one byte)
 * and returns the E8M0 scale byte. */
static uint8_t mx_block(const float v[32], int sr, uint64_t seed, uint32_t stream,
                        uint32_t r, uint32_t kbase, uint8_t codes_out[16])
{
    /* 1. block amax */
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        assert(isfinite(v[i]));
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    /* 2. scale */
    int E = oc_mx_shared_exponent(amax);
    float inv_scale = ldexpf(1.0f, -E); /* 2^-E, a normal binary32 for E in [-127, 125] */
    /* 3.-4. divide by the scale (an exact power of two) and convert */
    uint8_t c[32];
    for (int i = 0; i < 32; ++i) {
        float y = v[i] * inv_scale;
        c[i] = sr ? oc_e2m1_sr(y, oc_r16(seed, stream, r, kbase + (uint32_t)i))
                  : oc_e2m1_rne(y);
    }
    /* 5. pack */
    for (int t = 0; t < 16; ++t)
        codes_out[t] = (uint8_t)(c[2 * t] | (c[2 * t + 1] << 4));
    return (uint8_t)(E + 127);
}

/* Fetch logical element (r, k) of the operand from the bf16 source.
 * axis 0: operand = x (R = rows, K = cols); axis 1: operand = x^T
 * (R = cols, K = rows), i.e. the block runs down a column of x. */
static float fetch(const uint16_t *x, int64_t ld, int axis, int64_t r, int64_t k)
{
    return axis == 0 ? bf16_bits_to_float(x[r * ld + k]) : bf16_bits_to_float(x[k * ld + r]);
}

/* Fixed-sign 32-point Hadamard ([Fusion], section "Two Key Numerical
 * Techniques": a 32x32 Hadamard matrix with fixed signs, an orthogonal
 * transform).  v <- H32 * diag(d) * v with d_i = -1 where bit i of sign_mask
 * is set, H32 the unnormalised Sylvester matrix (entries (-1)^popcount(i&k)),
 * evaluated as five butterfly stages of span 1, 2, 4, 8, 16, each stage
 * replacing (a, b) by (a + b, a - b) in binary32. */
void oc_hadamard32(float v[32], uint32_t sign_mask)
{
    for (int i = 0; i < 32; ++i)
        if ((sign_mask >> i) & 1u) v[i] = -v[i];
    for (int h = 1; h < 32; h <<= 1) {
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
}

/* Shared driver for fp4_quantize_mx and fp4_hadamard32_quantize.
 * Outputs (linear layout): codes [R][K/2] bytes, scales [R][K/32] bytes. */
static int quantize_mx_impl(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                            int axis, int hadamard, uint32_t sign_mask, int sr,
                            uint64_t seed, uint32_t stream, uint8_t *codes, uint8_t *scales)
{
    int64_t R = axis == 0 ? rows : cols;
    int64_t K = axis == 0 ? cols : rows;
    if (K % 32 != 0) return 2;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t j = 0; j < K / 32; ++j) {
            float v[32];
            for (int i = 0; i < 32; ++i) v[i] = fetch(x, ld, axis, r, 32 * j + i);
            if (hadamard) oc_hadamard32(v, sign_mask);
            for (int i = 0; i < 32; ++i)
                if (!isfinite(v[i])) return 1; /* non-finite values are outside the contract */
            scales[r * (K / 32) + j] =
                mx_block(v, sr, seed, stream, (uint32_t)r, (uint32_t)(32 * j), codes + r * (K / 2) + 16 * j);
        }
    }
    return 0;
}

int oc_quantize_mx(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis, int sr,
                   uint64_t seed, uint32_t stream, uint8_t *codes, uint8_t *scales)
{
    return quantize_mx_impl(x, rows, cols, ld, axis, 0, 0u, sr, seed, stream, codes, scales);
}

int oc_hadamard32_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                           uint32_t sign_mask, int sr, uint64_t seed, uint32_t stream,
                           uint8_t *codes, uint8_t *scales)
{
    return quantize_mx_impl(x, rows, cols, ld, axis, 1, sign_mask, sr, seed, stream, codes, scales);
}

/* ------------------------------------------------------------------ */
/* NVFP4: 16-element blocks, E4M3 block scale, FP32 tensor scale       */
/* ([Stack], section "NVFP4 is more than a 4-bit value"; the three      */
/* scale domains of [Fusion], section "The Design Philosophy of         */
/* Format-Aware Fusion": global nvfp and CTA-local nvfp)                */
/* ------------------------------------------------------------------ */

/* FP32 tensor-level decode scale of a domain with amax A: the domain's largest
 * block then maps onto E4M3 448 times E2M1 6 = 2688.  A zero domain gets 1. */
float oc_nv_tensor_scale(float A)
{
    assert(isfinite(A) && A >= 0.0f);
    if (A == 0.0f) return 1.0f;
    float S = A / 2688.0f;
    return S;
}

/* E4M3 block scale for block amax b in a domain with tensor scale S,
 * clamped into [smallest positive E4M3, largest E4M3] ([Stack], section "The
 * third change": epsilon of the scale dtype <= scale <= max of the scale
 * dtype).  Two binary32 divisions, in this order. */
uint8_t oc_nv_block_scale(float b, float S)
{
    float sbf = (b / 6.0f) / S;
    uint8_t sb = oc_e4m3_rne_satfinite(sbf);
    if (sb == 0) sb = 1;
    return sb;
}

/* Quantize one 16-element block with block scale byte sb and tensor scale S:
 * decode scale d = e4m3(sb) * S, one reciprocal, one multiply per element. */
static void nv_block(const float v[16], uint8_t sb, float S, int sr, uint64_t seed, uint32_t stream,
                     uint32_t r, uint32_t kbase, uint8_t codes_out[8])
{
    float d = (float)oc_e4m3_value(sb) * S;
    float inv = 1.0f / d;
    uint8_t c[16];
    for (int i = 0; i < 16; ++i) {
        float y = v[i] * inv;
        c[i] = sr ? oc_e2m1_sr(y, oc_r16(seed, stream, r, kbase + (uint32_t)i)) : oc_e2m1_rne(y);
    }
    for (int t = 0; t < 8; ++t)
        codes_out[t] = (uint8_t)(c[2 * t] | (c[2 * t + 1] << 4));
}

/* Shared driver for oc_quantize_nv and oc_hadamard32_quantize_nv.
 * domain: 0 = one tensor scale for the whole operand ("global nvfp");
 *         1 = one tensor scale per 128 x 128 tile of the logical [R x K]
 *             operand ("CTA-local nvfp"); edge tiles are their own domains.
 * tensor_scale receives 1 float (global) or ceil(R/128) x ceil(K/128) floats
 * (row-major).  The logical operand is first materialized in binary32 (the
 * bf16 values widened, exactly; with hadamard set, each 32-element block
 * along K then transformed by oc_hadamard32), so that the domain amax, the
 * block amax and the codes all see the same values. */
static int quantize_nv_impl(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis, int hadamard,
                            uint32_t sign_mask, int sr, uint64_t seed, uint32_t stream, int domain,
                            uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    int64_t R = axis == 0 ? rows : cols;
    int64_t K = axis == 0 ? cols : rows;
    if (K % (hadamard ? 32 : 16) != 0) return 2;
    float *v = (float *)malloc((size_t)(R * K > 0 ? R * K : 1) * sizeof(float));
    if (!v) return 3;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t k = 0; k < K; ++k) v[r * K + k] = fetch(x, ld, axis, r, k);
        if (hadamard)
            for (int64_t j = 0; j < K / 32; ++j) oc_hadamard32(v + r * K + 32 * j, sign_mask);
    }
    for (int64_t i = 0; i < R * K; ++i)
        if (!isfinite(v[i])) { free(v); return 1; }
    int64_t TR = (R + 127) / 128, TK = (K + 127) / 128;
    /* domain amax, then the domain's tensor scale */
    if (domain == 0) {
        float A = 0.0f;
        for (int64_t i = 0; i < R * K; ++i) {
            float a = fabsf(v[i]);
            if (a > A) A = a;
        }
        if (A != 0.0f && A < 0x1p-100f) { free(v); return 1; } /* degenerate domain, outside the contract */
        tensor_scale[0] = oc_nv_tensor_scale(A);
    } else {
        for (int64_t tr = 0; tr < TR; ++tr)
            for (int64_t tk = 0; tk < TK; ++tk) {
                float A = 0.0f;
                for (int64_t r = 128 * tr; r < R && r < 128 * tr + 128; ++r)
                    for (int64_t k = 128 * tk; k < K && k < 128 * tk + 128; ++k) {
                        float a = fabsf(v[r * K + k]);
                        if (a > A) A = a;
                    }
                if (A != 0.0f && A < 0x1p-100f) { free(v); return 1; }
                tensor_scale[tr * TK + tk] = oc_nv_tensor_scale(A);
            }
    }
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t j = 0; j < K / 16; ++j) {
            float S = domain == 0 ? tensor_scale[0] : tensor_scale[(r / 128) * TK + (16 * j) / 128];
            const float *blk = v + r * K + 16 * j;
            float b = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(blk[i]);
                if (a > b) b = a;
            }
            uint8_t sb = oc_nv_block_scale(b, S);
            scales[r * (K / 16) + j] = sb;
            nv_block(blk, sb, S, sr, seed, stream, (uint32_t)r, (uint32_t)(16 * j), codes + r * (K / 2) + 8 * j);
        }
    }
    free(v);
    return 0;
}

int oc_quantize_nv(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis, int sr,
                   uint64_t seed, uint32_t stream, int domain, uint8_t *codes, uint8_t *scales,
                   float *tensor_scale)
{
    return quantize_nv_impl(x, rows, cols, ld, axis, 0, 0u, sr, seed, stream, domain, codes, scales, tensor_scale);
}

/* The fixed-sign Hadamard-32 ([Fusion], section "Two Key Numerical
 * Techniques") ahead of NVFP4: the transform runs along K in 32-element
 * blocks (two NV blocks each), as on the MX path, and the NV steps then apply
 * to the transformed values (K % 32 == 0). */
int oc_hadamard32_quantize_nv(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                              uint32_t sign_mask, int sr, uint64_t seed, uint32_t stream, int domain,
                              uint8_t *codes, uint8_t *scales, float *tensor_scale)
{
    return quantize_nv_impl(x, rows, cols, ld, axis, 1, sign_mask, sr, seed, stream, domain, codes, scales,
                            tensor_scale);
}

/* ------------------------------------------------------------------ */
/* dequantization and the brute-force GEMM reference                   */
/* ------------------------------------------------------------------ */

/* element k of row r of a packed operand (low nibble = even k) */
static uint8_t code_at(const uint8_t *codes, int64_t K, int64_t r, int64_t k)
{
    uint8_t byte = codes[r * (K / 2) + k / 2];
    return (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
}

/* MX: value = e2m1(code) * 2^(scale_byte - 127) */
void oc_dequant_mx(const uint8_t *codes, const uint8_t *scales, int64_t R, int64_t K, double *out)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) {
            int e = (int)scales[r * (K / 32) + k / 32] - 127;
            out[r * K + k] = ldexp(oc_e2m1_value(code_at(codes, K, r, k)), e);
        }
}

/* NV: value = e2m1(code) * e4m3(block scale) * S(domain of (r, k)) */
void oc_dequant_nv(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale, int domain,
                   int64_t R, int64_t K, double *out)
{
    int64_t TK = (K + 127) / 128;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) {
            double S = domain == 0 ? (double)tensor_scale[0] : (double)tensor_scale[(r / 128) * TK + k / 128];
            out[r * K + k] = oc_e2m1_value(code_at(codes, K, r, k)) * oc_e4m3_value(scales[r * (K / 16) + k / 16]) * S;
        }
}

/* C[m][n] = alpha * sum_k A[m][k] * B[n][k] and the error-bound weight
 * W[m][n] = |alpha| * sum_k |A[m][k] * B[n][k]|, by a plain triple loop in
 * fp64 (A, B are dequantized operands). */
void oc_gemm_bruteforce(const double *A, const double *B, int64_t M, int64_t N, int64_t K, double alpha,
                        double *C, double *W)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, w = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = A[m * K + k] * B[n * K + k];
                s += p;
                w += fabs(p);
            }
            C[m * N + n] = alpha * s;
            W[m * N + n] = fabs(alpha) * w;
        }
}

/* ------------------------------------------------------------------ */
/* SwiGLU: the MLP activation whose output H the fused producer        */
/* quantizes ([Fusion], section "The Design Philosophy of Format-Aware */
/* Fusion": the producer is fused with the operation that creates its  */
/* input).  Outside definition: SwiGLU(g, u) = SiLU(g) * u with        */
/* SiLU(x) = x / (1 + e^-x) (Shazeer, "GLU Variants Improve            */
/* Transformer", 2020).  H is that real number rounded once to bf16.   */
/* ------------------------------------------------------------------ */

/* float -> bf16 bits, round to nearest even (NaN -> a quiet NaN). */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint16_t oc_float_to_bf16(float f) { return float_to_bf16_rne(f); }

/* The bf16 spacing (as a power-of-two exponent) at a finite a > 0: bf16 has
 * 8 significant bits, so in [2^(e-1), 2^e) the step is 2^(e-8); below 2^-126
 * (subnormals) it is 2^-133. */
static int bf16_step_exp(double a)
{
    int e;
    frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1 */
    return e - 8 < -133 ? -133 : e - 8;
}

/* binary64 -> bf16 bits, rounded ONCE to nearest, ties to even (no binary32
 * step in between); magnitudes at or above 2^128 (1 - 2^-9), the midpoint
 * between the largest finite bf16 and 2^128, become infinities. */
uint16_t oc_double_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    const uint16_t s = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a == 0.0) return s;
    if (isinf(a)) return s | 0x7F80;
    const int q = bf16_step_exp(a);
    const double r = ldexp(rint(ldexp(a, -q)), q); /* exact scalings; rint: half to even */
    if (r >= 0x1p128) return s | 0x7F80;
    const float f = (float)r; /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(s | (u >> 16));
}

/* SiLU(g) * u evaluated in binary64: the product g u of two bf16 values is
 * exact, then one division by 1 + e^-g (libm exp).  Relative error a few
 * binary64 ulps (below 2^-50), far finer than the bf16 step (2^-8). */
double oc_swiglu_f64(float g, float u)
{
    const double p = (double)g * (double)u;
    return p / (1.0 + exp(-(double)g));
}

/* H[m][j] = bf16(SiLU(g) * u), g and u the bf16 gate and up values of
 * hidden column j read from the GEMM output C (row pitch ldc elements):
 * C's columns interleave gate and up in groups of `pair` columns -- gate
 * columns j of group b = j / pair sit at 2 pair b + (j mod pair), the up
 * columns `pair` further -- so pair = 32 is the layout whose 32-column gate
 * and up blocks share an accumulator lane, and pair = F is [gate | up].
 * Each element is oc_swiglu_f64 rounded once to bf16 (nearest, ties to
 * even).  This is the rounding of the real value SiLU(g) u except where
 * that value lies within the binary64 error (2^-50 relative) of a bf16
 * midpoint -- for example an exact tie g u when e^-g falls below the
 * binary64 resolution, whose real value lies just inside the midpoint.
 * If hv is not null it also receives the binary64 value of each element,
 * for tests that bound a kernel's deviation.  Returns 0, or -1 if pair does
 * not divide F. */
int oc_swiglu_bf16(const uint16_t *c, int64_t M, int64_t F, int64_t ldc, int64_t pair, uint16_t *h, double *hv)
{
    if (pair <= 0 || F % pair != 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < F; ++j) {
            const int64_t gcol = (j / pair) * 2 * pair + (j % pair);
            const float g = bf16_bits_to_float(c[m * ldc + gcol]);
            const float u = bf16_bits_to_float(c[m * ldc + gcol + pair]);
            const double v = oc_swiglu_f64(g, u);
            h[m * F + j] = oc_double_to_bf16(v);
            if (hv) hv[m * F + j] = v;
        }
    return 0;
}

/* bf16 bits of an array of binary64 values, each rounded once (the bf16
 * output of an exact GEMM result). */
void oc_double_to_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oc_double_to_bf16(v[i]);
}
