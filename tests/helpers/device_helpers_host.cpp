// Test helper: the scalar building blocks of the GPU kernels
// (fp4q_device.h), compiled for the host so the CPU tests can compare them
// with the oracle over large input sets.  Test infrastructure only.
#include "fp4q_device.h"

extern "C" {
// one value through slot `slot` (0..7) of the eight-value SR encode, the
// other slots holding zeros
uint32_t h_e2m1_sr_slot(float y, uint32_t r16, int slot)
{
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t w[4] = {0, 0, 0, 0};
    v[slot] = y;
    w[slot >> 1] = (slot & 1) ? r16 << 16 : r16;
    return (fp4q::e2m1_sr8(v, w) >> (4 * slot)) & 15u;
}
uint32_t h_e2m1_sr(float y, uint32_t r16) { return h_e2m1_sr_slot(y, r16, 0); }
uint32_t h_e4m3_rne_satfinite(float z) { return fp4q::e4m3_rne_satfinite(z); }
float h_e4m3_value(uint32_t c) { return fp4q::e4m3_value(c); }
uint32_t h_nv_block_scale(float b, float S) { return fp4q::nv_block_scale(b, S); }
float h_nv_inv_decode(uint32_t sb, float S) { return fp4q::nv_inv_decode(sb, S); }
float h_nv_tensor_scale(float A) { return fp4q::nv_tensor_scale(A); }
uint32_t h_mx_scale_byte(uint32_t amax_bits) { return fp4q::mx_scale_byte(amax_bits); }
float h_mx_inv_scale(uint32_t byte) { return fp4q::mx_inv_scale(byte); }
uint32_t h_f32_to_bf16_rne(float f) { return fp4q::f32_to_bf16_rne(f); }
void h_philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1, uint32_t *out)
{
    fp4q::philox4x32_10(c0, c1, c2, c3, k0, k1, out);
}
void h_e4m3_batch(const float *z, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)fp4q::e4m3_rne_satfinite(z[i]);
}
void h_silu_batch(const float *x, float *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = fp4q::silu_f32(x[i]);
}
// H = bf16(SiLU(g) u) as the SwiGLU kernels compute it: binary32 SiLU of the
// bf16 gate, one binary32 product, round to nearest even
void h_swiglu_batch(const uint16_t *g, const uint16_t *u, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = (uint16_t)fp4q::f32_to_bf16_rne(fp4q::silu_f32(fp4q::bf16_lo(g[i])) * fp4q::bf16_lo(u[i]));
}
// fast_div against the divisor d for n values
void h_fast_div(uint32_t d, const uint32_t *n, uint32_t *out, size_t count)
{
    const fp4q::FastDiv f = fp4q::fast_div_for(d);
    for (size_t i = 0; i < count; ++i) out[i] = fp4q::fast_div(n[i], f);
}
// chunks visited by one thread of the partial-maximum pass: count, index sum
// and the largest index (visit4 counts its four chunks)
void h_grid_stride(uint32_t start, uint32_t stride, uint32_t n, uint64_t *out)
{
    uint64_t cnt = 0, sum = 0, hi = 0;
    auto one = [&](uint32_t c) {
        ++cnt;
        sum += c;
        hi = c > hi ? c : hi;
    };
    fp4q::grid_stride_chunks(
        start, stride, n,
        [&](uint32_t c) {
            for (int i = 0; i < 4; ++i) one(c + (uint32_t)i * stride);
        },
        one);
    out[0] = cnt;
    out[1] = sum;
    out[2] = hi;
}
void h_e2m1_sr_batch(const float *y, const uint32_t *r, uint8_t *out, size_t n)
{
    // consecutive values share one eight-value encode: value i sits in slot i % 8
    for (size_t i = 0; i < n; i += 8) {
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t w[4] = {0, 0, 0, 0};
        for (size_t j = 0; j < 8 && i + j < n; ++j) {
            v[j] = y[i + j];
            w[j >> 1] |= (j & 1) ? r[i + j] << 16 : r[i + j];
        }
        const uint32_t p = fp4q::e2m1_sr8(v, w);
        for (size_t j = 0; j < 8 && i + j < n; ++j) out[i + j] = (uint8_t)((p >> (4 * j)) & 15u);
    }
}

// NV block scales for every bf16 domain amax A (step `astep` through the
// positive finite patterns) and every bf16 block amax b <= A: counts the
// pairs where the correction-step form differs from the two divisions in
// the code byte, and (where the block scale is at least 2^-10) in the
// binary32 block scale itself; also checks the decode table entries.
void h_nv_fast_sweep(uint32_t astep, uint64_t *out)
{
    uint64_t pairs = 0, code_diff = 0, value_diff = 0, fast_domains = 0;
    for (uint32_t a = 1; a < 0x7F80u; a += astep) {
        const float A = fp4q::u2f(a << 16);
        const float S = fp4q::nv_tensor_scale(A);
        const fp4q::NvDomain t = fp4q::nv_domain(S);
        fast_domains += t.fast ? 1 : 0;
        for (uint32_t b = 0; b <= a; ++b) {
            const float B = fp4q::u2f(b << 16);
            ++pairs;
            if (fp4q::nv_block_scale_fast(B, t) != fp4q::nv_block_scale(B, S)) ++code_diff;
            if (t.fast) {
                const float exact = (B / 6.0f) / S;
                const float fast = fp4q::div_by_recip(fp4q::div_by_recip(B, 6.0f, 0x1.555556p-3f), t.S, t.rS);
                if (exact >= 0x1p-10f && fp4q::f2u(exact) != fp4q::f2u(fast)) ++value_diff;
            }
        }
    }
    out[0] = pairs;
    out[1] = code_diff;
    out[2] = value_diff;
    out[3] = fast_domains;
}
}
