// Test helper: the scalar building blocks of the GPU kernels
// (fp4q_device.h), compiled for the host so the CPU tests can compare them
// with the oracle over large input sets.  Test infrastructure only.
#include "fp4q_device.h"

extern "C" {
uint32_t h_e2m1_sr(float y, uint32_t r16) { return fp4q::e2m1_sr(y, r16); }
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
void h_e2m1_sr_batch(const float *y, const uint32_t *r, uint8_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)fp4q::e2m1_sr(y[i], r[i]);
}
}
