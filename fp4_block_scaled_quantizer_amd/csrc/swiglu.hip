// swiglu.hip -- SwiGLU of a bf16 gate/up GEMM output, the activation whose
// output H the MX producer (or the fused GEMM epilogue) quantizes.
//
// Page cited: "Format-Aware Fusion: The Engineering Practice That Doubles FP4
// Pretraining Throughput", section "The Design Philosophy of Format-Aware
// Fusion" (the producer is fused with the operation that creates its input;
// this kernel is that operation on its own, the unfused reference point).
//
// h[m][j] = bf16(SiLU(g) * u), g and u the bf16 values of C at the gate and
// up columns of hidden column j: C's columns interleave gate and up in groups
// of `pair` columns (gate columns of group b at 2 pair b .. 2 pair b + pair-1,
// the up columns right after), so pair = 32 is the fused GEMM's weight layout
// and pair = F the plain [gate | up] one.  SiLU is fp4q_device.h's fixed
// binary32 sequence; the product is one binary32 multiply rounded to bf16
// (round to nearest even, v_cvt_pk_bf16_f32).
//
// HBM-bound: 4 bytes read and 2 written per hidden element.  A thread takes 8
// consecutive hidden columns of one row (one 16-byte load each of gate and up,
// one 16-byte store); a 256-thread workgroup covers 2048 columns of a row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t swiglu2(uint32_t g, uint32_t u)
{
    const float h0 = silu_f32(bf16_lo(g)) * bf16_lo(u);
    const float h1 = silu_f32(bf16_hi(g)) * bf16_hi(u);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){h0, h1}, bf16x2_t));
}

// grid.x covers F / 8 column chunks, grid.y strides over rows
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t *__restrict__ c, uint16_t *__restrict__ h,
                                                     int64_t M, int64_t F, int64_t ldc, int64_t ldh, int64_t pair)
{
    const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (j >= F) return;
    const int64_t gcol = (j / pair) * 2 * pair + (j % pair);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const uint16_t *row = c + m * ldc;
        const u32x4_t g = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(row + gcol));
        const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(row + gcol + pair));
        *reinterpret_cast<u32x4_t *>(h + m * ldh + j) =
            (u32x4_t){swiglu2(g[0], u[0]), swiglu2(g[1], u[1]), swiglu2(g[2], u[2]), swiglu2(g[3], u[3])};
    }
}

}  // namespace

int launch_swiglu(const void *c, int64_t M, int64_t F, int64_t ldc, int64_t pair, void *h, int64_t ldh,
                  hipStream_t st)
{
    if (M == 0 || F == 0) return 0;
    const int64_t chunks = F / 8;
    const unsigned gx = (unsigned)((chunks + 255) / 256);
    const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
    hipLaunchKernelGGL(swiglu_kernel, dim3(gx, gy), dim3(256), 0, st, reinterpret_cast<const uint16_t *>(c),
                       reinterpret_cast<uint16_t *>(h), M, F, ldc, ldh, pair);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
