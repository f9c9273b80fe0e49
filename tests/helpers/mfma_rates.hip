// Test helper: issue rates of the gfx950 matrix-core instructions an NVFP4
// GEMM could run on, measured on the GPU itself.  Test infrastructure only
// (not part of libfp4q).
//
// NVFP4 = E2M1 payload x E4M3 scale per 16 elements x FP32 tensor scale
// ("FP4 Is No Longer Just a Hardware Feature -- The NVFP4 Software Stack Is
// Taking Shape", section "NVFP4 is more than a 4-bit value").  libfp4q's NV
// GEMM dequantizes E2M1 x E4M3 exactly to fp16 and runs the 32x32x16 fp16
// instruction.  The alternative on 8-bit matrix cores needs each operand in
// two E4M3 parts (the dequantized value has up to 6 significant bits, E4M3
// holds 4), i.e. four fp8 products per fp16 one, so it pays only if the fp8
// instruction covers more than four times the K of the fp16 one per cycle.
// This measures exactly that ratio.
//
// Kernel: every wave runs `iters` rounds of 8 MFMAs of one kind into 8
// independent accumulators (no dependency between consecutive instructions)
// and lane 0 records the s_memtime cycles of the loop.  Grid: `blocks`
// workgroups of 256 threads; cycles has blocks * 4 entries, sink blocks * 256
// floats (the accumulators' sum, so nothing is optimized away).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

enum { kF16 = 0, kBF16 = 1, kFP8 = 2, kFP4 = 3, kFP4Data = 4 };

template <int kKind>
__device__ __forceinline__ v16f_t one(const v8i_t &a, const v8i_t &b, const v16f_t &c)
{
    if constexpr (kKind == kF16) {
        const half8_t x = __builtin_bit_cast(half8_t, (int4){a[0], a[1], a[2], a[3]});
        const half8_t y = __builtin_bit_cast(half8_t, (int4){b[0], b[1], b[2], b[3]});
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
    } else if constexpr (kKind == kBF16) {
        const bf16x8_t x = __builtin_bit_cast(bf16x8_t, (int4){a[0], a[1], a[2], a[3]});
        const bf16x8_t y = __builtin_bit_cast(bf16x8_t, (int4){b[0], b[1], b[2], b[3]});
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    } else if constexpr (kKind == kFP8) {  // E4M3 operands, unit (127) block scales
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    } else {                               // E2M1 operands, unit block scales
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, 127, 0, 127);
    }
}

template <int kKind>
__global__ __launch_bounds__(256) void rate_kernel(int iters, unsigned long long *cycles, float *sink)
{
    const int tid = threadIdx.x;
    v8i_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 ^ (tid * 0x01010101 + i);  // small finite codes in every format
        b[i] = 0x30303030 ^ (tid * 0x00010001 + 3 * i);
    }
    // kFP4Data: four random operand pairs per lane (xorshift32), rotated
    // every instruction, so that the matrix core sees changing data as in a
    // GEMM (every 4-bit pattern is an E2M1 value)
    v8i_t av[4], bv[4];
    uint32_t x = 0x9E3779B9u * (uint32_t)(blockIdx.x * 256 + tid + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x ^= x << 13; x ^= x >> 17; x ^= x << 5;
            av[j][i] = (int)x;
            x ^= x << 13; x ^= x >> 17; x ^= x << 5;
            bv[j][i] = (int)x;
        }
    v16f_t acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (v16f_t){};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (kKind == kFP4Data)
                acc[k] = one<kFP4>(av[k & 3], bv[(k + 1) & 3], acc[k]);
            else
                acc[k] = one<kKind>(a, b, acc[k]);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[k][r];
    sink[blockIdx.x * 256 + tid] = s;
    if ((tid & 63) == 0) cycles[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

// Launches the kernel of `kind` (0 fp16, 1 bf16, 2 fp8, 3 fp4, 4 fp4 on
// changing random operands) on `stream`;
// 0 on success, 1 for an unknown kind or a launch error.
extern "C" int mfma_rate_launch(int kind, int blocks, int iters, unsigned long long *cycles, float *sink,
                                void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (kind) {
    case kF16: hipLaunchKernelGGL(rate_kernel<kF16>, dim3(blocks), dim3(256), 0, st, iters, cycles, sink); break;
    case kBF16: hipLaunchKernelGGL(rate_kernel<kBF16>, dim3(blocks), dim3(256), 0, st, iters, cycles, sink); break;
    case kFP8: hipLaunchKernelGGL(rate_kernel<kFP8>, dim3(blocks), dim3(256), 0, st, iters, cycles, sink); break;
    case kFP4: hipLaunchKernelGGL(rate_kernel<kFP4>, dim3(blocks), dim3(256), 0, st, iters, cycles, sink); break;
    case kFP4Data:
        hipLaunchKernelGGL(rate_kernel<kFP4Data>, dim3(blocks), dim3(256), 0, st, iters, cycles, sink);
        break;
    default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
