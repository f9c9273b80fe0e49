// gemm_nv.hip -- NVFP4 GEMM: exact dequantization to bf16 in LDS, bf16
// matrix cores, FP32 tensor scales on the fp32 partial sums.
//
// Pages cited (titles as printed):
//   [Stack]  "FP4 Is No Longer Just a Hardware Feature -- The NVFP4 Software
//            Stack Is Taking Shape", section "NVFP4 is more than a 4-bit
//            value": value = E2M1 payload x E4M3 block scale (16 elements) x
//            FP32 tensor-level scale.
//   [Fusion] "Format-Aware Fusion: The Engineering Practice That Doubles FP4
//            Pretraining Throughput", section "The Design Philosophy of
//            Format-Aware Fusion": global nvfp and CTA-local nvfp domains.
//
// gfx950's scaled matrix-core instruction takes one power-of-two (E8M0)
// scale per 32 elements, which cannot carry an E4M3 scale per 16.  An E2M1
// value has at most 2 significant bits and an E4M3 value at most 4, so their
// product has at most 6 and is exact in bf16 (8 significant bits, the binary32
// exponent range).  The kernel therefore dequantizes each K slice of A and B
// into bf16 in LDS and multiplies on v_mfma_f32_32x32x16_bf16: every product
// is exact and only the fp32 accumulation rounds.  The tensor scales are
// applied to fp32 sums: once in the epilogue for the global domain, and per
// 128-wide K slice for the per-tile domain (a slice is one tile column of both
// operands, and a 128-row block of A or B lies in one tile row, so one factor
// S_A(tm, kt) * S_B(tn, kt) covers a workgroup's whole slice).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

namespace {

typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRowBytes = kBK * 2 + 16;                 // 64 bf16 + 16 pad
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;    // 36 KiB
constexpr int kLdsBytes = 2 * kStageBytes;

// E2M1 code (4 bits) -> binary32 bits: exponent field e = (c >> 1) & 3, mantissa
// bit c & 1; e = 0 is the subnormal 0 / 0.5.
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c)
{
    const uint32_t e = (c >> 1) & 3u, m = c & 1u, s = (c & 8u) << 28;
    const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
    return s | mag;
}

// Dequantize 32 codes (16 bytes, two 16-element NV blocks with scale values
// s0, s1) into 32 bf16 and store them as 64 bytes at dst.  Each product is
// exact, so truncating the binary32 to its upper half is the exact bf16.
__device__ __forceinline__ void dequant32(const uint4 &q, float s0, float s1, uint8_t *dst)
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float sc = d < 2 ? s0 : s1;
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float lo = u2f(e2m1_bits((w[d] >> (8 * p)) & 0xFu)) * sc;
            const float hi = u2f(e2m1_bits((w[d] >> (8 * p + 4)) & 0xFu)) * sc;
            o[p] = (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
        }
        *reinterpret_cast<uint4 *>(dst + 16 * d) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

template <bool kTile>
__global__ __launch_bounds__(256) void gemm_nv_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                      const float *__restrict__ Ats, const uint8_t *__restrict__ B,
                                                      const uint8_t *__restrict__ Bs, const float *__restrict__ Bts,
                                                      int M, int N, int K, float alpha, void *__restrict__ C,
                                                      int64_t ldc, int c_bf16, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const uint32_t KB = (uint32_t)K >> 1, KS = (uint32_t)K >> 4;
    const int nk = K / kBK;
    const int TK = (K + 127) >> 7;

    // dequant assignment: thread t handles 32 K-elements (half t & 1) of row
    // t >> 1 of both operands
    const int drow = tid >> 1, dh = tid & 1;
    const int ra = min(m0 + drow, M - 1), rb = min(n0 + drow, N - 1);
    const uint8_t *a_src = A + (size_t)ra * KB + dh * 16;
    const uint8_t *b_src = B + (size_t)rb * KB + dh * 16;
    const uint8_t *as_src = As + (size_t)ra * KS + dh * 2;
    const uint8_t *bs_src = Bs + (size_t)rb * KS + dh * 2;
    const int st_off = drow * kRowBytes + dh * 64;

    const int fr = lane & 31, fh = lane >> 5;
    const int fa_off = (wm * 64 + fr) * kRowBytes + fh * 16;
    const int fb_off = kBM * kRowBytes + (wn * 64 + fr) * kRowBytes + fh * 16;

    v16f_t acc[2][2], part[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = (v16f_t){};
            part[i][j] = (v16f_t){};
        }

    auto load_stage = [&](int ks, uint4 &qa, uint4 &qb, uint32_t &sa, uint32_t &sb) {
        qa = *reinterpret_cast<const uint4 *>(a_src + ks * (kBK / 2));
        qb = *reinterpret_cast<const uint4 *>(b_src + ks * (kBK / 2));
        sa = *reinterpret_cast<const uint16_t *>(as_src + ks * (kBK / 16));
        sb = *reinterpret_cast<const uint16_t *>(bs_src + ks * (kBK / 16));
    };
    auto store_stage = [&](int buf, const uint4 &qa, const uint4 &qb, uint32_t sa, uint32_t sb) {
        uint8_t *base = lds + buf * kStageBytes;
        dequant32(qa, e4m3_value(sa & 0xFFu), e4m3_value(sa >> 8), base + st_off);
        dequant32(qb, e4m3_value(sb & 0xFFu), e4m3_value(sb >> 8), base + kBM * kRowBytes + st_off);
    };

    uint4 qa, qb;
    uint32_t sa, sb;
    load_stage(0, qa, qb, sa, sb);
    store_stage(0, qa, qb, sa, sb);
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        load_stage(min(ks + 1, nk - 1), qa, qb, sa, sb);
        const uint8_t *base = lds + buf * kStageBytes;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            v8s_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 ta = *reinterpret_cast<const uint4 *>(base + fa_off + i * 32 * kRowBytes + kk * 32);
                const uint4 tb = *reinterpret_cast<const uint4 *>(base + fb_off + i * 32 * kRowBytes + kk * 32);
                af[i] = __builtin_bit_cast(v8s_t, ta);
                bfr[i] = __builtin_bit_cast(v8s_t, tb);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (kTile)
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], part[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                }
        }
        if (kTile && ((ks * kBK + kBK) % 128 == 0 || ks == nk - 1)) {
            // end of a 128-wide K slice: fold its partial sum with the slice's scales
            const int kt = (ks * kBK) >> 7;
            const float s = Ats[tm * TK + kt] * Bts[tn * TK + kt];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += s * part[i][j][r];
                    part[i][j] = (v16f_t){};
                }
        }
        store_stage(buf ^ 1, qa, qb, sa, sb);
        __syncthreads();
    }

    const float scale = kTile ? alpha : alpha * (Ats[0] * Bts[0]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + fr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
                if (row < M && col < N) {
                    const float v = scale * acc[i][j][r];
                    if (c_bf16)
                        reinterpret_cast<uint16_t *>(C)[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16_rne(v);
                    else
                        reinterpret_cast<float *>(C)[(int64_t)row * ldc + col] = v;
                }
            }
        }
}

__global__ void nv_fill_zero_kernel(void *__restrict__ C, int M, int N, int64_t ldc, int c_bf16)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int64_t r = i / N, c = i - r * N;
    if (c_bf16)
        reinterpret_cast<uint16_t *>(C)[r * ldc + c] = 0;
    else
        reinterpret_cast<float *>(C)[r * ldc + c] = 0.0f;
}

}  // namespace

int launch_gemm_nv(const GemmArgs &g, hipStream_t st)
{
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    if (M == 0 || N == 0) return 0;
    if (K == 0) {
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(nv_fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g.c, M, N,
                           g.ldc, (int)g.c_bf16);
        return hipGetLastError() == hipSuccess ? 0 : 1;
    }
    const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    auto *a = reinterpret_cast<const uint8_t *>(g.a_codes);
    auto *as = reinterpret_cast<const uint8_t *>(g.a_scales);
    auto *b = reinterpret_cast<const uint8_t *>(g.b_codes);
    auto *bs = reinterpret_cast<const uint8_t *>(g.b_scales);
    if (g.nv_domain == 1)
        hipLaunchKernelGGL(gemm_nv_kernel<true>, dim3(tiles_m * tiles_n), dim3(256), 0, st, a, as, g.a_ts, b, bs,
                           g.b_ts, M, N, K, g.alpha, g.c, g.ldc, (int)g.c_bf16, tiles_n);
    else
        hipLaunchKernelGGL(gemm_nv_kernel<false>, dim3(tiles_m * tiles_n), dim3(256), 0, st, a, as, g.a_ts, b, bs,
                           g.b_ts, M, N, K, g.alpha, g.c, g.ldc, (int)g.c_bf16, tiles_n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
