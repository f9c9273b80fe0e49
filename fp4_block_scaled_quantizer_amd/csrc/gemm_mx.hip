// gemm_mx.hip -- block-scaled MXFP4 GEMM on gfx950's scaled FP4 matrix cores.
//
// Page cited: "Format-Aware Fusion: The Engineering Practice That Doubles FP4
// Pretraining Throughput", sections "Why FP4 Speedups Often Remain
// Theoretical" (the FP4 matrix multiply the producers feed) and "The Design
// Philosophy of Format-Aware Fusion" (the consumer layout is bound to the
// producer: the GEMM reads the codes and E8M0 scales exactly as the MX
// producers store them).
//
// C[M x N] = alpha * sum_k e2m1(a[m][k]) 2^(sa[m][k/32]-127) e2m1(b[n][k]) 2^(sb[n][k/32]-127)
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1 does a
// 32 x 32 x 64 block per instruction and applies one E8M0 scale per lane:
// lane l supplies row (l mod 32), K elements 32*(l/32) .. +31 (16 bytes, low
// nibble = lower K) and the scale byte of exactly that 32-element block.  An
// MX block of the linear layout is therefore one lane's operand, and its
// scale byte is that lane's scale.  The accumulator holds
// D[8*(i/4) + 4*(l/32) + i%4][l mod 32] in register i of lane l.
//
// Tiling: a 256-thread workgroup owns a 256 x 256 tile of C (four waves, each
// 128 x 128 = 4 x 4 instructions, 256 fp32 accumulators per lane), walks K in
// steps of 128 and double-buffers the A and B code slices in LDS (rows padded
// from 64 to 80 bytes so the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks).  Scales go straight from global memory to registers (one
// 32-bit load covers the 4 blocks of a 128-wide step).  Tiles are numbered so
// that each of the 8 XCDs works on a contiguous group of tile rows and shares
// A and B slices through its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kRowBytes = 80;                              // 64 code bytes (128 K) + 16 pad
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;       // 40 KiB
constexpr int kLdsBytes = 2 * kStageBytes;                 // double buffer

// Tile order: XCD-contiguous ranges (workgroup b runs on XCD b mod 8), then
// groups of 8 tile rows swept column by column inside each range.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int nt = tiles_m * tiles_n;
    int t = bid;
    if ((nt & 7) == 0) t = (bid & 7) * (nt >> 3) + (bid >> 3);
    constexpr int G = 8;
    const int width = G * tiles_n;
    const int g = t / width;
    const int first = g * G;
    const int gsz = min(tiles_m - first, G);
    const int w = t - g * width;
    tm = first + w % gsz;
    tn = w / gsz;
}

__global__ __launch_bounds__(256) void gemm_mx_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                      const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                      int M, int N, int K, float alpha, void *__restrict__ C,
                                                      int64_t ldc, int c_bf16, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int64_t KB = K >> 1;  // code bytes per row
    const int64_t KS = K >> 5;  // scale bytes per row
    const int nk = K >> 7;      // 128-wide K steps

    // global -> LDS copy: thread t moves 16-byte chunk (t & 3) of rows
    // (t >> 2) + 64 i, i < 4, of both operands (rows past M / N re-read the
    // last row; their results are never stored)
    const int lrow = tid >> 2, lc = tid & 3;
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = min(m0 + lrow + 64 * i, M - 1);
        const int rb = min(n0 + lrow + 64 * i, N - 1);
        a_off[i] = (uint32_t)ra * (uint32_t)KB + lc * 16;
        b_off[i] = (uint32_t)rb * (uint32_t)KB + lc * 16;
    }
    const int st_off = lrow * kRowBytes + lc * 16;

    // this lane's fragment rows and scale rows (offsets in 32-bit words)
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t *As32 = reinterpret_cast<const uint32_t *>(As);
    const uint32_t *Bs32 = reinterpret_cast<const uint32_t *>(Bs);
    uint32_t as_off[4], bs_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = min(m0 + wm * 128 + i * 32 + fr, M - 1);
        const int rb = min(n0 + wn * 128 + i * 32 + fr, N - 1);
        as_off[i] = (uint32_t)ra * (uint32_t)(KS >> 2);
        bs_off[i] = (uint32_t)rb * (uint32_t)(KS >> 2);
    }
    const int fa_off = (wm * 128 + fr) * kRowBytes + fh * 16;
    const int fb_off = kBM * kRowBytes + (wn * 128 + fr) * kRowBytes + fh * 16;

    v16f_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f_t){};

    // prologue: stage 0 codes into LDS buffer 0, stage 0 scales into registers
    uint4 pa[4], pb[4];
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pa[i] = *reinterpret_cast<const uint4 *>(A + a_off[i]);
        pb[i] = *reinterpret_cast<const uint4 *>(B + b_off[i]);
        sa[i] = As32[as_off[i]];
        sb[i] = Bs32[bs_off[i]];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4 *>(lds + st_off + i * 64 * kRowBytes) = pa[i];
        *reinterpret_cast<uint4 *>(lds + kBM * kRowBytes + st_off + i * 64 * kRowBytes) = pb[i];
    }
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        // prefetch step ks+1 (the last step re-reads itself: always in bounds,
        // no branch, so the prefetch stays in registers)
        const int kn = min(ks + 1, nk - 1);
        uint32_t nsa[4], nsb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pa[i] = *reinterpret_cast<const uint4 *>(A + a_off[i] + kn * 64);
            pb[i] = *reinterpret_cast<const uint4 *>(B + b_off[i] + kn * 64);
            nsa[i] = As32[as_off[i] + kn];
            nsb[i] = Bs32[bs_off[i] + kn];
        }
        const uint8_t *base = lds + buf * kStageBytes;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 ta = *reinterpret_cast<const uint4 *>(base + fa_off + i * 32 * kRowBytes + kk * 32);
                const uint4 tb = *reinterpret_cast<const uint4 *>(base + fb_off + i * 32 * kRowBytes + kk * 32);
                af[i] = (v8i_t){(int)ta.x, (int)ta.y, (int)ta.z, (int)ta.w, 0, 0, 0, 0};
                bfr[i] = (v8i_t){(int)tb.x, (int)tb.y, (int)tb.z, (int)tb.w, 0, 0, 0, 0};
            }
            const int sh = 8 * (2 * kk + fh);  // this lane's block within the 128-wide step
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bfr[j], acc[i][j], 4, 4, 0, (int)(sa[i] >> sh), 0, (int)(sb[j] >> sh));
        }
        // the other buffer was last read before the previous barrier
        uint8_t *nb = lds + (buf ^ 1) * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4 *>(nb + st_off + i * 64 * kRowBytes) = pa[i];
            *reinterpret_cast<uint4 *>(nb + kBM * kRowBytes + st_off + i * 64 * kRowBytes) = pb[i];
            sa[i] = nsa[i];
            sb[i] = nsb[i];
        }
        __syncthreads();
    }

    // epilogue: C = alpha * acc, fp32 or bf16 (round to nearest even)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + j * 32 + fr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
                if (row < M && col < N) {
                    const float v = alpha * acc[i][j][r];
                    if (c_bf16)
                        reinterpret_cast<uint16_t *>(C)[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16_rne(v);
                    else
                        reinterpret_cast<float *>(C)[(int64_t)row * ldc + col] = v;
                }
            }
        }
    }
}

__global__ void fill_zero_kernel(void *__restrict__ C, int M, int N, int64_t ldc, int c_bf16)
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

int launch_gemm_mx(const GemmArgs &g, hipStream_t st)
{
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    if (M == 0 || N == 0) return 0;
    if (K == 0) {
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g.c, M, N, g.ldc,
                           (int)g.c_bf16);
        return hipGetLastError() == hipSuccess ? 0 : 1;
    }
    const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    hipLaunchKernelGGL(gemm_mx_kernel, dim3(tiles_m * tiles_n), dim3(256), 0, st,
                       reinterpret_cast<const uint8_t *>(g.a_codes), reinterpret_cast<const uint8_t *>(g.a_scales),
                       reinterpret_cast<const uint8_t *>(g.b_codes), reinterpret_cast<const uint8_t *>(g.b_scales), M,
                       N, K, g.alpha, g.c, g.ldc, (int)g.c_bf16, tiles_m, tiles_n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
