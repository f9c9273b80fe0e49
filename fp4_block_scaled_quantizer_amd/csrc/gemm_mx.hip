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
constexpr int kStages = 4;                                  // LDS ring depth (K steps in flight)
constexpr int kCodeBytes = kBM * 64;                        // one operand's codes per 128-wide K step
constexpr int kScaleOff = 2 * kCodeBytes;                   // A scales, then B scales (u32 per row)
constexpr int kStageBytes = 2 * kCodeBytes + (kBM + kBN) * 4;  // 34 KiB
constexpr int kLdsBytes = kStages * kStageBytes;            // 136 KiB
constexpr int kDmaPerStage = 10;                            // DMA instructions per wave per stage

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

// Global -> LDS copies that bypass VGPRs (gfx950 LDS DMA): lane i writes its
// 16 (or 4) bytes to LDS address m0 + 16 i (4 i).  They are issued from
// inline assembly so that the only waits on them are the explicit
// vmcnt waits of the K loop: every vector-memory instruction of the loop is
// one of these, so the count of DMA instructions issued after a stage is
// exactly the vmcnt value that guarantees that stage has landed.
// lds_addr must be the same in every lane (it is moved through
// readfirstlane into the scalar M0 register).
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr)
{
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *gptr, uint32_t lds_addr)
{
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(m) : "memory", "m0");
}

// All of this wave's LDS reads have returned and at most kAhead DMA
// instructions are still in flight; then the workgroup meets.
template <int kAhead>
__device__ __forceinline__ void wait_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kAhead) : "memory");
}

template <bool kTiled>
__global__ __launch_bounds__(256) void gemm_mx_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                      const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                      int M, int N, int K, float alpha, void *__restrict__ C,
                                                      int64_t ldc, int c_bf16, int vec_ok, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const uint32_t KB = (uint32_t)K >> 1;  // code bytes per row
    const uint32_t KS = (uint32_t)K >> 5;  // scale bytes per row
    const int nk = K >> 7;                 // 128-wide K steps
    const uint32_t Mp = ((uint32_t)M + 31) & ~31u, Np = ((uint32_t)N + 31) & ~31u;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    // LDS image of a stage: the codes of 32 rows x 64 K elements are one
    // 1 KiB block in matrix-core lane order (lane l's 16 bytes = row l mod 32,
    // K half l / 32), blocks ordered (row group g, K half kk) -> 2 g + kk.
    // Wave w copies blocks 4w .. 4w+3 of A and of B.  In the tiled layout a
    // block is 1 KiB of contiguous global memory; in the linear layout lane l
    // of block b reads row 32 (b / 2) + l mod 32, bytes 32 (b mod 2) +
    // 16 (l / 32) of the step.  Rows past the operand re-read its last row
    // (linear) or row group (tiled); their results are never stored.
    uint32_t a_goff[4], b_goff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = wave * 4 + i;
        if (kTiled) {
            const uint32_t ga = min((uint32_t)(m0 / 32 + (b >> 1)), Mp / 32 - 1);
            const uint32_t gb = min((uint32_t)(n0 / 32 + (b >> 1)), Np / 32 - 1);
            a_goff[i] = (ga * (uint32_t)(K >> 6) + (b & 1)) * 1024 + lane * 16;
            b_goff[i] = (gb * (uint32_t)(K >> 6) + (b & 1)) * 1024 + lane * 16;
        } else {
            const int r = 32 * (b >> 1) + (lane & 31);
            const uint32_t col = 32 * (b & 1) + 16 * (lane >> 5);
            a_goff[i] = (uint32_t)min(m0 + r, M - 1) * KB + col;
            b_goff[i] = (uint32_t)min(n0 + r, N - 1) * KB + col;
        }
    }
    const uint32_t code_step = kTiled ? 2048u : 64u;
    // scales: wave w copies rows 64 w + lane of A and of B (one u32 per row per step)
    uint32_t as_goff, bs_goff, as_step, bs_step;
    if (kTiled) {
        as_goff = min((uint32_t)(m0 + wave * 64 + lane), Mp - 1) * 4;
        bs_goff = min((uint32_t)(n0 + wave * 64 + lane), Np - 1) * 4;
        as_step = Mp * 4;
        bs_step = Np * 4;
    } else {
        as_goff = (uint32_t)min(m0 + wave * 64 + lane, M - 1) * KS;
        bs_goff = (uint32_t)min(n0 + wave * 64 + lane, N - 1) * KS;
        as_step = bs_step = 4;
    }

    auto issue = [&](int ks, int slot) {
        const uint32_t st = lds_base + slot * kStageBytes;
        const uint32_t kc = (uint32_t)ks * code_step;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(A + a_goff[i] + kc, st + (wave * 4 + i) * 1024);
            dma16(B + b_goff[i] + kc, st + kCodeBytes + (wave * 4 + i) * 1024);
        }
        dma4(As + as_goff + (uint32_t)ks * as_step, st + kScaleOff + wave * 256);
        dma4(Bs + bs_goff + (uint32_t)ks * bs_step, st + kScaleOff + kBM * 4 + wave * 256);
    };

    const int fr = lane & 31, fh = lane >> 5;

    v16f_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f_t){};

    // prologue: kStages - 1 steps in flight (steps past the end re-read the
    // last step into free slots, so the loop's wait count never changes)
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(min(s, nk - 1), s);

    for (int ks = 0; ks < nk; ++ks) {
        const int slot = ks % kStages;
        wait_and_barrier<(kStages - 2) * kDmaPerStage>();
        // the slot read in step ks-1 is free for step ks + kStages - 1
        issue(min(ks + kStages - 1, nk - 1), (ks + kStages - 1) % kStages);

        const uint8_t *st = lds + slot * kStageBytes;
        uint32_t sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i] = *reinterpret_cast<const uint32_t *>(st + kScaleOff + (wm * 128 + i * 32 + fr) * 4);
            sb[i] = *reinterpret_cast<const uint32_t *>(st + kScaleOff + kBM * 4 + (wn * 128 + i * 32 + fr) * 4);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 ta = *reinterpret_cast<const uint4 *>(st + ((wm * 4 + i) * 2 + kk) * 1024 + lane * 16);
                const uint4 tb =
                    *reinterpret_cast<const uint4 *>(st + kCodeBytes + ((wn * 4 + i) * 2 + kk) * 1024 + lane * 16);
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
    }
    // drain the re-read steps still in flight, and let every wave finish its
    // last LDS reads before the ring is reused for the epilogue
    wait_and_barrier<0>();

    // epilogue: each wave stages a 32 x 128 band of alpha * acc in its own LDS
    // region (row pitch padded by 16 bytes), then writes it out in contiguous
    // 16-byte pieces: 256 contiguous bytes per row of the band.
    const int esize = c_bf16 ? 2 : 4;
    const int pitch = 128 * esize + 16;
    uint8_t *ep = lds + wave * (32 * (128 * 4 + 16));
    const int row_base = m0 + wm * 128, col_base = n0 + wn * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = 8 * (r >> 2) + 4 * fh + (r & 3);
                const int cl = j * 32 + fr;
                const float v = alpha * acc[i][j][r];
                if (c_bf16)
                    *reinterpret_cast<uint16_t *>(ep + rl * pitch + cl * 2) = (uint16_t)f32_to_bf16_rne(v);
                else
                    *reinterpret_cast<float *>(ep + rl * pitch + cl * 4) = v;
            }
        }
        // the band is 32 rows x (128 * esize) bytes = 16-byte pieces per row: 16 (bf16) or 32 (fp32)
        const int per_row = 8 * esize;
        const int pieces = 32 * per_row;
        for (int pc = lane; pc < pieces; pc += 64) {
            const int rl = pc / per_row, cp = pc - rl * per_row;
            const int row = row_base + i * 32 + rl;
            const int col = col_base + cp * (16 / esize);
            if (row >= M) continue;
            const uint8_t *srcp = ep + rl * pitch + cp * 16;
            uint8_t *dstp = reinterpret_cast<uint8_t *>(C) + ((int64_t)row * ldc + col) * esize;
            if (vec_ok && col + 16 / esize <= N) {
                *reinterpret_cast<uint4 *>(dstp) = *reinterpret_cast<const uint4 *>(srcp);
            } else {
                for (int e = 0; e < 16 / esize; ++e)
                    if (col + e < N) {
                        if (c_bf16)
                            reinterpret_cast<uint16_t *>(dstp)[e] = reinterpret_cast<const uint16_t *>(srcp)[e];
                        else
                            reinterpret_cast<float *>(dstp)[e] = reinterpret_cast<const float *>(srcp)[e];
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
    const int esize = g.c_bf16 ? 2 : 4;
    const int vec_ok = ((uintptr_t)g.c % 16 == 0) && (g.ldc % (16 / esize) == 0);
    auto *a = reinterpret_cast<const uint8_t *>(g.a_codes);
    auto *as = reinterpret_cast<const uint8_t *>(g.a_scales);
    auto *b = reinterpret_cast<const uint8_t *>(g.b_codes);
    auto *bs = reinterpret_cast<const uint8_t *>(g.b_scales);
    if (g.tiled)
        hipLaunchKernelGGL(gemm_mx_kernel<true>, dim3(tiles_m * tiles_n), dim3(256), 0, st, a, as, b, bs, M, N, K,
                           g.alpha, g.c, g.ldc, (int)g.c_bf16, vec_ok, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(gemm_mx_kernel<false>, dim3(tiles_m * tiles_n), dim3(256), 0, st, a, as, b, bs, M, N, K,
                           g.alpha, g.c, g.ldc, (int)g.c_bf16, vec_ok, tiles_m, tiles_n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
