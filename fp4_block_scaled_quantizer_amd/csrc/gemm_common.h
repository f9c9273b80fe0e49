// gemm_common.h -- pieces shared by the block-scaled GEMM kernels of libfp4q
// (gemm_mx.hip, gemm_nv.hip): workgroup -> tile order, LDS DMA issue and
// waits, a compile-time loop, and the epilogue of a wave's 128 x 128 block.
// Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp4q_device.h"

namespace fp4q {
namespace gemm {

typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Epilogue staging of one wave: 32 rows x 64 fp32, rows padded by 16 bytes.
constexpr int kEpiPitch = 64 * 4 + 16;
constexpr int kEpiWaveBytes = 32 * kEpiPitch;

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

// Global -> LDS copies that bypass VGPRs (gfx950 LDS DMA): lane i reads
// base + voff_i (base a 64-bit scalar address, voff a 32-bit per-lane byte
// offset) and writes its 16 (or 4) bytes to LDS address m0 + 16 i (4 i),
// m0 = lds_slot + kLdsOff (the add clobbers SCC, declared as such; an LDS
// DMA needs one wait state after an SALU write of M0, hence the s_nop).
// They are issued from inline assembly so that the only waits on them are
// the explicit vmcnt waits of the K loop: every vector-memory instruction of
// the loop is one of these, so the count of DMA instructions issued after a
// stage is exactly the vmcnt value that guarantees that stage has landed.
// base and lds_slot must be the same in every lane (scalar operands).
template <uint32_t kLdsOff>
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_slot)
{
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_slot),
                 "n"(kLdsOff)
                 : "memory", "m0", "scc");
}
template <uint32_t kLdsOff>
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, uint32_t lds_slot)
{
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds_slot),
                 "n"(kLdsOff)
                 : "memory", "m0", "scc");
}

// All of this wave's LDS reads have returned and at most kAhead DMA
// instructions are still in flight; then the workgroup meets.
template <int kAhead>
__device__ __forceinline__ void wait_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kAhead) : "memory");
}

// wait_and_barrier<kAhead + kExtra> when `extra` (a wave-uniform scalar:
// kExtra more vector-memory instructions were issued, in order, before the
// DMA being waited for is younger than them), else wait_and_barrier<kAhead>.
// Each path meets the workgroup exactly once.
template <int kAhead, int kExtra>
__device__ __forceinline__ void wait_and_barrier_if(int extra)
{
    static_assert(kAhead + kExtra <= 63, "vmcnt holds at most 63");
    if (extra)
        wait_and_barrier<kAhead + kExtra>();
    else
        wait_and_barrier<kAhead>();
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>)
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Epilogue of a wave's 128 x 128 (or 128 x 64) block of C, held as a 4 x 4
// (4 x 2) grid of 32 x 32 accumulator blocks in which the B fragment was the matrix cores' first
// operand: register r of lane l holds C[row (l mod 32)][col 8 (r/4) +
// 4 (l/32) + r mod 4] of its block, so each aligned group of four
// accumulator registers is four consecutive columns of one row.  The block
// is written in chunks of 32 rows x 64 columns: 16-byte LDS writes
// straight from the accumulator registers into the wave's staging area `ep`
// (kEpiWaveBytes), then 16-byte LDS reads of row pieces, alpha (skipped when
// kScale is false), conversion (bf16: v_cvt_pk_bf16_f32, round to nearest
// even) and 16-byte global stores.  Fewest instructions per output: with one
// wave per SIMD every instruction costs an issue cycle that nothing hides.
// Rows >= M and columns >= N are not written; `full` says the whole block is
// inside C with 16-byte aligned rows (then no guards are evaluated); the
// lane index `el` is passed in from an opaque copy so that the lane-derived
// offsets are recomputed here rather than kept live across the K loop.
//
// amax_out (optional): max |C| over the values this wave stores, as they are
// stored, folded into *amax_out as binary32 bits with one atomic max per
// wave (the bits of non-negative floats order like the values).  The maximum
// is taken over the fp32 values and rounded to bf16 once at the end: round
// to nearest even is monotonic, so that is the maximum of the rounded values.

// Vector-memory instructions store_wave_block issues for a full bf16 block
// without amax: one 16-byte store per piece, four pieces per 32 x 64 chunk.
template <int kNJ>
constexpr int kEpiStoresBf16Full = 2 * kNJ * 4;

template <int kNJ, bool kScale, bool kBf16>
__device__ __forceinline__ void store_wave_block(const v16f_t (&acc)[4][kNJ], uint8_t *ep, int el, int row_base,
                                                 int col_base, int M, int N, float alpha, void *C, int64_t ldc,
                                                 bool vec_ok, bool full, uint32_t *amax_out)
{
    float amx = 0.0f;
    static_assert(kNJ == 2 || kNJ == 4, "a wave block is 128 rows x 64 or 128 columns");
    constexpr int kChunks = 2 * kNJ;  // 32 x 64 chunks
    constexpr int esize = kBf16 ? 2 : 4;
    const int efr = el & 31, efh = el >> 5;
    // A lane's pieces of a staged chunk: bf16 pieces are (row el/8 + 8u,
    // 8 columns at 8 (el mod 8)), two fp32 reads each; fp32 pieces
    // (row el/16 + 4u, 4 columns at 4 (el mod 16)).
    const int rl0 = kBf16 ? (el >> 3) : (el >> 4);
    constexpr int rstep = kBf16 ? 8 : 4;
    const int cpi = kBf16 ? (el & 7) : (el & 15);
    const uint32_t lds_lane = rl0 * kEpiPitch + cpi * (kBf16 ? 32 : 16);
    // lane's byte offset inside a chunk of C (the launcher keeps 32 rows of
    // C under 2 GiB for the unguarded path)
    const uint32_t lane_off = ((uint32_t)rl0 * (uint32_t)ldc + cpi * (kBf16 ? 8 : 4)) * esize;
    // chunk c = (i, jp): rows 32 i, columns 64 jp of the wave's block
    auto stage = [&](int c) {
        const int i = c / (kNJ / 2), jp = c % (kNJ / 2);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const v16f_t &a = acc[i][2 * jp + jj];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4 *>(ep + efr * kEpiPitch + (jj * 32 + 8 * g + 4 * efh) * 4) =
                    make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
    };
    auto fetch = [&](float4 (&r)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t o = kBf16 ? lds_lane + (u >> 1) * rstep * kEpiPitch + (u & 1) * 16
                                     : lds_lane + u * rstep * kEpiPitch;
            r[u] = *reinterpret_cast<const float4 *>(ep + o);
        }
    };
    auto store = [&](int c, float4 (&r)[8]) {
        const int i = c / (kNJ / 2), jp = c % (kNJ / 2);
        if (kScale) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                r[u].x *= alpha; r[u].y *= alpha; r[u].z *= alpha; r[u].w *= alpha;
            }
        }
        const int row0 = row_base + i * 32, col0 = col_base + jp * 64;
        constexpr int npieces = kBf16 ? 4 : 8;
        uint4 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if constexpr (kBf16) {
                if (u < 4) {
                    const float4 lo = r[2 * u], hi = r[2 * u + 1];
                    o[u].x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo.x, lo.y}, bf16x2_t));
                    o[u].y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo.z, lo.w}, bf16x2_t));
                    o[u].z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){hi.x, hi.y}, bf16x2_t));
                    o[u].w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){hi.z, hi.w}, bf16x2_t));
                }
            } else {
                o[u] = __builtin_bit_cast(uint4, r[u]);
            }
        }
        constexpr int ne = kBf16 ? 8 : 4;  // elements per piece
        if (full) {
            uint8_t *base = reinterpret_cast<uint8_t *>(C) + ((int64_t)row0 * ldc + col0) * esize;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u < npieces)
                    *reinterpret_cast<uint4 *>(base + (int64_t)u * rstep * ldc * esize + lane_off) = o[u];
            if (amax_out) {
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    amx = fmaxf(amx, fmaxf(fmaxf(fabsf(r[u].x), fabsf(r[u].y)), fmaxf(fabsf(r[u].z), fabsf(r[u].w))));
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u >= npieces) continue;
                const int row = row0 + rl0 + u * rstep, col = col0 + cpi * (kBf16 ? 8 : 4);
                if (row >= M) continue;
                if (amax_out) {
                    // the piece's ne values: r[2u], r[2u+1] (bf16) or r[u] (fp32)
                    const float *rv = reinterpret_cast<const float *>(&r[kBf16 ? 2 * u : u]);
#pragma unroll
                    for (int e = 0; e < ne; ++e)
                        if (col + e < N) amx = fmaxf(amx, fabsf(rv[e]));
                }
                uint8_t *dstp = reinterpret_cast<uint8_t *>(C) + ((int64_t)row * ldc + col) * esize;
                if (vec_ok && col + ne <= N) {
                    *reinterpret_cast<uint4 *>(dstp) = o[u];
                } else if constexpr (kBf16) {
                    const uint16_t *ov = reinterpret_cast<const uint16_t *>(&o[u]);
                    for (int e = 0; e < 8; ++e)
                        if (col + e < N) reinterpret_cast<uint16_t *>(dstp)[e] = ov[e];
                } else {
                    const float *ov = reinterpret_cast<const float *>(&o[u]);
                    for (int e = 0; e < 4; ++e)
                        if (col + e < N) reinterpret_cast<float *>(dstp)[e] = ov[e];
                }
            }
        }
    };
    // Two-deep pipeline over the eight chunks: the LDS writes and reads of
    // chunk c+1 are issued before chunk c is converted and stored, so one
    // chunk's LDS latency hides behind the other's stores.  A wave's LDS
    // operations run in issue order, so chunk c's reads complete before
    // chunk c+1's writes reuse the area.
    float4 r0[8], r1[8];
    stage(0);
    fetch(r0);
#pragma unroll
    for (int c = 0; c < kChunks; c += 2) {
        stage(c + 1);
        fetch(r1);
        store(c, r0);
        if (c + 2 < kChunks) {
            stage(c + 2);
            fetch(r0);
        }
        store(c + 1, r1);
    }
    if (amax_out) {
        uint32_t bits;
        if constexpr (kBf16)
            bits = (__builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){amx, 0.0f}, bf16x2_t)) & 0xFFFFu)
                   << 16;
        else
            bits = __builtin_bit_cast(uint32_t, amx);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) bits = max(bits, (uint32_t)__shfl_xor((int)bits, m, 64));
        if ((el & 63) == 0) atomicMax(amax_out, bits);
    }
}

// The epilogue for a runtime output type and alpha.
template <int kNJ>
__device__ __forceinline__ void store_wave_block_any(const v16f_t (&acc)[4][kNJ], uint8_t *ep, int el, int row_base,
                                                     int col_base, int M, int N, float alpha, void *C, int64_t ldc,
                                                     bool c_bf16, bool vec_ok, uint32_t *amax_out)
{
    const bool full = vec_ok && row_base + 128 <= M && col_base + 32 * kNJ <= N;
    if (c_bf16) {
        if (alpha != 1.0f)
            store_wave_block<kNJ, true, true>(acc, ep, el, row_base, col_base, M, N, alpha, C, ldc, vec_ok, full,
                                              amax_out);
        else
            store_wave_block<kNJ, false, true>(acc, ep, el, row_base, col_base, M, N, alpha, C, ldc, vec_ok, full,
                                               amax_out);
    } else {
        if (alpha != 1.0f)
            store_wave_block<kNJ, true, false>(acc, ep, el, row_base, col_base, M, N, alpha, C, ldc, vec_ok, full,
                                              amax_out);
        else
            store_wave_block<kNJ, false, false>(acc, ep, el, row_base, col_base, M, N, alpha, C, ldc, vec_ok, full,
                                                amax_out);
    }
}

// One accumulator register read in program order.  Read through plain C++,
// the accumulators of a whole wave block are copied out of the accumulator
// registers at once and spill; the opaque read keeps each copy next to its
// use.  The caller covers the matrix-core write-to-read distance.
__device__ __forceinline__ float acc_read(float a)
{
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// The value lane l ^ 32 holds (v_permlane32_swap: no LDS traffic); h = l / 32.
__device__ __forceinline__ uint32_t lane_half_exchange(uint32_t v, int h)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return h ? r[0] : r[1];
}

// One row's 32-column MX block of an epilogue output, held as bf16 pairs
// p[r] = columns 8 (r / 2) + 4 h + 2 (r mod 2) + {0, 1} in lane h = l / 32
// (the other 16 values in lane l ^ 32), with fmx = the largest |value|
// before the bf16 rounding: the block amax is fmx rounded once (rounding is
// monotonic) and exchanged with v_permlane32_swap, the codes come from the
// producers' scaled convert, and half of them are exchanged so that lane h
// writes bytes 8 h .. 8 h + 7 of the row's 16 code bytes, at column c of a
// ncols-wide output (tiled: 1 KiB lane-order blocks; a padding row writes
// zeros).  Returns the block's E8M0 byte.
template <bool kTiled>
__device__ __forceinline__ uint32_t emit_mx_block(const bf16x2_t (&p)[8], float fmx, int h, bool live, bool pad, int row,
                                                  int c, int ncols, uint8_t *codes)
{
    uint32_t amax = (__builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){fmx, 0.0f}, bf16x2_t)) & 0xFFFFu)
                    << 16;
    amax = max(amax, lane_half_exchange(amax, h));
    const uint32_t sbyte = mx_scale_byte(amax);
    const float scale = mx_scale_f32(sbyte);
    uint32_t grp[4];  // 4 codes (16 bits) of columns 8 g + 4 h .. + 3
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, p[2 * g], scale, 0);
        grp[g] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, p[2 * g + 1], scale, 1);
    }
    // lane h = 0 keeps groups 0, 1 of its half and takes the other half's;
    // lane h = 1 keeps groups 2, 3
    const uint32_t give = h ? (grp[0] | grp[1] << 16) : (grp[2] | grp[3] << 16);
    const uint32_t got = lane_half_exchange(give, h);
    uint2 out = h ? make_uint2((got & 0xFFFFu) | grp[2] << 16, (got >> 16) | grp[3] << 16)
                  : make_uint2(grp[0] | got << 16, grp[1] | (got & 0xFFFF0000u));
    if (pad) out = make_uint2(0u, 0u);
    if (live || pad) {
        uint8_t *dst = kTiled ? codes + ((int64_t)(row >> 5) * (ncols >> 6) + (c >> 6)) * 1024 +
                                    ((row & 31) + 32 * ((c >> 5) & 1)) * 16 + 8 * h
                              : codes + (int64_t)row * (ncols >> 1) + (c >> 1) + 8 * h;
        *reinterpret_cast<uint2 *>(dst) = out;
    }
    return live ? sbyte : 0u;
}

// Epilogue that writes a wave's 128 x 128 block of C as an MXFP4 operand
// along rows (the next GEMM's A operand) instead of as C itself.  Each value
// (times alpha) is rounded to bf16 first, so the output is exactly what the
// MX row producer makes of the bf16 C.  A row's 32-column block lies in
// lanes l and l ^ 32 (16 values each, four groups of four columns 8 g + 4 h),
// written by emit_mx_block; the lane h = 0 also writes the row's four scale
// bytes of the 128 columns as one word.  Requires N % 32 == 0 (N % 128 == 0
// tiled); in the tiled layout rows M .. Mp-1 are written as zero codes and
// zero scales, as the producers write them.
template <bool kScale, bool kTiled>
__device__ __forceinline__ void store_wave_block_mxq(const v16f_t (&acc)[4][4], int el, int row_base, int col_base,
                                                     int M, int N, int Mp, float alpha, uint8_t *codes,
                                                     uint8_t *scales)
{
    const int fr = el & 31, h = el >> 5;
    // the opaque reads hide the last matrix-core writes from the compiler's
    // hazard tracking: wait out the longest write-to-read distance here
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row_base + 32 * i + fr;
        const bool live = row < M;
        const bool pad = !live && kTiled && row < Mp;
        uint32_t sword = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = col_base + 32 * j;
            if (c >= N) continue;  // the same for every lane
            // bf16 pairs (round to nearest even, as the bf16 epilogue
            // stores them); the block amax is taken on the fp32 values
            bf16x2_t p[8];
            float fmx = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float a0 = acc_read(acc[i][j][2 * r]), a1 = acc_read(acc[i][j][2 * r + 1]);
                if (kScale) {
                    a0 *= alpha;
                    a1 *= alpha;
                }
                fmx = fmaxf(fmx, fmaxf(fabsf(a0), fabsf(a1)));
                p[r] = __builtin_convertvector((f32x2_t){a0, a1}, bf16x2_t);
            }
            sword |= emit_mx_block<kTiled>(p, fmx, h, live, pad, row, c, N, codes) << (8 * j);
        }
        if (h == 0 && (live || pad)) {
            if (kTiled) {
                *reinterpret_cast<uint32_t *>(scales + ((int64_t)(col_base >> 7) * Mp + row) * 4) = sword;
            } else {
                uint8_t *dst = scales + (int64_t)row * (N >> 5) + (col_base >> 5);
                if (col_base + 128 <= N) {
                    *reinterpret_cast<uint32_t *>(dst) = sword;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (col_base + 32 * j < N) dst[j] = (uint8_t)(sword >> (8 * j));
                }
            }
        }
    }
}

// Epilogue that applies SwiGLU to a wave's 128 x 128 block of C and writes
// the result H as an MXFP4 operand along rows.  The weight's rows (C's
// columns) interleave gate and up in groups of 32, so accumulator blocks
// j = 0, 2 hold gate columns and j = 1, 3 the up columns of the same 32
// hidden columns, lane for lane, and the wave's 128 columns of C are the
// 64 hidden columns hcol_base .. + 63 of H (F = N / 2 wide).  Per value:
// g and u = alpha C rounded to bf16 (as the bf16 GEMM stores C), then
// bf16(SiLU(g) * u) (silu_f32: the fixed binary32 sequence), then the MX
// block of emit_mx_block -- exactly what the bf16 GEMM, the SwiGLU kernel
// and the MX row producer compute one after another.  The lane h = 0 writes
// the row's two scale bytes as one 16-bit word.  Requires F % 32 == 0
// (F % 128 == 0 tiled).
template <bool kScale, bool kTiled>
__device__ __forceinline__ void store_wave_block_swiglu_mxq(const v16f_t (&acc)[4][4], int el, int row_base,
                                                            int hcol_base, int M, int F, int Mp, float alpha,
                                                            uint8_t *codes, uint8_t *scales)
{
    const int fr = el & 31, h = el >> 5;
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row_base + 32 * i + fr;
        const bool live = row < M;
        const bool pad = !live && kTiled && row < Mp;
        uint32_t sword = 0;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
            const int c = hcol_base + 32 * jp;
            if (c >= F) continue;  // the same for every lane
            bf16x2_t p[8];
            float fmx = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float g0 = acc_read(acc[i][2 * jp][2 * r]), g1 = acc_read(acc[i][2 * jp][2 * r + 1]);
                float u0 = acc_read(acc[i][2 * jp + 1][2 * r]), u1 = acc_read(acc[i][2 * jp + 1][2 * r + 1]);
                if (kScale) {
                    g0 *= alpha; g1 *= alpha; u0 *= alpha; u1 *= alpha;
                }
                const uint32_t gb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){g0, g1}, bf16x2_t));
                const uint32_t ub = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){u0, u1}, bf16x2_t));
                const float h0 = silu_f32(bf16_lo(gb)) * bf16_lo(ub);
                const float h1 = silu_f32(bf16_hi(gb)) * bf16_hi(ub);
                fmx = fmaxf(fmx, fmaxf(fabsf(h0), fabsf(h1)));
                p[r] = __builtin_convertvector((f32x2_t){h0, h1}, bf16x2_t);
            }
            sword |= emit_mx_block<kTiled>(p, fmx, h, live, pad, row, c, F, codes) << (8 * jp);
        }
        if (h == 0 && (live || pad)) {
            if (kTiled) {
                // bytes 2 (hcol_base / 64 mod 2) .. +1 of the row's word of
                // the 128-column step
                *reinterpret_cast<uint16_t *>(scales + ((int64_t)(hcol_base >> 7) * Mp + row) * 4 +
                                              ((hcol_base >> 5) & 2)) = (uint16_t)sword;
            } else {
                uint8_t *dst = scales + (int64_t)row * (F >> 5) + (hcol_base >> 5);
                if (hcol_base + 64 <= F)
                    *reinterpret_cast<uint16_t *>(dst) = (uint16_t)sword;
                else
                    dst[0] = (uint8_t)sword;
            }
        }
    }
}

// The quantizing epilogue for a runtime alpha and output layout.
__device__ __forceinline__ void store_wave_block_mxq_any(const v16f_t (&acc)[4][4], int el, int row_base,
                                                         int col_base, int M, int N, int Mp, float alpha,
                                                         uint8_t *codes, uint8_t *scales, bool tiled)
{
    if (tiled) {
        if (alpha != 1.0f)
            store_wave_block_mxq<true, true>(acc, el, row_base, col_base, M, N, Mp, alpha, codes, scales);
        else
            store_wave_block_mxq<false, true>(acc, el, row_base, col_base, M, N, Mp, alpha, codes, scales);
    } else {
        if (alpha != 1.0f)
            store_wave_block_mxq<true, false>(acc, el, row_base, col_base, M, N, Mp, alpha, codes, scales);
        else
            store_wave_block_mxq<false, false>(acc, el, row_base, col_base, M, N, Mp, alpha, codes, scales);
    }
}

// The SwiGLU epilogue for a runtime alpha and output layout.
__device__ __forceinline__ void store_wave_block_swiglu_mxq_any(const v16f_t (&acc)[4][4], int el, int row_base,
                                                                int hcol_base, int M, int F, int Mp, float alpha,
                                                                uint8_t *codes, uint8_t *scales, bool tiled)
{
    if (tiled) {
        if (alpha != 1.0f)
            store_wave_block_swiglu_mxq<true, true>(acc, el, row_base, hcol_base, M, F, Mp, alpha, codes, scales);
        else
            store_wave_block_swiglu_mxq<false, true>(acc, el, row_base, hcol_base, M, F, Mp, alpha, codes, scales);
    } else {
        if (alpha != 1.0f)
            store_wave_block_swiglu_mxq<true, false>(acc, el, row_base, hcol_base, M, F, Mp, alpha, codes, scales);
        else
            store_wave_block_swiglu_mxq<false, false>(acc, el, row_base, hcol_base, M, F, Mp, alpha, codes, scales);
    }
}

// n zero bytes (the quantized form of C = 0: zero codes, zero scales).
static __global__ void fill_bytes_zero_kernel(uint8_t *__restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// C = 0 (the K == 0 product); one thread per element.
static __global__ void fill_zero_kernel(void *__restrict__ C, int M, int N, int64_t ldc, int c_bf16)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int64_t r = i / N, c = i - r * N;
    if (c_bf16)
        reinterpret_cast<uint16_t *>(C)[r * ldc + c] = 0;
    else
        reinterpret_cast<float *>(C)[r * ldc + c] = 0.0f;
}

}  // namespace gemm
}  // namespace fp4q
