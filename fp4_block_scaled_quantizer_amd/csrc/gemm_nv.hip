// gemm_nv.hip -- NVFP4 GEMM on fp16 matrix cores with in-register exact
// dequantization; FP32 tensor scales applied to fp32 sums.
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
// scale per 32 elements, which cannot carry an E4M3 scale per 16.  The
// kernel therefore dequantizes the E2M1 codes times their E4M3 block scale
// exactly into fp16 and multiplies on v_mfma_f32_32x32x16_f16: every
// product is exact and only the fp32 accumulation rounds.  The tensor scales
// are applied to fp32 sums: once in the epilogue for the global domain, and
// per 128-wide K step for the per-tile domain (a step is one tile column of
// both operands, and a wave's 128-row block of A or 64-row block of B lies in
// one tile row, so one factor S_A(tm, kt) * S_B(tn, kt) covers a wave's whole
// partial sum of the step).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"
#include "fp4q_internal.h"
#include "gemm_common.h"

namespace fp4q {

namespace {

// ------------------------------------------------------------------
// Persistent kernel on fp16 matrix cores.
//
// An E2M1 value times an E4M3 scale has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in fp16 as well as bf16; fp16 has packed
// multiplies on gfx950 (bf16 has none), so each pair of elements dequantizes
// in two instructions: v_cvt_scalef32_pk_f16_fp4 (scale 1: the E2M1 values)
// and v_pk_mul_f16 by the block's E4M3 value.  (The scaled convert itself
// applies only the exponent of its scale operand, which an E4M3 value with a
// mantissa would lose.)  Products on v_mfma_f32_32x32x16_f16 are then exact
// and only the fp32 accumulation rounds.
//
// Structure as the MX kernel: one 256-thread workgroup per CU walks output
// tiles (B fragment first so the accumulators hold row pieces), a four-slot
// LDS ring of 128-wide K steps filled by LDS DMA three steps ahead, and the
// shared epilogue.  Each wave dequantizes the fragments it multiplies, in
// registers, one 16-wide K slice ahead of the matrix cores.
//
// Global domain: 256 x 256 tiles, four waves of 128 x 128; S_A * S_B * alpha
// scales the sum in the epilogue.  Per-tile domain: 256 x 128 tiles, four
// waves of 128 x 64, so that a second set of accumulators fits: each step's
// product starts from zero and is added, times S_A(tm, kt) * S_B(tn, kt),
// into the running sum.
//
// K order inside a step.  The matrix cores only need A and B to agree on
// which K a lane position carries, so slice s (0..7) of a 128-wide step
// gives lanes 0..31 the K values 8s .. 8s+7 and lanes 32..63 the values
// 64 + 8s .. 64 + 8s + 7.  A lane's 4 slices s = 4q .. 4q+3 are then 16
// contiguous code bytes (chunk 2h + q of its row's 64 bytes): one 16-byte
// LDS read per row per 4 slices.  Its 16-element NV block for slice s is
// 4h + s/2: byte s/2 of the 32-bit word at row offset 4h of the step's 8
// scale bytes.
//
// LDS image of a stage: codes of up to 256 rows x 64 bytes per operand with the
// 16-byte chunk c of local row r at r * 64 + 16 (c ^ ((r >> 1) & 3)) (the
// DMA lane mapping applies the swizzle, so 8 lanes reading one chunk of 8
// consecutive rows hit 8 distinct bank groups), then 8 scale bytes per row.
// ------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr int gStages = 4;
constexpr int gCodeBytes = 256 * 64;                     // one operand's codes per K step
constexpr int gScaleBytes = 256 * 8;                     // one operand's E4M3 bytes per K step
constexpr int gAS = 2 * gCodeBytes;                      // A scales, then B scales
constexpr int gBS = gAS + gScaleBytes;
constexpr int gStageBytes = 2 * gCodeBytes + 2 * gScaleBytes;  // 36 KiB
constexpr int gLdsBytes = gStages * gStageBytes;               // 144 KiB
static_assert(4 * gemm::kEpiWaveBytes <= gStageBytes, "epilogue staging must fit in one ring slot");

// 8 codes (one 32-bit word, element 2b in the low nibble of byte b) times a
// block scale given as two equal fp16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s2)
{
    const half2_t p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * s2;
    const half2_t p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * s2;
    const half2_t p2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * s2;
    const half2_t p3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * s2;
    return (half8_t){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Half of dequant8: elements 4 p .. 4 p + 3 of the fragment (codes of nibble
// pairs 2 p and 2 p + 1 of w), written into their two registers of out.
template <int p>
__device__ __forceinline__ void dequant4(half8_t &out, uint32_t w, half2_t s2)
{
    const half2_t lo = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2 * p)) * s2;
    const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2 * p + 1)) * s2;
    out[4 * p] = lo[0];
    out[4 * p + 1] = lo[1];
    out[4 * p + 2] = hi[0];
    out[4 * p + 3] = hi[1];
}

// E4M3 bytes 0, 1 (kHi: 2, 3) of word w as two fp16 (exact: every E4M3 value
// is an fp16 normal); a fragment's block scale is then one half of the pair,
// broadcast by bcast<h> into the op_sel of the packed multiply.
template <bool kHi>
__device__ __forceinline__ half2_t scale_pair(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi);
}

template <int h>
__device__ __forceinline__ half2_t bcast(half2_t p)
{
    return __builtin_shufflevector(p, p, h, h);
}

// kTiledIn: A and B in the tiled consumer layout (step-major 32-row blocks:
// a step's 64 code bytes of local row f of group g at ((g * nk + s) * 32 + f)
// * 64, its 8 scale bytes at ((g * nk + s) * 32 + f) * 8), so that each DMA
// instruction copies 1 KiB of contiguous codes (16 rows of one step) and
// each scale DMA 256 contiguous bytes; the chunk swizzle of the LDS image is
// applied by the lane -> source mapping, as in the linear layout.
template <bool kTile, bool kTiledIn>
__global__ __launch_bounds__(256) void gemm_nv_fp16_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const float *__restrict__ Ats,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs, const float *__restrict__ Bts, int M, int N, int K,
    float alpha, void *__restrict__ C, int64_t ldc, int c_bf16, int vec_ok, int tiles_m, int tiles_n,
    uint32_t *__restrict__ c_amax)
{
    using namespace gemm;
    // global domain: 256 x 256 tiles, wave blocks 128 x 128; per-tile domain:
    // 256 x 128 tiles, wave blocks 128 x 64 (room for a second accumulator set)
    constexpr int NJ = kTile ? 2 : 4;             // 32-column blocks per wave
    constexpr int BN = 64 * NJ;                   // workgroup tile columns (two waves across)
    constexpr int kBRowsPerWave = BN / 4;         // B rows one wave copies per step
    constexpr int kDma = 4 + NJ + 2 + NJ / 2;     // DMA instructions per wave per step
    __shared__ __attribute__((aligned(1024))) uint8_t lds[gLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t KB = (uint32_t)K >> 1;  // code bytes per row
    const uint32_t KS = (uint32_t)K >> 4;  // scale bytes per row
    const int nk = K >> 7;
    const uint32_t Mp = ((uint32_t)M + 31) & ~31u, Np = ((uint32_t)N + 31) & ~31u;
    constexpr uint32_t kCodeStep = kTiledIn ? 2048u : 64u;   // source advance per K step
    constexpr uint32_t kScaleStep = kTiledIn ? 256u : 8u;
    // source offset of the 64 code bytes (scale bytes) of stored row `row` in K step 0
    auto code_row = [&](uint32_t row) -> uint32_t {
        return kTiledIn ? ((row >> 5) * (uint32_t)nk * 32u + (row & 31u)) * 64u : row * KB;
    };
    auto scale_row = [&](uint32_t row) -> uint32_t {
        return kTiledIn ? ((row >> 5) * (uint32_t)nk * 32u + (row & 31u)) * 8u : row * KS;
    };
    const uint32_t Mlast = kTiledIn ? Mp - 1 : (uint32_t)M - 1, Nlast = kTiledIn ? Np - 1 : (uint32_t)N - 1;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    const int ntiles = tiles_m * tiles_n;

    // per-lane DMA sources of the current tile (see the stage image above)
    uint32_t a_goff[4], b_goff[NJ], as_goff[2], bs_goff[NJ / 2];
    int m0 = 0, n0 = 0;
    const uint8_t *pa = A, *pb = B, *pas = As, *pbs = Bs;
    int dstep = 0;
    auto setup = [&](int tile) {
        int tm, tn;
        tile_coords(tile, tiles_m, tiles_n, tm, tn);
        m0 = tm * 256;
        n0 = tn * BN;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t r = 64 * wave + 16 * t + (lane >> 2);  // local row
            const uint32_t c = (uint32_t)(lane & 3) ^ ((r >> 1) & 3u);
            a_goff[t] = code_row(min((uint32_t)m0 + r, Mlast)) + c * 16;
        }
#pragma unroll
        for (int t = 0; t < NJ; ++t) {
            const uint32_t r = kBRowsPerWave * wave + 16 * t + (lane >> 2);
            const uint32_t c = (uint32_t)(lane & 3) ^ ((r >> 1) & 3u);
            b_goff[t] = code_row(min((uint32_t)n0 + r, Nlast)) + c * 16;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t r = 64 * wave + 32 * t + (lane >> 1);
            as_goff[t] = scale_row(min((uint32_t)m0 + r, Mlast)) + (lane & 1) * 4;
        }
#pragma unroll
        for (int t = 0; t < NJ / 2; ++t) {
            const uint32_t r = kBRowsPerWave * wave + 32 * t + (lane >> 1);
            bs_goff[t] = scale_row(min((uint32_t)n0 + r, Nlast)) + (lane & 1) * 4;
        }
        pa = A;
        pb = B;
        pas = As;
        pbs = Bs;
        dstep = 0;
    };
    // the d-th of this wave's kDma DMA instructions of a step into the stage at slot_addr
    auto dma_piece = [&](uint32_t slot_addr, auto d_tag) {
        constexpr int d = decltype(d_tag)::value;
        if constexpr (d < 4)
            dma16<0>(pa, a_goff[d], slot_addr + (64 * wave + 16 * d) * 64);
        else if constexpr (d < 4 + NJ)
            dma16<gCodeBytes>(pb, b_goff[d - 4], slot_addr + (kBRowsPerWave * wave + 16 * (d - 4)) * 64);
        else if constexpr (d < 6 + NJ)
            dma4<gAS>(pas, as_goff[d - 4 - NJ], slot_addr + (64 * wave + 32 * (d - 4 - NJ)) * 8);
        else
            dma4<gBS>(pbs, bs_goff[d - 6 - NJ], slot_addr + (kBRowsPerWave * wave + 32 * (d - 6 - NJ)) * 8);
    };
    auto advance = [&]() {
        const uint32_t more = dstep < nk - 1 ? 1u : 0u;
        pa += more * kCodeStep;
        pb += more * kCodeStep;
        pas += more * kScaleStep;
        pbs += more * kScaleStep;
        dstep += (int)more;
    };
    auto prologue = [&]() {
#pragma unroll
        for (int s2 = 0; s2 < gStages - 1; ++s2) {
            const uint32_t slot_addr = lds_base + s2 * gStageBytes;
            static_for<kDma>([&](auto d) { dma_piece(slot_addr, d); });
            advance();
        }
    };

    // fragment sources: local rows of this wave's block rows / columns
    auto code_chunk = [&](const uint8_t *st, int operand, int i, int q) -> uint4 {
        const uint32_t r = (operand == 0 ? wm * 128 : wn * (32 * NJ)) + 32 * i + fr;
        const uint32_t c = (uint32_t)(2 * fh + q) ^ ((r >> 1) & 3u);
        return *reinterpret_cast<const uint4 *>(st + operand * gCodeBytes + r * 64 + c * 16);
    };
    auto scale_word = [&](const uint8_t *st, int operand, int i) -> uint32_t {
        const uint32_t r = (operand == 0 ? wm * 128 : wn * (32 * NJ)) + 32 * i + fr;
        return *reinterpret_cast<const uint32_t *>(st + gAS + operand * gScaleBytes + r * 8 + fh * 4);
    };

    v16f_t acc[4][NJ];              // the sum (global) or the current K tile's partial sum (per-tile)
    v16f_t tot[kTile ? 4 : 1][kTile ? NJ : 1];  // per-tile: the sum of the scaled partials
    uint4 rawA[4][2], rawB[NJ][2];  // code chunks of the step (q = 0, 1)
    uint32_t swA[4], swB[NJ];       // scale words of the step
    uint32_t nswA[4], nswB[NJ];     // scale words of the next step
    half2_t sAp[4], sBp[NJ];        // block scales of the current two slice pairs
    half8_t fa[4], fb[NJ];          // fragments of the slice on the matrix cores
    half8_t na[4], nb[NJ];          // fragments of the next slice

    auto word_of = [&](const uint4 &q, int d) -> uint32_t {
        return d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
    };

    int tile = blockIdx.x;
    setup(tile);
    prologue();
    for (;;) {
        // stages 0 and 1 of this tile have landed (only stage 2's DMA may be
        // in flight; loads complete in order)
        wait_and_barrier<kDma>();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rawA[i][0] = code_chunk(lds, 0, i, 0);
            rawA[i][1] = code_chunk(lds, 0, i, 1);
            swA[i] = scale_word(lds, 0, i);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            rawB[j][0] = code_chunk(lds, 1, j, 0);
            rawB[j][1] = code_chunk(lds, 1, j, 1);
            swB[j] = scale_word(lds, 1, j);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sAp[i] = scale_pair<false>(swA[i]);
            fa[i] = dequant8(rawA[i][0].x, bcast<0>(sAp[i]));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            sBp[j] = scale_pair<false>(swB[j]);
            fb[j] = dequant8(rawB[j][0].x, bcast<0>(sBp[j]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (kTile)
                    tot[kTile ? i : 0][kTile ? j : 0] = (v16f_t){};
                else
                    acc[i][j] = (v16f_t){};
            }
        // per-tile domain: the 128-row tiles of A and B this wave's block lies
        // in (a block wholly past row M, never stored, reads the last tile row)
        const int mt = min((m0 >> 7) + wm, (M - 1) >> 7), nt = n0 >> 7;

        uint32_t off_cur = 0, off_nxt = gStageBytes, off_n2 = 2 * gStageBytes, off_dma = 3 * gStageBytes;
        for (int ks = 0; ks < nk; ++ks) {
            // stage ks+1 has landed for every wave, and every wave is done
            // with stage ks-1 (read in steps ks-2 and ks-1): its slot takes
            // the DMA of step ks+3
            if (ks > 0) wait_and_barrier<kDma>();
            const uint8_t *stn = lds + off_nxt;
            const uint32_t dma_addr = lds_base + off_dma;
            const uint32_t more = dstep < nk - 1 ? 1u : 0u;
            // per-tile domain: this K tile's factor S_A(mt, ks) * S_B(nt, ks)
            const float fold = kTile ? Ats[mt * nk + ks] * Bts[nt * nk + ks] : 1.0f;
            constexpr int kSlots = 4 * NJ;  // MFMAs per slice
            // 8 slices of kSlots MFMAs; slice s+1 is dequantized while slice s runs
            static_for<8>([&](auto s_tag) {
                constexpr int s = decltype(s_tag)::value;
                constexpr int sn = s + 1;  // the slice being prepared (8 = slice 0 of step ks+1)
                static_for<kSlots>([&](auto t_tag) {
                    constexpr int t = decltype(t_tag)::value;
                    constexpr int i = t / NJ, j = t % NJ;
                    if constexpr (kTile && s == 0)  // a fresh partial sum per K tile
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], (v16f_t){}, 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
                    // an opaque use keeps each MFMA in its slot (the compiler
                    // would sink some below the DMA and dequantization of the
                    // following slots)
                    asm volatile("" ::"a"(acc[i][j]));
                    // DMA of step ks+3: two instructions per slice from slice 0 on
                    if constexpr (t < 2 && 2 * s + t < kDma)
                        dma_piece(dma_addr, std::integral_constant<int, 2 * s + t>{});
                    // next step's operands: q = 0 chunks and scale words once
                    // the current q = 0 chunks are consumed (slice 3 was
                    // prepared during slice 2), q = 1 chunks at the start of
                    // the next step (this step's slice 7 was prepared during
                    // slice 6)
                    if constexpr (s == 4 && t < 4) {
                        rawA[t][0] = code_chunk(stn, 0, t, 0);
                        nswA[t] = scale_word(stn, 0, t);
                    }
                    if constexpr (s == 4 && t >= 4 && t < 4 + NJ) {
                        rawB[t - 4][0] = code_chunk(stn, 1, t - 4, 0);
                        nswB[t - 4] = scale_word(stn, 1, t - 4);
                    }
                    if constexpr (s == 0 && t >= kSlots - 4 - NJ && t < kSlots - NJ) {
                        if (ks > 0) rawA[t - (kSlots - 4 - NJ)][1] = code_chunk(lds + off_cur, 0, t - (kSlots - 4 - NJ), 1);
                    }
                    if constexpr (s == 0 && t >= kSlots - NJ) {
                        if (ks > 0) rawB[t - (kSlots - NJ)][1] = code_chunk(lds + off_cur, 1, t - (kSlots - NJ), 1);
                    }
                    // pointer updates after the step's last DMA
                    if constexpr (s == 6 && t < 4) {
                        if (t == 0) { pa += more * kCodeStep; asm volatile("" : "+s"(pa)); }
                        if (t == 1) { pb += more * kCodeStep; asm volatile("" : "+s"(pb)); }
                        if (t == 2) { pas += more * kScaleStep; asm volatile("" : "+s"(pas)); }
                        if (t == 3) { pbs += more * kScaleStep; asm volatile("" : "+s"(pbs)); }
                    }
                    // dequantize slice sn.  Global domain (16 slots): fragment F = t / 2 (A F / 2 for
                    // even F, B F / 2 for odd F), half t % 2 of it per slot, so that every slot's
                    // VALU work (4 instructions) fits under its MFMA; block scales of a new slice
                    // pair before a fragment's first half.  Per-tile domain (8 slots, VALU-bound
                    // either way): fragment t / 2 of A (even t) or B (odd t) in slots 0..7.
                    if constexpr (!kTile) {
                        constexpr int F = t >> 1, part = t & 1, f = F >> 1;
                        constexpr int ss = sn & 7, q = ss >> 2, d = ss & 3, h = (ss >> 1) & 1;
                        if constexpr ((F & 1) == 0) {
                            if constexpr (part == 0 && (ss & 3) == 0)
                                sAp[f] = scale_pair<(ss >= 4)>(sn == 8 ? nswA[f] : swA[f]);
                            dequant4<part>(na[f], word_of(rawA[f][q], d), bcast<h>(sAp[f]));
                        } else {
                            if constexpr (part == 0 && (ss & 3) == 0)
                                sBp[f] = scale_pair<(ss >= 4)>(sn == 8 ? nswB[f] : swB[f]);
                            dequant4<part>(nb[f], word_of(rawB[f][q], d), bcast<h>(sBp[f]));
                        }
                    } else if constexpr (t < 8 && ((t & 1) == 0 || (t >> 1) < NJ)) {
                        constexpr int f = t >> 1;
                        // block scale byte ss / 2: half (ss / 2) % 2 of the pair of bytes ss / 4
                        constexpr int ss = sn & 7, q = ss >> 2, d = ss & 3, h = (ss >> 1) & 1;
                        if constexpr ((t & 1) == 0) {
                            if constexpr ((ss & 3) == 0) sAp[f] = scale_pair<(ss >= 4)>(sn == 8 ? nswA[f] : swA[f]);
                            na[f] = dequant8(word_of(rawA[f][q], d), bcast<h>(sAp[f]));
                        } else {
                            if constexpr ((ss & 3) == 0) sBp[f] = scale_pair<(ss >= 4)>(sn == 8 ? nswB[f] : swB[f]);
                            nb[f] = dequant8(word_of(rawB[f][q], d), bcast<h>(sBp[f]));
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
#pragma unroll
                for (int f = 0; f < 4; ++f) fa[f] = na[f];
#pragma unroll
                for (int f = 0; f < NJ; ++f) fb[f] = nb[f];
            });
            if constexpr (kTile) {
                // fold this K tile's partial sum with its factor (one rounding)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            tot[kTile ? i : 0][kTile ? j : 0][r] =
                                __builtin_fmaf(fold, acc[i][j][r], tot[kTile ? i : 0][kTile ? j : 0][r]);
            }
            dstep += (int)more;
#pragma unroll
            for (int f = 0; f < 4; ++f) swA[f] = nswA[f];
#pragma unroll
            for (int f = 0; f < NJ; ++f) swB[f] = nswB[f];
            const uint32_t o = off_cur;
            off_cur = off_nxt;
            off_nxt = off_n2;
            off_n2 = off_dma;
            off_dma = o;
        }
        wait_and_barrier<0>();
        const int tm0 = m0, tn0 = n0;
        const int next = tile + (int)gridDim.x;
        if (next < ntiles) {
            setup(next);
            prologue();
        }
        uint8_t *ep = lds + (gStages - 1) * gStageBytes + wave * kEpiWaveBytes;
        int el;
        asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
        if constexpr (kTile)
            store_wave_block_any<NJ>(tot, ep, el, tm0 + wm * 128, tn0 + wn * (32 * NJ), M, N, alpha, C, ldc,
                                     c_bf16 != 0, vec_ok != 0, c_amax);
        else
            store_wave_block_any<NJ>(acc, ep, el, tm0 + wm * 128, tn0 + wn * (32 * NJ), M, N,
                                     alpha * (Ats[0] * Bts[0]), C, ldc, c_bf16 != 0, vec_ok != 0, c_amax);
        if (next >= ntiles) break;
        tile = next;
    }
}

}  // namespace

int launch_gemm_nv(const GemmArgs &g, hipStream_t st)
{
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    if (M == 0 || N == 0) return 0;
    if (K == 0) {
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(gemm::fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g.c, M, N,
                           g.ldc, (int)g.c_bf16);
        return hipGetLastError() == hipSuccess ? 0 : 1;
    }
    auto *a = reinterpret_cast<const uint8_t *>(g.a_codes);
    auto *as = reinterpret_cast<const uint8_t *>(g.a_scales);
    auto *b = reinterpret_cast<const uint8_t *>(g.b_codes);
    auto *bs = reinterpret_cast<const uint8_t *>(g.b_scales);
    const int esize = g.c_bf16 ? 2 : 4;
    const int vec_ok = ((uintptr_t)g.c % 16 == 0) && (g.ldc % (16 / esize) == 0) && g.ldc <= (int64_t(1) << 26);
    const bool tile = g.nv_domain == 1;
    const int tiles_m = (M + 255) / 256, tiles_n = tile ? (N + 127) / 128 : (N + 255) / 256;
    const int cus = device_cu_count();
    if (cus <= 0) return 1;
    const int grid = min(tiles_m * tiles_n, cus);
#define FP4Q_GEMM_NV(TILE, TIN)                                                                                 \
    hipLaunchKernelGGL((gemm_nv_fp16_kernel<TILE, TIN>), dim3(grid), dim3(256), 0, st, a, as, g.a_ts, b, bs, g.b_ts, \
                       M, N, K, g.alpha, g.c, g.ldc, (int)g.c_bf16, vec_ok, tiles_m, tiles_n, g.c_amax)
    if (tile) { if (g.tiled) FP4Q_GEMM_NV(true, true); else FP4Q_GEMM_NV(true, false); }
    else { if (g.tiled) FP4Q_GEMM_NV(false, true); else FP4Q_GEMM_NV(false, false); }
#undef FP4Q_GEMM_NV
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
