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
// MX block is therefore one lane's operand, and its scale byte is that
// lane's scale.  The B fragment is passed as the instruction's first
// operand, so register i of lane l holds C[row l mod 32][column
// 8*(i/4) + 4*(l/32) + i%4] of its 32 x 32 block: each group of four
// registers is four consecutive columns of one row.
//
// Structure: one 256-thread workgroup per CU (a persistent grid) walks
// 256 x 256 tiles of C in an XCD-aware order; each wave owns 128 x 128
// (4 x 4 instructions, 256 fp32 accumulators per lane).  K runs in 128-wide
// steps through a four-slot LDS ring filled by LDS DMA (global_load_lds)
// three steps ahead: in the tiled layout every 1 KiB block of codes is one
// instruction's operand in lane order, copied as is, and the scale words are
// copied with rows permuted so that a wave reads its four words of a step in
// one 16-byte LDS read.  The next tile's first steps are put in flight
// before the finished tile's epilogue (gemm_common.h) runs.  The linear
// layout takes the same kernel with per-lane DMA addresses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp4q_device.h"
#include "fp4q_internal.h"
#include "gemm_common.h"

namespace fp4q {

namespace {

using namespace gemm;

typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256;
constexpr int kStages = 4;                                  // LDS ring depth (K steps in flight)
constexpr int kCodeBytes = kBM * 64;                        // one operand's codes per 128-wide K step
constexpr int kScaleOff = 2 * kCodeBytes;                   // A scales, then B scales (u32 per row)
constexpr int kStageBytes = 2 * kCodeBytes + (kBM + kBN) * 4;  // 34 KiB
constexpr int kRingBytes = kStages * kStageBytes;           // 136 KiB
// The epilogue stages its chunks in the last ring slot, which the next
// tile's prologue (K steps 0 .. kStages-2) leaves free.
static_assert(4 * kEpiWaveBytes <= kStageBytes, "epilogue staging must fit in one ring slot");
constexpr int kLdsBytes = kRingBytes;
constexpr int kDmaPerStage = 10;                            // DMA instructions per wave per stage
constexpr int kDmaA = kDmaPerStage / 2;                    // DMA instructions in phase A; the rest in phase B
constexpr int kDmaB = kDmaPerStage - kDmaA;

// Persistent kernel: one workgroup per CU walks tiles b, b + G, b + 2G, ...
// (G = grid size).  Each tile: 256 x 256 outputs, four waves of 128 x 128.
// Between two tiles the next tile's first two K steps are put in flight
// before the finished tile's epilogue runs, so the epilogue hides the start
// latency of the next tile.
// kOut: 0 writes C (bf16 or fp32); 1 writes C as an MXFP4 operand along
// rows; 2 writes SwiGLU(C) (gate and up columns interleaved in groups of 32)
// as an MXFP4 operand along rows.
template <bool kTiled, int kOut>
__global__ __launch_bounds__(256) void gemm_mx_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                      const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                      int M, int N, int K, float alpha, void *__restrict__ C,
                                                      int64_t ldc, int c_bf16, int vec_ok, int tiles_m, int tiles_n,
                                                      uint32_t *__restrict__ c_amax, uint8_t *__restrict__ q_codes,
                                                      uint8_t *__restrict__ q_scales, int q_tiled)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: keeps LDS addresses scalar
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t KB = (uint32_t)K >> 1;  // code bytes per row
    const uint32_t KS = (uint32_t)K >> 5;  // scale bytes per row
    const int nk = K >> 7;                 // 128-wide K steps
    const uint32_t Mp = ((uint32_t)M + 31) & ~31u, Np = ((uint32_t)N + 31) & ~31u;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    const int ntiles = tiles_m * tiles_n;
    const uint32_t code_step = kTiled ? 2048u : 64u;

    // Per-tile DMA sources.  LDS image of a stage: the codes of 32 rows x 64 K
    // elements are one 1 KiB block in matrix-core lane order (lane l's 16
    // bytes = row l mod 32, K half l / 32), blocks ordered (row group g, K
    // half kk) -> 2 g + kk.  Wave w copies blocks 4w .. 4w+3 of A and of B
    // and 64 scale words of each operand.  The scale words are stored so that
    // the four a consuming lane needs (rows 32 i + l mod 32 of its 128-row
    // block, i = 0..3) are one 16-byte read: word 4 f + i of 128-row block c
    // holds row 128 c + 32 i + f, so lane l of wave w's copy takes row
    // 128 (w / 2) + 32 (l mod 4) + 16 (w mod 2) + l / 4.  In the tiled layout a block is
    // 1 KiB of contiguous global memory; in the linear layout lane l of block
    // b reads row 32 (b / 2) + l mod 32, bytes 32 (b mod 2) + 16 (l / 32) of
    // the step.  Rows past the operand re-read its last row (linear) or row
    // group (tiled); their results are never stored.
    uint32_t a_goff[4], b_goff[4], as_goff, bs_goff, as_step, bs_step;
    int m0 = 0, n0 = 0;
    // Scalar sources of the K step the next DMA copies (dstep): advanced by
    // one step after each step's DMA, never past the last step, so a
    // pipeline running past the end re-reads the last step.
    const uint8_t *pa = A, *pb = B, *pas = As, *pbs = Bs;
    int dstep = 0;
    auto setup = [&](int tile) {
        int tm, tn;
        tile_coords(tile, tiles_m, tiles_n, tm, tn);
        m0 = tm * kBM;
        n0 = tn * kBN;
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
        const int srow = 128 * (wave >> 1) + 32 * (lane & 3) + 16 * (wave & 1) + (lane >> 2);
        if (kTiled) {
            as_goff = min((uint32_t)(m0 + srow), Mp - 1) * 4;
            bs_goff = min((uint32_t)(n0 + srow), Np - 1) * 4;
            as_step = Mp * 4;
            bs_step = Np * 4;
        } else {
            as_goff = (uint32_t)min(m0 + srow, M - 1) * KS;
            bs_goff = (uint32_t)min(n0 + srow, N - 1) * KS;
            as_step = bs_step = 4;
        }
        pa = A;
        pb = B;
        pas = As;
        pbs = Bs;
        dstep = 0;
    };
    // the d-th of this wave's 10 DMA instructions of a step, into the stage
    // at LDS address slot_addr
    auto dma_piece = [&](uint32_t slot_addr, auto d_tag) {
        constexpr int d = decltype(d_tag)::value;
        const uint32_t wslot = slot_addr + wave * 4096;  // this wave's 4 KiB of each operand's codes
        if constexpr (d < 8) {
            constexpr int i = d >> 1;
            if constexpr ((d & 1) == 0)
                dma16<i * 1024>(pa, a_goff[i], wslot);
            else
                dma16<kCodeBytes + i * 1024>(pb, b_goff[i], wslot);
        } else if constexpr (d == 8) {
            dma4<kScaleOff>(pas, as_goff, slot_addr + wave * 256);
        } else {
            dma4<kScaleOff + kBM * 4>(pbs, bs_goff, slot_addr + wave * 256);
        }
    };
    // Branch-free (a branch here would let the compiler sink the MFMAs of
    // the step below it, out of their interleaved slots); the K loop spreads
    // the four pointer updates over separate MFMA slots.
    auto advance_ptr = [&](int which, uint32_t more) {
        if (which == 0) {
            pa += more * code_step;
            asm volatile("" : "+s"(pa));
        }
        if (which == 1) {
            pb += more * code_step;
            asm volatile("" : "+s"(pb));
        }
        if (which == 2) {
            pas += more * as_step;
            asm volatile("" : "+s"(pas));
        }
        if (which == 3) {
            pbs += more * bs_step;
            asm volatile("" : "+s"(pbs));
        }
    };
    auto advance = [&]() {
        const uint32_t more = dstep < nk - 1 ? 1u : 0u;
        for (int w = 0; w < 4; ++w) advance_ptr(w, more);
        dstep += (int)more;
    };
    // a tile's first two K steps, into ring slots 0 and 1
    auto prologue = [&]() {
#pragma unroll
        for (int s2 = 0; s2 < kStages - 1; ++s2) {
            const uint32_t slot_addr = lds_base + s2 * kStageBytes;
            static_for<kDmaPerStage>([&](auto d) { dma_piece(slot_addr, d); });
            advance();
        }
    };

    auto frag = [&](const uint8_t *st, int operand, int i, int kk) -> v8i_t {
        const int g = operand == 0 ? wm * 4 + i : wn * 4 + i;
        const uint4 t = *reinterpret_cast<const uint4 *>(st + operand * kCodeBytes + (g * 2 + kk) * 1024 + lane * 16);
        return (v8i_t){(int)t.x, (int)t.y, (int)t.z, (int)t.w, 0, 0, 0, 0};
    };
    // A lane's scale word of a 128-wide step holds the E8M0 bytes of K
    // blocks 0..3; lanes 32..63 feed the matrix cores K blocks 1 and 3, so
    // their word is shifted down one byte and both halves select byte 0
    // (K half 0) or byte 2 (K half 1) with the instruction's byte select.
    auto scale_words = [&](const uint8_t *st, int operand) -> uint4 {
        const int c = operand == 0 ? wm : wn;
        return *reinterpret_cast<const uint4 *>(st + kScaleOff + operand * kBM * 4 + (c * 128 + fr * 4) * 4);
    };

    v16f_t acc[4][4];
    v8i_t fa0[4], fb0[4], fa1[4], fb1[4];
    uint32_t sa[4], sb[4], nsa[4], nsb[4];

    // The previous tile's bf16 epilogue issued exactly kEpiStores stores after
    // this tile's prologue (full block, no amax; wave-uniform): the waits of
    // this tile's first two K steps then allow that many more outstanding
    // vector-memory instructions, so the stores drain while the matrix cores
    // run instead of before the first step (the counter completes in issue
    // order; from step 2 on the stores are older than the awaited DMA).
    constexpr int kEpiStores = kEpiStoresBf16Full<4>;
    int stores_pending = 0;
    int tile = blockIdx.x;
    setup(tile);
    prologue();
    for (;;) {
        // stage 0 of this tile has landed: loads complete in issue order, so
        // once at most (kStages-2) stages' DMA instructions (plus the
        // previous tile's pending stores) are outstanding the oldest stage is
        // in LDS
        wait_and_barrier_if<(kStages - 2) * kDmaPerStage, kEpiStores>(stores_pending);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa0[i] = frag(lds, 0, i, 0);
            fb0[i] = frag(lds, 1, i, 0);
        }
        {
            const uint4 wa = scale_words(lds, 0), wb = scale_words(lds, 1);
            sa[0] = wa.x >> (8 * fh); sa[1] = wa.y >> (8 * fh); sa[2] = wa.z >> (8 * fh); sa[3] = wa.w >> (8 * fh);
            sb[0] = wb.x >> (8 * fh); sb[1] = wb.y >> (8 * fh); sb[2] = wb.z >> (8 * fh); sb[3] = wb.w >> (8 * fh);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = (v16f_t){};

        // Software pipeline.  A 128-wide K step is two 64-wide halves
        // (kk = 0, 1); its fragments are read from LDS one half ahead of the
        // matrix cores and every memory instruction is issued between two
        // MFMAs, so LDS reads, DMA issue and MFMAs overlap:
        //   phase A of step ks: MFMAs of half 0 (operands in registers),
        //     interleaved with half of the DMA of step ks+3 (into the slot of
        //     step ks-1, free since the previous barrier) and the LDS reads
        //     of half 1 of step ks;
        //   barrier: step ks+1 has landed in LDS for every wave;
        //   phase B: MFMAs of half 1, interleaved with the rest of the DMA of
        //     step ks+3 and the LDS reads of half 0 and the scales of ks+1.
        // The DMA runs three steps ahead: the K slices of all workgroups on
        // an XCD are requested together, so every one of them waits for the
        // full HBM latency of the first request of a slice.
        // Ring slots rotate through four scalar offsets (current step, the
        // two next steps, DMA target) so that every LDS address is a scalar plus a
        // constant.
        static_assert(kStages == 4, "the slot rotation below is written for four slots");
        uint32_t off_cur = 0, off_nxt = kStageBytes, off_n2 = 2 * kStageBytes, off_dma = 3 * kStageBytes;
        for (int ks = 0; ks < nk; ++ks) {
            const uint8_t *st = lds + off_cur;
            const uint8_t *stn = lds + off_nxt;  // a re-read copy past the end
            const uint32_t dma_addr = lds_base + off_dma;
            static_for<16>([&](auto t_tag) {
                constexpr int t = decltype(t_tag)::value;
                constexpr int i = t >> 2, j = t & 3;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb0[j], fa0[i], acc[i][j], 4, 4, 0,
                                                                             (int)sb[j], 0, (int)sa[i]);
                // an opaque use keeps each MFMA in its slot: left alone, the
                // compiler sinks the first MFMAs of a phase below the DMA and
                // LDS reads of the following slots
                asm volatile("" ::"a"(acc[i][j]));
                if constexpr (t < kDmaA) dma_piece(dma_addr, t_tag);
                if constexpr (t < 4) fa1[t] = frag(st, 0, t, 1);
                else if constexpr (t < 8) fb1[t - 4] = frag(st, 1, t - 4, 1);
                __builtin_amdgcn_sched_barrier(0);
            });
            // step ks+1's DMA was issued two steps ago; after it only step
            // ks+2's DMA and this step's first kDmaA instructions may
            // still be in flight
            wait_and_barrier_if<(kStages - 3) * kDmaPerStage + kDmaA, kEpiStores>(ks < 2 ? stores_pending : 0);
            const uint32_t more = dstep < nk - 1 ? 1u : 0u;
            static_for<16>([&](auto t_tag) {
                constexpr int t = decltype(t_tag)::value;
                constexpr int i = t >> 2, j = t & 3;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb1[j], fa1[i], acc[i][j], 4, 4, 2,
                                                                             (int)sb[j], 2, (int)sa[i]);
                asm volatile("" ::"a"(acc[i][j]));
                if constexpr (t < kDmaB)
                    dma_piece(dma_addr, std::integral_constant<int, kDmaA + t>{});
                // next step's operands, in the order phase A consumes them,
                // two per slot so they land well before the phase ends
                // the scale words first: LDS reads return in order, so the
                // shifts below then wait on these two reads only
                if constexpr (t == 0) {
                    const uint4 wb = scale_words(stn, 1), wa = scale_words(stn, 0);
                    nsb[0] = wb.x; nsb[1] = wb.y; nsb[2] = wb.z; nsb[3] = wb.w;
                    nsa[0] = wa.x; nsa[1] = wa.y; nsa[2] = wa.z; nsa[3] = wa.w;
                }
                if constexpr (t < 8) {
                    constexpr int q = t >> 1;
                    if constexpr ((t & 1) == 0)
                        fb0[q] = frag(stn, 1, q, 0);
                    else
                        fa0[q] = frag(stn, 0, q, 0);
                }
                // lanes 32..63 take the odd K blocks: shift their scale
                // words down one byte, well after the reads were issued
                // (the empty asm statements pin each update to its slot: the
                // compiler would otherwise fold it into the loop's back edge)
                if constexpr (t >= 8) {
                    constexpr int q = (t - 8) >> 1;
                    if constexpr ((t & 1) == 0) {
                        nsb[q] >>= 8 * fh;
                        asm volatile("" : "+v"(nsb[q]));
                    } else {
                        nsa[q] >>= 8 * fh;
                        asm volatile("" : "+v"(nsa[q]));
                    }
                }
                if constexpr (t >= kDmaB && t < kDmaB + 4) advance_ptr(t - kDmaB, more);
                __builtin_amdgcn_sched_barrier(0);
            });
            dstep += (int)more;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa[i] = nsa[i];
                sb[i] = nsb[i];
            }
            const uint32_t o = off_cur;
            off_cur = off_nxt;
            off_nxt = off_n2;
            off_n2 = off_dma;
            off_dma = o;
        }
        // the ring is idle: every DMA landed, every wave finished its reads
        wait_and_barrier<0>();
        const int tm0 = m0, tn0 = n0;
        const int next = tile + (int)gridDim.x;
        if (next < ntiles) {
            setup(next);
            prologue();
        }

        // Epilogue (store_wave_block): the B fragment is the matrix cores'
        // first operand, so the accumulators hold row pieces; staged through
        // LDS in the ring slot the prologue left free.
        uint8_t *ep = lds + (kStages - 1) * kStageBytes + wave * kEpiWaveBytes;
        const int row_base = tm0 + wm * 128, col_base = tn0 + wn * 128;
        // Lane-derived offsets are recomputed per tile from an opaque copy of
        // the lane index: hoisted out of the tile loop they would stay live
        // across the K loop and spill to scratch, whose reloads wait on the
        // whole vector-memory counter (the next tile's DMA included).
        int el;
        asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
        if constexpr (kOut == 1)  // C leaves as the next GEMM's MXFP4 operand
            store_wave_block_mxq_any(acc, el, row_base, col_base, M, N, q_tiled ? (int)Mp : M, alpha, q_codes,
                                     q_scales, q_tiled != 0);
        else if constexpr (kOut == 2)  // so does SwiGLU(C), N / 2 columns wide
            store_wave_block_swiglu_mxq_any(acc, el, row_base, col_base >> 1, M, N >> 1, q_tiled ? (int)Mp : M, alpha,
                                            q_codes, q_scales, q_tiled != 0);
        else
            store_wave_block_any(acc, ep, el, row_base, col_base, M, N, alpha, C, ldc, c_bf16 != 0, vec_ok != 0,
                                 c_amax);
        // the full-block condition of store_wave_block_any, as a scalar
        stores_pending = __builtin_amdgcn_readfirstlane(
            (kOut == 0 && c_bf16 && !c_amax && vec_ok && row_base + 128 <= M && col_base + 128 <= N) ? 1 : 0);
        if (next >= ntiles) break;
        tile = next;
    }
}

}  // namespace

int launch_gemm_mx(const GemmArgs &g, hipStream_t st)
{
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    if (M == 0 || N == 0) return 0;
    auto *q_codes = reinterpret_cast<uint8_t *>(g.q_codes);
    auto *q_scales = reinterpret_cast<uint8_t *>(g.q_scales);
    if (K == 0 && q_codes) {  // C = 0 and SwiGLU(0) = 0: zero codes and scales
        const int64_t ms = g.q_tiled ? (M + 31) / 32 * 32 : M;
        const int64_t cols = g.q_swiglu ? N / 2 : N;  // the quantized output's width
        const int64_t nc = ms * cols / 2, ns = ms * cols / 32;
        hipLaunchKernelGGL(fill_bytes_zero_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, st, q_codes, nc);
        hipLaunchKernelGGL(fill_bytes_zero_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, q_scales, ns);
        return hipGetLastError() == hipSuccess ? 0 : 1;
    }
    if (K == 0) {
        const int64_t n = (int64_t)M * N;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g.c, M, N, g.ldc,
                           (int)g.c_bf16);
        return hipGetLastError() == hipSuccess ? 0 : 1;
    }
    const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    const int esize = g.c_bf16 ? 2 : 4;
    // 16-byte output stores need a 16-byte aligned C and ldc; the fast
    // epilogue also keeps a lane's in-chunk byte offset in 32 bits
    const int vec_ok = ((uintptr_t)g.c % 16 == 0) && (g.ldc % (16 / esize) == 0) && g.ldc <= (int64_t(1) << 26);
    auto *a = reinterpret_cast<const uint8_t *>(g.a_codes);
    auto *as = reinterpret_cast<const uint8_t *>(g.a_scales);
    auto *b = reinterpret_cast<const uint8_t *>(g.b_codes);
    auto *bs = reinterpret_cast<const uint8_t *>(g.b_scales);
    // persistent grid: one workgroup per CU (the kernel's 136 KiB of LDS
    // allows no more), never more workgroups than tiles
    const int cus = device_cu_count();
    if (cus <= 0) return 1;
    const int grid = min(tiles_m * tiles_n, cus);
#define FP4Q_GEMM_MX(T, Q)                                                                                     \
    hipLaunchKernelGGL((gemm_mx_kernel<T, Q>), dim3(grid), dim3(256), 0, st, a, as, b, bs, M, N, K, g.alpha, g.c, \
                       g.ldc, (int)g.c_bf16, vec_ok, tiles_m, tiles_n, g.c_amax, q_codes, q_scales, (int)g.q_tiled)
    const int out = !q_codes ? 0 : g.q_swiglu ? 2 : 1;
    if (g.tiled) {
        if (out == 2) FP4Q_GEMM_MX(true, 2); else if (out == 1) FP4Q_GEMM_MX(true, 1); else FP4Q_GEMM_MX(true, 0);
    } else {
        if (out == 2) FP4Q_GEMM_MX(false, 2); else if (out == 1) FP4Q_GEMM_MX(false, 1); else FP4Q_GEMM_MX(false, 0);
    }
#undef FP4Q_GEMM_MX
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
