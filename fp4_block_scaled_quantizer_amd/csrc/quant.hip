// quant.hip -- FP4 quantization producers for gfx950 (MXFP4, MXFP4 with the
// fixed-sign Hadamard-32, the dual-output MX producer, NVFP4 global -- two
// passes, or one with a given amax -- and per-128x128-tile domains).
//
// Pages cited (titles as printed):
//   [Fusion] "Format-Aware Fusion: The Engineering Practice That Doubles FP4
//            Pretraining Throughput"
//   [Stack]  "FP4 Is No Longer Just a Hardware Feature -- The NVFP4 Software
//            Stack Is Taking Shape"
//
// Each producer is one pass over the bf16 input: block amax -> scale ->
// divide -> E2M1 -> pack -> store, with nothing materialised in between
// ([Stack] section "The first change: PyTorch is bringing FP4 packing into
// compiler fusion" describes the unfused chain this avoids).  The kernels are
// HBM-bound: 2 bytes read and 0.53 (MX) / 0.56 (NV) bytes written per element.
//
// Work split (along rows): a lane owns 8 consecutive elements (one 16-byte
// load of bf16, one 4-byte store of codes).  Four lanes make an MX block of 32
// and two lanes an NV block of 16; block maxima are combined with cross-lane
// exchanges inside the wavefront.  Consecutive lanes read consecutive 16-byte
// chunks, so every wavefront load is a contiguous 1 KiB.  In the tiled
// (consumer) layout a workgroup assembles whole 1 KiB matrix-core blocks in
// LDS and writes them out contiguously; along columns a 128 x 128 tile is
// staged in LDS and transposed there.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerThread = 4;  // 16-byte chunks per lane per launch slot
// The global-domain NVFP4 quantize pass: chunks per lane.  Each workgroup
// first folds every partial maximum and fills its decode table, so it is
// given more input to amortize that over.
constexpr int kNvgChunks = 8;

// Cross-lane exchange inside a quad of lanes (DPP quad_perm): mask 1 swaps
// lanes 0<->1 and 2<->3, mask 2 swaps 0<->2 and 1<->3.
template <int kMask>
__device__ __forceinline__ uint32_t quad_xor(uint32_t v)
{
    static_assert(kMask == 1 || kMask == 2, "quad exchange");
    constexpr int ctrl = kMask == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, false);
}
template <int kMask>
__device__ __forceinline__ uint32_t xor_max(uint32_t v)
{
    return max(v, quad_xor<kMask>(v));
}
template <int kMask>
__device__ __forceinline__ float xor_get(float v)
{
    return u2f(quad_xor<kMask>(f2u(v)));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming loads of the bf16 input: each byte is read once, so the loads
// carry the non-temporal hint.
__device__ __forceinline__ uint4 load_nt16(const uint16_t *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt8(const uint16_t *p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
}

// E2M1 round-to-nearest-even of x / scale for 8 values, by gfx950's scaled
// FP4 convert (2 values per instruction, element 2j in the low nibble of byte
// j).  scale must be an exact power of two 2^E.  For such scales the
// instruction equals the E2M1 RNE rule of this library (ties to even,
// saturation at 6, sign kept on zero) bit for bit for every finite input:
// all 65536 bf16 patterns, and binary32 values with random low mantissa
// bits, were compared with the CPU reference for every E in [-127, 127].
__device__ __forceinline__ uint32_t cvt8_bf16(const uint4 &q, float scale)
{
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, q.x), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, q.y), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, q.z), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, q.w), scale, 3);
    return r;
}


// Largest |bf16| bit pattern (15 bits) among the 8 values of a chunk: the
// sign bits cleared in each word, then packed 16-bit maxima (v_pk_max_u16,
// two values per instruction) and one max of the two halves.
__device__ __forceinline__ uint32_t amax8_bf16(const uint4 &q)
{
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    const u16x2_t a = __builtin_bit_cast(u16x2_t, q.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2_t, q.y & 0x7FFF7FFFu);
    const u16x2_t c = __builtin_bit_cast(u16x2_t, q.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2_t, q.w & 0x7FFF7FFFu);
    const u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// The 8 bf16 of a chunk as binary32.
__device__ __forceinline__ void unpack8(const uint4 &q, float f[8])
{
    f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x);
    f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
    f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z);
    f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
}

// Butterfly stages of span 1, 2, 4 inside the lane's 8 elements, then 8 and
// 16 across the lanes of the quad (lane bit 0 and bit 1), in the fixed
// order of the fixed-sign Hadamard-32 ([Fusion] section "Two Key Numerical
// Techniques"): (a, b) -> (a + b, a - b) with a the lower index.
__device__ __forceinline__ void hadamard32_quad(float f[8], uint32_t sign_bits8, int quad_lane)
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if ((sign_bits8 >> i) & 1u) f[i] = -f[i];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & h) continue;
            const float a = f[i], b = f[i + h];
            f[i] = a + b;
            f[i + h] = a - b;
        }
    }
#pragma unroll
    for (int bit = 0; bit < 2; ++bit) {
        const bool upper = (quad_lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = bit == 0 ? xor_get<1>(f[i]) : xor_get<2>(f[i]);
            f[i] = upper ? (p - f[i]) : (f[i] + p);
        }
    }
}

// ------------------------------------------------------------------
// MXFP4 along rows (optionally Hadamard-32 first, optionally SR)
// ------------------------------------------------------------------
template <bool kSR, bool kHad, bool kContig>
__global__ __launch_bounds__(kThreads) void quant_mx_rows_kernel(const uint16_t *__restrict__ x, uint32_t K,
                                                                 uint32_t ld, uint32_t nchunks,
                                                                 uint32_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales, uint32_t seed_lo,
                                                                 uint32_t seed_hi, uint32_t stream_id,
                                                                 uint32_t sign_mask)
{
    const uint32_t cpr = K >> 3;  // 16-byte chunks per row
    // chunk indices in 64 bits for the bounds test: nchunks may lie within a
    // workgroup's span of 2^32, where a 32-bit index would wrap below it
    const uint64_t base = (uint64_t)blockIdx.x * (kThreads * kChunksPerThread) + threadIdx.x;
    const int quad_lane = threadIdx.x & 3;
    uint4 q[kChunksPerThread];
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
        const uint32_t c = (uint32_t)(base + i * kThreads);
        q[i] = make_uint4(0u, 0u, 0u, 0u);
        if (base + i * kThreads < nchunks) {
            size_t off;
            if (kContig) {
                off = (size_t)c * 8;
            } else {
                const uint32_t r = c / cpr;
                off = (size_t)r * ld + (size_t)(c - r * cpr) * 8;
            }
            q[i] = load_nt16(x + off);
        }
    }
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
        const uint32_t c = (uint32_t)(base + i * kThreads);
        const bool valid = base + i * kThreads < nchunks;
        uint32_t packed = 0, sbyte;
        if (!kHad && !kSR) {
            // bf16 straight into the scaled convert: no binary32 unpack
            uint32_t amax = amax8_bf16(q[i]);
            amax = xor_max<1>(amax);
            amax = xor_max<2>(amax);
            sbyte = mx_scale_byte(amax << 16);
            packed = cvt8_bf16(q[i], mx_scale_f32(sbyte));
        } else {
            float f[8];
            unpack8(q[i], f);
            if (kHad) hadamard32_quad(f, (sign_mask >> (8 * quad_lane)) & 0xFFu, quad_lane);
            uint32_t amax = 0;
            if (kHad) {
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = max(amax, f2u(f[j]) & 0x7FFFFFFFu);
            } else {
                amax = amax8_bf16(q[i]) << 16;  // the values are still the bf16 inputs
            }
            amax = xor_max<1>(amax);
            amax = xor_max<2>(amax);
            sbyte = mx_scale_byte(amax);
            if (kSR) {
                const float inv = mx_inv_scale(sbyte);
                const uint32_t r = c / cpr;
                const uint32_t c8 = c - r * cpr;
                uint32_t w[4];
                philox4x32_10(c8, r, stream_id, 0u, seed_lo, seed_hi, w);
                float y[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) y[j] = f[j] * inv;
                packed |= e2m1_sr8(y, w);
            } else {
                packed = cvt8_f32(f, mx_scale_f32(sbyte));
            }
        }
        if (valid) {
            __builtin_nontemporal_store(packed, codes + c);
            if (quad_lane == 0) scales[c >> 2] = (uint8_t)sbyte;
        }
    }
}

// One 8-element chunk of an MX operand along rows, encoded by a quad of lanes
// (the four chunks of a 32-element block sit in lanes 4m .. 4m+3): returns
// the packed codes of the chunk and sets the block's scale byte.  Every lane
// of the wavefront must call it (the block amax is a quad shuffle).  `chunk`
// is the chunk's index along K and `row` its row in the logical operand (the
// SR counter), as in the row kernels.
template <bool kSR>
__device__ __forceinline__ uint32_t encode_row_chunk(const uint4 &q, uint32_t row, uint32_t chunk, uint32_t stream_id,
                                                     uint32_t seed_lo, uint32_t seed_hi, uint32_t &sbyte)
{
    if (!kSR) {
        uint32_t amax = amax8_bf16(q);
        amax = xor_max<1>(amax);
        amax = xor_max<2>(amax);
        sbyte = mx_scale_byte(amax << 16);
        return cvt8_bf16(q, mx_scale_f32(sbyte));
    }
    float f[8];
    unpack8(q, f);
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = max(amax, f2u(f[j]) & 0x7FFFFFFFu);
    amax = xor_max<1>(amax);
    amax = xor_max<2>(amax);
    sbyte = mx_scale_byte(amax);
    const float inv = mx_inv_scale(sbyte);
    uint32_t w[4];
    philox4x32_10(chunk, row, stream_id, 0u, seed_lo, seed_hi, w);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = f[j] * inv;
    return e2m1_sr8(y, w);
}

// ------------------------------------------------------------------
// MXFP4 along columns: the logical operand is x^T, blocks run down 32 rows of
// one column of x.  A workgroup owns 128 rows (4 blocks along K) x 128
// columns.  It reads the tile with row-contiguous 16-byte loads (256 bytes
// of each row), stages it in LDS, and then each thread quantizes two
// adjacent columns of one 32-row block, reading them as 32-bit words down
// the block (a wavefront reads 256 contiguous bytes of one staged row per
// instruction, so neither phase has bank conflicts).  Each (output row,
// block) gives 16 bytes of codes: in the tiled layout the thread's two
// columns are adjacent lane slots of one 1 KiB block, and the 4 scale bytes
// of an output row form one 32-bit word, assembled in LDS and written 128
// words at a time.
// ------------------------------------------------------------------
constexpr int kColTile = 128;            // rows and columns of a workgroup tile
constexpr int kColPitch = kColTile * 2;  // bytes per staged row

// Thread t's share of the 128 x 128 tile at (r0, c0) of x (rows >= 1,
// cols % 4 == 0): 8 passes of 16 rows, thread = (row t / 16, 16-byte chunk
// t mod 16); zeros outside the operand.  With cols % 8 == 0 a chunk is full
// or empty, and the eight loads are issued unconditionally from clamped
// in-bounds addresses (row rows - 1, the row's first chunk) and masked
// afterwards: a load under a branch is waited for inside the branch, which
// serialized them.  Otherwise a row's last chunk may be half full and the
// guarded loads are kept.
__device__ __forceinline__ void load_col_tile(const uint16_t *__restrict__ x, uint32_t rows, uint32_t cols,
                                              uint32_t ld, uint32_t r0, uint32_t c0, uint4 (&q)[8])
{
    const int t = threadIdx.x;
    const uint32_t rr = t >> 4, c = c0 + (t & 15) * 8;
    if ((cols & 7u) == 0) {
        const bool cv = c < cols;
#pragma unroll
        for (int p = 0; p < 8; ++p)
            q[p] = load_nt16(x + (size_t)min(r0 + p * 16 + rr, rows - 1) * ld + (cv ? c : 0u));
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const uint32_t keep = r0 + p * 16 + rr < rows && cv ? ~0u : 0u;
            q[p] = make_uint4(q[p].x & keep, q[p].y & keep, q[p].z & keep, q[p].w & keep);
        }
    } else {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const uint32_t r = r0 + p * 16 + rr;
            q[p] = make_uint4(0u, 0u, 0u, 0u);
            if (r < rows) {
                const uint16_t *src = x + (size_t)r * ld + c;
                if (c + 8 <= cols) {
                    q[p] = load_nt16(src);
                } else if (c + 4 <= cols) {  // cols % 4 == 0: a chunk is full, half or empty
                    const uint2 h = load_nt8(src);
                    q[p] = make_uint4(h.x, h.y, 0u, 0u);
                }
            }
        }
    }
}

// Dual output (kRowsOut = 1: RNE, 2: SR): while the tile is in registers
// the kernel also writes x along rows ([rows x cols], no Hadamard) to
// codes_r / scales_r, bit-identical to the row producers, so one read of x
// yields both operands a training step needs from it.  The dual launch
// requires rows and cols to be multiples of 32 (linear) or 128 (tiled).
template <bool kSR, bool kHad, bool kTiled, int kRowsOut = 0>
__global__ __launch_bounds__(kThreads) void quant_mx_cols_kernel(const uint16_t *__restrict__ x, uint32_t rows,
                                                                 uint32_t cols, uint32_t ld, uint32_t Rp,
                                                                 uint8_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales, uint32_t seed_lo,
                                                                 uint32_t seed_hi, uint32_t stream_id,
                                                                 uint32_t sign_mask,
                                                                 uint8_t *__restrict__ codes_r = nullptr,
                                                                 uint8_t *__restrict__ scales_r = nullptr,
                                                                 uint32_t stream_id_r = 0)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kColTile * kColPitch];
    __shared__ __attribute__((aligned(16))) uint8_t sc[kColTile * 4];
    const uint32_t c0 = blockIdx.x * kColTile, r0 = blockIdx.y * kColTile;
    const uint32_t span = kTiled ? Rp : cols;  // output rows; the tiled layout pads with zero rows
    const uint32_t nblk = min(4u, (rows - r0) >> 5);
    const int t = threadIdx.x;
    {
        // 8 passes of 16 rows; thread = (row t / 16, 16-byte chunk t mod 16)
        const uint32_t ch = t & 15, rr = t >> 4, c = c0 + ch * 8;
        uint4 q[8];
        load_col_tile(x, rows, cols, ld, r0, c0, q);
#pragma unroll
        for (int p = 0; p < 8; ++p) *reinterpret_cast<uint4 *>(tile + (p * 16 + rr) * kColPitch + ch * 16) = q[p];
        if constexpr (kRowsOut != 0) {
            // x along rows: chunk c / 8 of row r; lanes 4m .. 4m+3 hold one
            // 32-element block
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t r = r0 + p * 16 + rr;
                uint32_t sbyte;
                const uint32_t packed =
                    encode_row_chunk<kRowsOut == 2>(q[p], r, c >> 3, stream_id_r, seed_lo, seed_hi, sbyte);
                if (r < rows && c < cols) {
                    if (kTiled) {
                        *reinterpret_cast<uint32_t *>(codes_r + ((size_t)(r >> 5) * (cols >> 6) + (c >> 6)) * 1024 +
                                                      ((r & 31) + 32 * ((c >> 5) & 1)) * 16 + ((c >> 3) & 3) * 4) =
                            packed;
                        if ((ch & 3) == 0) scales_r[((size_t)(c >> 7) * rows + r) * 4 + ((c >> 5) & 3)] = (uint8_t)sbyte;
                    } else {
                        *reinterpret_cast<uint32_t *>(codes_r + (size_t)r * (cols >> 1) + (c >> 1)) = packed;
                        if ((ch & 3) == 0) scales_r[(size_t)r * (cols >> 5) + (c >> 5)] = (uint8_t)sbyte;
                    }
                }
            }
        }
    }
    __syncthreads();
    const uint32_t cp = t & 63, jb = t >> 6;
    const uint32_t col = c0 + 2 * cp;  // first column of the pair; cols % 4 == 0, so both or neither exist
    if (jb < nblk && col < span) {
        const uint32_t j = (r0 >> 5) + jb;  // block index along K
        float v[2][32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(tile + (jb * 32 + i) * kColPitch + cp * 4);
            v[0][i] = bf16_lo(w);
            v[1][i] = bf16_hi(w);
        }
        uint4 o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (kHad) {
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    if ((sign_mask >> i) & 1u) v[h][i] = -v[h][i];
#pragma unroll
                for (int st = 1; st < 32; st <<= 1) {
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        if (i & st) continue;
                        const float a = v[h][i], b = v[h][i + st];
                        v[h][i] = a + b;
                        v[h][i + st] = a - b;
                    }
                }
            }
            uint32_t amax = 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = max(amax, f2u(v[h][i]) & 0x7FFFFFFFu);
            const uint32_t sbyte = mx_scale_byte(amax);
            uint32_t out[4];
            if (kSR) {
                const float inv = mx_inv_scale(sbyte);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t w[4];
                    philox4x32_10(4 * j + g, col + h, stream_id, 0u, seed_lo, seed_hi, w);
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = v[h][8 * g + e] * inv;
                    out[g] = e2m1_sr8(y, w);
                }
            } else {
                const float scale = mx_scale_f32(sbyte);
#pragma unroll
                for (int g = 0; g < 4; ++g) out[g] = cvt8_f32(&v[h][8 * g], scale);
            }
            o[h] = make_uint4(out[0], out[1], out[2], out[3]);
            if (kTiled) {
                sc[(2 * cp + h) * 4 + jb] = (uint8_t)sbyte;
            } else {
                scales[(size_t)(col + h) * (rows >> 5) + j] = (uint8_t)sbyte;
            }
        }
        if (kTiled) {
            // lane slots (col mod 32) + 32 (j mod 2) of block (col / 32, j / 2): the pair is 32 contiguous bytes
            uint8_t *dst = codes + ((size_t)(col >> 5) * (rows >> 6) + (j >> 1)) * 1024 + ((col & 31) + 32 * (j & 1)) * 16;
            *reinterpret_cast<uint4 *>(dst) = o[0];
            *reinterpret_cast<uint4 *>(dst + 16) = o[1];
        } else {
            const uint32_t K2 = rows >> 1;
            *reinterpret_cast<uint4 *>(codes + (size_t)col * K2 + (size_t)j * 16) = o[0];
            *reinterpret_cast<uint4 *>(codes + (size_t)(col + 1) * K2 + (size_t)j * 16) = o[1];
        }
    }
    if (kTiled) {
        // rows % 128 == 0 in the tiled layout: the tile is exactly one 128-wide K step
        __syncthreads();
        if ((uint32_t)t < kColTile && c0 + t < span)
            *reinterpret_cast<uint32_t *>(scales + ((size_t)(r0 >> 7) * Rp + c0 + t) * 4) =
                *reinterpret_cast<const uint32_t *>(sc + t * 4);
    }
}

// ------------------------------------------------------------------
// MXFP4 along rows into the tiled layout.  A workgroup owns 32 rows x kWin K
// (kWin = 512 or 256: up to kWin / 128 K steps).  Each load instruction of a
// wavefront covers 512 contiguous elements: one row of a 512-wide window, or
// two rows of a 256-wide one (lane = 8-element chunk); the rows are
// quantized exactly like the linear kernel, the group's 1 KiB lane-order
// code blocks and its step-major scale words are assembled in LDS, then
// written out contiguously.
// ------------------------------------------------------------------
template <bool kSR, bool kHad, int kWin>
__global__ __launch_bounds__(kThreads) void quant_mx_rows_tiled_kernel(
    const uint16_t *__restrict__ x, uint32_t R, uint32_t K, uint32_t ld, uint32_t Rp, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales, uint32_t seed_lo, uint32_t seed_hi, uint32_t stream_id, uint32_t sign_mask)
{
    static_assert(kWin == 512 || kWin == 256 || kWin == 128, "window of 4, 2 or 1 K steps");
    constexpr int kRowsPerLoad = 512 / kWin;       // rows one load instruction covers
    constexpr int kLoads = 8 / kRowsPerLoad;       // load instructions per thread
    constexpr int kCodeTile = kWin * 16;           // 32 rows x kWin codes, bytes
    __shared__ __attribute__((aligned(16))) uint8_t tile[kCodeTile + kWin];
    const uint32_t g = blockIdx.y;         // 32-row group
    const uint32_t k0 = blockIdx.x * kWin; // first K of this workgroup
    const uint32_t nsteps = min((uint32_t)(kWin / 128), (K - k0) >> 7);
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int quad_lane = lane & 3;
    const uint32_t c8 = lane % (kWin / 8);  // 8-element chunk within the window
    const uint32_t sub = lane / (kWin / 8); // which row of the load instruction
    const bool kvalid = (c8 >> 4) < nsteps;
    // Unconditional loads from a clamped address (row R - 1, or a chunk of the
    // first K step, which the launch guarantees in bounds: R >= 1, K % 128 ==
    // 0, k0 < K), zeroed afterwards: a load under a branch lets the compiler
    // wait for it inside the branch, which serializes the four loads.
    uint4 q[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const uint32_t row = g * 32 + (i * 4 + wave) * kRowsPerLoad + sub;
        const uint32_t rc = min(row, R - 1), cc = kvalid ? c8 : (c8 & 15u);
        q[i] = load_nt16(x + (size_t)rc * ld + k0 + 8 * cc);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const uint32_t row = g * 32 + (i * 4 + wave) * kRowsPerLoad + sub;
        if (!(row < R && kvalid)) q[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const uint32_t rl = (i * 4 + wave) * kRowsPerLoad + sub, row = g * 32 + rl;
        uint32_t packed = 0, sbyte;
        if (!kHad && !kSR) {
            uint32_t amax = amax8_bf16(q[i]);
            amax = xor_max<1>(amax);
            amax = xor_max<2>(amax);
            sbyte = mx_scale_byte(amax << 16);
            packed = cvt8_bf16(q[i], mx_scale_f32(sbyte));
        } else {
            float f[8];
            unpack8(q[i], f);
            if (kHad) hadamard32_quad(f, (sign_mask >> (8 * quad_lane)) & 0xFFu, quad_lane);
            uint32_t amax = 0;
            if (kHad) {
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = max(amax, f2u(f[j]) & 0x7FFFFFFFu);
            } else {
                amax = amax8_bf16(q[i]) << 16;  // the values are still the bf16 inputs
            }
            amax = xor_max<1>(amax);
            amax = xor_max<2>(amax);
            sbyte = mx_scale_byte(amax);
            if (kSR) {
                const float inv = mx_inv_scale(sbyte);
                uint32_t w[4];
                philox4x32_10((k0 >> 3) + c8, row, stream_id, 0u, seed_lo, seed_hi, w);
                float y[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) y[j] = f[j] * inv;
                packed |= e2m1_sr8(y, w);
            } else {
                packed = cvt8_f32(f, mx_scale_f32(sbyte));
            }
        }
        // lane-order block (c8 / 8), slot = row + 32 * (32-element half), 4 bytes per chunk
        *reinterpret_cast<uint32_t *>(tile + (c8 >> 3) * 1024 + (rl + 32 * ((c8 >> 2) & 1)) * 16 + (c8 & 3) * 4) =
            packed;
        if (quad_lane == 0) {
            const uint32_t jb = c8 >> 2;  // MX block within the window
            tile[kCodeTile + (jb >> 2) * 128 + rl * 4 + (jb & 3)] = (uint8_t)sbyte;
        }
    }
    __syncthreads();
    uint8_t *dst = codes + ((size_t)g * (K >> 6) + (k0 >> 6)) * 1024;
    for (uint32_t o = t * 16; o < nsteps * 2048; o += kThreads * 16)
        *reinterpret_cast<uint4 *>(dst + o) = *reinterpret_cast<const uint4 *>(tile + o);
    if ((uint32_t)t < 8 * nsteps) {
        const uint32_t s = t >> 3, part = t & 7;
        *reinterpret_cast<uint4 *>(scales + ((size_t)((k0 >> 7) + s) * Rp + 32 * g) * 4 + part * 16) =
            *reinterpret_cast<const uint4 *>(tile + kCodeTile + s * 128 + part * 16);
    }
}

// ------------------------------------------------------------------
// NVFP4, global domain: pass 1 writes one partial maximum per workgroup,
// pass 2 folds them into the domain amax A, derives S and quantizes.
// ------------------------------------------------------------------
constexpr int kAmaxBlocks = 1024;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *sh)
{
    for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    uint32_t r = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = max(r, sh[w]);
    __syncthreads();
    return r;
}

// kFlat: the rows are contiguous (ld == K), so chunk c starts at element 8 c
// (no division); four 16-byte loads per thread are in flight per iteration
template <bool kFlat>
__global__ __launch_bounds__(kThreads) void nv_amax_partial_kernel(const uint16_t *__restrict__ x, uint32_t K,
                                                                   uint32_t ld, uint32_t nchunks,
                                                                   uint32_t *__restrict__ partial)
{
    __shared__ uint32_t sh[kThreads / 64];
    const uint32_t cpr = K >> 3;
    const uint32_t stride = gridDim.x * kThreads;
    auto src = [&](uint32_t c) -> const uint16_t * {
        if (kFlat) return x + (size_t)c * 8;
        const uint32_t r = c / cpr;
        return x + (size_t)r * ld + (size_t)(c - r * cpr) * 8;
    };
    uint32_t m = 0;
    grid_stride_chunks(
        blockIdx.x * kThreads + threadIdx.x, stride, nchunks,
        [&](uint32_t c) {
            const uint4 q0 = load_nt16(src(c)), q1 = load_nt16(src(c + stride));
            const uint4 q2 = load_nt16(src(c + 2 * stride)), q3 = load_nt16(src(c + 3 * stride));
            m = max(m, max(max(amax8_bf16(q0), amax8_bf16(q1)), max(amax8_bf16(q2), amax8_bf16(q3))));
        },
        [&](uint32_t c) { m = max(m, amax8_bf16(load_nt16(src(c)))); });
    m = block_max_u32(m, sh);
    if (threadIdx.x == 0) partial[blockIdx.x] = m << 16;  // binary32 bits of the partial amax
}

// One lane's 8 bf16 values (q) of a 16-element NV block shared with lane ^ 1:
// block amax (packed 16-bit maxima, then across the lane pair), E4M3 block
// scale by correction steps (nv_block_scale_fast), its decode reciprocal
// 1 / (e4m3(sb) S) from the workgroup's table inv_tab (filled with the
// correctly rounded divisions), y = x * inv and the E2M1 codes.
template <bool kSR>
__device__ __forceinline__ uint32_t nv_encode8(const uint4 &q, const NvDomain &dom, const float *inv_tab,
                                               uint32_t *sb_out, uint32_t r, uint32_t c8, uint32_t stream_id,
                                               uint32_t seed_lo, uint32_t seed_hi)
{
    const uint32_t bmax = xor_max<1>(amax8_bf16(q) << 16);  // binary32 bits of the block amax
    const uint32_t sb = nv_block_scale_fast(u2f(bmax), dom);
    const float inv = inv_tab[sb];
    float f[8], y[8];
    unpack8(q, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = f[j] * inv;
    uint32_t packed = 0;
    if (kSR) {
        uint32_t w[4];
        philox4x32_10(c8, r, stream_id, 0u, seed_lo, seed_hi, w);
        packed = e2m1_sr8(y, w);
    } else {
        packed = cvt8_f32(y, 1.0f);  // scale 2^0: plain RNE of y, saturating
    }
    *sb_out = sb;
    return packed;
}

// The decode reciprocals 1 / (e4m3(k) S) of a scale domain, k = 1 .. 126,
// correctly rounded (entry 0 is unused: block scales are at least 1).
__device__ __forceinline__ void nv_fill_inv_table(float *inv_tab, float S, int i)
{
    if (i >= 1 && i < 127) inv_tab[i] = nv_inv_decode((uint32_t)i, S);
}

// kFlat: contiguous rows (ld == K), chunk c starts at element 8 c.  The
// data loads go out first and the domain amax is reduced from the partial
// maxima while they are in flight; four scale bytes (lanes +0, +2, +4, +6:
// consecutive chunks) are gathered by DPP row shifts into one 32-bit store
// when the chunk count is a multiple of 8 and the scales are word-aligned.
// kTiled: the outputs go to the tiled consumer layout (K % 128 == 0) and the
// chunks are walked in that layout's order: chunk c is 16 chunks (one row's
// 128-element K step) of row (c >> 4) % 32 of 32-row block / K step c >> 9,
// so the codes word of chunk c lands at word c and its scale bytes at byte
// 2 c -- both output streams are written linearly, and a wave reads four
// 256-byte row pieces.  The grid also covers the padding rows up to a
// multiple of 32 (nchunks_out chunks), whose codes and scale bytes are
// written as zeros.  `by` divides by K / 8 (row split of the linear order)
// or, tiled, by K / 128 (the K steps per 32-row block).
// a readable 16-byte chunk for loads that an empty operand cannot serve
__device__ __align__(16) uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};  // never written

template <bool kSR, bool kFlat, bool kTiled>
__global__ __launch_bounds__(kThreads) void nv_quant_global_kernel(const uint16_t *__restrict__ x, uint32_t K,
                                                                   uint32_t ld, uint32_t nchunks,
                                                                   const uint32_t *__restrict__ partial,
                                                                   uint32_t npartial, uint32_t *__restrict__ codes,
                                                                   uint8_t *__restrict__ scales,
                                                                   float *__restrict__ tensor_scale,
                                                                   uint32_t seed_lo, uint32_t seed_hi,
                                                                   uint32_t stream_id, uint32_t nchunks_out,
                                                                   FastDiv by)
{
    __shared__ uint32_t sh[kThreads / 64];
    const uint32_t cpr = K >> 3;
    // chunk indices in 64 bits for the bounds tests: the chunk count may lie
    // within a workgroup's span of 2^32, where a 32-bit index would wrap
    const uint64_t base = (uint64_t)blockIdx.x * (kThreads * kNvgChunks) + threadIdx.x;
    const uint64_t cend = kTiled ? nchunks_out : nchunks;
    // The partial maxima are loaded before the data: loads complete in issue
    // order, so the domain amax, the barriers and the decode table proceed
    // while the data is in flight, and chunk i's encode waits for its own load.
    static_assert(kAmaxBlocks % kThreads == 0, "partial maxima per lane");
    // (Unconditional loads from a clamped index, npartial >= 1: a repeated
    // element does not change a maximum, and a guarded load would be waited
    // for inside its branch.)
    uint32_t pm[kAmaxBlocks / kThreads];
#pragma unroll
    for (int j = 0; j < kAmaxBlocks / kThreads; ++j) pm[j] = partial[min(threadIdx.x + j * kThreads, npartial - 1)];
    asm volatile("" ::: "memory");  // keep the data loads after these
    const uint16_t *fallback = nchunks != 0 ? x : reinterpret_cast<const uint16_t *>(kZeroChunk);
    uint4 q[kNvgChunks];
    uint32_t rows[kNvgChunks], cols[kNvgChunks];  // (row, chunk in row) of each chunk
#pragma unroll
    for (int i = 0; i < kNvgChunks; ++i) {
        const uint32_t c = (uint32_t)(base + i * kThreads);
        const bool in = base + i * kThreads < cend;
        // every load is issued (an invalid chunk reads the operand's first
        // chunk, or a zero chunk when the operand is empty, and is zeroed
        // below), so the loads' completion count is exact
        bool valid;
        const uint16_t *src;
        if (kTiled) {
            const uint32_t blk = c >> 9, rb = fast_div(blk, by);
            rows[i] = rb * 32u + ((c >> 4) & 31u);
            cols[i] = (blk - rb * (K >> 7)) * 16u + (c & 15u);
            valid = in && (uint64_t)rows[i] * cpr < nchunks;
            src = x + (size_t)rows[i] * ld + (size_t)cols[i] * 8;
        } else {
            rows[i] = 0;
            cols[i] = 0;
            if (kSR || !kFlat) {
                rows[i] = fast_div(c, by);
                cols[i] = c - rows[i] * cpr;
            }
            valid = in;
            src = kFlat ? x + (size_t)c * 8 : x + (size_t)rows[i] * ld + (size_t)cols[i] * 8;
        }
        const uint4 v = load_nt16(valid ? src : fallback);
        const uint32_t keep = valid ? ~0u : 0u;
        q[i] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
    __shared__ float inv_tab[128];
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < kAmaxBlocks / kThreads; ++j) a = max(a, pm[j]);
    a = block_max_u32(a, sh);
    const float S = nv_tensor_scale(u2f(a));
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = S;
    const NvDomain dom = nv_domain(S);
    nv_fill_inv_table(inv_tab, S, threadIdx.x);
    __syncthreads();
    const bool word_scales = kTiled || ((nchunks & 7u) == 0 && ((uintptr_t)scales & 3u) == 0);
#pragma unroll
    for (int i = 0; i < kNvgChunks; ++i) {
        const uint32_t c = (uint32_t)(base + i * kThreads);
        const bool in = base + i * kThreads < cend;
        const uint32_t r = rows[i], col = cols[i];  // stochastic rounding keys on them
        uint32_t sb;
        uint32_t packed = nv_encode8<kSR>(q[i], dom, inv_tab, &sb, r, col, stream_id, seed_lo, seed_hi);
        if (kTiled && (uint64_t)r * cpr >= nchunks) {  // a padding row
            packed = 0;
            sb = 0;
        }
        const uint32_t s2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x102, 0xF, 0xF, true);
        const uint32_t s4 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x104, 0xF, 0xF, true);
        const uint32_t s6 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x106, 0xF, 0xF, true);
        if (kTiled) {
            if (in) {  // tiled order: word c, scale bytes 2 c .. (nv_code_off / nv_scale_off)
                __builtin_nontemporal_store(packed, codes + c);
                if ((threadIdx.x & 7) == 0)  // chunks col .. col + 7: four blocks of one row and K step
                    *reinterpret_cast<uint32_t *>(scales + (c >> 1)) = sb | s2 << 8 | s4 << 16 | s6 << 24;
            }
        } else if (in) {
            __builtin_nontemporal_store(packed, codes + c);
            if (word_scales) {
                if ((threadIdx.x & 7) == 0)  // c % 8 == 0 and c + 7 < nchunks
                    *reinterpret_cast<uint32_t *>(scales + (c >> 1)) = sb | s2 << 8 | s4 << 16 | s6 << 24;
            } else if ((threadIdx.x & 1) == 0) {
                scales[c >> 1] = (uint8_t)sb;
            }
        }
    }
}

// ------------------------------------------------------------------
// NVFP4, per-128x128-tile domain ("CTA-local"): a 512-thread workgroup
// owns two horizontally adjacent tiles (128 rows x 256 K): each tile's
// amax, its S, then the codes from registers.  No grid-wide
// dependency.  Thread t handles chunk t mod 32 (tile (t mod 32) / 16) of
// rows t / 32 + 16 i (i < 8), so a row's 32 codes words are one full
// 128-byte line and the two tiles' maxima reduce over lane bits 0-3 and 5
// (then over the 8 waves through LDS).  Four scale bytes
// (lanes +0, +2, +4, +6 of the row's 32) are gathered with DPP row shifts
// and written as one 32-bit word when K % 64 == 0 and the scales are
// 4-byte aligned (word-aligned rows); else one byte per even lane.
// ------------------------------------------------------------------
constexpr int kTileThreads = 512, kTileRowsPerIter = kTileThreads / 32, kTileIters = 128 / kTileRowsPerIter;

// The quantization of tile pair (tr, tp) from this thread's 8 chunks q[i]
// (zero outside the operand).  sh: 2 * 8 words, inv_tab: two 128-entry
// tables, both in LDS; the function meets the workgroup twice.
// kTiled: outputs in the tiled consumer layout (K % 128 == 0), padding rows
// R .. Rp-1 (inside the last tile row) written as zeros.
template <bool kSR, bool kTiled>
__device__ __forceinline__ void nv_tile_pair_encode(const uint4 (&q)[kTileIters], uint32_t tr, uint32_t tp, uint32_t R,
                                                    uint32_t K, uint32_t *__restrict__ codes,
                                                    uint8_t *__restrict__ scales, float *__restrict__ tensor_scale,
                                                    uint32_t seed_lo, uint32_t seed_hi, uint32_t stream_id,
                                                    uint32_t Rp, uint32_t *sh, float (*inv_tab)[128])
{
    const uint32_t TK = (K + 127) >> 7;
    const uint32_t cpr = K >> 3;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint32_t cc = t & 31, half = cc >> 4;  // chunk within the pair, its tile
    const uint32_t c8 = tp * 32 + cc;
    const bool cvalid = c8 < cpr;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kTileIters; ++i) m = max(m, amax8_bf16(q[i]));
    // per tile: lanes with the same bit 4 (and any bits 0-3, 5) share it
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 4, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 8, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
    if (lane == 0) sh[2 * wave] = m;
    if (lane == 16) sh[2 * wave + 1] = m;
    __syncthreads();
    uint32_t tm = sh[half];
#pragma unroll
    for (int w = 1; w < kTileThreads / 64; ++w) tm = max(tm, sh[2 * w + half]);
    const float S = nv_tensor_scale(u2f(tm << 16));
    const uint32_t tk = tp * 2 + half;
    if ((t == 0 || t == 16) && tk < TK) tensor_scale[tr * TK + tk] = S;
    // decode tables of the two tiles: threads 0..127 fill tile 0's, 128..255 tile 1's
    if (t < 256) {
        const uint32_t h = (uint32_t)t >> 7;
        uint32_t th = sh[h];
#pragma unroll
        for (int w = 1; w < kTileThreads / 64; ++w) th = max(th, sh[2 * w + h]);
        nv_fill_inv_table(inv_tab[h], nv_tensor_scale(u2f(th << 16)), t & 127);
    }
    __syncthreads();
    const NvDomain dom = nv_domain(S);
    const bool word_scales = kTiled || ((K & 63u) == 0 && ((uintptr_t)scales & 3u) == 0);
#pragma unroll
    for (int i = 0; i < kTileIters; ++i) {
        const uint32_t r = tr * 128 + (t >> 5) + kTileRowsPerIter * i;
        uint32_t sb;
        uint32_t packed = nv_encode8<kSR>(q[i], dom, inv_tab[half], &sb, r, c8, stream_id, seed_lo, seed_hi);
        if (kTiled && r >= R) {  // a padding row
            packed = 0;
            sb = 0;
        }
        // scale bytes of chunks cc, cc + 2, cc + 4, cc + 6 (one per 16-element block)
        const uint32_t s2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x102, 0xF, 0xF, true);
        const uint32_t s4 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x104, 0xF, 0xF, true);
        const uint32_t s6 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x106, 0xF, 0xF, true);
        if (kTiled) {
            if (r < Rp && cvalid) {
                __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(codes) +
                                                                                 nv_code_off(r, c8, K, true)));
                if ((cc & 7) == 0)  // four blocks of one row and K step
                    *reinterpret_cast<uint32_t *>(scales + nv_scale_off(r, c8 >> 1, K, true)) =
                        sb | s2 << 8 | s4 << 16 | s6 << 24;
            }
        } else if (r < R && cvalid) {
            const size_t c = (size_t)r * cpr + c8;
            __builtin_nontemporal_store(packed, codes + c);
            if (word_scales) {
                if ((cc & 7) == 0)  // chunks c8 .. c8 + 7 lie inside the row (cpr % 8 == 0)
                    *reinterpret_cast<uint32_t *>(scales + (c >> 1)) = sb | s2 << 8 | s4 << 16 | s6 << 24;
            } else if ((cc & 1) == 0) {
                scales[c >> 1] = (uint8_t)sb;
            }
        }
    }
}

// One tile pair per workgroup (grid: pairs x tile rows), the chunks loaded
// into registers.  Unconditional loads from clamped in-bounds addresses (row
// R - 1, the row's first chunk), zeroed afterwards: a load under a branch
// lets the compiler wait for it inside the branch.
template <bool kSR, bool kTiled>
__global__ __launch_bounds__(kTileThreads) void nv_quant_tile_kernel(const uint16_t *__restrict__ x, uint32_t R,
                                                                 uint32_t K, uint32_t ld,
                                                                 uint32_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales,
                                                                 float *__restrict__ tensor_scale,
                                                                 uint32_t seed_lo, uint32_t seed_hi,
                                                                 uint32_t stream_id, uint32_t Rp)
{
    __shared__ uint32_t sh[2 * (kTileThreads / 64)];
    __shared__ float inv_tab[2][128];
    const uint32_t tr = blockIdx.y, tp = blockIdx.x;  // tile row, tile pair
    const int t = threadIdx.x;
    const uint32_t c8 = tp * 32 + (t & 31);
    const bool cvalid = c8 < (K >> 3);
    uint4 q[kTileIters];
#pragma unroll
    for (int i = 0; i < kTileIters; ++i) {
        const uint32_t r = tr * 128 + (t >> 5) + kTileRowsPerIter * i;
        q[i] = load_nt16(x + (size_t)min(r, R - 1) * ld + (size_t)(cvalid ? c8 : 0u) * 8);
    }
#pragma unroll
    for (int i = 0; i < kTileIters; ++i) {
        const uint32_t r = tr * 128 + (t >> 5) + kTileRowsPerIter * i;
        const uint32_t keep = r < R && cvalid ? ~0u : 0u;
        q[i] = make_uint4(q[i].x & keep, q[i].y & keep, q[i].z & keep, q[i].w & keep);
    }
    nv_tile_pair_encode<kSR, kTiled>(q, tr, tp, R, K, codes, scales, tensor_scale, seed_lo, seed_hi, stream_id, Rp,
                                     sh, inv_tab);
}

// ------------------------------------------------------------------
// NVFP4 along columns (the logical operand is x^T; optionally the fixed-sign
// Hadamard-32 along K first).  A workgroup owns one 128 x 128 tile of x,
// i.e. one 128 x 128 tile of the logical operand: exactly one per-tile scale
// domain.  The tile is staged in LDS as in the MX column kernel; thread t
// then holds two adjacent columns (output rows) x 32 rows (K) in registers:
// two 16-element NV blocks per column.
//   kMode 0, per-tile domain: tile amax (of the transformed values with
//            Hadamard) by a workgroup reduction -> S -> quantize.
//   kMode 1, global domain: S from the partial maxima -> quantize.
//   kMode 2, global domain with Hadamard, pass 1: the amax of the
//            transformed values of tiles blockIdx.x, + gridDim.x, ... into
//            partial[blockIdx.x].
// Requires cols % 4 == 0 and rows % 16 == 0 (rows % 32 == 0 with Hadamard).
// ------------------------------------------------------------------
// kTiled: outputs in the tiled consumer layout (rows % 128 == 0), output
// rows cols .. Rp-1 (padding up to a multiple of 32) written as zeros.
template <bool kSR, bool kHad, int kMode, bool kTiled = false>
__global__ __launch_bounds__(kThreads) void nv_quant_cols_kernel(const uint16_t *__restrict__ x, uint32_t rows,
                                                                 uint32_t cols, uint32_t ld,
                                                                 uint8_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales,
                                                                 float *__restrict__ tensor_scale,
                                                                 uint32_t *__restrict__ partial, uint32_t npartial,
                                                                 uint32_t seed_lo, uint32_t seed_hi,
                                                                 uint32_t stream_id, uint32_t sign_mask,
                                                                 uint32_t Rp = 0)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kColTile * kColPitch];
    __shared__ uint32_t sh[kThreads / 64];
    const int t = threadIdx.x;
    const uint32_t tiles_c = (cols + kColTile - 1) / kColTile, tiles_r = (rows + kColTile - 1) / kColTile;
    const uint32_t ntile = tiles_c * tiles_r;
    uint32_t run_max = 0;  // kMode 2: over this workgroup's tiles
    for (uint32_t tt = blockIdx.x; tt < ntile; tt += (kMode == 2 ? gridDim.x : ntile)) {
        const uint32_t c0 = (tt % tiles_c) * kColTile, r0 = (tt / tiles_c) * kColTile;
        if (kMode == 2 && tt != blockIdx.x) __syncthreads();  // the previous tile's LDS reads are done
        {
            const uint32_t ch = t & 15, rr = t >> 4;
            uint4 q[8];
            load_col_tile(x, rows, cols, ld, r0, c0, q);
#pragma unroll
            for (int p = 0; p < 8; ++p) *reinterpret_cast<uint4 *>(tile + (p * 16 + rr) * kColPitch + ch * 16) = q[p];
        }
        __syncthreads();
        const uint32_t cp = t & 63, jb = t >> 6;
        const uint32_t col = c0 + 2 * cp;               // output rows col, col + 1
        const uint32_t k0 = r0 + 32 * jb;               // first K of the thread's 32
        const uint32_t kvalid = k0 < rows ? min(32u, rows - k0) : 0u;  // 0, 16 or 32
        float v[2][32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(tile + (jb * 32 + i) * kColPitch + cp * 4);
            v[0][i] = bf16_lo(w);
            v[1][i] = bf16_hi(w);
        }
        if (kHad) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    if ((sign_mask >> i) & 1u) v[h][i] = -v[h][i];
#pragma unroll
                for (int st = 1; st < 32; st <<= 1) {
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        if (i & st) continue;
                        const float a = v[h][i], b = v[h][i + st];
                        v[h][i] = a + b;
                        v[h][i + st] = a - b;
                    }
                }
            }
        }
        // block maxima (rows past the end and missing columns are zeros in the
        // tile, so they never raise a maximum)
        uint32_t bmax[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) m = max(m, f2u(v[h][16 * b + i]) & 0x7FFFFFFFu);
                bmax[h][b] = m;
            }
        float S;
        if (kMode == 1) {
            uint32_t a = 0;
            for (uint32_t i = t; i < npartial; i += kThreads) a = max(a, partial[i]);
            S = nv_tensor_scale(u2f(block_max_u32(a, sh)));
            if (blockIdx.x == 0 && t == 0) *tensor_scale = S;
        } else {
            const uint32_t a = block_max_u32(max(max(bmax[0][0], bmax[0][1]), max(bmax[1][0], bmax[1][1])), sh);
            if (kMode == 2) {
                run_max = max(run_max, a);
                continue;
            }
            S = nv_tensor_scale(u2f(a));
            if (t == 0) tensor_scale[(c0 / kColTile) * tiles_r + r0 / kColTile] = S;
        }
        if (kTiled && kvalid != 0 && col >= cols && col < Rp) {
            // padding output rows of the tiled layout: zero codes and scales
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                *reinterpret_cast<uint4 *>(codes + nv_code_off(col + h, k0 >> 3, rows, true)) = make_uint4(0u, 0u, 0u, 0u);
                *reinterpret_cast<uint16_t *>(scales + nv_scale_off(col + h, k0 >> 4, rows, true)) = 0;
            }
        }
        if (kvalid == 0 || col >= cols) continue;
        const NvDomain dom = nv_domain(S);
        const uint32_t K2 = rows >> 1, K16 = rows >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t out[4], sbs = 0;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t sb = nv_block_scale_fast(u2f(bmax[h][b]), dom);
                const float inv = nv_inv_decode(sb, S);
                sbs |= sb << (8 * b);
#pragma unroll
                for (int g2 = 0; g2 < 2; ++g2) {
                    const int g = 2 * b + g2;  // 8-element group within the 32
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = v[h][8 * g + e] * inv;
                    if (kSR) {
                        uint32_t w[4];
                        philox4x32_10((k0 >> 3) + g, col + h, stream_id, 0u, seed_lo, seed_hi, w);
                        out[g] = e2m1_sr8(y, w);
                    } else {
                        out[g] = cvt8_f32(y, 1.0f);
                    }
                }
            }
            if (kTiled) {  // 32 K of one row and K step: 16 contiguous code bytes, 2 scale bytes
                *reinterpret_cast<uint4 *>(codes + nv_code_off(col + h, k0 >> 3, rows, true)) =
                    make_uint4(out[0], out[1], out[2], out[3]);
                *reinterpret_cast<uint16_t *>(scales + nv_scale_off(col + h, k0 >> 4, rows, true)) = (uint16_t)sbs;
                continue;
            }
            uint8_t *crow = codes + (size_t)(col + h) * K2 + (k0 >> 1);
            uint8_t *srow = scales + (size_t)(col + h) * K16 + (k0 >> 4);
            if (kvalid == 32 && (rows & 31u) == 0) {  // 16- and 2-byte aligned rows
                *reinterpret_cast<uint4 *>(crow) = make_uint4(out[0], out[1], out[2], out[3]);
                *reinterpret_cast<uint16_t *>(srow) = (uint16_t)sbs;
            } else {  // rows % 32 == 16: 8-byte aligned code rows, byte scales
                *reinterpret_cast<uint2 *>(crow) = make_uint2(out[0], out[1]);
                srow[0] = (uint8_t)sbs;
                if (kvalid == 32) {
                    *reinterpret_cast<uint2 *>(crow + 8) = make_uint2(out[2], out[3]);
                    srow[1] = (uint8_t)(sbs >> 8);
                }
            }
        }
    }
    if (kMode == 2 && t == 0) partial[blockIdx.x] = run_max;
    if (kMode == 1 && ntile == 0 && t == 0) *tensor_scale = 1.0f;  // an empty operand: S = 1
}

}  // namespace

// ------------------------------------------------------------------ launchers

int launch_quant_mx(const QuantArgs &a, hipStream_t st)
{
    const uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32);
    auto *x = reinterpret_cast<const uint16_t *>(a.x);
    auto *scales = reinterpret_cast<uint8_t *>(a.scales);
    if (a.axis == 0 && a.tiled) {
        const uint32_t R = (uint32_t)a.rows, K = (uint32_t)a.cols;
        if (R == 0 || K == 0) return 0;
        const uint32_t Rp = (R + 31) / 32 * 32;
        constexpr int kWin = 256;  // two K steps per workgroup: 4096 workgroups for an 8192 x 4096 input
        dim3 grid((K + kWin - 1) / kWin, Rp / 32);
        auto *codes = reinterpret_cast<uint8_t *>(a.codes);
#define FP4Q_LAUNCH_ROWS_T(SR, HAD)                                                                                  \
    hipLaunchKernelGGL((quant_mx_rows_tiled_kernel<SR, HAD, kWin>), grid, dim3(kThreads), 0, st, x, R, K,            \
                       (uint32_t)a.ld, Rp, codes, scales, seed_lo, seed_hi, a.stream_id, a.sign_mask)
        if (a.sr) { if (a.hadamard) FP4Q_LAUNCH_ROWS_T(true, true); else FP4Q_LAUNCH_ROWS_T(true, false); }
        else { if (a.hadamard) FP4Q_LAUNCH_ROWS_T(false, true); else FP4Q_LAUNCH_ROWS_T(false, false); }
#undef FP4Q_LAUNCH_ROWS_T
    } else if (a.axis == 0) {
        const uint32_t R = (uint32_t)a.rows, K = (uint32_t)a.cols;
        const uint64_t nchunks = (uint64_t)R * (K >> 3);
        if (nchunks == 0) return 0;
        const uint32_t grid = (uint32_t)((nchunks + kThreads * kChunksPerThread - 1) / (kThreads * kChunksPerThread));
        const bool contig = a.ld == a.cols;
        auto *codes = reinterpret_cast<uint32_t *>(a.codes);
#define FP4Q_LAUNCH_ROWS(SR, HAD, CONTIG)                                                                   \
    hipLaunchKernelGGL((quant_mx_rows_kernel<SR, HAD, CONTIG>), dim3(grid), dim3(kThreads), 0, st, x, K,       \
                       (uint32_t)a.ld, (uint32_t)nchunks, codes, scales, seed_lo, seed_hi, a.stream_id, a.sign_mask)
        if (a.sr) {
            if (a.hadamard) { if (contig) FP4Q_LAUNCH_ROWS(true, true, true); else FP4Q_LAUNCH_ROWS(true, true, false); }
            else { if (contig) FP4Q_LAUNCH_ROWS(true, false, true); else FP4Q_LAUNCH_ROWS(true, false, false); }
        } else {
            if (a.hadamard) { if (contig) FP4Q_LAUNCH_ROWS(false, true, true); else FP4Q_LAUNCH_ROWS(false, true, false); }
            else { if (contig) FP4Q_LAUNCH_ROWS(false, false, true); else FP4Q_LAUNCH_ROWS(false, false, false); }
        }
#undef FP4Q_LAUNCH_ROWS
    } else {
        const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
        if (rows == 0 || cols == 0) return 0;
        const uint32_t Rp = (cols + 31) / 32 * 32;
        const uint32_t span = a.tiled ? Rp : cols;
        dim3 grid((span + kColTile - 1) / kColTile, (rows + kColTile - 1) / kColTile);
        auto *codes = reinterpret_cast<uint8_t *>(a.codes);
        auto *codes_r = reinterpret_cast<uint8_t *>(a.codes_rows);
        auto *scales_r = reinterpret_cast<uint8_t *>(a.scales_rows);
#define FP4Q_LAUNCH_COLS(SR, HAD, T, RO)                                                                          \
    hipLaunchKernelGGL((quant_mx_cols_kernel<SR, HAD, T, RO>), grid, dim3(kThreads), 0, st, x, rows, cols,          \
                       (uint32_t)a.ld, Rp, codes, scales, seed_lo, seed_hi, a.stream_id, a.sign_mask, codes_r,      \
                       scales_r, a.stream_id_rows)
#define FP4Q_LAUNCH_COLS1(SR, HAD, T)                                       \
    do {                                                                    \
        if (a.rows_round == 1) FP4Q_LAUNCH_COLS(SR, HAD, T, 1);             \
        else if (a.rows_round == 2) FP4Q_LAUNCH_COLS(SR, HAD, T, 2);        \
        else FP4Q_LAUNCH_COLS(SR, HAD, T, 0);                               \
    } while (0)
#define FP4Q_LAUNCH_COLS2(SR, HAD) \
    do { if (a.tiled) FP4Q_LAUNCH_COLS1(SR, HAD, true); else FP4Q_LAUNCH_COLS1(SR, HAD, false); } while (0)
        if (a.sr) { if (a.hadamard) FP4Q_LAUNCH_COLS2(true, true); else FP4Q_LAUNCH_COLS2(true, false); }
        else { if (a.hadamard) FP4Q_LAUNCH_COLS2(false, true); else FP4Q_LAUNCH_COLS2(false, false); }
#undef FP4Q_LAUNCH_COLS2
#undef FP4Q_LAUNCH_COLS1
#undef FP4Q_LAUNCH_COLS
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

size_t nv_workspace_bytes(int domain) { return domain == 0 ? (size_t)kAmaxBlocks * sizeof(uint32_t) : 0; }

int launch_quant_nv(const QuantArgs &a, int domain, float *tensor_scale, void *workspace, const float *given_amax,
                    hipStream_t st)
{
    const uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32);
    const uint32_t R = (uint32_t)a.rows, K = (uint32_t)a.cols;
    auto *x = reinterpret_cast<const uint16_t *>(a.x);
    auto *codes = reinterpret_cast<uint32_t *>(a.codes);
    auto *scales = reinterpret_cast<uint8_t *>(a.scales);
    if (a.axis == 1) {
        // along columns (x^T), optionally with the Hadamard: rows = K
        const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
        const uint32_t ntile = ((cols + kColTile - 1) / kColTile) * ((rows + kColTile - 1) / kColTile);
        auto *c8 = reinterpret_cast<uint8_t *>(a.codes);
        const uint32_t Rp = (cols + 31) / 32 * 32;  // output rows of the tiled layout
#define FP4Q_NVC_T(SR, HAD, MODE, T, G, PART, NP)                                                                   \
    hipLaunchKernelGGL((nv_quant_cols_kernel<SR, HAD, MODE, T>), dim3(G), dim3(kThreads), 0, st, x, rows, cols,     \
                       (uint32_t)a.ld, c8, scales, tensor_scale, PART, NP, seed_lo, seed_hi, a.stream_id, a.sign_mask, \
                       Rp)
#define FP4Q_NVC(SR, HAD, MODE, G, PART, NP)                                      \
    do {                                                                          \
        if (a.tiled) FP4Q_NVC_T(SR, HAD, MODE, true, G, PART, NP);                \
        else FP4Q_NVC_T(SR, HAD, MODE, false, G, PART, NP);                       \
    } while (0)
        if (domain == 1) {
            if (ntile == 0) return 0;
            if (a.sr) { if (a.hadamard) FP4Q_NVC(true, true, 0, ntile, nullptr, 0u); else FP4Q_NVC(true, false, 0, ntile, nullptr, 0u); }
            else { if (a.hadamard) FP4Q_NVC(false, true, 0, ntile, nullptr, 0u); else FP4Q_NVC(false, false, 0, ntile, nullptr, 0u); }
        } else {
            // pass 1: partial maxima of the (transformed) values; an empty
            // operand still gets S = 1 from pass 2
            auto *part = reinterpret_cast<uint32_t *>(workspace);
            const uint32_t np = ntile == 0 ? 1u : min(ntile, (uint32_t)kAmaxBlocks);
            if (a.hadamard) FP4Q_NVC_T(false, true, 2, false, np, part, 0u);
            else FP4Q_NVC_T(false, false, 2, false, np, part, 0u);
            const uint32_t g = ntile == 0 ? 1u : ntile;
            if (a.sr) { if (a.hadamard) FP4Q_NVC(true, true, 1, g, part, np); else FP4Q_NVC(true, false, 1, g, part, np); }
            else { if (a.hadamard) FP4Q_NVC(false, true, 1, g, part, np); else FP4Q_NVC(false, false, 1, g, part, np); }
        }
#undef FP4Q_NVC
#undef FP4Q_NVC_T
        return hipGetLastError() == hipSuccess ? 0 : 1;
    }
    if (domain == 0) {
        const uint64_t nchunks = (uint64_t)R * (K >> 3);
        const uint32_t *partial;
        uint32_t np;
        if (given_amax) {
            // single pass: the caller supplies the domain amax (binary32; its
            // bits are the one "partial maximum")
            partial = reinterpret_cast<const uint32_t *>(given_amax);
            np = 1;
        } else {
            auto *part = reinterpret_cast<uint32_t *>(workspace);
            np = (uint32_t)((nchunks + kThreads - 1) / kThreads);
            if (np > (uint32_t)kAmaxBlocks) np = kAmaxBlocks;
            if (np == 0) np = 1;
            // pass 1 (also runs for an empty operand so that S = 1 is written)
            if (a.ld == (int64_t)K)
                hipLaunchKernelGGL(nv_amax_partial_kernel<true>, dim3(np), dim3(kThreads), 0, st, x, K,
                                   (uint32_t)a.ld, (uint32_t)nchunks, part);
            else
                hipLaunchKernelGGL(nv_amax_partial_kernel<false>, dim3(np), dim3(kThreads), 0, st, x, K,
                                   (uint32_t)a.ld, (uint32_t)nchunks, part);
            partial = part;
        }
        // the tiled layout's padding rows (up to a multiple of 32) are written too
        const uint64_t nchunks_out = a.tiled ? (uint64_t)((R + 31) / 32 * 32) * (K >> 3) : nchunks;
        const uint32_t grid =
            (uint32_t)((nchunks_out + kThreads * kNvgChunks - 1) / (kThreads * kNvgChunks));
        const uint32_t g = grid == 0 ? 1 : grid;
#define FP4Q_NVG(SR, FLAT, T)                                                                                  \
    hipLaunchKernelGGL((nv_quant_global_kernel<SR, FLAT, T>), dim3(g), dim3(kThreads), 0, st, x, K, (uint32_t)a.ld,    \
                       (uint32_t)nchunks, partial, np, codes, scales, tensor_scale, seed_lo, seed_hi, a.stream_id, \
                       (uint32_t)nchunks_out, by)
        const bool flat = a.ld == (int64_t)K;
        const uint32_t div = a.tiled ? K >> 7 : K >> 3;
        const FastDiv by = fast_div_for(div ? div : 1);
        if (a.tiled) {  // the tiled walk computes each chunk's row itself: one form for any ld
            if (a.sr) FP4Q_NVG(true, false, true); else FP4Q_NVG(false, false, true);
        } else {
            if (a.sr) { if (flat) FP4Q_NVG(true, true, false); else FP4Q_NVG(true, false, false); }
            else { if (flat) FP4Q_NVG(false, true, false); else FP4Q_NVG(false, false, false); }
        }
#undef FP4Q_NVG
    } else {
        if (R == 0 || K == 0) return 0;
        dim3 grid(((K + 127) / 128 + 1) / 2, (R + 127) / 128);  // pairs of tiles
        const uint32_t Rp = (R + 31) / 32 * 32;
#define FP4Q_NVT(SR, T)                                                                                            \
    hipLaunchKernelGGL((nv_quant_tile_kernel<SR, T>), grid, dim3(kTileThreads), 0, st, x, R, K, (uint32_t)a.ld, codes, \
                       scales, tensor_scale, seed_lo, seed_hi, a.stream_id, Rp)
        if (a.tiled) { if (a.sr) FP4Q_NVT(true, true); else FP4Q_NVT(false, true); }
        else { if (a.sr) FP4Q_NVT(true, false); else FP4Q_NVT(false, false); }
#undef FP4Q_NVT
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fp4q
