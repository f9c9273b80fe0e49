/*
 * fp4q.h -- C ABI of libfp4q: FP4 block-scaled quantization producers and the
 * block-scaled FP4 GEMM that consumes them, for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as printed):
 *   [Fusion] "Format-Aware Fusion: The Engineering Practice That Doubles FP4
 *            Pretraining Throughput"
 *   [Stack]  "FP4 Is No Longer Just a Hardware Feature -- The NVFP4 Software
 *            Stack Is Taking Shape"
 *   [OnGPUs] "4-Bit Floating Point (FP4) on GPUs: How It Works and When It Pays Off"
 *
 * What the library computes.  A quantization producer turns a bf16 matrix
 * into a two-part FP4 operand ([OnGPUs], section "How Does 4-Bit Floating
 * Point Work in Practice?": packed 4-bit payload plus per-block scales) in one
 * pass: block amax -> scale -> divide by the scale -> E2M1 -> pack two codes
 * per byte ([Stack], section "The first change: PyTorch is bringing FP4
 * packing into compiler fusion").  Each producer is bound to its scale domain
 * and to the layout its GEMM loads ([Fusion], section "The Design Philosophy
 * of Format-Aware Fusion": native mxfp, global nvfp, CTA-local nvfp).
 *
 * Numerical contract (bit-exact; every output byte is a pure function of the
 * inputs):
 *   E2M1 code  = sign<<3 | k, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}[k];
 *                the sign bit is kept for negative values that round to zero.
 *   RNE        round to nearest, ties to even k; |y| >= 6 saturates to k = 7.
 *   SR         with lo <= |y| < hi the neighbouring magnitudes, round up iff
 *              r16 < 65536 * (|y| - lo) / (hi - lo); r16 = 16 bits of
 *              Philox4x32-10 (Salmon et al., SC'11) with counter
 *              {k/8, r, stream_id, 0} and key {seed low, seed high}, word
 *              (k/2) mod 4, high half for odd k; (r, k) are coordinates in the
 *              logical operand, so results do not depend on the launch shape.
 *   MX         32-element blocks along K; shared exponent
 *              E = clamp(floor(log2 amax) - 2, -127, 127) (OCP MX v1.0; an
 *              all-zero block gets -127); scale byte = E + 127 (E8M0);
 *              y = x * 2^-E in binary32.
 *   NV         16-element blocks along K; tensor scale S = A / 2688 (A = amax
 *              of the domain; S = 1 when A = 0); block scale
 *              sb = E4M3_RNE_satfinite((b / 6) / S) clamped to >= 0x01
 *              ([Stack], section "The third change: oneDNN is defining a safe
 *              numerical range for FP4 scales"); d = e4m3(sb) * S;
 *              y = x * (1 / d) in binary32.
 *   Hadamard   before MX: x <- H32 * diag(d) * x per 32-block along K, d_i = -1
 *              where bit i of sign_mask is set, H32 the unnormalised Sylvester
 *              matrix, evaluated as butterflies of span 1, 2, 4, 8, 16 in
 *              binary32 ([Fusion], section "Two Key Numerical Techniques").
 *              H32 * H32^T = 32 I, so a GEMM of two such operands takes
 *              alpha = 1/32.
 *
 * Operands.  The input x is a row-major bf16 [rows x cols] matrix with leading
 * dimension ld_x >= cols (elements).  The logical quantized operand [R x K] is
 * x itself for FP4Q_ALONG_ROWS (R = rows, K = cols) and x^T for
 * FP4Q_ALONG_COLS (R = cols, K = rows): blocks then run down the columns of x
 * (the transpose-quantize a wgrad/dgrad operand needs).
 * Linear layout (FP4Q_LAYOUT_LINEAR):
 *   codes   [R x K/2] bytes, row-major; element 2j in the low nibble of byte j,
 *           element 2j+1 in the high nibble ([Stack] pairs even and odd
 *           elements into one byte);
 *   scales  MX: [R x K/32] E8M0 bytes; NV: [R x K/16] E4M3 bytes, row-major;
 *   tensor_scale  NV global: 1 float; NV tile128: [ceil(R/128) x ceil(K/128)]
 *           floats, row-major, one per 128 x 128 tile of the logical operand.
 * Tiled layout (FP4Q_LAYOUT_TILED; K % 128 == 0): the consumer layout of
 * the GEMMs ([Fusion], section "The Design Philosophy of Format-Aware
 * Fusion": the producer writes what the consumer loads).  With
 * Rp = 32 * ceil(R/32), for MX operands:
 *   codes   [Rp/32][K/64][64][16] bytes.  The 16 bytes at (g, kb, l) hold row
 *           32 g + (l mod 32), K elements 64 kb + 32 (l / 32) .. +31, element
 *           2j in the low nibble of byte j: one 1 KiB block is exactly the
 *           operand of one gfx950 scaled-MFMA instruction, lane l's 16 bytes
 *           at offset 16 l.  Rows R .. Rp-1 hold zero codes.
 *   scales  [K/128][Rp][4] bytes: byte q of (s, r) is the E8M0 scale of row r,
 *           K block 4 s + q (one 32-bit word per row per 128-wide K step).
 *           Rows R .. Rp-1 hold 0.
 *   Sizes: codes Rp * K / 2 bytes, scales Rp * K / 32 bytes, both 16-byte
 *   aligned.  Producers write every byte, padding included.
 * For NV operands (step-major 32-row blocks):
 *   codes   [Rp/32][K/128][32][64] bytes: the 64 bytes at (g, s, f) are the
 *           codes of row 32 g + f, K elements 128 s .. 128 s + 127, in the
 *           order of the linear layout (element 2j of the step in the low
 *           nibble of byte j); a K step of a 32-row group is 2 KiB.
 *   scales  [Rp/32][K/128][32][8] bytes: the eight E4M3 bytes of row 32 g + f,
 *           K blocks 8 s .. 8 s + 7.
 *   tensor_scale as in the linear layout.  Rows R .. Rp-1 hold zero codes
 *   and zero scale bytes.  Sizes: codes Rp * K / 2, scales Rp * K / 16
 *   bytes, both 16-byte aligned.
 *
 * GEMM.  C[M x N] = alpha * A * B^T, A the logical [M x K] operand and B the
 * logical [N x K] operand, both quantized along K; fp32 accumulation; C is
 * row-major with leading dimension ldc >= N, fp32 or bf16 (round to nearest
 * even from the fp32 result).  For Y = X * W^T pass X as A and W as B.
 *
 * Ownership and execution.  Every pointer is device memory owned by the
 * caller (for example PyTorch tensors).  The library never allocates, frees
 * or synchronizes; every call enqueues its kernels on `stream` (a hipStream_t;
 * NULL = the default stream) and returns once they are enqueued.  Outputs are
 * valid after the stream is synchronized.  Inputs must not overlap outputs.
 *
 * Errors.  Arguments are checked on the host before any launch; a failing
 * check returns a status and enqueues nothing:
 *   FP4Q_EINVAL       null pointer, unknown enum value, overlapping buffers,
 *                     workspace too small;
 *   FP4Q_ESHAPE       negative size, K not a multiple of the block (32 MX,
 *                     16 NV), GEMM K not a multiple of 128, ld_x < cols,
 *                     ldc < N, a dimension above 2^31 - 1;
 *   FP4Q_EALIGN       x, codes or GEMM operand pointers not 16-byte aligned,
 *                     ld_x not a multiple of 8 elements;
 *   FP4Q_EUNSUPPORTED a valid combination this build does not implement
 *                     (listed at each call);
 *   FP4Q_ELAUNCH      the kernel launch failed (hipGetLastError).
 * Inputs outside the numerical contract (NaN or Inf anywhere in x, an NV
 * domain with 0 < amax < 2^-100) are not detected and give unspecified codes.
 * Empty operands (R == 0 or K == 0, or M, N or K == 0) are valid and enqueue
 * nothing, except that a GEMM with K == 0 writes C = 0.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 1

/* Symbols of the C ABI are the only ones the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define FP4Q_API __attribute__((visibility("default")))
#else
#define FP4Q_API
#endif

typedef enum {
    FP4Q_OK = 0,
    FP4Q_EINVAL = 1,
    FP4Q_ESHAPE = 2,
    FP4Q_EALIGN = 3,
    FP4Q_ELAUNCH = 4,
    FP4Q_EUNSUPPORTED = 5
} fp4q_status;

typedef enum { FP4Q_ALONG_ROWS = 0, FP4Q_ALONG_COLS = 1 } fp4q_axis;
typedef enum { FP4Q_RNE = 0, FP4Q_SR = 1 } fp4q_round;
typedef enum { FP4Q_NV_GLOBAL = 0, FP4Q_NV_TILE128 = 1 } fp4q_nv_domain;
typedef enum { FP4Q_LAYOUT_LINEAR = 0, FP4Q_LAYOUT_TILED = 1 } fp4q_layout;
typedef enum { FP4Q_OUT_F32 = 0, FP4Q_OUT_BF16 = 1 } fp4q_out;

/* MXFP4 producer ("native mxfp", [Fusion] section "The Design Philosophy of
 * Format-Aware Fusion"; steps of [Stack] section "The first change").
 * x: bf16 [rows x ld_x]; writes codes [R x K/2] and E8M0 scales [R x K/32].
 * round = FP4Q_SR uses (seed, stream_id) as stated above ("row-gradient
 * stochastic rounding", [Fusion] section "Two Key Numerical Techniques").
 * Requires K % 32 == 0 (linear) or K % 128 == 0 (tiled).  Both axes, both
 * rounding modes, both layouts. */
FP4Q_API fp4q_status fp4_quantize_mx(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                            int round, uint64_t seed, uint32_t stream_id, void *codes, void *scales,
                            int layout, void *stream);

/* Fixed-sign 32-point Hadamard, then MXFP4 ("fixed-sign 32-value Hadamard
 * weight-gradient preconditioning", [Fusion] section "Two Key Numerical
 * Techniques").  Same outputs and requirements as fp4_quantize_mx; the
 * transform runs along K in the same 32-blocks as the scales. */
FP4Q_API fp4q_status fp4_hadamard32_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                                    uint32_t sign_mask, int round, uint64_t seed, uint32_t stream_id,
                                    void *codes, void *scales, int layout, void *stream);

/* One read of x, both MXFP4 operands a training step takes from it: x along
 * rows (the forward / dgrad operand, [rows x cols], no Hadamard) and x^T
 * along columns with an optional fixed-sign Hadamard (the wgrad operand,
 * [cols x rows]).  Saving the second one at forward time keeps the backward
 * pass from reading x again ([Fusion] section "Why FP4 Speedups Often Remain
 * Theoretical": the state kept for backpropagation is one of the overheads;
 * section "The Design Philosophy of Format-Aware Fusion": each producer is
 * bound to the layout its consumer loads).
 * Outputs: codes_rows / scales_rows exactly as fp4_quantize_mx(x, rows, cols,
 * ld_x, FP4Q_ALONG_ROWS, round_rows, seed, stream_id_rows, ...) writes them,
 * and codes_cols / scales_cols exactly as fp4_hadamard32_quantize (when
 * hadamard_cols = 1, with sign_mask) or fp4_quantize_mx (hadamard_cols = 0)
 * with FP4Q_ALONG_COLS, round_cols, seed, stream_id_cols; every byte is
 * identical to those calls'.  Requires rows and cols to be multiples of 32
 * (linear) or 128 (tiled); both outputs in `layout`.  Errors as the two
 * producers, plus FP4Q_EINVAL for hadamard_cols other than 0 or 1 and for
 * outputs that overlap each other. */
FP4Q_API fp4q_status fp4_quantize_mx_dual(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int round_rows,
                                 uint32_t stream_id_rows, void *codes_rows, void *scales_rows, int hadamard_cols,
                                 uint32_t sign_mask, int round_cols, uint32_t stream_id_cols, void *codes_cols,
                                 void *scales_cols, uint64_t seed, int layout, void *stream);

/* Bytes of device workspace fp4_quantize_nv needs (the global domain's
 * partial maxima; 0 for the tile domain). */
FP4Q_API size_t fp4q_nv_workspace_bytes(int64_t rows, int64_t cols, int axis, int domain);

/* NVFP4 producer: "global nvfp" (domain FP4Q_NV_GLOBAL, one FP32 tensor scale
 * from the whole operand's amax; two kernels: partial maxima into `workspace`,
 * then quantize) or "CTA-local nvfp" (FP4Q_NV_TILE128, one tensor scale per
 * 128 x 128 tile, one kernel) ([Fusion] section "The Design Philosophy of
 * Format-Aware Fusion"; the two-level scale of [Stack] section "NVFP4 is more
 * than a 4-bit value").  Writes codes [R x K/2], E4M3 scales [R x K/16] and
 * tensor_scale.  Both axes: along columns (the transpose a wgrad operand
 * needs) a 128 x 128 tile of x is one tile domain of x^T.  Requires
 * K % 16 == 0 (linear) or K % 128 == 0 (tiled), and cols % 4 == 0 along
 * columns.  Both layouts, axes and domains, RNE and SR. */
FP4Q_API fp4q_status fp4_quantize_nv(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, int round,
                            uint64_t seed, uint32_t stream_id, int domain, void *codes, void *scales,
                            float *tensor_scale, void *workspace, size_t workspace_bytes, int layout,
                            void *stream);

/* fp4_quantize_nv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The global domain's partial maxima go
 * to a 4 KiB buffer inside the library (a file-scope device array; every GPU
 * the library runs on holds its own copy until the process ends), so the
 * call allocates nothing; the tile domain needs none.  Every output byte
 * equals fp4_quantize_nv's for the same arguments.  The work runs on the
 * current device, which must be the one `stream` belongs to.  All calls on
 * one GPU share its buffer: calls that overlap in time on one GPU (on
 * different streams, or from several host threads without ordering) race
 * and give unspecified outputs; calls ordered on one stream do not (each
 * call writes every slot it reads before reading it, so nothing needs
 * clearing).  The buffer holds at most 1024 partial maxima, enough for any
 * operand size; FP4Q_EINVAL if a build ever needed more.  Errors as
 * fp4_quantize_nv, plus FP4Q_ELAUNCH if the buffer's device address cannot
 * be obtained. */
FP4Q_API fp4q_status fp4_quantize_nv_noalloc(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                                            int round, uint64_t seed, uint32_t stream_id, int domain, void *codes,
                                            void *scales, float *tensor_scale, int layout, void *stream);

/* Fixed-sign 32-point Hadamard along K, then NVFP4 ([Fusion] section "Two Key
 * Numerical Techniques" names it for the weight-gradient operands; here on
 * the NVFP4 path): as fp4_quantize_nv on the transformed values, which the
 * domain amax, the block amax and the codes all see.  Along columns only
 * (the wgrad operands, quantized along tokens); requires K % 32 == 0
 * (linear) or K % 128 == 0 (tiled) and cols % 4 == 0.  FP4Q_EUNSUPPORTED:
 * FP4Q_ALONG_ROWS. */
FP4Q_API fp4q_status fp4_hadamard32_quantize_nv(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                                       uint32_t sign_mask, int round, uint64_t seed, uint32_t stream_id, int domain,
                                       void *codes, void *scales, float *tensor_scale, void *workspace,
                                       size_t workspace_bytes, int layout, void *stream);

/* MXFP4 GEMM on gfx950's scaled FP4 MFMA (E8M0 scales applied by the matrix
 * core): C = alpha * A * B^T.  a_codes [M x K/2], a_scales [M x K/32],
 * b_codes [N x K/2], b_scales [N x K/32] as written by the MX producers,
 * in the layout given by `layout` (both operands in the same layout; the
 * tiled layout is the fast one).  Requires K % 128 == 0; M and N are
 * arbitrary. */
FP4Q_API fp4q_status fp4_gemm_mx(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                        int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type,
                        int64_t ldc, void *stream);

/* NVFP4 GEMM: E2M1 x E4M3 is dequantized exactly to fp16 and multiplied on
 * fp16 MFMA with fp32 accumulation; the FP32 tensor scales multiply the fp32
 * partial sums (once in the epilogue for the global domain, per 128-wide K
 * slice for tile128).
 * a_tensor_scale / b_tensor_scale as written by fp4_quantize_nv with the same
 * domain; A and B both in `layout` (the tiled layout's 2 KiB step blocks
 * are what the GEMM's LDS DMA copies, whole).  Requires K % 128 == 0. */
FP4Q_API fp4q_status fp4_gemm_nv(const void *a_codes, const void *a_scales, const float *a_tensor_scale,
                        const void *b_codes, const void *b_scales, const float *b_tensor_scale, int domain,
                        int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type,
                        int64_t ldc, void *stream);

/* MXFP4 GEMM whose output leaves as the next GEMM's MXFP4 operand: C =
 * alpha * A * B^T is rounded to bf16 and quantized along rows (RNE, E8M0
 * per 32) in the epilogue, so that no bf16 C is written and read back
 * ([Fusion] section "Why FP4 Speedups Often Remain Theoretical": unfused
 * quantization steps around the matrix multiply cost the gain; section "The
 * Design Philosophy of Format-Aware Fusion": the producer writes the layout
 * its consumer loads).  c_codes / c_scales are exactly what fp4_quantize_mx
 * (FP4Q_ALONG_ROWS, FP4Q_RNE, c_layout) writes for the bf16 C that
 * fp4_gemm_mx would produce.  A, B in `layout`; requires K % 128 == 0 and
 * N % 32 == 0 (linear output) or N % 128 == 0 (tiled output, rows padded to
 * 32 with zero codes and scales).  Errors as fp4_gemm_mx. */
FP4Q_API fp4q_status fp4_gemm_mx_quant(const void *a_codes, const void *a_scales, const void *b_codes,
                              const void *b_scales, int64_t M, int64_t N, int64_t K, float alpha, int layout,
                              void *c_codes, void *c_scales, int c_layout, void *stream);

/* SwiGLU of a bf16 gate/up GEMM output (the activation before the MX
 * producer of the MLP's hidden operand H; [Fusion] section "The Design
 * Philosophy of Format-Aware Fusion": the producer is fused with the op that
 * makes its input -- this is that op on its own).  c: bf16 [M x >= 2F],
 * row pitch ldc elements, whose columns interleave gate and up in groups of
 * `pair` columns (gate column j at 2 pair (j / pair) + j mod pair, its up
 * column `pair` further; pair = 32 is the layout fp4_gemm_mx_swiglu_quant
 * takes, pair = F the plain [gate | up]).  h: bf16 [M x F], pitch ldh:
 * h[m][j] = bf16(SiLU(g) * u), SiLU(x) = x / (1 + e^-x), evaluated in
 * binary32 by one fixed division-free sequence: e = e^-min(|x|, 112) by
 * Cody-Waite reduction with a two-part ln 2, a degree-7 Horner polynomial p
 * and scaling by 2^k; the reciprocal y of 1 + e by three Newton steps from a
 * bit-pattern seed; SiLU = x y for x >= 0 and (x p y) 2^k for x < 0.  Its
 * error over every finite bf16 x is below 4 binary32 half-ulps (relative)
 * for normal results and 2^-149 in the subnormal range; then one binary32
 * product with u, rounded to bf16 to nearest even.  So h is the real
 * SiLU(g) u rounded to bf16, except where that value lies within this
 * error of a bf16 rounding midpoint (then either neighbour).  Requires F % 8 == 0, pair % 8 == 0, F % pair == 0,
 * ldc >= 2F and ldh >= F both multiples of 8 (FP4Q_ESHAPE), c and h 16-byte
 * aligned (FP4Q_EALIGN), h not overlapping c (FP4Q_EINVAL). */
FP4Q_API fp4q_status fp4_swiglu_bf16(const void *c, int64_t M, int64_t F, int64_t ldc, int64_t pair, void *h,
                            int64_t ldh, void *stream);

/* MXFP4 gate/up GEMM whose output leaves as SwiGLU(C) quantized along rows:
 * the MLP's hidden operand H for the down projection, with neither the
 * bf16 C nor the bf16 H written ([Fusion] sections "Why FP4 Speedups Often
 * Remain Theoretical" and "The Design Philosophy of Format-Aware Fusion").
 * B's N rows (N = 2F) interleave the gate and up weight rows in groups of 32
 * (B rows 64 b .. 64 b + 31 = gate rows 32 b .. 32 b + 31, the next 32 = the
 * up rows of the same hidden units), so that each 32-column gate block of C
 * shares the accumulator lanes of its up block.  h_codes / h_scales: H
 * [M x F] exactly as fp4_quantize_mx (FP4Q_ALONG_ROWS, FP4Q_RNE, h_layout)
 * writes it for the bf16 H that fp4_gemm_mx (bf16 C) followed by
 * fp4_swiglu_bf16 (pair 32) produces.  A, B in `layout`; requires K % 128
 * == 0 and N % 64 == 0 (linear output) or N % 256 == 0 (tiled output, rows
 * padded to 32 with zero codes and scales).  Errors as fp4_gemm_mx_quant. */
FP4Q_API fp4q_status fp4_gemm_mx_swiglu_quant(const void *a_codes, const void *a_scales, const void *b_codes,
                                     const void *b_scales, int64_t M, int64_t N, int64_t K, float alpha,
                                     int layout, void *h_codes, void *h_scales, int h_layout, void *stream);

/* The GEMMs above, also reporting max |C| for a following NVFP4 "global
 * nvfp" quantization of C, so that it needs no amax pass over C (the amax is
 * produced by the op before the quantizer: [Fusion] section "The Design
 * Philosophy of Format-Aware Fusion", the global nvfp scenario; [Stack]
 * section "NVFP4 is more than a 4-bit value": the FP32 tensor scale comes
 * from the tensor's amax).  c_amax: one device float, 4-byte aligned, not
 * inside C; the epilogue folds max |C| over the values it stores, as stored
 * (after the bf16 rounding), into *c_amax with an atomic max: initialize it
 * to 0 (or to a running maximum) before the call.  The result is then
 * exactly the amax fp4_quantize_nv computes for a bf16 C.  NaN or Inf in C
 * give an unspecified *c_amax.  Otherwise identical to fp4_gemm_mx /
 * fp4_gemm_nv; FP4Q_EINVAL if c_amax is null or overlaps C. */
FP4Q_API fp4q_status fp4_gemm_mx_amax(const void *a_codes, const void *a_scales, const void *b_codes,
                             const void *b_scales, int64_t M, int64_t N, int64_t K, float alpha, int layout,
                             void *c, int c_type, int64_t ldc, float *c_amax, void *stream);
FP4Q_API fp4q_status fp4_gemm_nv_amax(const void *a_codes, const void *a_scales, const float *a_tensor_scale,
                             const void *b_codes, const void *b_scales, const float *b_tensor_scale, int domain,
                             int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type,
                             int64_t ldc, float *c_amax, void *stream);

/* NVFP4 "global nvfp" producer in one pass: the domain amax is read from
 * `amax` (a device float, e.g. written by fp4_gemm_*_amax for this x)
 * instead of being computed from x.  With *amax == max |x| every output byte
 * equals fp4_quantize_nv(..., FP4Q_NV_GLOBAL, ...)'s; another finite value >= 0 gives
 * the codes of the tensor scale S = *amax / 2688.  Along rows, linear layout;
 * requires cols % 16 == 0.  Errors as fp4_quantize_nv, plus FP4Q_EINVAL for
 * a null or overlapping `amax`, FP4Q_EALIGN if it is not 4-byte aligned. */
FP4Q_API fp4q_status fp4_quantize_nv_amax(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int round,
                                 uint64_t seed, uint32_t stream_id, const float *amax, void *codes, void *scales,
                                 float *tensor_scale, void *stream);

/* Human-readable text for a status code (static storage). */
FP4Q_API const char *fp4q_status_str(int status);

/* FP4Q_ABI_VERSION of the built library. */
FP4Q_API int fp4q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
