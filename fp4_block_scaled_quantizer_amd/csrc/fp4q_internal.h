// fp4q_internal.h -- argument bundles shared by the C-ABI layer and the
// kernel launchers of libfp4q.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4q {

struct QuantArgs {
    const void *x;   // bf16 [rows x ld]
    int64_t rows, cols, ld;
    int axis;        // 0: along rows, 1: along columns (x^T)
    bool sr;
    bool hadamard;
    bool tiled;      // FP4Q_LAYOUT_TILED outputs
    uint64_t seed;
    uint32_t stream_id;
    uint32_t sign_mask;
    void *codes;
    void *scales;
    // dual output (axis 1 only): x along rows as well, rounded per rows_round
    // (0 none, 1 RNE, 2 SR) with its own stream id
    int rows_round;
    uint32_t stream_id_rows;
    void *codes_rows;
    void *scales_rows;
};

struct GemmArgs {
    const void *a_codes, *a_scales, *b_codes, *b_scales;
    const float *a_ts, *b_ts;  // NV tensor scales (null for MX)
    int nv_domain;             // NV only: 0 global, 1 tile128
    bool tiled;                // FP4Q_LAYOUT_TILED operands
    int64_t M, N, K;
    float alpha;
    void *c;
    bool c_bf16;
    int64_t ldc;
    uint32_t *c_amax;  // optional: max |C| as stored, folded in as binary32 bits
    // MX only, optional: C written as an MXFP4 operand along rows instead;
    // with q_swiglu, SwiGLU(C) (N / 2 columns: gate and up columns of C
    // interleaved in groups of 32)
    void *q_codes, *q_scales;
    bool q_tiled;
    bool q_swiglu;
};

// Compute units of the current device (the persistent GEMMs' grid), looked
// up once per device; <= 0 if the device cannot be queried.
int device_cu_count();

int launch_quant_mx(const QuantArgs &a, hipStream_t st);
// given_amax: optional device pointer to the global domain's amax (skips the
// amax pass); null for the two-pass global path and the tile domain
int launch_quant_nv(const QuantArgs &a, int domain, float *tensor_scale, void *workspace, const float *given_amax,
                    hipStream_t st);
size_t nv_workspace_bytes(int domain);
int launch_gemm_mx(const GemmArgs &g, hipStream_t st);
int launch_gemm_nv(const GemmArgs &g, hipStream_t st);
// h[m][j] = bf16(SiLU(gate) * up) from a bf16 C whose columns interleave gate
// and up in groups of `pair` (a multiple of 8 dividing F)
int launch_swiglu(const void *c, int64_t M, int64_t F, int64_t ldc, int64_t pair, void *h, int64_t ldh,
                  hipStream_t st);

}  // namespace fp4q
