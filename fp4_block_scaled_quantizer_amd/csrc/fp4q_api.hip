// fp4q_api.hip -- the extern "C" entry points declared in include/fp4q.h:
// argument checks (all before any HIP call, so they run without a GPU), then
// one call into the kernel launchers.  The library allocates nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/fp4q.h"
#include "fp4q_internal.h"

namespace fp4q {

int device_cu_count()
{
    static std::atomic<int> cached[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
    if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace fp4q

namespace {

constexpr int64_t kMaxDim = INT32_MAX;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range bytes(const void *p, uint64_t n) { return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)n}; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// bytes spanned by a row-major bf16 [rows x ld] input whose rows hold `cols` used elements
uint64_t input_span(int64_t rows, int64_t cols, int64_t ld)
{
    return rows == 0 || cols == 0 ? 0 : ((uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * 2u;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

fp4q_status launched(int rc) { return rc == 0 ? FP4Q_OK : FP4Q_ELAUNCH; }

// Shared checks of the two MX producers.
fp4q_status check_mx_producer(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, int round,
                              const void *codes, const void *scales, int layout, bool *empty)
{
    if ((axis != FP4Q_ALONG_ROWS && axis != FP4Q_ALONG_COLS) || (round != FP4Q_RNE && round != FP4Q_SR) ||
        (layout != FP4Q_LAYOUT_LINEAR && layout != FP4Q_LAYOUT_TILED))
        return FP4Q_EINVAL;
    if (rows < 0 || cols < 0 || ld_x < cols || rows > kMaxDim || cols > kMaxDim || ld_x > kMaxDim)
        return FP4Q_ESHAPE;
    const bool tiled = layout == FP4Q_LAYOUT_TILED;
    const int64_t R = axis == FP4Q_ALONG_ROWS ? rows : cols;
    const int64_t K = axis == FP4Q_ALONG_ROWS ? cols : rows;
    if (K % (tiled ? 128 : 32) != 0) return FP4Q_ESHAPE;
    if (axis == FP4Q_ALONG_COLS && cols % 4 != 0) return FP4Q_ESHAPE;
    const int64_t Rs = tiled ? (R + 31) / 32 * 32 : R;  // rows of the stored operand
    if ((uint64_t)Rs * (uint64_t)(K / 8) >= (1ull << 32)) return FP4Q_ESHAPE;
    *empty = (R == 0 || K == 0);
    if (*empty) return FP4Q_OK;
    if (!x || !codes || !scales) return FP4Q_EINVAL;
    if (!aligned(x, 16) || !aligned(codes, 16) || ld_x % 8 != 0) return FP4Q_EALIGN;
    if (tiled && !aligned(scales, 16)) return FP4Q_EALIGN;
    const Range rx = bytes(x, input_span(rows, cols, ld_x));
    const Range rc = bytes(codes, (uint64_t)Rs * (uint64_t)K / 2);
    const Range rs = bytes(scales, (uint64_t)Rs * (uint64_t)K / 32);
    if (overlap(rx, rc) || overlap(rx, rs) || overlap(rc, rs)) return FP4Q_EINVAL;
    return FP4Q_OK;
}

fp4q_status run_mx_producer(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, bool hadamard,
                            uint32_t sign_mask, int round, uint64_t seed, uint32_t stream_id, void *codes,
                            void *scales, int layout, void *stream)
{
    bool empty = false;
    const fp4q_status st = check_mx_producer(x, rows, cols, ld_x, axis, round, codes, scales, layout, &empty);
    if (st != FP4Q_OK || empty) return st;
    fp4q::QuantArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld_x;
    a.axis = axis;
    a.sr = round == FP4Q_SR;
    a.hadamard = hadamard;
    a.tiled = layout == FP4Q_LAYOUT_TILED;
    a.seed = seed;
    a.stream_id = stream_id;
    a.sign_mask = sign_mask;
    a.codes = codes;
    a.scales = scales;
    (void)hipGetLastError();  // report only this call's launch status
    return launched(fp4q::launch_quant_mx(a, as_stream(stream)));
}

fp4q_status check_gemm_common(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                              int64_t M, int64_t N, int64_t K, int layout, const void *c, int c_type, int64_t ldc,
                              int scale_div, bool *empty)
{
    if ((layout != FP4Q_LAYOUT_LINEAR && layout != FP4Q_LAYOUT_TILED) ||
        (c_type != FP4Q_OUT_F32 && c_type != FP4Q_OUT_BF16))
        return FP4Q_EINVAL;
    const bool tiled = layout == FP4Q_LAYOUT_TILED;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || ldc < N || ldc > kMaxDim)
        return FP4Q_ESHAPE;
    if (K % 128 != 0) return FP4Q_ESHAPE;
    const uint64_t Ms = tiled ? (uint64_t)(M + 31) / 32 * 32 : (uint64_t)M;  // stored rows
    const uint64_t Ns = tiled ? (uint64_t)(N + 31) / 32 * 32 : (uint64_t)N;
    if (Ms * (uint64_t)K / 2 >= (1ull << 32) || Ns * (uint64_t)K / 2 >= (1ull << 32)) return FP4Q_ESHAPE;
    *empty = (M == 0 || N == 0);
    if (*empty) return FP4Q_OK;
    if (!c) return FP4Q_EINVAL;
    const uint64_t esize = c_type == FP4Q_OUT_F32 ? 4 : 2;
    if (!aligned(c, esize)) return FP4Q_EALIGN;
    if (K == 0) return FP4Q_OK;
    if (!a_codes || !a_scales || !b_codes || !b_scales) return FP4Q_EINVAL;
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4))
        return FP4Q_EALIGN;
    const Range rc = bytes(c, ((uint64_t)(M - 1) * (uint64_t)ldc + (uint64_t)N) * esize);
    const Range ins[4] = {bytes(a_codes, Ms * K / 2), bytes(a_scales, Ms * K / scale_div),
                          bytes(b_codes, Ns * K / 2), bytes(b_scales, Ns * K / scale_div)};
    for (const Range &r : ins)
        if (overlap(rc, r)) return FP4Q_EINVAL;
    return FP4Q_OK;
}

// An optional output amax: one 4-byte aligned float outside C.
bool amax_ok(const float *c_amax, const void *c, int64_t M, int64_t N, int64_t ldc, int c_type)
{
    if (!aligned(c_amax, 4)) return false;
    const uint64_t esize = c_type == FP4Q_OUT_F32 ? 4 : 2;
    return !overlap(bytes(c_amax, 4), bytes(c, ((uint64_t)(M - 1) * (uint64_t)ldc + (uint64_t)N) * esize));
}

fp4q_status run_gemm_mx(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                        int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type, int64_t ldc,
                        float *c_amax, void *stream)
{
    bool empty = false;
    const fp4q_status st =
        check_gemm_common(a_codes, a_scales, b_codes, b_scales, M, N, K, layout, c, c_type, ldc, 32, &empty);
    if (st != FP4Q_OK || empty) return st;
    if (c_amax && !amax_ok(c_amax, c, M, N, ldc, c_type)) return aligned(c_amax, 4) ? FP4Q_EINVAL : FP4Q_EALIGN;
    fp4q::GemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.b_codes = b_codes;
    g.b_scales = b_scales;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.c = c;
    g.c_bf16 = c_type == FP4Q_OUT_BF16;
    g.ldc = ldc;
    g.tiled = layout == FP4Q_LAYOUT_TILED;
    g.c_amax = reinterpret_cast<uint32_t *>(c_amax);
    (void)hipGetLastError();
    return launched(fp4q::launch_gemm_mx(g, as_stream(stream)));
}

// MX GEMM whose C leaves as an MXFP4 operand along rows (codes + E8M0
// scales in c_layout) instead of as bf16 / fp32.
// swiglu: the output is SwiGLU(C) (N / 2 columns) instead of C
fp4q_status run_gemm_mx_quant(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                              int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c_codes,
                              void *c_scales, int c_layout, bool swiglu, void *stream)
{
    if ((layout != FP4Q_LAYOUT_LINEAR && layout != FP4Q_LAYOUT_TILED) ||
        (c_layout != FP4Q_LAYOUT_LINEAR && c_layout != FP4Q_LAYOUT_TILED))
        return FP4Q_EINVAL;
    const bool tiled = layout == FP4Q_LAYOUT_TILED, ctiled = c_layout == FP4Q_LAYOUT_TILED;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP4Q_ESHAPE;
    if (K % 128 != 0 || N % ((ctiled ? 128 : 32) * (swiglu ? 2 : 1)) != 0) return FP4Q_ESHAPE;
    const int64_t Nq = swiglu ? N / 2 : N;  // the quantized output's columns
    const uint64_t Ms = tiled ? (uint64_t)(M + 31) / 32 * 32 : (uint64_t)M;
    const uint64_t Ns = tiled ? (uint64_t)(N + 31) / 32 * 32 : (uint64_t)N;
    const uint64_t Mq = ctiled ? (uint64_t)(M + 31) / 32 * 32 : (uint64_t)M;  // stored output rows
    if (Ms * (uint64_t)K / 2 >= (1ull << 32) || Ns * (uint64_t)K / 2 >= (1ull << 32) ||
        Mq * (uint64_t)Nq / 2 >= (1ull << 32))
        return FP4Q_ESHAPE;
    if (M == 0 || N == 0) return FP4Q_OK;
    if (!c_codes || !c_scales) return FP4Q_EINVAL;
    if (!aligned(c_codes, 16) || !aligned(c_scales, 4)) return FP4Q_EALIGN;
    const Range oc = bytes(c_codes, Mq * Nq / 2), os = bytes(c_scales, Mq * Nq / 32);
    if (overlap(oc, os)) return FP4Q_EINVAL;
    if (K > 0) {
        if (!a_codes || !a_scales || !b_codes || !b_scales) return FP4Q_EINVAL;
        if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4))
            return FP4Q_EALIGN;
        const Range ins[4] = {bytes(a_codes, Ms * K / 2), bytes(a_scales, Ms * K / 32), bytes(b_codes, Ns * K / 2),
                              bytes(b_scales, Ns * K / 32)};
        for (const Range &r : ins)
            if (overlap(oc, r) || overlap(os, r)) return FP4Q_EINVAL;
    }
    fp4q::GemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.b_codes = b_codes;
    g.b_scales = b_scales;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.c_bf16 = true;
    g.ldc = N;
    g.tiled = tiled;
    g.q_codes = c_codes;
    g.q_scales = c_scales;
    g.q_tiled = ctiled;
    g.q_swiglu = swiglu;
    (void)hipGetLastError();
    return launched(fp4q::launch_gemm_mx(g, as_stream(stream)));
}

fp4q_status run_gemm_nv(const void *a_codes, const void *a_scales, const float *a_tensor_scale, const void *b_codes,
                        const void *b_scales, const float *b_tensor_scale, int domain, int64_t M, int64_t N,
                        int64_t K, float alpha, int layout, void *c, int c_type, int64_t ldc, float *c_amax,
                        void *stream)
{
    if (domain != FP4Q_NV_GLOBAL && domain != FP4Q_NV_TILE128) return FP4Q_EINVAL;
    bool empty = false;
    const fp4q_status st =
        check_gemm_common(a_codes, a_scales, b_codes, b_scales, M, N, K, layout, c, c_type, ldc, 16, &empty);
    if (st != FP4Q_OK || empty) return st;
    if (c_amax && !amax_ok(c_amax, c, M, N, ldc, c_type)) return aligned(c_amax, 4) ? FP4Q_EINVAL : FP4Q_EALIGN;
    if (K > 0) {
        if (!a_tensor_scale || !b_tensor_scale) return FP4Q_EINVAL;
        if (!aligned(a_tensor_scale, 4) || !aligned(b_tensor_scale, 4)) return FP4Q_EALIGN;
        const uint64_t TK = (uint64_t)(K + 127) / 128;
        const uint64_t na = domain == FP4Q_NV_GLOBAL ? 1 : (uint64_t)((M + 127) / 128) * TK;
        const uint64_t nb = domain == FP4Q_NV_GLOBAL ? 1 : (uint64_t)((N + 127) / 128) * TK;
        const uint64_t esize = c_type == FP4Q_OUT_F32 ? 4 : 2;
        const Range rc = bytes(c, ((uint64_t)(M - 1) * (uint64_t)ldc + (uint64_t)N) * esize);
        if (overlap(rc, bytes(a_tensor_scale, na * 4)) || overlap(rc, bytes(b_tensor_scale, nb * 4)))
            return FP4Q_EINVAL;
    }
    fp4q::GemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.b_codes = b_codes;
    g.b_scales = b_scales;
    g.a_ts = a_tensor_scale;
    g.b_ts = b_tensor_scale;
    g.nv_domain = domain;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.c = c;
    g.c_bf16 = c_type == FP4Q_OUT_BF16;
    g.ldc = ldc;
    g.c_amax = reinterpret_cast<uint32_t *>(c_amax);
    g.tiled = layout == FP4Q_LAYOUT_TILED;
    (void)hipGetLastError();
    return launched(fp4q::launch_gemm_nv(g, as_stream(stream)));
}


// The allocation-free variant's workspace: the global domain's partial
// maxima (at most 1024 x 4 bytes, whatever the operand's size), in a
// file-scope device array.  Each GPU holds its own copy until the process
// ends; host code uses the address hipGetSymbolAddress returns for the
// current device, never the array's name.
constexpr size_t kScratchBytes = 4096;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device).
fp4q_status scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4Q_ELAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP4Q_ELAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FP4Q_OK;
}

// use_scratch: the workspace is the library's `scratch` (workspace and
// workspace_bytes are ignored); looked up after every argument check.
fp4q_status run_quantize_nv(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, int round,
                            uint64_t seed, uint32_t stream_id, int domain, void *codes, void *scales,
                            float *tensor_scale, void *workspace, size_t workspace_bytes, int layout,
                            const float *given_amax, bool hadamard, uint32_t sign_mask, void *stream,
                            bool use_scratch = false)
{
    if ((axis != FP4Q_ALONG_ROWS && axis != FP4Q_ALONG_COLS) || (round != FP4Q_RNE && round != FP4Q_SR) ||
        (domain != FP4Q_NV_GLOBAL && domain != FP4Q_NV_TILE128) ||
        (layout != FP4Q_LAYOUT_LINEAR && layout != FP4Q_LAYOUT_TILED))
        return FP4Q_EINVAL;
    const bool tiled = layout == FP4Q_LAYOUT_TILED;
    if (rows < 0 || cols < 0 || ld_x < cols || rows > kMaxDim || cols > kMaxDim || ld_x > kMaxDim)
        return FP4Q_ESHAPE;
    if (hadamard && axis == FP4Q_ALONG_ROWS) return FP4Q_EUNSUPPORTED;
    const int64_t R = axis == FP4Q_ALONG_ROWS ? rows : cols, K = axis == FP4Q_ALONG_ROWS ? cols : rows;
    if (K % (tiled ? 128 : hadamard ? 32 : 16) != 0) return FP4Q_ESHAPE;
    if (axis == FP4Q_ALONG_COLS && cols % 4 != 0) return FP4Q_ESHAPE;
    const int64_t Rs = tiled ? (R + 31) / 32 * 32 : R;  // rows of the stored operand
    if ((uint64_t)Rs * (uint64_t)(K / 8) >= (1ull << 32)) return FP4Q_ESHAPE;
    const bool empty = R == 0 || K == 0;
    if (empty && domain == FP4Q_NV_TILE128) return FP4Q_OK;  // no tiles, no tensor scales
    if (!tensor_scale) return FP4Q_EINVAL;
    if (!empty && (!x || !codes || !scales)) return FP4Q_EINVAL;
    if (!empty && (!aligned(x, 16) || !aligned(codes, 16) || ld_x % 8 != 0)) return FP4Q_EALIGN;
    if (!empty && tiled && !aligned(scales, 16)) return FP4Q_EALIGN;
    if (!aligned(tensor_scale, 4)) return FP4Q_EALIGN;
    const size_t need = given_amax ? 0 : fp4q_nv_workspace_bytes(rows, cols, axis, domain);
    if (use_scratch) {
        if (need > kScratchBytes) return FP4Q_EINVAL;  // the partial maxima never need more
        workspace = nullptr;
    } else {
        if (need > 0 && (!workspace || workspace_bytes < need)) return FP4Q_EINVAL;
        if (need > 0 && !aligned(workspace, 4)) return FP4Q_EALIGN;
    }
    const uint64_t nts = domain == FP4Q_NV_GLOBAL ? 1 : (uint64_t)((R + 127) / 128) * (uint64_t)((K + 127) / 128);
    const Range rx = bytes(x, input_span(rows, cols, ld_x));
    const Range outs[4] = {bytes(codes, (uint64_t)Rs * K / 2), bytes(scales, (uint64_t)Rs * K / 16),
                           bytes(tensor_scale, nts * 4), bytes(workspace, use_scratch ? 0 : need)};
    for (int i = 0; i < 4; ++i) {
        if (overlap(rx, outs[i])) return FP4Q_EINVAL;
        if (given_amax && overlap(bytes(given_amax, 4), outs[i])) return FP4Q_EINVAL;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FP4Q_EINVAL;
    }
    fp4q::QuantArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld_x;
    a.axis = axis;
    a.sr = round == FP4Q_SR;
    a.seed = seed;
    a.stream_id = stream_id;
    a.hadamard = hadamard;
    a.sign_mask = sign_mask;
    a.tiled = tiled;
    a.codes = codes;
    a.scales = scales;
    if (use_scratch && need > 0) {
        const fp4q_status st = scratch_of_current_device(&workspace);
        if (st != FP4Q_OK) return st;
    }
    (void)hipGetLastError();
    return launched(fp4q::launch_quant_nv(a, domain, tensor_scale, workspace, given_amax, as_stream(stream)));
}

}  // namespace

extern "C" {

fp4q_status fp4_quantize_mx(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, int round,
                            uint64_t seed, uint32_t stream_id, void *codes, void *scales, int layout, void *stream)
{
    return run_mx_producer(x, rows, cols, ld_x, axis, false, 0u, round, seed, stream_id, codes, scales, layout,
                           stream);
}

fp4q_status fp4_hadamard32_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                                    uint32_t sign_mask, int round, uint64_t seed, uint32_t stream_id, void *codes,
                                    void *scales, int layout, void *stream)
{
    return run_mx_producer(x, rows, cols, ld_x, axis, true, sign_mask, round, seed, stream_id, codes, scales, layout,
                           stream);
}

fp4q_status fp4_quantize_mx_dual(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int round_rows,
                                 uint32_t stream_id_rows, void *codes_rows, void *scales_rows, int hadamard_cols,
                                 uint32_t sign_mask, int round_cols, uint32_t stream_id_cols, void *codes_cols,
                                 void *scales_cols, uint64_t seed, int layout, void *stream)
{
    if (hadamard_cols != 0 && hadamard_cols != 1) return FP4Q_EINVAL;
    bool empty = false;
    fp4q_status st = check_mx_producer(x, rows, cols, ld_x, FP4Q_ALONG_ROWS, round_rows, codes_rows, scales_rows,
                                       layout, &empty);
    if (st != FP4Q_OK) return st;
    st = check_mx_producer(x, rows, cols, ld_x, FP4Q_ALONG_COLS, round_cols, codes_cols, scales_cols, layout, &empty);
    if (st != FP4Q_OK || empty) return st;
    // K % 32 (or 128) of both operands makes rows and cols multiples of the
    // block, so neither operand has padding rows
    const uint64_t n = (uint64_t)rows * (uint64_t)cols;
    const Range outs[4] = {bytes(codes_rows, n / 2), bytes(scales_rows, n / 32), bytes(codes_cols, n / 2),
                           bytes(scales_cols, n / 32)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FP4Q_EINVAL;
    fp4q::QuantArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld_x;
    a.axis = FP4Q_ALONG_COLS;
    a.sr = round_cols == FP4Q_SR;
    a.hadamard = hadamard_cols != 0;
    a.tiled = layout == FP4Q_LAYOUT_TILED;
    a.seed = seed;
    a.stream_id = stream_id_cols;
    a.sign_mask = sign_mask;
    a.codes = codes_cols;
    a.scales = scales_cols;
    a.rows_round = round_rows == FP4Q_SR ? 2 : 1;
    a.stream_id_rows = stream_id_rows;
    a.codes_rows = codes_rows;
    a.scales_rows = scales_rows;
    (void)hipGetLastError();
    return launched(fp4q::launch_quant_mx(a, as_stream(stream)));
}

size_t fp4q_nv_workspace_bytes(int64_t rows, int64_t cols, int axis, int domain)
{
    (void)rows;
    (void)cols;
    (void)axis;
    return domain == FP4Q_NV_GLOBAL ? fp4q::nv_workspace_bytes(0) : 0;
}

fp4q_status fp4_quantize_nv(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, int round,
                            uint64_t seed, uint32_t stream_id, int domain, void *codes, void *scales,
                            float *tensor_scale, void *workspace, size_t workspace_bytes, int layout, void *stream)
{
    return run_quantize_nv(x, rows, cols, ld_x, axis, round, seed, stream_id, domain, codes, scales, tensor_scale,
                           workspace, workspace_bytes, layout, nullptr, false, 0u, stream);
}

fp4q_status fp4_quantize_nv_noalloc(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis, int round,
                                    uint64_t seed, uint32_t stream_id, int domain, void *codes, void *scales,
                                    float *tensor_scale, int layout, void *stream)
{
    return run_quantize_nv(x, rows, cols, ld_x, axis, round, seed, stream_id, domain, codes, scales, tensor_scale,
                           nullptr, 0, layout, nullptr, false, 0u, stream, true);
}

fp4q_status fp4_hadamard32_quantize_nv(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                                       uint32_t sign_mask, int round, uint64_t seed, uint32_t stream_id, int domain,
                                       void *codes, void *scales, float *tensor_scale, void *workspace,
                                       size_t workspace_bytes, int layout, void *stream)
{
    return run_quantize_nv(x, rows, cols, ld_x, axis, round, seed, stream_id, domain, codes, scales, tensor_scale,
                           workspace, workspace_bytes, layout, nullptr, true, sign_mask, stream);
}

fp4q_status fp4_gemm_mx(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                        int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type, int64_t ldc,
                        void *stream)
{
    return run_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, alpha, layout, c, c_type, ldc, nullptr, stream);
}

fp4q_status fp4_gemm_mx_amax(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                             int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type,
                             int64_t ldc, float *c_amax, void *stream)
{
    if (!c_amax) return FP4Q_EINVAL;
    return run_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, alpha, layout, c, c_type, ldc, c_amax, stream);
}

fp4q_status fp4_gemm_mx_quant(const void *a_codes, const void *a_scales, const void *b_codes, const void *b_scales,
                              int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c_codes, void *c_scales,
                              int c_layout, void *stream)
{
    return run_gemm_mx_quant(a_codes, a_scales, b_codes, b_scales, M, N, K, alpha, layout, c_codes, c_scales,
                             c_layout, false, stream);
}

fp4q_status fp4_gemm_mx_swiglu_quant(const void *a_codes, const void *a_scales, const void *b_codes,
                                     const void *b_scales, int64_t M, int64_t N, int64_t K, float alpha, int layout,
                                     void *h_codes, void *h_scales, int h_layout, void *stream)
{
    return run_gemm_mx_quant(a_codes, a_scales, b_codes, b_scales, M, N, K, alpha, layout, h_codes, h_scales,
                             h_layout, true, stream);
}

fp4q_status fp4_swiglu_bf16(const void *c, int64_t M, int64_t F, int64_t ldc, int64_t pair, void *h, int64_t ldh,
                            void *stream)
{
    if (M < 0 || F < 0 || M > kMaxDim || F > kMaxDim) return FP4Q_ESHAPE;
    if (F % 8 != 0 || pair <= 0 || pair % 8 != 0 || (F > 0 && F % pair != 0) || ldc < 2 * F || ldh < F ||
        ldc % 8 != 0 || ldh % 8 != 0 || ldc > kMaxDim * 2 || ldh > kMaxDim)
        return FP4Q_ESHAPE;
    if (M == 0 || F == 0) return FP4Q_OK;
    if (!c || !h) return FP4Q_EINVAL;
    if (!aligned(c, 16) || !aligned(h, 16)) return FP4Q_EALIGN;
    const Range rc = bytes(c, ((uint64_t)(M - 1) * (uint64_t)ldc + 2 * (uint64_t)F) * 2);
    const Range rh = bytes(h, ((uint64_t)(M - 1) * (uint64_t)ldh + (uint64_t)F) * 2);
    if (overlap(rc, rh)) return FP4Q_EINVAL;
    (void)hipGetLastError();
    return launched(fp4q::launch_swiglu(c, M, F, ldc, pair, h, ldh, as_stream(stream)));
}

fp4q_status fp4_gemm_nv(const void *a_codes, const void *a_scales, const float *a_tensor_scale, const void *b_codes,
                        const void *b_scales, const float *b_tensor_scale, int domain, int64_t M, int64_t N,
                        int64_t K, float alpha, int layout, void *c, int c_type, int64_t ldc, void *stream)
{
    return run_gemm_nv(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, domain, M, N, K, alpha,
                       layout, c, c_type, ldc, nullptr, stream);
}

fp4q_status fp4_gemm_nv_amax(const void *a_codes, const void *a_scales, const float *a_tensor_scale,
                             const void *b_codes, const void *b_scales, const float *b_tensor_scale, int domain,
                             int64_t M, int64_t N, int64_t K, float alpha, int layout, void *c, int c_type,
                             int64_t ldc, float *c_amax, void *stream)
{
    if (!c_amax) return FP4Q_EINVAL;
    return run_gemm_nv(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, domain, M, N, K, alpha,
                       layout, c, c_type, ldc, c_amax, stream);
}

fp4q_status fp4_quantize_nv_amax(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int round, uint64_t seed,
                                 uint32_t stream_id, const float *amax, void *codes, void *scales,
                                 float *tensor_scale, void *stream)
{
    if (!amax) return FP4Q_EINVAL;
    if (!aligned(amax, 4)) return FP4Q_EALIGN;
    return run_quantize_nv(x, rows, cols, ld_x, FP4Q_ALONG_ROWS, round, seed, stream_id, FP4Q_NV_GLOBAL, codes,
                           scales, tensor_scale, nullptr, 0, FP4Q_LAYOUT_LINEAR, amax, false, 0u, stream);
}

const char *fp4q_status_str(int status)
{
    switch (status) {
    case FP4Q_OK: return "ok";
    case FP4Q_EINVAL: return "invalid argument (null pointer, unknown enum, overlapping buffers or small workspace)";
    case FP4Q_ESHAPE: return "unsupported shape (block multiple, leading dimension or size limit)";
    case FP4Q_EALIGN: return "misaligned pointer or leading dimension";
    case FP4Q_ELAUNCH: return "kernel launch failed";
    case FP4Q_EUNSUPPORTED: return "valid combination not implemented by this build";
    default: return "unknown status";
    }
}

int fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

}  // extern "C"
