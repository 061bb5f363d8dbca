// C ABI entry points of libw4a4.so: argument validation on the host, workspace carving, launches.
// Every check runs before anything is enqueued, so a failing call launches nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>

#include "w4a4_internal.h"

namespace w4a4 {

static thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(W4A4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return W4A4_OK;
}

int ensure_dynamic_lds(const void *kernel, size_t bytes, const char *what)
{
    static std::mutex mu;
    static std::map<std::pair<const void *, int>, size_t> granted;  // (kernel, device) -> bytes
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4A4_ERR_HIP, "%s LDS request: %s", what, hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    size_t &have = granted[{kernel, dev}];
    if (have >= bytes) return W4A4_OK;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return fail(W4A4_ERR_HIP, "%s LDS request: %s", what, hipGetErrorString(e));
    have = bytes;
    return W4A4_OK;
}

static int ok()
{
    g_err[0] = '\0';
    return W4A4_OK;
}

static bool pow2_block(int B) { return B >= 1 && B <= 256 && (B & (B - 1)) == 0; }

static int check_dtype(int dt, const char *name)
{
    if (dt != W4A4_F16 && dt != W4A4_F32) return fail(W4A4_ERR_ARG, "%s dtype %d unknown", name, dt);
    return W4A4_OK;
}

static size_t dtype_bytes(int dt) { return dt == W4A4_F16 ? 2 : 4; }

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shape rules shared by every call that takes K and a block size.
static int check_kb(int K, int B)
{
    if (!pow2_block(B))
        return fail(W4A4_ERR_UNSUPPORTED, "block %d is not a power of two in [1, 256]", B);
    if (K <= 0) return fail(W4A4_ERR_ARG, "K = %d must be positive", K);
    if (K % 2) return fail(W4A4_ERR_SHAPE, "K = %d must be even (two int4 codes per byte)", K);
    if (K % B) return fail(W4A4_ERR_SHAPE, "K = %d is not a multiple of the block %d", K, B);
    if (K > (1 << 24)) return fail(W4A4_ERR_UNSUPPORTED, "K = %d above 2^24", K);
    return W4A4_OK;
}

static int check_matrix(const void *A, int dt, int rows, int K, int64_t ld, const char *name)
{
    int rc = check_dtype(dt, name);
    if (rc) return rc;
    if (rows < 0) return fail(W4A4_ERR_ARG, "%s rows = %d negative", name, rows);
    if (ld < K) return fail(W4A4_ERR_SHAPE, "%s leading dimension %lld < K = %d", name,
                            (long long)ld, K);
    if (rows > 0 && !A) return fail(W4A4_ERR_ARG, "%s is NULL", name);
    if (!aligned(A, dtype_bytes(dt))) return fail(W4A4_ERR_ALIGN, "%s misaligned for its dtype", name);
    if ((int64_t)rows * ld > ((int64_t)1 << 40))
        return fail(W4A4_ERR_UNSUPPORTED, "%s larger than 2^40 elements", name);
    return W4A4_OK;
}

static int check_ws(const void *ws, size_t have, size_t need)
{
    if (need == 0) return W4A4_OK;
    if (!ws || have < need)
        return fail(W4A4_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, have,
                    ws ? "" : " (NULL)");
    if (!aligned(ws, 256)) return fail(W4A4_ERR_ALIGN, "workspace must be 256-byte aligned");
    return W4A4_OK;
}

// ---- activation path plumbing shared by rotate_quant_act and calibrate_act_scale -------------
enum ActKind { KIND_STEP = 0, KIND_TOKEN = 1, KIND_CALIB = 2 };

static bool act_on_mfma(int xdt, int B) { return xdt == W4A4_F16 && (B == 64 || B == 128); }

static size_t act_ws_bytes(int M, int K, int B, int kind)
{
    // maxima: one per row (per-token), one per rotation block (calibration, grouped or not)
    const int nmax = (kind == KIND_CALIB) ? max(max(M, 1), K / B) : max(M, 1);
    size_t n = (kind == KIND_STEP) ? 0 : align_up((size_t)nmax * sizeof(uint32_t), 256);
    if (M > 0 && (B == 64 || B == 128) && act_uses_permute_pass(M, K, kind != KIND_STEP))
        n += act_permute_bytes(M, K);
    return n;
}

// xf (FP6 output, int4 codes only): the codes are written in the FP6 operand layout, by the
// streaming kernel itself when it runs (block 128), else as packed int4 into the workspace after
// act_ws_bytes and re-encoded from there.
static int run_activation(const void *X, int xdt, int M, int K, int64_t ldx, int B,
                          const int32_t *perm, const void *rot, const float *table, int step,
                          int kind, uint8_t *xq, float *x_scale, float *xrot, void *ws,
                          float *calib_out, hipStream_t s, bool q8 = false, bool grouped = false,
                          uint8_t *xf = nullptr)
{
    int rc;
    char *w = reinterpret_cast<char *>(ws);
    uint8_t *f6_tmp = xf ? reinterpret_cast<uint8_t *>(w + act_ws_bytes(M, K, B, kind)) : nullptr;
    if (xf) xq = f6_tmp;
    auto finish_f6 = [&](bool direct) {
        return (xf && !direct) ? launch_codes_to_f6(f6_tmp, M, K, xf, s) : W4A4_OK;
    };
    uint32_t *rowmax = reinterpret_cast<uint32_t *>(w);
    const int nb = K / B;
    const int nmax = (kind == KIND_CALIB) ? max(max(M, 1), nb) : max(M, 1);
    const size_t off = (kind == KIND_STEP) ? 0 : align_up((size_t)nmax * sizeof(uint32_t), 256);
    const bool permute_pass = act_on_mfma(xdt, B) && perm && act_uses_permute_pass(M, K, kind != KIND_STEP);
    // the maxima start at zero: cleared by the permutation pass (its first M entries) when there
    // is one; group-wise scales (grouped) index the table row and the maxima by rotation block
    const int nclear = (kind == KIND_CALIB) ? (grouped ? nb : 1) : M;
    if (kind != KIND_STEP && (!permute_pass || nclear > M) &&
        (rc = launch_fill_u32(rowmax, 0u, nclear, s)))
        return rc;
    const int gstride = grouped ? 1 : 0;
    if (grouped && kind == KIND_STEP) {
        table += (size_t)step * nb;
        step = 0;
    }
    if (act_on_mfma(xdt, B)) {
        const uint16_t *xperm = nullptr;
        if (permute_pass) {
            uint16_t *xp = reinterpret_cast<uint16_t *>(w + off);
            if ((rc = launch_permute_rows(X, M, K, ldx, perm, xp,
                                          kind == KIND_STEP ? nullptr : rowmax, s)))
                return rc;
            xperm = xp;
        }
        const bool f6_direct = xf && B == 128 && !xrot && rq_ring_path(M, X, ldx, perm, xperm, K);
        uint8_t *qout = f6_direct ? xf : xq;
        if (kind == KIND_STEP) {
            if ((rc = launch_rotate_quant_mfma(X, M, K, ldx, B, perm, rot, table, step, ACT_PER_STEP,
                                               nullptr, qout, x_scale, xrot, xperm, q8, s, gstride,
                                               f6_direct)))
                return rc;
            return finish_f6(f6_direct);
        }
        if (kind == KIND_CALIB) {
            if ((rc = launch_rotate_quant_mfma(X, M, K, ldx, B, perm, rot, nullptr, 0,
                                               ACT_CALIB_MAX, rowmax, nullptr, nullptr, nullptr,
                                               xperm, false, s, gstride)))
                return rc;
            return launch_scale_from_absmax(rowmax, calib_out, q8, s, grouped ? nb : 1);
        }
        if ((rc = launch_rotate_quant_mfma(X, M, K, ldx, B, perm, rot, nullptr, 0, ACT_TOKEN_MAX,
                                           rowmax, nullptr, nullptr, nullptr, xperm, false, s)))
            return rc;
        if ((rc = launch_rotate_quant_mfma(X, M, K, ldx, B, perm, rot, nullptr, 0, ACT_TOKEN_QUANT,
                                           rowmax, qout, x_scale, xrot, xperm, q8, s, 0, f6_direct)))
            return rc;
        return finish_f6(f6_direct);
    }
    if (kind == KIND_STEP) {
        if ((rc = launch_rotate_quant(X, xdt, M, K, ldx, B, perm, rot, table, step, ACT_PER_STEP,
                                      nullptr, xq, x_scale, xrot, q8, s)))
            return rc;
        return finish_f6(false);
    }
    if (kind == KIND_CALIB) {
        if ((rc = launch_rotate_quant(X, xdt, M, K, ldx, B, perm, rot, nullptr, 0, ACT_CALIB_MAX,
                                      rowmax, nullptr, nullptr, nullptr, false, s)))
            return rc;
        return launch_scale_from_absmax(rowmax, calib_out, q8, s);
    }
    if ((rc = launch_rotate_quant(X, xdt, M, K, ldx, B, perm, rot, nullptr, 0, ACT_TOKEN_MAX,
                                  rowmax, nullptr, nullptr, nullptr, false, s)))
        return rc;
    if ((rc = launch_rotate_quant(X, xdt, M, K, ldx, B, perm, rot, nullptr, 0, ACT_TOKEN_QUANT,
                                  rowmax, xq, x_scale, xrot, q8, s)))
        return rc;
    return finish_f6(false);
}

}  // namespace w4a4

using namespace w4a4;

extern "C" {

int w4a4_abi_version(void) { return 1; }

const char *w4a4_last_error(void) { return g_err; }

const char *w4a4_status_string(int status)
{
    switch (status) {
    case W4A4_OK: return "W4A4_OK";
    case W4A4_ERR_ARG: return "W4A4_ERR_ARG";
    case W4A4_ERR_SHAPE: return "W4A4_ERR_SHAPE";
    case W4A4_ERR_STEP_RANGE: return "W4A4_ERR_STEP_RANGE";
    case W4A4_ERR_UNSUPPORTED: return "W4A4_ERR_UNSUPPORTED";
    case W4A4_ERR_ALIGN: return "W4A4_ERR_ALIGN";
    case W4A4_ERR_WORKSPACE: return "W4A4_ERR_WORKSPACE";
    case W4A4_ERR_HIP: return "W4A4_ERR_HIP";
    default: return "W4A4_ERR_UNKNOWN";
    }
}

// ------------------------------------------------------------------ calibration

size_t w4a4_zigzag_workspace_bytes(int K) { return K > 0 ? zigzag_workspace(K) : 0; }

int w4a4_zigzag_perm(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                     int32_t *perm, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if (N <= 0) return fail(W4A4_ERR_ARG, "N = %d must be positive", N);
    if ((rc = check_matrix(W, w_dtype, N, K, ldw, "W"))) return rc;
    if (!perm) return fail(W4A4_ERR_ARG, "perm is NULL");
    if ((rc = check_ws(ws, ws_bytes, zigzag_workspace(K)))) return rc;
    if ((rc = launch_zigzag(W, w_dtype, N, K, ldw, block, perm, ws, stream))) return rc;
    return ok();
}

size_t w4a4_block_svd_workspace_bytes(int N, int K, int block)
{
    if (N <= 0 || K <= 0 || !pow2_block(block) || K % block) return 0;
    return block_svd_workspace(N, K, block);
}

int w4a4_block_svd(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                   const int32_t *perm, float *U, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if (block > 128) return fail(W4A4_ERR_UNSUPPORTED, "device SVD supports block <= 128");
    if (N <= 0) return fail(W4A4_ERR_ARG, "N = %d must be positive", N);
    if ((rc = check_matrix(W, w_dtype, N, K, ldw, "W"))) return rc;
    if (!U) return fail(W4A4_ERR_ARG, "U is NULL");
    if ((rc = check_ws(ws, ws_bytes, block_svd_workspace(N, K, block)))) return rc;
    if ((rc = launch_block_svd(W, w_dtype, N, K, ldw, block, perm, U, ws, stream))) return rc;
    return ok();
}

size_t w4a4_calibrate_workspace_bytes(int M, int K, int block)
{
    if (M < 0 || K <= 0 || !pow2_block(block) || K % block) return 0;
    return act_ws_bytes(M, K, block, KIND_CALIB);
}

static int calibrate_entry(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                           const int32_t *perm, const void *rot, float *table_entry, void *ws,
                           size_t ws_bytes, hipStream_t stream, bool q8)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if ((rc = check_matrix(X, x_dtype, M, K, ldx, "X"))) return rc;
    if (!rot) return fail(W4A4_ERR_ARG, "rot is NULL");
    if (!aligned(rot, 16)) return fail(W4A4_ERR_ALIGN, "rot must be 16-byte aligned");
    if (!table_entry) return fail(W4A4_ERR_ARG, "table_entry is NULL");
    if (!aligned(perm, 4)) return fail(W4A4_ERR_ALIGN, "perm misaligned");
    if ((rc = check_ws(ws, ws_bytes, act_ws_bytes(M, K, block, KIND_CALIB)))) return rc;
    if ((rc = run_activation(X, x_dtype, M, K, ldx, block, perm, rot, nullptr, 0, KIND_CALIB,
                             nullptr, nullptr, nullptr, ws, table_entry, stream, q8)))
        return rc;
    return ok();
}

int w4a4_calibrate_act_scale(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                             const int32_t *perm, const void *rot, float *table_entry,
                             void *ws, size_t ws_bytes, hipStream_t stream)
{
    return calibrate_entry(X, x_dtype, M, K, ldx, block, perm, rot, table_entry, ws, ws_bytes,
                           stream, false);
}

int w4a4_calibrate_act_scale_a8(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                                const int32_t *perm, const void *rot, float *table_entry,
                                void *ws, size_t ws_bytes, hipStream_t stream)
{
    return calibrate_entry(X, x_dtype, M, K, ldx, block, perm, rot, table_entry, ws, ws_bytes,
                           stream, true);
}

// ------------------------------------------------------------------ weight pack

size_t w4a4_rot_bytes(int K, int block)
{
    if (K <= 0 || !pow2_block(block) || K % block) return 0;
    return rot_layout(K, block).total;
}

size_t w4a4_pack_workspace_bytes(int N, int K, int block)
{
    if (N <= 0 || K <= 0 || !pow2_block(block) || K % block) return 0;
    return align_up((size_t)K * block * sizeof(double), 256) + align_up((size_t)N * 8, 256);
}

static int pack_entry(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                      const int32_t *perm, const float *U, uint8_t *wq, float *w_scale, void *rot,
                      void *ws, size_t ws_bytes, hipStream_t stream, int bits)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if (N <= 0) return fail(W4A4_ERR_ARG, "N = %d must be positive", N);
    if ((rc = check_matrix(W, w_dtype, N, K, ldw, "W"))) return rc;
    if (!wq || !w_scale || !rot) return fail(W4A4_ERR_ARG, "wq, w_scale and rot are required");
    if (!aligned(U, 4) || !aligned(w_scale, 4)) return fail(W4A4_ERR_ALIGN, "U / w_scale misaligned");
    if (!aligned(rot, 16)) return fail(W4A4_ERR_ALIGN, "rot must be 16-byte aligned");
    if (!aligned(perm, 4)) return fail(W4A4_ERR_ALIGN, "perm misaligned");
    if ((rc = check_ws(ws, ws_bytes, w4a4_pack_workspace_bytes(N, K, block)))) return rc;
    double *R64 = reinterpret_cast<double *>(ws);
    unsigned long long *rowmax = reinterpret_cast<unsigned long long *>(
        reinterpret_cast<char *>(ws) + align_up((size_t)K * block * sizeof(double), 256));
    const double hinv = 1.0 / std::sqrt((double)block);
    if ((rc = launch_rotation(U, K, block, hinv, R64, rot, stream))) return rc;
    if (bits == 8 && !aligned(wq, 2)) return fail(W4A4_ERR_ALIGN, "int8 wq must be 2-byte aligned");
    if ((rc = launch_weight_pack(W, w_dtype, N, K, ldw, block, perm, R64, rowmax, wq, w_scale, bits,
                                 stream)))
        return rc;
    return ok();
}

int w4a4_pack_weights(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                      const int32_t *perm, const float *U, uint8_t *wq, float *w_scale, void *rot,
                      void *ws, size_t ws_bytes, hipStream_t stream)
{
    return pack_entry(W, w_dtype, N, K, ldw, block, perm, U, wq, w_scale, rot, ws, ws_bytes, stream,
                      4);
}

int w4a4_pack_weights_w8(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                         const int32_t *perm, const float *U, uint8_t *wq, float *w_scale,
                         void *rot, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return pack_entry(W, w_dtype, N, K, ldw, block, perm, U, wq, w_scale, rot, ws, ws_bytes, stream,
                      8);
}

// ------------------------------------------------------------------ activation path

size_t w4a4_act_workspace_bytes(int M, int K, int block, int per_token)
{
    if (M <= 0 || K <= 0 || !pow2_block(block) || K % block) return 0;
    return act_ws_bytes(M, K, block, per_token ? KIND_TOKEN : KIND_STEP);
}

static size_t act_f6_ws_bytes(int M, int K, int block, int per_token)
{
    return act_ws_bytes(M, K, block, per_token ? KIND_TOKEN : KIND_STEP) +
           align_up((size_t)M * (K / 2), 256);
}

static int rq_entry(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                    const int32_t *perm, const void *rot, const float *act_scale_table,
                    int num_steps, int step, uint8_t *xq, float *x_scale, float *xrot_dbg,
                    void *ws, size_t ws_bytes, hipStream_t stream, bool q8, uint8_t *xf = nullptr)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if ((rc = check_matrix(X, x_dtype, M, K, ldx, "X"))) return rc;
    if (!rot) return fail(W4A4_ERR_ARG, "rot is NULL");
    if (!aligned(rot, 16)) return fail(W4A4_ERR_ALIGN, "rot must be 16-byte aligned");
    if (!aligned(perm, 4)) return fail(W4A4_ERR_ALIGN, "perm misaligned");
    const bool per_step = act_scale_table != nullptr;
    if (per_step) {
        if (num_steps <= 0) return fail(W4A4_ERR_STEP_RANGE, "num_steps = %d must be positive",
                                        num_steps);
        if (step < 0 || step >= num_steps)
            return fail(W4A4_ERR_STEP_RANGE, "step %d outside [0, %d)", step, num_steps);
        if (!aligned(act_scale_table, 4)) return fail(W4A4_ERR_ALIGN, "table misaligned");
    }
    if (xf) {
        if (block != 128)
            return fail(W4A4_ERR_UNSUPPORTED, "FP6 activation output needs block 128 (got %d)", block);
        if (!aligned(xf, 16)) return fail(W4A4_ERR_ALIGN, "xf must be 16-byte aligned");
        if ((int64_t)((M + 1) & ~1) * (K / 32) > INT32_MAX)
            return fail(W4A4_ERR_UNSUPPORTED, "FP6 operand of %d x %d beyond int32 indexing", M, K);
    } else if (M > 0 && !xq) {
        return fail(W4A4_ERR_ARG, "xq and x_scale are required");
    }
    if (M > 0 && !x_scale) return fail(W4A4_ERR_ARG, "xq and x_scale are required");
    if (!aligned(x_scale, 4) || !aligned(xrot_dbg, 4))
        return fail(W4A4_ERR_ALIGN, "x_scale / xrot_dbg misaligned");
    const size_t need = xf ? (M > 0 ? act_f6_ws_bytes(M, K, block, !per_step) : 0)
                           : w4a4_act_workspace_bytes(M, K, block, !per_step);
    if ((rc = check_ws(ws, ws_bytes, need))) return rc;
    if (M == 0) return ok();
    if (q8 && !aligned(xq, 4)) return fail(W4A4_ERR_ALIGN, "int8 xq must be 4-byte aligned");
    if ((rc = run_activation(X, x_dtype, M, K, ldx, block, perm, rot, act_scale_table, step,
                             per_step ? KIND_STEP : KIND_TOKEN, xq, x_scale, xrot_dbg, ws, nullptr,
                             stream, q8, false, xf)))
        return rc;
    return ok();
}

int w4a4_rotate_quant_act(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                          const int32_t *perm, const void *rot, const float *act_scale_table,
                          int num_steps, int step, uint8_t *xq, float *x_scale, float *xrot_dbg,
                          void *ws, size_t ws_bytes, hipStream_t stream)
{
    return rq_entry(X, x_dtype, M, K, ldx, block, perm, rot, act_scale_table, num_steps, step, xq,
                    x_scale, xrot_dbg, ws, ws_bytes, stream, false);
}

// ---- rotate-quantize without allocation: scratch in a file-scope device array ---------------
//
// The array is part of the library's code object, so every GPU the library runs on holds its own
// copy from module load until the process ends. Host code never passes the array's name to a
// kernel (on the host it is a stand-in symbol, not a device address): the device address is taken
// once per device with hipGetSymbolAddress, with that device current, and kept per device.
}  // extern "C"

namespace w4a4 {
namespace {
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void *g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

int scratch_for_current_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4A4_ERR_HIP, "scratch: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(W4A4_ERR_UNSUPPORTED, "scratch: device %d beyond %d", dev, NOALLOC_MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(W4A4_ERR_HIP, "scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4A4_OK;
}
}  // namespace
}  // namespace w4a4

extern "C" {

size_t w4a4_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

int w4a4_rotate_quant_act_noalloc(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                                  const int32_t *perm, const void *rot,
                                  const float *act_scale_table, int num_steps, int step,
                                  uint8_t *xq, float *x_scale, float *xrot_dbg, hipStream_t stream)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    const size_t need = w4a4_act_workspace_bytes(M, K, block, act_scale_table == nullptr);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(W4A4_ERR_UNSUPPORTED,
                    "rotate-quantize of %d x %d needs %zu scratch bytes, above the %zu-byte maximum "
                    "of the allocation-free call", M, K, need, NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0 && (rc = scratch_for_current_device(&ws))) return rc;
    return rq_entry(X, x_dtype, M, K, ldx, block, perm, rot, act_scale_table, num_steps, step, xq,
                    x_scale, xrot_dbg, ws, need > 0 ? NOALLOC_SCRATCH_BYTES : 0, stream, false);
}

size_t w4a4_act_f6_workspace_bytes(int M, int K, int block, int per_token)
{
    if (M <= 0 || K <= 0 || block != 128 || K % block) return 0;
    return act_f6_ws_bytes(M, K, block, per_token);
}

int w4a4_rotate_quant_act_f6(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                             const int32_t *perm, const void *rot, const float *act_scale_table,
                             int num_steps, int step, uint8_t *xf, float *x_scale, void *ws,
                             size_t ws_bytes, hipStream_t stream)
{
    if (M > 0 && !xf) return fail(W4A4_ERR_ARG, "xf is required");
    return rq_entry(X, x_dtype, M, K, ldx, block, perm, rot, act_scale_table, num_steps, step,
                    nullptr, x_scale, nullptr, ws, ws_bytes, stream, false, xf);
}

int w4a4_rotate_quant_act_a8(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                             const int32_t *perm, const void *rot, const float *act_scale_table,
                             int num_steps, int step, uint8_t *xq, float *x_scale,
                             float *xrot_dbg, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return rq_entry(X, x_dtype, M, K, ldx, block, perm, rot, act_scale_table, num_steps, step, xq,
                    x_scale, xrot_dbg, ws, ws_bytes, stream, true);
}

int w4a4_rotate_quant_act_hadamard(const void *X, int x_dtype, int M, int K, int64_t ldx,
                                   int block, const int32_t *perm, const float *act_scale_table,
                                   int num_steps, int step, uint8_t *xq, float *x_scale,
                                   float *xrot_dbg, hipStream_t stream)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if (block != 64 && block != 128)
        return fail(W4A4_ERR_UNSUPPORTED, "Hadamard-only rotation supports block 64 or 128, not %d",
                    block);
    if ((rc = check_matrix(X, x_dtype, M, K, ldx, "X"))) return rc;
    if (hadamard_lds_bytes(1, K, block, x_dtype, nullptr) > 128 * 1024)
        return fail(W4A4_ERR_UNSUPPORTED, "K = %d too long for the staged-row Hadamard kernel "
                    "(at most 65536 fp16 or 32768 fp32 values per row)", K);
    if (!aligned(perm, 4)) return fail(W4A4_ERR_ALIGN, "perm misaligned");
    const bool per_step = act_scale_table != nullptr;
    if (per_step) {
        if (num_steps <= 0) return fail(W4A4_ERR_STEP_RANGE, "num_steps = %d must be positive",
                                        num_steps);
        if (step < 0 || step >= num_steps)
            return fail(W4A4_ERR_STEP_RANGE, "step %d outside [0, %d)", step, num_steps);
        if (!aligned(act_scale_table, 4)) return fail(W4A4_ERR_ALIGN, "table misaligned");
    }
    if (M > 0 && (!xq || !x_scale)) return fail(W4A4_ERR_ARG, "xq and x_scale are required");
    if (!aligned(xq, 16)) return fail(W4A4_ERR_ALIGN, "xq must be 16-byte aligned");
    if (!aligned(x_scale, 4) || !aligned(xrot_dbg, 4))
        return fail(W4A4_ERR_ALIGN, "x_scale / xrot_dbg misaligned");
    if (M == 0) return ok();
    if ((rc = launch_rotate_quant_hadamard(X, x_dtype, M, K, ldx, block, perm, act_scale_table, step,
                                           xq, x_scale, xrot_dbg, stream)))
        return rc;
    return ok();
}

// ------------------------------------------------------------------ GEMM

size_t w4a4_gemm_workspace_bytes(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return gemm_workspace(M, N, K, false);
}

size_t w4a4_gemm_w8a8_workspace_bytes(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return gemm_workspace(M, N, K, true);
}

}  // extern "C"

namespace w4a4 {

// operand formats of the GEMM entry points
enum { OPF_I4 = 0, OPF_I8 = 1, OPF_F6 = 2 };

static size_t gemm_ws_for(int M, int N, int K, int fmt)
{
    return fmt == OPF_F6 ? gemm_f6_workspace(M, N, K) : gemm_workspace(M, N, K, fmt == OPF_I8);
}

static int check_gemm_common(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, int fmt)
{
    if (M < 0 || N <= 0 || K <= 0) return fail(W4A4_ERR_ARG, "bad sizes M=%d N=%d K=%d", M, N, K);
    if ((M > 0 && !xq) || !wq) return fail(W4A4_ERR_ARG, "xq / wq is NULL");
    if (fmt == OPF_I4) {
        if (K % 2) return fail(W4A4_ERR_SHAPE, "K = %d must be even", K);
        if (K > (1 << 24)) return fail(W4A4_ERR_UNSUPPORTED, "K = %d above 2^24", K);
        return W4A4_OK;
    }
    if (fmt == OPF_F6) {
        if (K % 128) return fail(W4A4_ERR_SHAPE, "fp6 GEMM needs K a multiple of 128, not %d", K);
        if (K > (1 << 18))
            return fail(W4A4_ERR_UNSUPPORTED, "fp6 GEMM K = %d above 2^18 (exact fp32 sums)", K);
        if (!aligned(xq, 16) || !aligned(wq, 16))
            return fail(W4A4_ERR_ALIGN, "fp6 operands must be 16-byte aligned");
        return W4A4_OK;
    }
    if (K % 64) return fail(W4A4_ERR_SHAPE, "int8 GEMM needs K a multiple of 64, not %d", K);
    if (K > (1 << 16))
        return fail(W4A4_ERR_UNSUPPORTED, "int8 GEMM K = %d above 2^16 (int32 sums)", K);
    if (!aligned(xq, 16) || !aligned(wq, 16))
        return fail(W4A4_ERR_ALIGN, "int8 operands must be 16-byte aligned");
    return W4A4_OK;
}

static int gemm_entry(const uint8_t *xq, const float *x_scale, int x_scale_per_token,
                      const uint8_t *wq, const float *w_scale, int M, int N, int K, uint16_t *Y,
                      int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr, void *ws,
                      size_t ws_bytes, hipStream_t stream, int fmt, const RqNext *rq = nullptr,
                      bool *rq_done = nullptr, const int32_t *res_cols = nullptr,
                      const int32_t *res_order = nullptr)
{
    int rc;
    if ((rc = check_gemm_common(xq, wq, M, N, K, fmt))) return rc;
    if (epilogue != W4A4_EPI_NONE && epilogue != W4A4_EPI_GELU && epilogue != W4A4_EPI_RESIDUAL)
        return fail(W4A4_ERR_ARG, "unknown epilogue %d", epilogue);
    if (!w_scale || (M > 0 && (!x_scale || !Y)))
        return fail(W4A4_ERR_ARG, "x_scale, w_scale and Y are required");
    if (ldy < N) return fail(W4A4_ERR_SHAPE, "ldy %lld < N = %d", (long long)ldy, N);
    if (epilogue == W4A4_EPI_RESIDUAL) {
        if (M > 0 && !residual) return fail(W4A4_ERR_ARG, "residual epilogue without residual");
        if (ldr < N) return fail(W4A4_ERR_SHAPE, "ldr %lld < N = %d", (long long)ldr, N);
        if (!aligned(residual, 2)) return fail(W4A4_ERR_ALIGN, "residual misaligned");
    }
    if (!aligned(Y, 2) || !aligned(x_scale, 4) || !aligned(w_scale, 4))
        return fail(W4A4_ERR_ALIGN, "Y / scales misaligned");
    if ((rc = check_ws(ws, ws_bytes, M > 0 ? gemm_ws_for(M, N, K, fmt) : 0))) return rc;
    if (M == 0) return ok();
    GemmEpilogue epi{};
    epi.x_scale = x_scale;
    epi.x_scale_per_token = x_scale_per_token ? 1 : 0;
    epi.w_scale = w_scale;
    epi.Y = Y;
    epi.ldy = ldy;
    epi.mode = epilogue;
    epi.residual = residual;
    epi.ldr = ldr;
    epi.res_cols = res_cols;
    epi.res_order = res_order;
    if (rq) epi.rq = *rq;
    if ((rc = fmt == OPF_F6 ? launch_gemm_f6(xq, wq, M, N, K, epi, ws, ws_bytes, stream)
                         : launch_gemm(xq, wq, M, N, K, epi, ws, ws_bytes, stream, fmt == OPF_I8,
                                       rq_done)))
        return rc;
    return ok();
}

static int gemm_i32_entry(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, int32_t *acc,
                          void *ws, size_t ws_bytes, hipStream_t stream, int fmt)
{
    int rc;
    if ((rc = check_gemm_common(xq, wq, M, N, K, fmt))) return rc;
    if (M > 0 && !acc) return fail(W4A4_ERR_ARG, "acc is NULL");
    if (!aligned(acc, 4)) return fail(W4A4_ERR_ALIGN, "acc misaligned");
    if ((rc = check_ws(ws, ws_bytes, M > 0 ? gemm_ws_for(M, N, K, fmt) : 0))) return rc;
    if (M == 0) return ok();
    GemmEpilogue epi{};
    epi.mode = GEMM_OUT_I32;
    epi.acc_out = acc;
    if ((rc = fmt == OPF_F6 ? launch_gemm_f6(xq, wq, M, N, K, epi, ws, ws_bytes, stream)
                         : launch_gemm(xq, wq, M, N, K, epi, ws, ws_bytes, stream, fmt == OPF_I8)))
        return rc;
    return ok();
}

}  // namespace w4a4

extern "C" {

int w4a4_gemm(const uint8_t *xq, const float *x_scale, int x_scale_per_token, const uint8_t *wq,
              const float *w_scale, int M, int N, int K, uint16_t *Y, int64_t ldy, int epilogue,
              const uint16_t *residual, int64_t ldr, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return gemm_entry(xq, x_scale, x_scale_per_token, wq, w_scale, M, N, K, Y, ldy, epilogue,
                      residual, ldr, ws, ws_bytes, stream, OPF_I4);
}

size_t w4a4_gemm_rq_next_workspace_bytes(int M, int N, int K, int K_next, int block_next,
                                         int mapped_residual)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const size_t gemm = mapped_residual ? gemm_mapped_residual_workspace(M, N, K)
                                        : w4a4_gemm_workspace_bytes(M, N, K);
    return K_next > 0 ? std::max(gemm, w4a4_act_workspace_bytes(M, K_next, block_next, 0)) : gemm;
}

int w4a4_gemm_rq_next(const uint8_t *xq, const float *x_scale, int x_scale_per_token,
                      const uint8_t *wq, const float *w_scale, int M, int N, int K, uint16_t *Y,
                      int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr,
                      const int32_t *res_cols, const int32_t *res_order, int col0, int K_next,
                      int block_next,
                      const void *rot_next, const float *table_next, int num_steps, int step,
                      uint8_t *xq_next, float *x_scale_next, int store_next_cols, void *ws,
                      size_t ws_bytes, hipStream_t stream)
{
    // every argument of the rotate-quantize half and of the residual map is checked before
    // anything is launched
    int rc;
    if (res_cols) {
        if (epilogue != W4A4_EPI_RESIDUAL)
            return fail(W4A4_ERR_ARG, "res_cols needs the residual epilogue");
        if (!aligned(res_cols, 4)) return fail(W4A4_ERR_ALIGN, "res_cols misaligned");
        if (N > 65536) return fail(W4A4_ERR_UNSUPPORTED, "res_cols with N = %d > 65536", N);
    }
    if (res_order) {
        if (!res_cols) return fail(W4A4_ERR_ARG, "res_order without res_cols");
        if (!aligned(res_order, 4)) return fail(W4A4_ERR_ALIGN, "res_order misaligned");
    }
    if (K_next < 0 || col0 < 0 || (int64_t)col0 + K_next > N || (K_next == 0 && col0 != 0))
        return fail(W4A4_ERR_SHAPE, "columns [%d, %d + %d) outside the N = %d outputs", col0, col0,
                    K_next, N);
    if (K_next > 0) {
        if ((rc = check_kb(K_next, block_next))) return rc;
        if (!rot_next) return fail(W4A4_ERR_ARG, "rot_next is NULL");
        if (!aligned(rot_next, 16)) return fail(W4A4_ERR_ALIGN, "rot_next must be 16-byte aligned");
        if (!table_next) return fail(W4A4_ERR_ARG, "table_next is required (per-step scale)");
        if (!aligned(table_next, 4)) return fail(W4A4_ERR_ALIGN, "table_next misaligned");
        if (num_steps <= 0)
            return fail(W4A4_ERR_STEP_RANGE, "num_steps = %d must be positive", num_steps);
        if (step < 0 || step >= num_steps)
            return fail(W4A4_ERR_STEP_RANGE, "step %d outside [0, %d)", step, num_steps);
        if (M > 0 && (!xq_next || !x_scale_next))
            return fail(W4A4_ERR_ARG, "xq_next and x_scale_next are required");
        if (!aligned(x_scale_next, 4)) return fail(W4A4_ERR_ALIGN, "x_scale_next misaligned");
    }
    if (M > 0 && (!Y || !aligned(Y + col0, 2)))
        return fail(W4A4_ERR_ARG, "Y is required");
    if ((rc = check_ws(ws, ws_bytes,
                       M > 0 ? w4a4_gemm_rq_next_workspace_bytes(M, N, K, K_next, block_next,
                                                                 res_cols != nullptr)
                             : 0)))
        return rc;
    if (K_next == 0)
        return gemm_entry(xq, x_scale, x_scale_per_token, wq, w_scale, M, N, K, Y, ldy, epilogue,
                          residual, ldr, ws, ws_bytes, stream, OPF_I4, nullptr, nullptr, res_cols,
                          res_order);
    const RotLayout L = rot_layout(K_next, block_next);
    const char *rb = reinterpret_cast<const char *>(rot_next);
    const RqNext rq{reinterpret_cast<const _Float16 *>(rb + L.r32),
                    reinterpret_cast<const _Float16 *>(rb + L.r32 + L.r16),
                    table_next, step, col0, K_next, xq_next, x_scale_next, store_next_cols ? 1 : 0};
    bool done = false;
    if ((rc = gemm_entry(xq, x_scale, x_scale_per_token, wq, w_scale, M, N, K, Y, ldy, epilogue,
                         residual, ldr, ws, ws_bytes, stream, OPF_I4,
                         block_next == 128 ? &rq : nullptr, &done, res_cols, res_order)))
        return rc;
    if (done || M == 0) return ok();
    // no fused tile plan for this shape: the rotate-quantize of the columns, after the GEMM on
    // the same stream (they are already in the next linear's zigzag order: no gather)
    return rq_entry(Y + col0, W4A4_F16, M, K_next, ldy, block_next, nullptr, rot_next, table_next,
                    num_steps, step, xq_next, x_scale_next, nullptr, ws, ws_bytes, stream, false);
}

int w4a4_gemm_i32(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, int32_t *acc,
                  void *ws, size_t ws_bytes, hipStream_t stream)
{
    return gemm_i32_entry(xq, wq, M, N, K, acc, ws, ws_bytes, stream, OPF_I4);
}

int w4a4_gemm_w8a8(const uint8_t *xq, const float *x_scale, int x_scale_per_token,
                   const uint8_t *wq, const float *w_scale, int M, int N, int K, uint16_t *Y,
                   int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr, void *ws,
                   size_t ws_bytes, hipStream_t stream)
{
    return gemm_entry(xq, x_scale, x_scale_per_token, wq, w_scale, M, N, K, Y, ldy, epilogue,
                      residual, ldr, ws, ws_bytes, stream, OPF_I8);
}

int w4a4_gemm_w8a8_i32(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, int32_t *acc,
                       void *ws, size_t ws_bytes, hipStream_t stream)
{
    return gemm_i32_entry(xq, wq, M, N, K, acc, ws, ws_bytes, stream, OPF_I8);
}

// ------------------------------------------------------------------ FP6 operands

size_t w4a4_f6_operand_bytes(int rows, int K)
{
    if (rows <= 0 || K <= 0 || K % 128) return 0;
    return f6_operand_bytes(rows, K);
}

int w4a4_codes_to_f6(const uint8_t *codes, int rows, int K, uint8_t *out, hipStream_t stream)
{
    if (rows < 0 || K <= 0) return fail(W4A4_ERR_ARG, "bad sizes rows=%d K=%d", rows, K);
    if (K % 128) return fail(W4A4_ERR_SHAPE, "fp6 operands need K a multiple of 128, not %d", K);
    if ((int64_t)((rows + 1) & ~1) * (K / 32) > INT32_MAX)
        return fail(W4A4_ERR_UNSUPPORTED, "fp6 operand of %d x %d beyond int32 indexing", rows, K);
    if (rows > 0 && (!codes || !out)) return fail(W4A4_ERR_ARG, "codes / out is NULL");
    if (!aligned(codes, 16) || !aligned(out, 16))
        return fail(W4A4_ERR_ALIGN, "codes and out must be 16-byte aligned");
    if (rows == 0) return ok();
    int rc;
    if ((rc = launch_codes_to_f6(codes, rows, K, out, stream))) return rc;
    return ok();
}

size_t w4a4_gemm_f6_workspace_bytes(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 128) return 0;
    return gemm_f6_workspace(M, N, K);
}

int w4a4_gemm_f6(const uint8_t *xf, const float *x_scale, int x_scale_per_token, const uint8_t *wf,
                 const float *w_scale, int M, int N, int K, uint16_t *Y, int64_t ldy, int epilogue,
                 const uint16_t *residual, int64_t ldr, void *ws, size_t ws_bytes,
                 hipStream_t stream)
{
    return gemm_entry(xf, x_scale, x_scale_per_token, wf, w_scale, M, N, K, Y, ldy, epilogue,
                      residual, ldr, ws, ws_bytes, stream, OPF_F6);
}

int w4a4_gemm_f6_i32(const uint8_t *xf, const uint8_t *wf, int M, int N, int K, int32_t *acc,
                     void *ws, size_t ws_bytes, hipStream_t stream)
{
    return gemm_i32_entry(xf, wf, M, N, K, acc, ws, ws_bytes, stream, OPF_F6);
}

// ------------------------------------------------------------------ group-wise scales

static int check_grouped(int x_dtype, int block)
{
    if (block != 128)
        return fail(W4A4_ERR_UNSUPPORTED, "group-wise scales need block 128 (got %d)", block);
    if (x_dtype != W4A4_F16)
        return fail(W4A4_ERR_UNSUPPORTED, "group-wise scales need fp16 activations");
    return W4A4_OK;
}

int w4a4_calibrate_act_scale_grouped(const void *X, int x_dtype, int M, int K, int64_t ldx,
                                     int block, const int32_t *perm, const void *rot,
                                     float *table_row, void *ws, size_t ws_bytes,
                                     hipStream_t stream)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if ((rc = check_grouped(x_dtype, block))) return rc;
    if ((rc = check_matrix(X, x_dtype, M, K, ldx, "X"))) return rc;
    if (!rot) return fail(W4A4_ERR_ARG, "rot is NULL");
    if (!aligned(rot, 16)) return fail(W4A4_ERR_ALIGN, "rot must be 16-byte aligned");
    if (!table_row) return fail(W4A4_ERR_ARG, "table_row is NULL");
    if (!aligned(perm, 4) || !aligned(table_row, 4)) return fail(W4A4_ERR_ALIGN, "perm / table_row misaligned");
    if ((rc = check_ws(ws, ws_bytes, act_ws_bytes(M, K, block, KIND_CALIB)))) return rc;
    if ((rc = run_activation(X, x_dtype, M, K, ldx, block, perm, rot, nullptr, 0, KIND_CALIB,
                             nullptr, nullptr, nullptr, ws, table_row, stream, false, true)))
        return rc;
    return ok();
}

int w4a4_rotate_quant_act_grouped(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                                  const int32_t *perm, const void *rot,
                                  const float *act_scale_table, int num_steps, int step,
                                  uint8_t *xq, float *x_scale, float *xrot_dbg, void *ws,
                                  size_t ws_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if ((rc = check_grouped(x_dtype, block))) return rc;
    if ((rc = check_matrix(X, x_dtype, M, K, ldx, "X"))) return rc;
    if (!rot) return fail(W4A4_ERR_ARG, "rot is NULL");
    if (!aligned(rot, 16)) return fail(W4A4_ERR_ALIGN, "rot must be 16-byte aligned");
    if (!aligned(perm, 4)) return fail(W4A4_ERR_ALIGN, "perm misaligned");
    if (!act_scale_table) return fail(W4A4_ERR_ARG, "group-wise scales need the table");
    if (num_steps <= 0) return fail(W4A4_ERR_STEP_RANGE, "num_steps = %d must be positive", num_steps);
    if (step < 0 || step >= num_steps)
        return fail(W4A4_ERR_STEP_RANGE, "step %d outside [0, %d)", step, num_steps);
    if (!aligned(act_scale_table, 4)) return fail(W4A4_ERR_ALIGN, "table misaligned");
    if (M > 0 && (!xq || !x_scale)) return fail(W4A4_ERR_ARG, "xq and x_scale are required");
    if (!aligned(x_scale, 4) || !aligned(xrot_dbg, 4))
        return fail(W4A4_ERR_ALIGN, "x_scale / xrot_dbg misaligned");
    if ((rc = check_ws(ws, ws_bytes, w4a4_act_workspace_bytes(M, K, block, 0)))) return rc;
    if (M == 0) return ok();
    if ((rc = run_activation(X, x_dtype, M, K, ldx, block, perm, rot, act_scale_table, step,
                             KIND_STEP, xq, x_scale, xrot_dbg, ws, nullptr, stream, false, true)))
        return rc;
    return ok();
}

int w4a4_gemm_grouped(const uint8_t *xq, const float *x_scales, const uint8_t *wq,
                      const float *w_scale, int M, int N, int K, int block, uint16_t *Y,
                      int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr,
                      hipStream_t stream)
{
    int rc;
    if ((rc = check_gemm_common(xq, wq, M, N, K, OPF_I4))) return rc;
    if (block != 128)
        return fail(W4A4_ERR_UNSUPPORTED, "group-wise scales need block 128 (got %d)", block);
    if (K % block) return fail(W4A4_ERR_SHAPE, "K = %d not a multiple of block %d", K, block);
    if (epilogue != W4A4_EPI_NONE && epilogue != W4A4_EPI_GELU && epilogue != W4A4_EPI_RESIDUAL)
        return fail(W4A4_ERR_ARG, "unknown epilogue %d", epilogue);
    if (!wq || !w_scale || !x_scales || (M > 0 && (!xq || !Y)))
        return fail(W4A4_ERR_ARG, "NULL operand");
    if (ldy < N) return fail(W4A4_ERR_SHAPE, "ldy = %lld < N = %d", (long long)ldy, N);
    if (epilogue == W4A4_EPI_RESIDUAL && (!residual || ldr < N))
        return fail(W4A4_ERR_ARG, "residual epilogue needs residual with ldr >= N");
    if (!aligned(xq, 16) || !aligned(wq, 16))
        return fail(W4A4_ERR_ALIGN, "group-wise GEMM needs 16-byte aligned xq and wq");
    if (!aligned(x_scales, 4) || !aligned(w_scale, 4) || !aligned(Y, 2) || !aligned(residual, 2))
        return fail(W4A4_ERR_ALIGN, "scales / Y / residual misaligned");
    if (M == 0) return ok();
    GemmEpilogue epi{};
    epi.x_scale = x_scales;
    epi.x_scale_per_token = 0;
    epi.w_scale = w_scale;
    epi.Y = Y;
    epi.ldy = ldy;
    epi.mode = epilogue;
    epi.residual = residual;
    epi.ldr = ldr;
    epi.acc_out = nullptr;
    rc = launch_gemm_grouped(xq, wq, M, N, K, epi, stream);
    return rc ? rc : ok();
}

// ------------------------------------------------------------------ GPTQ weight solver

static int check_gptq_k(int K, int block)
{
    int rc;
    if ((rc = check_kb(K, block))) return rc;
    if (K > GPTQ_MAX_K)
        return fail(W4A4_ERR_UNSUPPORTED, "GPTQ solver supports K <= %d (got %d)", GPTQ_MAX_K, K);
    return W4A4_OK;
}

size_t w4a4_gptq_hessian_workspace_bytes(int M, int K, int block)
{
    if (M < 0 || K <= 0 || !pow2_block(block) || K % block) return 0;
    return align_up((size_t)K * block * sizeof(double), 256) +
           align_up((size_t)(M > 0 ? M : 1) * K * sizeof(double), 256);
}

int w4a4_gptq_hessian(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                      const int32_t *perm, const float *U, double *H, int accumulate, void *ws,
                      size_t ws_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_gptq_k(K, block))) return rc;
    if ((rc = check_matrix(X, x_dtype, M, K, ldx, "X"))) return rc;
    if (!H) return fail(W4A4_ERR_ARG, "H is NULL");
    if (!aligned(H, 8) || !aligned(U, 4) || !aligned(perm, 4))
        return fail(W4A4_ERR_ALIGN, "H / U / perm misaligned");
    if ((rc = check_ws(ws, ws_bytes, w4a4_gptq_hessian_workspace_bytes(M, K, block)))) return rc;
    double *R64 = reinterpret_cast<double *>(ws);
    double *Xr = reinterpret_cast<double *>(reinterpret_cast<char *>(ws) +
                                            align_up((size_t)K * block * sizeof(double), 256));
    if ((rc = launch_rotation(U, K, block, 1.0 / std::sqrt((double)block), R64, nullptr, stream)))
        return rc;
    if ((rc = launch_rotate_rows_f64(X, x_dtype, M, K, ldx, block, perm, R64, Xr, stream))) return rc;
    if ((rc = launch_gram_f64(Xr, M, K, H, accumulate != 0, stream))) return rc;
    return ok();
}

size_t w4a4_gptq_factor_workspace_bytes(int K)
{
    if (K <= 0) return 0;
    return align_up(((size_t)K * K + 1) * sizeof(double), 256);
}

int w4a4_gptq_factor(const double *H, int K, double damp_percent, double *Hf, uint8_t *dead,
                     void *ws, size_t ws_bytes, hipStream_t stream)
{
    int rc;
    if (K <= 0) return fail(W4A4_ERR_ARG, "K = %d must be positive", K);
    if (K > GPTQ_MAX_K)
        return fail(W4A4_ERR_UNSUPPORTED, "GPTQ solver supports K <= %d (got %d)", GPTQ_MAX_K, K);
    if (!H || !Hf) return fail(W4A4_ERR_ARG, "H and Hf are required");
    if (!(damp_percent >= 0.0) || !std::isfinite(damp_percent))
        return fail(W4A4_ERR_ARG, "damp_percent must be finite and non-negative");
    if (!aligned(H, 8) || !aligned(Hf, 8)) return fail(W4A4_ERR_ALIGN, "H / Hf misaligned");
    if ((rc = check_ws(ws, ws_bytes, w4a4_gptq_factor_workspace_bytes(K)))) return rc;
    if ((rc = launch_gptq_factor(H, K, damp_percent, Hf, dead, reinterpret_cast<double *>(ws),
                                 stream)))
        return rc;
    return ok();
}

size_t w4a4_pack_gptq_workspace_bytes(int N, int K, int block)
{
    if (N <= 0 || K <= 0 || !pow2_block(block) || K % block) return 0;
    return align_up((size_t)K * block * sizeof(double), 256) + align_up((size_t)N * 8, 256) +
           align_up((size_t)N * K * sizeof(double), 256) + align_up((size_t)N * K, 256);
}

int w4a4_pack_weights_gptq(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                           const int32_t *perm, const float *U, const double *Hf,
                           const uint8_t *dead, uint8_t *wq, float *w_scale, void *rot, void *ws,
                           size_t ws_bytes, hipStream_t stream)
{
    int rc;
    if ((rc = check_gptq_k(K, block))) return rc;
    if (N <= 0) return fail(W4A4_ERR_ARG, "N = %d must be positive", N);
    if ((rc = check_matrix(W, w_dtype, N, K, ldw, "W"))) return rc;
    if (!wq || !w_scale || !rot || !Hf) return fail(W4A4_ERR_ARG, "wq, w_scale, rot and Hf are required");
    if (!aligned(U, 4) || !aligned(w_scale, 4) || !aligned(Hf, 8) || !aligned(perm, 4))
        return fail(W4A4_ERR_ALIGN, "U / w_scale / Hf / perm misaligned");
    if (!aligned(rot, 16)) return fail(W4A4_ERR_ALIGN, "rot must be 16-byte aligned");
    if ((rc = check_ws(ws, ws_bytes, w4a4_pack_gptq_workspace_bytes(N, K, block)))) return rc;
    char *w = reinterpret_cast<char *>(ws);
    double *R64 = reinterpret_cast<double *>(w);
    w += align_up((size_t)K * block * sizeof(double), 256);
    unsigned long long *rowmax = reinterpret_cast<unsigned long long *>(w);
    w += align_up((size_t)N * 8, 256);
    double *Wr = reinterpret_cast<double *>(w);
    w += align_up((size_t)N * K * sizeof(double), 256);
    int8_t *codes = reinterpret_cast<int8_t *>(w);
    if ((rc = launch_rotation(U, K, block, 1.0 / std::sqrt((double)block), R64, rot, stream))) return rc;
    if ((rc = launch_weight_rowmax_rot(W, w_dtype, N, K, ldw, block, perm, R64, rowmax, Wr, stream)))
        return rc;
    if ((rc = launch_gptq_sweep(Wr, N, K, Hf, dead, rowmax, codes, w_scale, stream))) return rc;
    if ((rc = launch_pack_codes(codes, N, K, wq, stream))) return rc;
    return ok();
}

}  // extern "C"
