// Internal declarations shared by the translation units of libw4a4.so (not part of the ABI).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "w4a4.h"

namespace w4a4 {

// ---- host-side status handling ---------------------------------------------------------------
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char *what);  // W4A4_OK, or W4A4_ERR_HIP with the HIP error text
// Allows `kernel` at least `bytes` of dynamic LDS on the current device: the limit is raised once
// per (kernel, device) and again only when a launch needs more (thread-safe).
int ensure_dynamic_lds(const void *kernel, size_t bytes, const char *what);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- device helpers --------------------------------------------------------------------------
__device__ __forceinline__ float load_as_f32(const void *p, int dtype, int64_t idx)
{
    if (dtype == W4A4_F16) return __half2float(reinterpret_cast<const __half *>(p)[idx]);
    return reinterpret_cast<const float *>(p)[idx];
}

// fp16 and fp32 values widen to fp64 exactly.
__device__ __forceinline__ double load_as_f64(const void *p, int dtype, int64_t idx)
{
    return (double)load_as_f32(p, dtype, idx);
}

// FP6 operand encoding (see the FP6 GEMM in k_gemm.hip).
// E3M2 codes of four two's-complement nibbles held one per byte (values 0..15): two byte lookups
// with v_perm_b32 (nibbles 0..7 -> codes of 0..7, nibbles 8..15 -> codes of -8..-1) blended on bit 3.
__device__ __forceinline__ uint32_t e3m2_of_nibble_bytes(uint32_t nb)
{
    const uint32_t sel = nb & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x17161514u, 0x12100C00u, sel);  // 0x00 0x0C 0x10 0x12 0x14..0x17
    const uint32_t neg = __builtin_amdgcn_perm(0x2C303234u, 0x35363738u, sel);  // 0x38 0x37 0x36 0x35 0x34 0x32 0x30 0x2C
    const uint32_t b = (nb >> 3) & 0x01010101u;
    const uint32_t m = (b << 6) - b;  // 0x3F in the bytes of negative nibbles
    return (neg & m) | (pos & ~m);
}

// Four 6-bit values held one per byte -> one 24-bit run, byte i at bits 6i..6i+5.
__device__ __forceinline__ uint32_t pack6x4(uint32_t x)
{
    return (x & 0x3Fu) | ((x >> 2) & 0xFC0u) | ((x >> 4) & 0x3F000u) | ((x >> 6) & 0xFC0000u);
}

// 16 packed bytes (32 int4 codes, low nibble first) -> the 192-bit string of their E3M2 fields,
// code i at bits 6i..6i+5: w[0..3] is the group's head, w[4..5] its tail.
__device__ __forceinline__ void f6_encode_group(const uint4 p, uint32_t (&w)[6])
{
    const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
    uint32_t c[8];  // 24-bit runs of k = 4j .. 4j+3
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = e3m2_of_nibble_bytes(pw[d] & 0x0F0F0F0Fu);          // k = 8d + 0, 2, 4, 6
        const uint32_t hi = e3m2_of_nibble_bytes((pw[d] >> 4) & 0x0F0F0F0Fu);   // k = 8d + 1, 3, 5, 7
        c[2 * d] = pack6x4(__builtin_amdgcn_perm(hi, lo, 0x05010400u));        // k = 8d .. 8d+3
        c[2 * d + 1] = pack6x4(__builtin_amdgcn_perm(hi, lo, 0x07030602u));    // k = 8d+4 .. 8d+7
    }
    // run j starts at bit 24 j
    w[0] = c[0] | (c[1] << 24);
    w[1] = (c[1] >> 8) | (c[2] << 16);
    w[2] = (c[2] >> 16) | (c[3] << 8);
    w[3] = c[4] | (c[5] << 24);
    w[4] = (c[5] >> 8) | (c[6] << 16);
    w[5] = (c[6] >> 16) | (c[7] << 8);
}

// Natural-order Sylvester Hadamard sign: (-1)^popcount(l & j).
__device__ __forceinline__ bool hadamard_negative(int l, int j) { return __popc(l & j) & 1; }

// Layout of the activation rotation operand written by the pack call (all offsets 256-aligned):
//   [0, r32)          fp32 R_b[i][j] for every block, [nb][B][B] row-major
//   [r32, r32 + r16)  fp16 high parts of R_b, in MFMA operand order (rot16_index)
//   [.., .. + r16)    fp16 low parts scaled by 2^ROT_LO_SHIFT, same order
// with R_b ~= hi + lo * 2^-ROT_LO_SHIFT to about 22 significant bits.
constexpr int ROT_LO_SHIFT = 12;
struct RotLayout {
    size_t r32, r16, total;
};
// Position of R_b[i][j]'s fp16 part. For B a multiple of 32 the parts are stored as the A operand
// of v_mfma_f32_16x16x32_f16 with R_b^T as the matrix: per block b, 16-channel group j / 16 and
// 32-input chunk i / 32, one contiguous 1 KB run in which lane l = (j % 16) + 16 ((i % 32) / 8)
// holds inputs 32 (i / 32) + 8 (l / 16) + 0..7 of channel j, so a wave loads a fragment with one
// fully used 16-byte-per-lane load. Other block sizes use the plain transpose [b][j][i].
__host__ __device__ inline int64_t rot16_index(int b, int i, int j, int B)
{
    if (B % 32 != 0) return ((int64_t)b * B + j) * B + i;
    const int64_t run = ((int64_t)b * (B / 16) + j / 16) * (B / 32) + i / 32;
    return (run * 64 + (j % 16) + 16 * ((i % 32) / 8)) * 8 + (i % 8);
}
// Element offset of the fragment (16-channel group jt, chunk kk) of block b for lane `lane`.
__host__ __device__ inline int64_t rot16_fragment(int b, int jt, int kk, int lane, int B)
{
    return ((((int64_t)b * (B / 16) + jt) * (B / 32) + kk) * 64 + lane) * 8;
}
inline RotLayout rot_layout(int K, int B)
{
    RotLayout L;
    L.r32 = align_up((size_t)K * B * sizeof(float), 256);
    L.r16 = align_up((size_t)K * B * sizeof(uint16_t), 256);
    L.total = L.r32 + 2 * L.r16;
    return L;
}

// ---- launchers (one per kernel family) --------------------------------------------------------
// offline weight side (k_pack.hip)
int launch_rotation(const float *U, int K, int B, double hinv, double *R64, void *rot,
                    hipStream_t s);
int launch_weight_pack(const void *W, int wdt, int N, int K, int64_t ldw, int B,
                       const int32_t *perm, const double *R64, unsigned long long *rowmax,
                       uint8_t *wq, float *w_scale, int bits, hipStream_t s);
int launch_weight_rowmax_rot(const void *W, int wdt, int N, int K, int64_t ldw, int B,
                             const int32_t *perm, const double *R64, unsigned long long *rowmax,
                             double *wrot, hipStream_t s);
// fp64 rows A[:, perm] . blockdiag(R_b) into out [rows][K] (the weight pack's fixed-order arithmetic)
int launch_rotate_rows_f64(const void *A, int adt, int rows, int K, int64_t lda, int B,
                           const int32_t *perm, const double *R64, double *out, hipStream_t s);
// GPTQ solver (k_gptq.hip)
int launch_gram_f64(const double *A, int rows, int K, double *H, bool accumulate, hipStream_t s);
int launch_gptq_factor(const double *H, int K, double damp_percent, double *Hf, uint8_t *dead,
                       double *work, hipStream_t s);
int launch_gptq_sweep(const double *Wr, int N, int K, const double *Hf, const uint8_t *dead,
                      const unsigned long long *rowmax, int8_t *codes, float *w_scale,
                      hipStream_t s);
int launch_pack_codes(const int8_t *codes, int N, int K, uint8_t *wq, hipStream_t s);
constexpr int GPTQ_MAX_K = 4096;

// activation side (k_act.hip)
enum ActMode { ACT_PER_STEP = 0, ACT_TOKEN_MAX = 1, ACT_TOKEN_QUANT = 2, ACT_CALIB_MAX = 3 };
int launch_fill_u32(uint32_t *p, uint32_t value, int64_t count, hipStream_t s);
int launch_rotate_quant(const void *X, int xdt, int M, int K, int64_t ldx, int B,
                        const int32_t *perm, const void *rot, const float *table, int step,
                        ActMode mode, uint32_t *rowmax, uint8_t *xq, float *x_scale,
                        float *xrot_dbg, bool q8, hipStream_t s);
// q8 (here and below): int8 codes [M][K] with scales max / 127 instead of packed int4 and max / 7
int launch_scale_from_absmax(const uint32_t *amax, float *out, bool q8, hipStream_t s,
                             int count = 1);
// fp16 activations with block 64 or 128: MFMA rotation; xperm (optional) holds rows already in
// zigzag order, written by launch_permute_rows (which also clears zero_row[0..M) when given).
bool act_uses_permute_pass(int M, int K, int per_token);
size_t act_permute_bytes(int M, int K);
int launch_permute_rows(const void *X, int M, int K, int64_t ldx, const int32_t *perm, uint16_t *xp,
                        uint32_t *zero_row, hipStream_t s);
// Hadamard-only rotation (U_b = I), B in {64, 128}: LDS bytes of the staged rows (and the rows per
// workgroup), and the single-kernel rotate-quantize (table == NULL selects per-token scales).
size_t hadamard_lds_bytes(int M, int K, int B, int x_dtype, int *rows_per_wg);
int launch_rotate_quant_hadamard(const void *X, int x_dtype, int M, int K, int64_t ldx, int B,
                                 const int32_t *perm, const float *table, int step, uint8_t *xq,
                                 float *x_scale, float *xrot_dbg, hipStream_t s);
// f6: xq is an FP6 operand (the layout of launch_gemm_f6) written by the streaming kernel (B = 128,
// int4 codes, per-step or per-token quantize pass); only where rq_ring_path holds.
int launch_rotate_quant_mfma(const void *X, int M, int K, int64_t ldx, int B, const int32_t *perm,
                             const void *rot, const float *table, int step, ActMode mode,
                             uint32_t *rowmax, uint8_t *xq, float *x_scale, float *xrot_dbg,
                             const uint16_t *xperm, bool q8, hipStream_t s, int gstride = 0,
                             bool f6 = false);
// whether launch_rotate_quant_mfma takes the streaming (LDS-ring) kernel for these rows
bool rq_ring_path(int M, const void *X, int64_t ldx, const int32_t *perm, const uint16_t *xperm,
                  int K);

// GEMM (k_gemm.hip)
// The next linear's rotate-quantize fused into a GEMM epilogue (per-step scale, block 128): the
// output columns [col0, col0 + kn), which hold that linear's input in its zigzag order, become its
// packed int4 codes xq [M][kn / 2] and its scale x_scale[0] = table[step]. xq == nullptr: none.
struct RqNext {
    const _Float16 *rhi, *rlo;  // the next linear's rotation operand (fp16 high and low parts)
    const float *table;
    int step, col0, kn;
    uint8_t *xq;
    float *x_scale;
    int store_y;  // 0: the columns [col0, col0 + kn) of Y need not be written
};
struct GemmEpilogue {
    const float *x_scale;
    int x_scale_per_token;
    const float *w_scale;
    uint16_t *Y;
    int64_t ldy;
    int mode;  // W4A4_EPI_* or GEMM_OUT_I32
    const uint16_t *residual;
    int64_t ldr;
    int32_t *acc_out;  // GEMM_OUT_I32 destination, dense [M][N]
    RqNext rq;
    // residual column map (W4A4_EPI_RESIDUAL): output column n adds residual column res_cols[n]
    // (nullptr: column n). launch_gemm reads it in the split-group kernel's staged epilogue, or
    // gathers the residual into its workspace first. res_order (optional, with res_cols): for each
    // 128-column tile, the order in which that kernel's lanes gather the tile's columns.
    const int32_t *res_cols;
    const int32_t *res_order;
};
constexpr int GEMM_OUT_I32 = 100;
// q8: int8 operands [rows][K] (W8A8) instead of packed int4 [rows][K/2]
size_t gemm_workspace(int M, int N, int K, bool q8);
// With epi.rq.xq set, *rq_done tells whether the GEMM kernel also wrote the next linear's codes
// (a 128-column tile plan with the staged epilogue); otherwise the caller runs the rotate-quantize.
int launch_gemm(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, const GemmEpilogue &epi,
                void *ws, size_t ws_bytes, hipStream_t s, bool q8, bool *rq_done = nullptr);
// Workspace of a launch_gemm call with a residual column map: the split-K partials of its plan, or
// the gathered residual [M][N] fp16 when the plan cannot read the map in its epilogue.
size_t gemm_mapped_residual_workspace(int M, int N, int K);
// group-wise activation scales epi.x_scale[K / 128] (int4, K % 128 == 0, 16-byte aligned operands)
int launch_gemm_grouped(const uint8_t *xq, const uint8_t *wq, int M, int N, int K,
                        const GemmEpilogue &epi, hipStream_t s);

// FP6 (E3M2) operands of the FP6 matrix-core GEMM: packed int4 codes [rows][K/2] re-encoded into
// f6_operand_bytes(rows, K) bytes (K % 128 == 0), and the GEMM on two such operands (K <= 2^18).
inline size_t f6_operand_bytes(int rows, int K) { return (size_t)((rows + 1) & ~1) * (size_t)K * 3 / 4; }
int launch_codes_to_f6(const uint8_t *q, int rows, int K, uint8_t *out, hipStream_t s);
size_t gemm_f6_workspace(int M, int N, int K);
int launch_gemm_f6(const uint8_t *xf, const uint8_t *wf, int M, int N, int K,
                   const GemmEpilogue &epi, void *ws, size_t ws_bytes, hipStream_t s);

// calibration (k_calib.hip)
size_t zigzag_workspace(int K);
int launch_zigzag(const void *W, int wdt, int N, int K, int64_t ldw, int B, int32_t *perm,
                  void *ws, hipStream_t s);
size_t block_svd_workspace(int N, int K, int B);
int launch_block_svd(const void *W, int wdt, int N, int K, int64_t ldw, int B, const int32_t *perm,
                     float *U, void *ws, hipStream_t s);

}  // namespace w4a4
