/*
 * w4a4.h -- C ABI of libw4a4.so, an MI355X (gfx950) implementation of the W4A4 quantized linear of
 * Omega-QVLA: zigzag channel permutation, blockwise composite SVD.Hadamard rotation, symmetric int4
 * activations (per-denoising-step table scale or dynamic per-token scale), int4 RTN weights with a
 * per-output-channel scale, integer GEMM on int8 MFMA (for large batches also on FP6 MFMA, with the
 * codes re-encoded exactly as E3M2 floats), fp16 output.
 *
 * Passages the calls follow (pages cited by title and section):
 *  - gist.science (pt/fr) summary of arXiv 2605.28803, "Metodologia" / "Methodologie", item 1: the SVD
 *    W = U Sigma V^T gives R_SVD, a normalized Hadamard H is composed with it, R = R_SVD . H, the
 *    rotation is applied block by block along the input channels after a zigzag permutation ordered
 *    by weight column norms, before quantization. Item 2: a per-step activation scale table built
 *    offline from calibration trajectories and looked up at inference time.
 *  - vnrobo.com "Omega-QVLA: Nen VLA W4A4 tren Edge", "Y tuong paper" (per-step act_scale_table,
 *    runtime lookup of the current step's scale) and "Build DiT action head pack" (--use-rtn,
 *    --w-bits 4, --a-bits 4, --num-steps 8, --duquant-block-size 64).
 *  - aiexpert.news "Omega-QVLA Reduce el Modelo ... 71%": a step-count mismatch or a truncated table
 *    is a failure mode, so a step outside the table is an error here, never clamped.
 *  - radar.vhtltd.com FoldQuantVLA summary, key change 2: dynamic per-token activation quantization.
 *
 * Conventions for every call:
 *  - Every pointer argument is a caller-owned DEVICE pointer (hipMalloc'd or torch CUDA memory)
 *    unless stated otherwise. The library allocates nothing; scratch memory comes from the `ws`
 *    argument, sized by the matching *_workspace_bytes() query (ws may be NULL when that is 0).
 *  - Work is enqueued on `stream` (NULL = the null stream) and the call returns without waiting.
 *    Arguments are validated on the host before anything is launched; a failing call launches
 *    nothing and leaves every output untouched. Calls that share a workspace must not overlap.
 *  - Layouts: X [M][K] and W [N][K] are row-major with row strides ldx / ldw in elements, dtype
 *    W4A4_F16 (IEEE binary16) or W4A4_F32. perm is int32 [K]: permuted position j takes original
 *    channel perm[j]; perm == NULL means the identity (the caller already stores channels in
 *    zigzag order). U is fp32 [K/block][block][block] row-major: entry (i, j) of block b's factor
 *    U_b is U[(b*block + i)*block + j]; a row vector x_b of block b is rotated as (x_b U_b) H_B, with
 *    H_B the natural-order Sylvester Hadamard matrix scaled by 1/sqrt(block).
 *    Packed int4: uint8 [rows][K/2], two's-complement nibbles, low nibble = even k.
 *    Scales are fp32. Y and residual are IEEE binary16 bit patterns, row-major with strides ldy/ldr.
 *  - block must be a power of two in [1, 256] dividing K, and K must be even.
 *  - Return value: W4A4_OK or one of the W4A4_ERR_* codes; w4a4_last_error() then describes the
 *    failure (thread-local, valid until the next call on the same thread).
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w4a4_status {
    W4A4_OK = 0,
    W4A4_ERR_ARG = 1,         /* NULL where a pointer is required, negative size, unknown enum */
    W4A4_ERR_SHAPE = 2,       /* K odd or not a multiple of block, leading dimension too small */
    W4A4_ERR_STEP_RANGE = 3,  /* step outside [0, num_steps) */
    W4A4_ERR_UNSUPPORTED = 4, /* block not a power of two in [1, 256]; size beyond int32 indexing */
    W4A4_ERR_ALIGN = 5,       /* pointer not aligned as the argument requires */
    W4A4_ERR_WORKSPACE = 6,   /* ws NULL or smaller than the *_workspace_bytes() figure */
    W4A4_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed */
};

enum w4a4_dtype { W4A4_F16 = 0, W4A4_F32 = 1 };

enum w4a4_epilogue {
    W4A4_EPI_NONE = 0,     /* Y = fp16(dequant) */
    W4A4_EPI_GELU = 1,     /* Y = fp16(gelu_erf(dequant)), GELU evaluated in fp32 */
    W4A4_EPI_RESIDUAL = 2  /* Y = fp16(fp32(dequant) + fp32(residual)) */
};

/* ---------------------------------------------------------------------------------------------
 * Offline calibration on the device (done once per linear, before packing).
 * ------------------------------------------------------------------------------------------- */

/* Zigzag permutation [gist.science Metodologia 1, "Implementacao em Blocos"]: rank the input
 * channels by descending weight column norm (the fp64 sum over rows n = 0..N-1, in that order, of
 * W[n][k]^2; ties go to the lower channel index), then deal ranks over the nb = K/block blocks like
 * a boustrophedon: rank r = p*nb + j lands in block j when pass p is even and in block nb-1-j when p
 * is odd, at position p inside the block. Writes perm[b*block + p] = original channel (int32 [K]).
 * Bit-exact (integer result of fp64 comparisons). */
size_t w4a4_zigzag_workspace_bytes(int K);
int w4a4_zigzag_perm(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                     int32_t *perm, void *ws, size_t ws_bytes, hipStream_t stream);

/* Per-block SVD factor [gist.science Metodologia 1, "Rotacao SVD": W = U Sigma V^T, R_SVD]: for each
 * block b, the right singular vectors of W_b = W[:, perm[b*block .. b*block+block-1]] (N x block),
 * columns in descending singular value, each column's sign chosen so that its largest-magnitude
 * entry is positive; computed as the fp64 cyclic-Jacobi eigenbasis of W_b^T W_b and rounded once to
 * fp32. Writes U fp32 [K/block][block][block]. Singular vectors are unique only up to the sign fixed
 * here and up to rotations inside repeated singular values (e.g. N < block). block <= 128 here
 * (W4A4_ERR_UNSUPPORTED above). */
size_t w4a4_block_svd_workspace_bytes(int N, int K, int block);
int w4a4_block_svd(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                   const int32_t *perm, float *U, void *ws, size_t ws_bytes, hipStream_t stream);

/* Per-step activation scale for one table entry [vnrobo.com "Y tuong paper"; gist.science item 2
 * "Calibracao por Passo"]: *table_entry = fp32(max |fp32(x')| / 7) over every row of the stacked
 * calibration activations X [M][K] (several calibration samples of one denoising step stacked along
 * M), x' being the rotated activation; 1.0f if that max is 0. `rot` is the operand written by
 * w4a4_pack_weights for this linear. */
size_t w4a4_calibrate_workspace_bytes(int M, int K, int block);
int w4a4_calibrate_act_scale(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                             const int32_t *perm, const void *rot, float *table_entry,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Offline weight rotate + RTN + pack [gist.science Metodologia 1; vnrobo.com "Build DiT action head
 * pack": --use-rtn --w-bits 4 --svd-rank 0, i.e. RTN on the whole rotated weight].
 *
 * W' = W[:, perm] . blockdiag(R_b), R_b = U_b . H_B, all in fp64 with every dot product summed in
 * increasing index order without fused multiply-add; s_w[n] = fp32(max_k |W'[n][k]| / 7) (1.0f for a
 * zero row); codes p = clamp(rint(W' / s_w), -8, 7) (half to even), packed into wq [N][K/2].
 * Also writes `rot`, the activation-side rotation operand (w4a4_rot_bytes(K, block) bytes, 16-byte
 * aligned, opaque device layout) that w4a4_rotate_quant_act and w4a4_calibrate_act_scale read.
 * wq and w_scale are bit-exact functions of (W, perm, U). U == NULL stands for U_b = I (R_b = H_B,
 * the Hadamard-only mode of w4a4_rotate_quant_act_hadamard).
 * ------------------------------------------------------------------------------------------- */
size_t w4a4_rot_bytes(int K, int block);
size_t w4a4_pack_workspace_bytes(int N, int K, int block);
int w4a4_pack_weights(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                      const int32_t *perm, const float *U, uint8_t *wq, float *w_scale, void *rot,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Runtime activation path: zigzag gather, block rotation x' = X[:, perm] . blockdiag(R_b) computed
 * on the device in fp32, activation scale, int4 quantization and packing.
 *  - Per-step mode (act_scale_table != NULL) [vnrobo.com "Y tuong paper"]: s = table[step] for every
 *    row; step must lie in [0, num_steps) (else W4A4_ERR_STEP_RANGE) and the table must hold at
 *    least num_steps device floats. x_scale[0] receives s. Only a positive finite entry is a
 *    scale: for any other entry (zero, negative, infinite, NaN -- an uncalibrated or damaged table)
 *    every code is 0 and x_scale[0] receives NaN, so every output of the GEMM that consumes them is
 *    NaN (the device cannot report the table's contents through the return value without a wait).
 *  - Per-token mode (act_scale_table == NULL) [FoldQuantVLA key change 2]: s_m = fp32(max_k |x'_mk|
 *    / 7) (1.0f for a zero row); x_scale[m] receives s_m for m in [0, M). num_steps/step ignored.
 *  Codes: r = fp32(1/s), q = clamp(rint(fp32(x' * r)), -8, 7), packed into xq [M][K/2].
 *  xrot_dbg: NULL in production; otherwise fp32 [M][K] receives x' (test hook).
 *  M == 0 is a valid empty call.
 * ------------------------------------------------------------------------------------------- */
size_t w4a4_act_workspace_bytes(int M, int K, int block, int per_token);
int w4a4_rotate_quant_act(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                          const int32_t *perm, const void *rot, const float *act_scale_table,
                          int num_steps, int step, uint8_t *xq, float *x_scale, float *xrot_dbg,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of w4a4_rotate_quant_act, for callers that cannot allocate device
 * memory or own a workspace (code under HIP graph capture that may not allocate, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, modes, layouts, outputs and errors as
 * w4a4_rotate_quant_act without ws / ws_bytes: the scratch it needs (per-token row maxima, the
 * staged zigzag-ordered rows of large batches) lives in a fixed device array inside the library,
 * w4a4_noalloc_scratch_bytes() = 16 MiB, one copy per GPU, held until the process ends. A call
 * whose w4a4_act_workspace_bytes(M, K, block, per_token) exceeds that maximum returns
 * W4A4_ERR_UNSUPPORTED and launches nothing. The call performs no allocation or free of any kind.
 * All calls on one GPU share that array and it keeps the last call's contents (everything that
 * must start at zero is cleared by a kernel of the call): calls that can overlap on one GPU --
 * on different streams, or from different host threads -- race and must be serialized by the
 * caller. */
size_t w4a4_noalloc_scratch_bytes(void);
int w4a4_rotate_quant_act_noalloc(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                                  const int32_t *perm, const void *rot,
                                  const float *act_scale_table, int num_steps, int step,
                                  uint8_t *xq, float *x_scale, float *xrot_dbg,
                                  hipStream_t stream);

/* Hadamard-only rotation mode: the same runtime call for R_b = H_B (U_b = I), the block Hadamard
 * transform on its own [FoldQuantVLA summary, key change 2: block Hadamard transform with dynamic
 * per-token quantization; gist.science Metodologia 1 names the Hadamard factor of the composite
 * rotation]. Weights for this mode are packed by w4a4_pack_weights with U == NULL. No rotation
 * operand and no workspace: each row is staged on chip and transformed with fp64 butterflies, so x'
 * is the fp32 rounding of a value within a few fp64 ulps of X[:, perm] . blockdiag(H_B). Scales and
 * codes follow w4a4_rotate_quant_act (per-step with act_scale_table, per-token without). block must
 * be 64 or 128 and K at most 65536 (fp16 X) or 32768 (fp32 X), else W4A4_ERR_UNSUPPORTED; xq must
 * be 16-byte aligned (W4A4_ERR_ALIGN). */
int w4a4_rotate_quant_act_hadamard(const void *X, int x_dtype, int M, int K, int64_t ldx,
                                   int block, const int32_t *perm, const float *act_scale_table,
                                   int num_steps, int step, uint8_t *xq, float *x_scale,
                                   float *xrot_dbg, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * W4A4 GEMM with fused dequantization [vnrobo.com "Vi sao W4A4 kho hon W4A16?": activations must be
 * low-bit too for the compute path to be truly low-bit]. acc[m][n] = sum_k q[m][k] p[n][k] is exact
 * in int32 (int8 MFMA, |acc| <= 64 K, K <= 2^24); Y[m][n] = fp16(fp32(fp32(float(acc) * s_x) *
 * w_scale[n])) with s_x = x_scale[m] (x_scale_per_token != 0) or x_scale[0], then the epilogue.
 * xq [M][K/2], wq [N][K/2]; residual [M][N] fp16 (stride ldr) is read only by W4A4_EPI_RESIDUAL.
 * M == 0 is a valid empty call.
 * ------------------------------------------------------------------------------------------- */
size_t w4a4_gemm_workspace_bytes(int M, int N, int K);
int w4a4_gemm(const uint8_t *xq, const float *x_scale, int x_scale_per_token, const uint8_t *wq,
              const float *w_scale, int M, int N, int K, uint16_t *Y, int64_t ldy, int epilogue,
              const uint16_t *residual, int64_t ldr, void *ws, size_t ws_bytes, hipStream_t stream);

/* The GEMM above followed by the next linear's per-step rotate-quantize of part of its output:
 * the columns [col0, col0 + K_next) of Y, which the caller has arranged to hold the next linear's
 * input already in that linear's zigzag order (its perm folded into this linear's weight rows
 * offline), become the next linear's packed int4 codes xq_next [M][K_next / 2] and its scale
 * x_scale_next[0] = act_scale_table_next[step], exactly as
 *   w4a4_rotate_quant_act(Y + col0, W4A4_F16, M, K_next, ldy, block_next, NULL, rot_next,
 *                         table_next, num_steps, step, xq_next, x_scale_next, NULL, ...)
 * would give them after this GEMM [gist.science summary, "Metodologia" 1: rotate, then quantize the
 * next layer's input; vnrobo.com "Y tuong paper": the step's scale is a table lookup]. Y is written
 * in full when store_next_cols != 0; with store_next_cols == 0 the columns [col0, col0 + K_next) of
 * Y may be left unwritten (their contents are then unspecified: for a caller whose only consumer of
 * them is the next linear), but Y must still be a valid [M][N] buffer, since the non-fused case
 * below computes them there. With block_next 128 and a 128-column tile plan (M above 64, no K
 * split, 16-byte aligned rows) the rotation and quantization run in the GEMM's epilogue on the
 * finished fp16 tile, with the same arithmetic as the standalone call, so the codes are identical
 * bit for bit; any other case runs the standalone call on the same stream after the GEMM.
 * K_next == 0 (with col0 == 0) means no next linear: the call is the GEMM alone, and block_next,
 * rot_next, table_next, num_steps, step, xq_next, x_scale_next and store_next_cols are ignored.
 * res_cols (optional, device int32 [N], 4-byte aligned; residual epilogue only, N <= 65536): a
 * residual column map, so that output column n adds residual[m][res_cols[n]] instead of
 * residual[m][n]. It lets a residual stream be kept in one linear's zigzag order while the next
 * linear's output comes out in another's. Entries must lie in [0, N); the kernels clamp any other
 * entry into that range (no out-of-bounds access, but the sum is then meaningless). The tile plan
 * of the stack's 64 x 128 split-group GEMM gathers the mapped residual in its epilogue; other plans
 * gather it into the workspace first. res_order (optional, with res_cols; device int32 [N], 4-byte
 * aligned) is a gather-order hint for that epilogue: for each tile of 128 output columns starting
 * at column n0, res_order[n0 + j] is the output column (in [n0, n0 + 128)) whose residual the
 * tile's j-th lane fetches. Sorting each tile's columns by res_cols makes adjacent lanes read
 * adjacent residual columns. It must permute each tile's columns (unchecked: a column left out
 * gets an unspecified residual); NULL means column order. Other tile plans ignore it.
 * Arguments and errors as w4a4_gemm and w4a4_rotate_quant_act (per-step scale only: table_next is
 * required when K_next > 0); every argument is checked before anything is launched. ws:
 * w4a4_gemm_rq_next_workspace_bytes(M, N, K, K_next, block_next, res_cols != NULL) bytes, 256-byte
 * aligned. */
size_t w4a4_gemm_rq_next_workspace_bytes(int M, int N, int K, int K_next, int block_next,
                                         int mapped_residual);
int w4a4_gemm_rq_next(const uint8_t *xq, const float *x_scale, int x_scale_per_token,
                      const uint8_t *wq, const float *w_scale, int M, int N, int K, uint16_t *Y,
                      int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr,
                      const int32_t *res_cols, const int32_t *res_order, int col0, int K_next,
                      int block_next, const void *rot_next, const float *table_next,
                      int num_steps, int step, uint8_t *xq_next, float *x_scale_next,
                      int store_next_cols, void *ws, size_t ws_bytes, hipStream_t stream);

/* Test hook: the raw int32 accumulators acc [M][N] (row-major, dense) of the same integer GEMM. */
int w4a4_gemm_i32(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, int32_t *acc,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * FP6 matrix-core operands for the large-M GEMM [the same integer GEMM as w4a4_gemm; vnrobo.com
 * "Vi sao W4A4 kho hon W4A16?": the compute path itself must run on the low-bit codes]. Every int4
 * code is exactly representable in the OCP Microscaling E3M2 six-bit float (sign bit, 3 exponent
 * bits with bias 3, 2 mantissa bits), and gfx950's FP6 matrix instructions run at twice the int8
 * rate without any widening work. Products of two codes are exact integers and so is every fp32
 * partial sum (|sum| <= 64 K < 2^24 for K <= 2^18), so acc and Y equal those of w4a4_gemm /
 * w4a4_gemm_i32 on the same codes, bit for bit.
 * Operand layout of a code matrix [rows][K], K % 128 == 0, R2 = rows rounded up to even (the last
 * row is zeros when rows is odd), total w4a4_f6_operand_bytes(rows, K) = R2 * K * 3/4 bytes: k is
 * cut into stages of 128 and each stage into four groups of 32 consecutive k; a group's codes, as
 * E3M2 fields with code i at bits 6i..6i+5 of a 192-bit little-endian string, are split into a
 * 16-byte head (bits 0..127) and an 8-byte tail (bits 128..191). Stage s occupies the R2*96 bytes
 * from s*R2*96: heads at row*64 + 16*group, then tails at R2*64 + (group*R2 + row)*8.
 *  - w4a4_codes_to_f6: packed int4 codes [rows][K/2] -> that layout (out must hold
 *    w4a4_f6_operand_bytes(rows, K) bytes). Both pointers 16-byte aligned (W4A4_ERR_ALIGN); K not a
 *    multiple of 128 is W4A4_ERR_SHAPE. Weights are converted once, offline; activation codes after
 *    each rotate-quantize call. Bit-exact (an encoding).
 *  - w4a4_rotate_quant_act_f6: w4a4_rotate_quant_act (same arguments, per-step or per-token scales,
 *    same codes and x_scale) writing the codes in that layout (xf: w4a4_f6_operand_bytes(M, K)
 *    bytes, 16-byte aligned) instead of packed int4. block must be 128 (W4A4_ERR_UNSUPPORTED), so
 *    one rotation block is one 128-k stage; no xrot_dbg; workspace
 *    w4a4_act_f6_workspace_bytes(M, K, block, per_token). The streaming (large-batch) kernel writes
 *    the layout itself; other batch shapes quantize into the workspace and re-encode from there.
 *  - w4a4_gemm_f6 / w4a4_gemm_f6_i32: the arguments, scales, epilogues and outputs of w4a4_gemm /
 *    w4a4_gemm_i32 with xf / wf FP6 operands of M / N rows. K % 128 == 0 (W4A4_ERR_SHAPE),
 *    K <= 2^18 (W4A4_ERR_UNSUPPORTED), xf and wf 16-byte aligned (W4A4_ERR_ALIGN). Meant for
 *    M > 64, where the GEMM is bound by the matrix cores; the workspace holds split-K partials.
 * ------------------------------------------------------------------------------------------- */
size_t w4a4_f6_operand_bytes(int rows, int K);
int w4a4_codes_to_f6(const uint8_t *codes, int rows, int K, uint8_t *out, hipStream_t stream);
size_t w4a4_act_f6_workspace_bytes(int M, int K, int block, int per_token);
int w4a4_rotate_quant_act_f6(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                             const int32_t *perm, const void *rot, const float *act_scale_table,
                             int num_steps, int step, uint8_t *xf, float *x_scale, void *ws,
                             size_t ws_bytes, hipStream_t stream);
size_t w4a4_gemm_f6_workspace_bytes(int M, int N, int K);
int w4a4_gemm_f6(const uint8_t *xf, const float *x_scale, int x_scale_per_token, const uint8_t *wf,
                 const float *w_scale, int M, int N, int K, uint16_t *Y, int64_t ldy, int epilogue,
                 const uint16_t *residual, int64_t ldr, void *ws, size_t ws_bytes,
                 hipStream_t stream);
int w4a4_gemm_f6_i32(const uint8_t *xf, const uint8_t *wf, int M, int N, int K, int32_t *acc,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * W8A8 linears [radar.vhtltd.com FoldQuantVLA summary, key change 5: the attention-output and FFN
 * down projections kept at W8A8 raise the real-robot success rate at about 1 ms of latency]: the
 * same rotation, scales and calls on the symmetric int8 grid. Codes are int8, one per byte, two's
 * complement, stored [rows][K]; 7 becomes 127 in every scale (s_w[n] = fp32(max |W'| / 127),
 * per-token s_m = fp32(max |x'| / 127), calibrated table entries fp32(max |x'| / 127)) and codes are
 * clamp(rint(.), -128, 127). The rotation operand `rot` is the one w4a4_pack_weights_w8 writes (the
 * same layout as w4a4_pack_weights), and the activation workspace is w4a4_act_workspace_bytes /
 * w4a4_calibrate_workspace_bytes. Alignment: int8 wq 2 bytes, int8 xq 4 bytes (W4A4_ERR_ALIGN).
 * GEMM: acc = sum_k q p is exact in int32 for K <= 2^16 (W4A4_ERR_UNSUPPORTED above); K must be a
 * multiple of 64 (W4A4_ERR_SHAPE) and xq, wq 16-byte aligned (W4A4_ERR_ALIGN); the dequantization
 * and epilogues are those of w4a4_gemm.
 * ------------------------------------------------------------------------------------------- */
int w4a4_pack_weights_w8(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                         const int32_t *perm, const float *U, uint8_t *wq, float *w_scale,
                         void *rot, void *ws, size_t ws_bytes, hipStream_t stream);
int w4a4_calibrate_act_scale_a8(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                                const int32_t *perm, const void *rot, float *table_entry,
                                void *ws, size_t ws_bytes, hipStream_t stream);
int w4a4_rotate_quant_act_a8(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                             const int32_t *perm, const void *rot, const float *act_scale_table,
                             int num_steps, int step, uint8_t *xq, float *x_scale,
                             float *xrot_dbg, void *ws, size_t ws_bytes, hipStream_t stream);
size_t w4a4_gemm_w8a8_workspace_bytes(int M, int N, int K);
int w4a4_gemm_w8a8(const uint8_t *xq, const float *x_scale, int x_scale_per_token,
                   const uint8_t *wq, const float *w_scale, int M, int N, int K, uint16_t *Y,
                   int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr, void *ws,
                   size_t ws_bytes, hipStream_t stream);
/* Test hook: int32 accumulators of the int8 GEMM. */
int w4a4_gemm_w8a8_i32(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, int32_t *acc,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Group-wise per-step activation scales [vnrobo.com "Y tuong paper": the act_scale_table is per
 * layer, per step and per channel; gist.science item 2 "Calibracao por Passo"]: the integer-GEMM
 * form of a channel-varying table keeps one scale per (step, rotation block), and the GEMM folds
 * each block's exact int32 partial in with that block's scale. int4 codes, fp16 activations and
 * block 128 only (else W4A4_ERR_UNSUPPORTED); same weights, perm and `rot` as the per-step mode.
 *  - Calibration: table_row[g] = fp32(max |fp32(x')| / 7) over every row of X and the channels of
 *    block g (1.0f for a zero max), g in [0, K/128). Workspace: w4a4_calibrate_workspace_bytes.
 *  - Rotate-quantize: act_scale_table is [num_steps][K/128] device floats; position k of step
 *    `step` is quantized with s = table[step][k / 128] (r = fp32(1/s), q = clamp(rint(fp32(x' *
 *    r)), -8, 7)); x_scale[g] receives the K/128 scales used. Step range and entry rules as in the
 *    per-step mode, block by block (an unusable entry zeroes that block's codes and its x_scale[g]
 *    is NaN). Workspace: w4a4_act_workspace_bytes(M, K, block, 0).
 *  - GEMM: acc_g[m][n] = sum over k in block g of q p (exact), y = 0 then y = fmaf(float(acc_g),
 *    x_scales[g], y) for g = 0, 1, ... in order (one correctly rounded fused multiply-add per
 *    block), then Y = fp16(fp32(y * w_scale[n])) with the epilogues of w4a4_gemm. xq and wq must
 *    be 16-byte aligned (W4A4_ERR_ALIGN); no workspace.
 * ------------------------------------------------------------------------------------------- */
int w4a4_calibrate_act_scale_grouped(const void *X, int x_dtype, int M, int K, int64_t ldx,
                                     int block, const int32_t *perm, const void *rot,
                                     float *table_row, void *ws, size_t ws_bytes,
                                     hipStream_t stream);
int w4a4_rotate_quant_act_grouped(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                                  const int32_t *perm, const void *rot,
                                  const float *act_scale_table, int num_steps, int step,
                                  uint8_t *xq, float *x_scale, float *xrot_dbg, void *ws,
                                  size_t ws_bytes, hipStream_t stream);
int w4a4_gemm_grouped(const uint8_t *xq, const float *x_scales, const uint8_t *wq,
                      const float *w_scale, int M, int N, int K, int block, uint16_t *Y,
                      int64_t ldy, int epilogue, const uint16_t *residual, int64_t ldr,
                      hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * GPTQ weight solver, offline [vnrobo.com "Kien truc thuc thi": the backbone pack is "SVD-Hadamard
 * rotation + GPTQ pack"; "Build LLM pack": --gptq-block-size 128 --gptq-damp-percent 0.05]. It
 * replaces round-to-nearest in the weight pack; the runtime calls are unchanged. K <= 4096 (else
 * W4A4_ERR_UNSUPPORTED); int4 codes.
 *  - w4a4_gptq_hessian: H = X'^T X' (accumulate != 0: H += X'^T X') in fp64 [K][K], X' = X[:, perm]
 *    . blockdiag(U_b H_B) the rotated calibration activations (rotated in fp64 with the weight
 *    pack's fixed-order arithmetic; every entry of H summed over rows in increasing order).
 *  - w4a4_gptq_factor: dead[k] = (H[k][k] == 0) (dead may be NULL); H' = H with those diagonal
 *    entries set to 1, plus damp_percent * mean(diag H') on the diagonal; Hf (fp64 [K][K], row-major)
 *    = the upper Cholesky factor of H'^-1 (Hf^T Hf = H'^-1), computed as the reversed inverse of
 *    the lower Cholesky factor of the index-reversed H' (no explicit inverse).
 *  - w4a4_pack_weights_gptq: W' = W[:, perm] . blockdiag(R_b) in fp64 as in w4a4_pack_weights;
 *    s_w[n] = fp32(max_k |W'[n][k]| / 7) (the RTN scale, fixed); dead input channels are zeroed;
 *    then for each row and k = 0, 1, ... in order: q = clamp(rint(w[k] / s_w), -8, 7),
 *    err = (w[k] - q s_w) / Hf[k][k], w[j] -= err * Hf[k][j] for j > k (fp64, separate multiply
 *    and subtract). Codes packed into wq [N][K/2]; `rot` written as by w4a4_pack_weights. Given Hf,
 *    wq and w_scale are bit-exact functions of (W, perm, U, Hf, dead).
 * ------------------------------------------------------------------------------------------- */
size_t w4a4_gptq_hessian_workspace_bytes(int M, int K, int block);
int w4a4_gptq_hessian(const void *X, int x_dtype, int M, int K, int64_t ldx, int block,
                      const int32_t *perm, const float *U, double *H, int accumulate, void *ws,
                      size_t ws_bytes, hipStream_t stream);
size_t w4a4_gptq_factor_workspace_bytes(int K);
int w4a4_gptq_factor(const double *H, int K, double damp_percent, double *Hf, uint8_t *dead,
                     void *ws, size_t ws_bytes, hipStream_t stream);
size_t w4a4_pack_gptq_workspace_bytes(int N, int K, int block);
int w4a4_pack_weights_gptq(const void *W, int w_dtype, int N, int K, int64_t ldw, int block,
                           const int32_t *perm, const float *U, const double *Hf,
                           const uint8_t *dead, uint8_t *wq, float *w_scale, void *rot, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Diagnostics (host only).
 * ------------------------------------------------------------------------------------------- */
const char *w4a4_last_error(void);
const char *w4a4_status_string(int status);
int w4a4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
