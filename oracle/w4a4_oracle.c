/*
 * CPU oracle of the W4A4 quantized linear (Omega-QVLA composite SVD.Hadamard rotation + int4 RTN).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library. The GPU library shares no code, header or table with it.
 *
 * Plain single-threaded scalar loops. Floating point is IEEE fp64 unless a step says fp32, built with
 * -O2 -ffp-contract=off so that every product and sum is rounded exactly where it is written.
 * Every sum runs over its index in increasing order.
 *
 * Sources (the pages, cited by title and section):
 *  [P1] "Omega-QVLA: Nen VLA W4A4 tren Edge" (vnrobo.com): sections "Y tuong paper" (SVD then
 *       Hadamard, per-step act_scale_table) and "Build DiT action head pack" (--w-bits 4 --a-bits 4,
 *       --use-rtn, --duquant-block-size 64, --num-steps 8).
 *  [P2] gist.science (pt) technical summary of arXiv 2605.28803, section "Metodologia", item 1
 *       "Rotacao Composta SVD.Hadamard": W = U Sigma V^T, R = R_SVD . H, block implementation with a
 *       zigzag permutation ordered by weight column norms; item 2 "Escalonamento ... por Passo".
 *  [P4] the same summary in French, "Methodologie" items 1 and 2.
 *  [P5] FoldQuantVLA summary (radar.vhtltd.com): dynamic per-token activation quantization.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Squared L2 norm of every input channel k of W[N][K] (row-major, nn.Linear layout):
 * c2[k] = sum_n W[n][k]^2, n increasing. The zigzag order ranks channels by weight column norm
 * [P2 Metodologia 1, "Implementacao em Blocos"]; ranking by the square gives the same order. */
void orc_colnorm2(const double *W, int64_t N, int64_t K, double *c2)
{
    for (int64_t k = 0; k < K; ++k) c2[k] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double *row = W + n * K;
        for (int64_t k = 0; k < K; ++k) {
            double v = row[k];
            double sq = v * v;
            c2[k] = c2[k] + sq;
        }
    }
}

/* Entry (l, j) of the normalized natural-order Sylvester Hadamard matrix of size B (power of two):
 * (-1)^popcount(l & j) / sqrt(B) [P2 Metodologia 1, "Rotacao Hadamard": normalized Hadamard H]. */
static double orc_hadamard_entry(int64_t l, int64_t j, int64_t B)
{
    int64_t bits = l & j;
    int parity = 0;
    while (bits) { parity ^= (int)(bits & 1); bits >>= 1; }
    double inv = 1.0 / sqrt((double)B);
    return parity ? -inv : inv;
}

void orc_hadamard(int64_t B, double *H)
{
    for (int64_t l = 0; l < B; ++l)
        for (int64_t j = 0; j < B; ++j) H[l * B + j] = orc_hadamard_entry(l, j, B);
}

/* Composite rotation of every block, R_b = U_b . H_B [P2 Metodologia 1: R = R_SVD . H], fp64.
 * U is fp32 [nb][B][B] row-major (U_b[i][l] = U[(b*B+i)*B + l]); R is fp64 in the same layout.
 * R_b[i][j] = sum_l U_b[i][l] * H[l][j], l increasing. */
void orc_rotation(const float *U, int64_t K, int64_t B, double *R)
{
    int64_t nb = K / B;
    double *H = (double *)malloc((size_t)(B * B) * sizeof(double));
    orc_hadamard(B, H);
    for (int64_t b = 0; b < nb; ++b)
        for (int64_t i = 0; i < B; ++i)
            for (int64_t j = 0; j < B; ++j) {
                double s = 0.0;
                for (int64_t l = 0; l < B; ++l) {
                    double p = (double)U[(b * B + i) * B + l] * H[l * B + j];
                    s = s + p;
                }
                R[(b * B + i) * B + j] = s;
            }
    free(H);
}

/* Rotated rows: Y = A[:, perm] . blockdiag(R_0 .. R_{nb-1}) for A[rows][K] fp64 (row stride lda).
 * Y[r][b*B + j] = sum_i A[r][perm[b*B + i]] * R_b[i][j], i increasing. perm[j] is the original
 * channel that lands at permuted position j. Used for both weights (rows = output channels) and
 * activations (rows = tokens): X' W'^T = X P R R^T P^T W^T = X W^T. */
void orc_rotate_rows(const double *A, int64_t rows, int64_t K, int64_t lda, int64_t B,
                     const int32_t *perm, const double *R, double *Y)
{
    int64_t nb = K / B;
    double *g = (double *)malloc((size_t)B * sizeof(double));
    for (int64_t r = 0; r < rows; ++r) {
        const double *a = A + r * lda;
        for (int64_t b = 0; b < nb; ++b) {
            for (int64_t i = 0; i < B; ++i) g[i] = a[perm[b * B + i]];
            const double *Rb = R + b * B * B;
            for (int64_t j = 0; j < B; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < B; ++i) {
                    double p = g[i] * Rb[i * B + j];
                    s = s + p;
                }
                Y[r * K + b * B + j] = s;
            }
        }
    }
    free(g);
}

static int8_t orc_clamp_code(double v)
{
    if (v < -8.0) return -8;
    if (v > 7.0) return 7;
    return (int8_t)v;
}

/* The same symmetric grid at another width: codes in [-(qmax + 1), qmax], qmax = 2^(bits-1) - 1
 * (7 for int4; 127 for the int8 codes of the W8A8 linears that the FoldQuantVLA summary keeps for
 * the attention-output and FFN-down projections, key change 5). */
static int8_t orc_clamp_q(double v, int qmax)
{
    if (v < -(double)qmax - 1.0) return (int8_t)(-qmax - 1);
    if (v > (double)qmax) return (int8_t)qmax;
    return (int8_t)v;
}

/* Per-output-channel symmetric RTN at width qmax: s_w[n] = fp32(max_k |W'[n][k]| / qmax) (1.0f for a
 * zero row), p = clamp(rint(W' / s_w), -(qmax + 1), qmax), in fp64. */
void orc_weight_rtn_q(const double *Wr, int64_t N, int64_t K, int qmax, float *s_w, int8_t *p)
{
    for (int64_t n = 0; n < N; ++n) {
        const double *w = Wr + n * K;
        double m = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = fabs(w[k]);
            if (a > m) m = a;
        }
        float s = (m > 0.0) ? (float)(m / (double)qmax) : 1.0f;
        s_w[n] = s;
        for (int64_t k = 0; k < K; ++k) p[n * K + k] = orc_clamp_q(rint(w[k] / (double)s), qmax);
    }
}

/* Activation quantization at width qmax, as orc_act_quant with 7 replaced by qmax:
 * per-token s_m = fp32(max_k |x32[m][k]| / qmax); q = clamp(rint(fp32(x32 * r)), -(qmax + 1), qmax). */
void orc_act_quant_q(const double *Xr, int64_t rows, int64_t K, int mode, float table_scale,
                     int qmax, float *x32, float *v, int8_t *q, float *scale)
{
    for (int64_t m = 0; m < rows; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float x = (float)Xr[m * K + k];
            x32[m * K + k] = x;
            float a = fabsf(x);
            if (a > amax) amax = a;
        }
        float s;
        if (mode == 0) s = table_scale;
        else s = (amax > 0.0f) ? (float)((double)amax / (double)qmax) : 1.0f;
        scale[m] = s;
        float r = (float)(1.0 / (double)s);
        for (int64_t k = 0; k < K; ++k) {
            float y = x32[m * K + k] * r;
            v[m * K + k] = y;
            float t = rintf(y);
            q[m * K + k] = orc_clamp_q((double)t, qmax);
        }
    }
}

/* Per-output-channel symmetric 4-bit round-to-nearest of the rotated weights
 * [P1 "Build DiT action head pack": --use-rtn --w-bits 4]:
 * s_w[n] = fp32(max_k |W'[n][k]| / 7) (divided in fp64, then rounded once to fp32), 1.0f for an
 * all-zero row; p = clamp(rint(W' / s_w), -8, 7) with rint rounding half to even. */
void orc_weight_rtn(const double *Wr, int64_t N, int64_t K, float *s_w, int8_t *p)
{
    for (int64_t n = 0; n < N; ++n) {
        const double *w = Wr + n * K;
        double m = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = fabs(w[k]);
            if (a > m) m = a;
        }
        float s = (m > 0.0) ? (float)(m / 7.0) : 1.0f;
        s_w[n] = s;
        for (int64_t k = 0; k < K; ++k) p[n * K + k] = orc_clamp_code(rint(w[k] / (double)s));
    }
}

/* Activation quantization in fp32 (the precision in which the decision is taken on the device too).
 * x32 = fp32(x'); r = fp32(1/s); q = clamp(rint(fp32(x32 * r)), -8, 7).
 * mode 0, per-step [P1 "Y tuong paper": the runtime looks up the current denoising step's scale in the
 *   act_scale_table]: s = table_scale for every row.
 * mode 1, per-token [P5 key change 2: dynamic per-token quantization]:
 *   s_m = fp32(max_k |x32[m][k]| / 7), 1.0f for an all-zero row.
 * Writes x32 [rows][K], the fp32 pre-rounding value v = x32*r [rows][K], codes, and the scale per row. */
void orc_act_quant(const double *Xr, int64_t rows, int64_t K, int mode, float table_scale,
                   float *x32, float *v, int8_t *q, float *scale)
{
    for (int64_t m = 0; m < rows; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float x = (float)Xr[m * K + k];
            x32[m * K + k] = x;
            float a = fabsf(x);
            if (a > amax) amax = a;
        }
        float s;
        if (mode == 0) s = table_scale;
        else s = (amax > 0.0f) ? (float)((double)amax / 7.0) : 1.0f;
        scale[m] = s;
        float r = (float)(1.0 / (double)s);
        for (int64_t k = 0; k < K; ++k) {
            float y = x32[m * K + k] * r;
            v[m * K + k] = y;
            float t = rintf(y);
            q[m * K + k] = orc_clamp_code((double)t);
        }
    }
}

/* Group-wise per-step activation quantization (one scale per rotation block, the integer-GEMM
 * form of a per-channel act_scale_table): position k uses s[k / B];
 * q = clamp(rint(fp32(x32 * fp32(1 / s_g))), -8, 7), every step as in orc_act_quant. */
void orc_act_quant_grouped(const double *Xr, int64_t rows, int64_t K, int64_t B, const float *s,
                           float *x32, float *v, int8_t *q)
{
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float x = (float)Xr[m * K + k];
            x32[m * K + k] = x;
            float r = (float)(1.0 / (double)s[k / B]);
            float y = x * r;
            v[m * K + k] = y;
            q[m * K + k] = orc_clamp_code((double)rintf(y));
        }
}

/* Integer GEMM split by rotation block: acc[g][m][n] = sum over k in block g of q[m][k] p[n][k],
 * in int64, k increasing. */
void orc_int_gemm_grouped(const int8_t *q, const int8_t *p, int64_t M, int64_t N, int64_t K,
                          int64_t B, int64_t *acc)
{
    int64_t nb = K / B;
    for (int64_t g = 0; g < nb; ++g)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                int64_t t = 0;
                for (int64_t k = g * B; k < (g + 1) * B; ++k)
                    t += (int64_t)q[m * K + k] * (int64_t)p[n * K + k];
                acc[(g * M + m) * N + n] = t;
            }
}

/* Group-wise dequantization: y = 0, then for g = 0, 1, ..., nb - 1: y = fmaf((float)acc_g, s_g, y)
 * (one correctly rounded fused multiply-add per block, in block order), then y = fp32(y * s_w[n]). */
void orc_dequant_grouped(const int64_t *acc, int64_t nb, int64_t M, int64_t N, const float *sg,
                         const float *sw, float *y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float t = 0.0f;
            for (int64_t g = 0; g < nb; ++g)
                t = fmaf((float)acc[(g * M + m) * N + n], sg[g], t);
            y[m * N + n] = t * sw[n];
        }
}

/* GPTQ column sweep over the rotated weights (optimal-brain-quantization updates with the inverse
 * Hessian's upper Cholesky factor Hf, row-major K x K): for every row n independently and for
 * k = 0, 1, ..., K-1 in order, q = clamp(rint(w[k] / s_w[n]), -8, 7) (the row's RTN scale, fixed),
 * err = (w[k] - q * s_w[n]) / Hf[k][k], and w[j] = w[j] - err * Hf[k][j] for j > k; fp64 with
 * separate multiply and subtract. `w` is a K-double scratch row. */
void orc_gptq_sweep(const double *Wr, int64_t N, int64_t K, const double *Hf, const float *s_w,
                    double *w, int8_t *q)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) w[k] = Wr[n * K + k];
        double s = (double)s_w[n];
        for (int64_t k = 0; k < K; ++k) {
            int8_t c = orc_clamp_code(rint(w[k] / s));
            q[n * K + k] = c;
            double err = (w[k] - (double)c * s) / Hf[k * K + k];
            for (int64_t j = k + 1; j < K; ++j) {
                double t = err * Hf[k * K + j];
                w[j] = w[j] - t;
            }
        }
    }
}

/* Two's-complement nibble packing, two codes per byte, low nibble = even k. */
void orc_pack(const int8_t *q, int64_t rows, int64_t K, uint8_t *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t lo = (uint8_t)(q[r * K + 2 * j] & 0xF);
            uint8_t hi = (uint8_t)(q[r * K + 2 * j + 1] & 0xF);
            out[r * (K / 2) + j] = (uint8_t)(lo | (uint8_t)(hi << 4));
        }
}

void orc_unpack(const uint8_t *in, int64_t rows, int64_t K, int8_t *q)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = in[r * (K / 2) + j];
            int lo = b & 0xF, hi = (b >> 4) & 0xF;
            q[r * K + 2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            q[r * K + 2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
}

/* Integer GEMM: acc[m][n] = sum_k q[m][k] * p[n][k] in int64 (the low-bit integer product that W4A4
 * exists for [P1 "Vi sao W4A4 kho hon W4A16?"]). q is [M][K], p is [N][K]. */
void orc_int_gemm(const int8_t *q, const int8_t *p, int64_t M, int64_t N, int64_t K, int64_t *acc)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)q[m * K + k] * (int64_t)p[n * K + k];
            acc[m * N + n] = s;
        }
}

/* Dot products for sampled output positions (m_i, n_i) only. */
void orc_int_gemm_sampled(const int8_t *q, const int8_t *p, int64_t K, int64_t count,
                          const int64_t *mi, const int64_t *ni, int64_t *acc)
{
    for (int64_t t = 0; t < count; ++t) {
        const int8_t *a = q + mi[t] * K, *b = p + ni[t] * K;
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
        acc[t] = s;
    }
}

/* Dequantization to fp32: y = fp32(fp32(float(acc) * s_x) * s_w[n]), s_x the row's per-token scale
 * or the step's table scale. The fp16 rounding and the optional epilogues are applied by the caller. */
void orc_dequant(const int64_t *acc, int64_t M, int64_t N, const float *sx, int sx_per_token,
                 const float *sw, float *y)
{
    for (int64_t m = 0; m < M; ++m) {
        float s = sx_per_token ? sx[m] : sx[0];
        for (int64_t n = 0; n < N; ++n) {
            float a = (float)acc[m * N + n];
            float t = a * s;
            y[m * N + n] = t * sw[n];
        }
    }
}

/* Exact erf-GELU in fp64 of an fp32 input: 0.5 v (1 + erf(v / sqrt 2)). */
void orc_gelu(const float *in, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        double v = (double)in[i];
        out[i] = 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
    }
}
