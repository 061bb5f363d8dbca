// GPTQ weight solver on the device (offline): Hessian of the rotated calibration activations,
// damped inverse-Hessian Cholesky factor, and the per-row column sweep that chooses the int4 codes
// [vnrobo.com "Kien truc thuc thi": the backbone pack is "SVD-Hadamard rotation + GPTQ pack";
// "Build LLM pack": --gptq-block-size 128 --gptq-damp-percent 0.05]. The sweep runs the plain
// sequential form (the 128-column lazy batches of the flag only reorder the same updates), in fp64
// with separate multiply and subtract, so given the factor its codes are exactly reproducible.
#include <cmath>

#include "w4a4_internal.h"

namespace w4a4 {

// ------------------------------------------------------------------ Hessian: H (+)= A^T A
// 16 x 16 output tile per workgroup, rows of A streamed through LDS 16 at a time; every entry sums
// its products in increasing row order, and H[i][j], H[j][i] use the same products in the same
// order, so H is exactly symmetric and reproducible.
constexpr int GT = 16;

__global__ __launch_bounds__(GT * GT) void k_gram_f64(const double *__restrict__ A, int rows, int K,
                                                      double *__restrict__ H, int accumulate)
{
#pragma clang fp contract(off)
    __shared__ double si[GT][GT], sj[GT][GT];
    const int ti = threadIdx.x / GT, tj = threadIdx.x % GT;
    const int i0 = blockIdx.y * GT, j0 = blockIdx.x * GT;
    double acc = 0.0;
    for (int m0 = 0; m0 < rows; m0 += GT) {
        const int m = m0 + ti;
        si[ti][tj] = (m < rows && i0 + tj < K) ? A[(int64_t)m * K + i0 + tj] : 0.0;
        sj[ti][tj] = (m < rows && j0 + tj < K) ? A[(int64_t)m * K + j0 + tj] : 0.0;
        __syncthreads();
        const int mlen = min(GT, rows - m0);
        for (int t = 0; t < mlen; ++t) {
            const double p = si[t][ti] * sj[t][tj];
            acc = acc + p;
        }
        __syncthreads();
    }
    const int i = i0 + ti, j = j0 + tj;
    if (i < K && j < K) {
        double *h = H + (int64_t)i * K + j;
        *h = accumulate ? *h + acc : acc;
    }
}

int launch_gram_f64(const double *A, int rows, int K, double *H, bool accumulate, hipStream_t s)
{
    dim3 grid((K + GT - 1) / GT, (K + GT - 1) / GT);
    hipLaunchKernelGGL(k_gram_f64, grid, dim3(GT * GT), 0, s, A, rows, K, H, accumulate ? 1 : 0);
    return check_launch("gptq hessian");
}

// ------------------------------------------------------------------ inverse-Hessian factor
// Hf = upper Cholesky factor of (H')^-1, H' = H with dead channels (zero diagonal) given a unit
// diagonal, plus damp * mean(diag H') on the diagonal. With P the index reversal, G = P H' P =
// L L^T (lower Cholesky) gives (H')^-1 = (P L^-1 P)^T (P L^-1 P), and P L^-1 P is upper
// triangular with a positive diagonal, so Hf = P L^-1 P: one Cholesky and one triangular inverse,
// no explicit inverse.

// one workgroup: dead flags and the damping term (diagonal summed in a fixed order)
__global__ __launch_bounds__(256) void k_gptq_damp(const double *__restrict__ H, int K,
                                                   double damp_percent, uint8_t *__restrict__ dead,
                                                   double *__restrict__ damp)
{
    __shared__ double part[256];
    double s = 0.0;
    for (int k = threadIdx.x; k < K; k += 256) {
        const double d = H[(int64_t)k * K + k];
        const bool z = (d == 0.0);
        if (dead) dead[k] = z ? 1 : 0;
        s = s + (z ? 1.0 : d);
    }
    part[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < 256; ++i) t = t + part[i];
        damp[0] = damp_percent * (t / (double)K);
    }
}

// G[i][j] = H'[K-1-i][K-1-j] + damp on the diagonal
__global__ void k_gptq_reverse(const double *__restrict__ H, int K, const double *__restrict__ damp,
                               double *__restrict__ G)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)K * K) return;
    const int i = (int)(idx / K), j = (int)(idx % K);
    double v = H[(int64_t)(K - 1 - i) * K + (K - 1 - j)];
    if (i == j) v = ((v == 0.0) ? 1.0 : v) + damp[0];
    G[idx] = v;
}

// right-looking Cholesky step j: G[i][k] -= L[i][j] L[k][j] for j < k <= i, with L[x][j] =
// G[x][j] / sqrt(G[j][j]) read from the (still unscaled) column j, which this step never writes
__global__ void k_chol_step(double *__restrict__ G, int K, int j)
{
#pragma clang fp contract(off)
    const int i = j + 1 + blockIdx.y * 16 + threadIdx.x / 16;
    const int k = j + 1 + blockIdx.x * 16 + threadIdx.x % 16;
    if (i >= K || k > i) return;
    const double d = sqrt(G[(int64_t)j * K + j]);
    const double lij = G[(int64_t)i * K + j] / d;
    const double lkj = G[(int64_t)k * K + j] / d;
    const double p = lij * lkj;
    G[(int64_t)i * K + k] = G[(int64_t)i * K + k] - p;
}

// final column scaling: L[i][j] = G[i][j] / sqrt(G[j][j]) (i > j), L[j][j] = sqrt(G[j][j])
__global__ void k_chol_scale(double *__restrict__ G, int K)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)K * K) return;
    const int i = (int)(idx / K), j = (int)(idx % K);
    if (j > i) return;
    const double d = sqrt(G[(int64_t)j * K + j]);
    // the diagonal is read by every entry of its column: write it in a second kernel
    if (i > j) G[idx] = G[idx] / d;
}

__global__ void k_chol_diag(double *__restrict__ G, int K)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < K) G[(int64_t)j * K + j] = sqrt(G[(int64_t)j * K + j]);
}

// column c of L^-1 by forward substitution (one wave per column, the column kept in LDS), written
// reversed into the upper factor: Hf[K-1-i][K-1-c] = (L^-1)[i][c]; entries below Hf's diagonal are
// zeroed
__global__ __launch_bounds__(64) void k_tri_inverse(const double *__restrict__ L, int K,
                                                    double *__restrict__ Hf)
{
#pragma clang fp contract(off)
    extern __shared__ double x[];
    const int c = blockIdx.x, lane = threadIdx.x;
    if (lane == 0) x[c] = 1.0 / L[(int64_t)c * K + c];
    __syncthreads();
    for (int i = c + 1; i < K; ++i) {
        const double *li = L + (int64_t)i * K;
        double s = 0.0;
        for (int k = c + lane; k < i; k += 64) {
            const double p = li[k] * x[k];
            s = s + p;
        }
        for (int off = 32; off > 0; off >>= 1) s = s + __shfl_xor(s, off);
        if (lane == 0) x[i] = -s / li[i];
        __syncthreads();
    }
    const int col = K - 1 - c;
    for (int i = lane; i < K; i += 64) {
        // Hf row K-1-i, column K-1-c holds (L^-1)[i][c], zero for i < c
        Hf[(int64_t)(K - 1 - i) * K + col] = (i >= c) ? x[i] : 0.0;
    }
}

int launch_gptq_factor(const double *H, int K, double damp_percent, double *Hf, uint8_t *dead,
                       double *work, hipStream_t s)
{
    double *G = work;
    double *damp = work + (int64_t)K * K;
    const int64_t KK = (int64_t)K * K;
    hipLaunchKernelGGL(k_gptq_damp, dim3(1), dim3(256), 0, s, H, K, damp_percent, dead, damp);
    hipLaunchKernelGGL(k_gptq_reverse, dim3((unsigned)((KK + 255) / 256)), dim3(256), 0, s, H, K,
                       damp, G);
    for (int j = 0; j + 1 < K; ++j) {
        const int rem = K - 1 - j;
        dim3 grid((rem + 15) / 16, (rem + 15) / 16);
        hipLaunchKernelGGL(k_chol_step, grid, dim3(256), 0, s, G, K, j);
    }
    hipLaunchKernelGGL(k_chol_scale, dim3((unsigned)((KK + 255) / 256)), dim3(256), 0, s, G, K);
    hipLaunchKernelGGL(k_chol_diag, dim3((K + 255) / 256), dim3(256), 0, s, G, K);
    hipLaunchKernelGGL(k_tri_inverse, dim3(K), dim3(64), (size_t)K * sizeof(double), s, G, K, Hf);
    return check_launch("gptq factor");
}

// ------------------------------------------------------------------ column sweep
// One wave per weight row, ROWS rows per workgroup sharing the factor rows, which are staged in
// LDS one step ahead (only the part a later step reads: Hf[k][j], j >= k). Lane l holds positions
// l + 64 t (t < SLOTS) of its row in registers (ROWS is 8 for the longest rows, so the workgroup's
// register budget holds them; 4 rows at 4096). Step k: the owning lane quantizes w[k] with the row's fixed RTN
// scale, err = (w[k] - q s) / Hf[k][k] is broadcast, and every position j > k takes
// w[j] = w[j] - err * Hf[k][j].
template <int SLOTS, int ROWS>
__global__ __launch_bounds__(64 * ROWS) void k_gptq_sweep(
    const double *__restrict__ Wr, int N, int K, const double *__restrict__ Hf,
    const uint8_t *__restrict__ dead, const unsigned long long *__restrict__ rowmax,
    int8_t *__restrict__ codes, float *__restrict__ w_scale)
{
#pragma clang fp contract(off)
    extern __shared__ double hrow[];  // [2][K]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * ROWS + wave;
    const bool live = n < N;
    double w[SLOTS];
    float sf = 1.0f;
    if (live) {
        const double m = __longlong_as_double((long long)rowmax[n]);
        sf = (m > 0.0) ? (float)(m / 7.0) : 1.0f;
        if (lane == 0) w_scale[n] = sf;
    }
    const double s = (double)sf;
#pragma unroll
    for (int t = 0; t < SLOTS; ++t) {
        const int j = lane + 64 * t;
        w[t] = (live && j < K && !(dead && dead[j])) ? Wr[(int64_t)n * K + j] : 0.0;
    }
    for (int e = threadIdx.x; e < K; e += blockDim.x) hrow[e] = Hf[e];
    __syncthreads();
    for (int k = 0; k < K; ++k) {
        const double *h = hrow + (k & 1) * K;
        if (k + 1 < K) {
            double *nx = hrow + ((k + 1) & 1) * K;
            for (int e = k + 1 + threadIdx.x; e < K; e += blockDim.x)
                nx[e] = Hf[(int64_t)(k + 1) * K + e];
        }
        double wk = 0.0;
#pragma unroll
        for (int t = 0; t < SLOTS; ++t)
            if (t == (k >> 6)) wk = w[t];
        double qd = rint(wk / s);
        qd = fmin(fmax(qd, -8.0), 7.0);
        const double r = qd * s;
        double err = (wk - r) / h[k];
        err = __shfl(err, k & 63);
        if (live && lane == (k & 63)) codes[(int64_t)n * K + k] = (int8_t)qd;
#pragma unroll
        for (int t = 0; t < SLOTS; ++t) {
            const int j = lane + 64 * t;
            if (j > k && j < K) {
                const double p = err * h[j];
                w[t] = w[t] - p;
            }
        }
        __syncthreads();
    }
}

int launch_gptq_sweep(const double *Wr, int N, int K, const double *Hf, const uint8_t *dead,
                      const unsigned long long *rowmax, int8_t *codes, float *w_scale,
                      hipStream_t s)
{
    const size_t lds = 2 * (size_t)K * sizeof(double);
#define W4A4_SWEEP(SL, RW)                                                                         \
    do {                                                                                           \
        const int lrc = ensure_dynamic_lds((const void *)k_gptq_sweep<SL, RW>, lds, "gptq sweep"); \
        if (lrc != W4A4_OK) return lrc;                                                            \
        hipLaunchKernelGGL((k_gptq_sweep<SL, RW>), dim3((N + RW - 1) / RW), dim3(64 * RW), lds, s, \
                           Wr, N, K, Hf, dead, rowmax, codes, w_scale);                            \
    } while (0)
    if (K <= 256) W4A4_SWEEP(4, 16);
    else if (K <= 1024) W4A4_SWEEP(16, 16);
    else if (K <= 2048) W4A4_SWEEP(32, 8);
    else W4A4_SWEEP(64, 4);
#undef W4A4_SWEEP
    return check_launch("gptq sweep");
}

// two int4 codes per byte, low nibble = even k
__global__ void k_pack_codes(const int8_t *__restrict__ codes, int64_t bytes, uint8_t *__restrict__ wq)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= bytes) return;
    wq[i] = (uint8_t)((codes[2 * i] & 0xF) | ((codes[2 * i + 1] & 0xF) << 4));
}

int launch_pack_codes(const int8_t *codes, int N, int K, uint8_t *wq, hipStream_t s)
{
    const int64_t bytes = (int64_t)N * (K / 2);
    hipLaunchKernelGGL(k_pack_codes, dim3((unsigned)((bytes + 255) / 256)), dim3(256), 0, s, codes,
                       bytes, wq);
    return check_launch("pack codes");
}

}  // namespace w4a4
