// Offline calibration on the device: the zigzag channel permutation and the per-block SVD factor.
//
// Zigzag (gist.science summary, "Metodologia" 1, "Implementacao em Blocos"): channels are ranked by
// weight column norm and dealt over the rotation blocks so that high- and low-norm channels spread
// evenly. SVD factor ("Rotacao SVD", W = U Sigma V^T): for each block the right singular vectors of
// the block's N x B weight slice, i.e. the eigenbasis of its B x B Gram matrix, found here by a
// parallel cyclic Jacobi iteration in fp64 (Brent-Luk round-robin pairing, B/2 disjoint rotations
// per step).
#include "w4a4_internal.h"

namespace w4a4 {

// ------------------------------------------------------------------ zigzag
// c2[k] = sum over rows n = 0..N-1, in order, of W[n][k]^2 (fp64, no fused multiply-add), so the
// ranking decisions are bit-identical to any other evaluation in that order.
__global__ void k_colnorm2(const void *__restrict__ W, int wdt, int N, int K, int64_t ldw,
                           double *__restrict__ c2)
{
#pragma clang fp contract(off)
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    double s = 0.0;
    for (int n = 0; n < N; ++n) {
        double v = load_as_f64(W, wdt, (int64_t)n * ldw + k);
        double sq = v * v;
        s = s + sq;
    }
    c2[k] = s;
}

// rank(k) = #{j : c2[j] > c2[k]} + #{j < k : c2[j] == c2[k]} (stable descending order), then the
// boustrophedon deal: pass p = rank / nb, j = rank % nb, block j (p even) or nb-1-j (p odd).
__global__ __launch_bounds__(256) void k_zigzag(const double *__restrict__ c2, int K, int B,
                                                int32_t *__restrict__ perm)
{
    __shared__ double sc[1024];
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    const double mine = (k < K) ? c2[k] : 0.0;
    int rank = 0;
    for (int base = 0; base < K; base += 1024) {
        __syncthreads();
        for (int t = threadIdx.x; t < 1024; t += blockDim.x)
            sc[t] = (base + t < K) ? c2[base + t] : 0.0;
        __syncthreads();
        const int lim = min(1024, K - base);
        if (k < K) {
            for (int t = 0; t < lim; ++t) {
                const double v = sc[t];
                rank += (v > mine) || (v == mine && base + t < k);
            }
        }
    }
    if (k >= K) return;
    const int nb = K / B;
    const int pass = rank / nb, j = rank % nb;
    const int b = (pass & 1) ? nb - 1 - j : j;
    perm[b * B + pass] = k;
}

size_t zigzag_workspace(int K) { return align_up((size_t)K * sizeof(double), 256); }

int launch_zigzag(const void *W, int wdt, int N, int K, int64_t ldw, int B, int32_t *perm,
                  void *ws, hipStream_t s)
{
    double *c2 = reinterpret_cast<double *>(ws);
    hipLaunchKernelGGL(k_colnorm2, dim3((K + 255) / 256), dim3(256), 0, s, W, wdt, N, K, ldw, c2);
    hipLaunchKernelGGL(k_zigzag, dim3((K + 255) / 256), dim3(256), 0, s, c2, K, B, perm);
    return check_launch("zigzag");
}

// ------------------------------------------------------------------ Gram matrices
// Partial Gram matrices G_b^(c) = W_b[rows of chunk c]^T W_b[rows of chunk c] (fp64), one workgroup
// per (block, row chunk); the Jacobi kernel sums the chunks in order, so the result is deterministic.
constexpr int GRAM_ROWS = 2048;  // rows per chunk
constexpr int GRAM_STAGE = 16;   // rows staged in LDS at a time
constexpr int SVD_MAX_B = 128;

__global__ __launch_bounds__(256) void k_gram(const void *__restrict__ W, int wdt, int N, int K,
                                              int64_t ldw, int B, const int32_t *__restrict__ perm,
                                              double *__restrict__ partial)
{
    __shared__ double sw[GRAM_STAGE][SVD_MAX_B];
    const int b = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
    const int r0 = chunk * GRAM_ROWS, r1 = min(r0 + GRAM_ROWS, N);
    const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
    const int T = (B + 15) / 16;  // outputs per thread per dimension: i = ti + 16 a, j = tj + 16 c
    double acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = 0.0;
    for (int n0 = r0; n0 < r1; n0 += GRAM_STAGE) {
        __syncthreads();
        for (int e = threadIdx.x; e < GRAM_STAGE * B; e += blockDim.x) {
            int r = e / B, i = e % B;
            int n = n0 + r;
            int ch = perm ? perm[b * B + i] : b * B + i;
            sw[r][i] = (n < r1) ? load_as_f64(W, wdt, (int64_t)n * ldw + ch) : 0.0;
        }
        __syncthreads();
        for (int r = 0; r < GRAM_STAGE; ++r) {
            double xi[8], xj[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                int i = ti + 16 * a, j = tj + 16 * a;
                xi[a] = (a < T && i < B) ? sw[r][i] : 0.0;
                xj[a] = (a < T && j < B) ? sw[r][j] : 0.0;
            }
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[a][c] = fma(xi[a], xj[c], acc[a][c]);
        }
    }
    double *G = partial + ((int64_t)b * nchunks + chunk) * B * B;
    for (int a = 0; a < T; ++a)
        for (int c = 0; c < T; ++c) {
            int i = ti + 16 * a, j = tj + 16 * c;
            if (i < B && j < B) G[i * B + j] = acc[a][c];
        }
}

static int gram_chunks(int N) { return (N + GRAM_ROWS - 1) / GRAM_ROWS; }

// ------------------------------------------------------------------ Jacobi eigensolver
constexpr int JACOBI_MAX_SWEEPS = 40;

__global__ __launch_bounds__(256) void k_jacobi(const double *__restrict__ partial, int nchunks,
                                                int B, double *__restrict__ Vws,
                                                float *__restrict__ U)
{
    extern __shared__ double sG[];                 // B x B
    __shared__ double sc[SVD_MAX_B / 2], ss[SVD_MAX_B / 2];
    __shared__ int sp[SVD_MAX_B / 2], sq[SVD_MAX_B / 2];
    __shared__ double sred[256];
    __shared__ int sflag;
    __shared__ int srank[SVD_MAX_B];
    __shared__ double ssign[SVD_MAX_B];
    const int b = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const int half = B / 2;
    double *V = Vws + (int64_t)b * B * B;

    for (int e = tid; e < B * B; e += nt) {
        double g = 0.0;
        for (int c = 0; c < nchunks; ++c) g += partial[((int64_t)b * nchunks + c) * B * B + e];
        sG[e] = g;
        V[e] = (e / B == e % B) ? 1.0 : 0.0;
    }
    __syncthreads();
    // symmetrize exactly (the partial Grams are symmetric up to rounding order only)
    for (int e = tid; e < B * B; e += nt) {
        int i = e / B, j = e % B;
        if (i < j) {
            double v = 0.5 * (sG[i * B + j] + sG[j * B + i]);
            sG[i * B + j] = v;
            sG[j * B + i] = v;
        }
    }
    __syncthreads();

    for (int sweep = 0; sweep < JACOBI_MAX_SWEEPS && B > 1; ++sweep) {
        // convergence: off-diagonal mass against the diagonal
        double off = 0.0, dia = 0.0;
        for (int e = tid; e < B * B; e += nt) {
            double g = sG[e];
            if (e / B == e % B) dia += g * g;
            else off += g * g;
        }
        sred[tid] = off;
        __syncthreads();
        for (int w = nt / 2; w > 0; w >>= 1) {
            if (tid < w) sred[tid] += sred[tid + w];
            __syncthreads();
        }
        const double offs = sred[0];
        __syncthreads();
        sred[tid] = dia;
        __syncthreads();
        for (int w = nt / 2; w > 0; w >>= 1) {
            if (tid < w) sred[tid] += sred[tid + w];
            __syncthreads();
        }
        if (tid == 0) sflag = (offs <= 1e-30 * sred[0]) ? 1 : 0;
        __syncthreads();
        if (sflag) break;

        for (int round = 0; round < B - 1; ++round) {
            if (tid < half) {
                int p, q;
                if (tid == 0) {
                    p = 0;
                    q = 1 + (round % (B - 1));
                } else {
                    p = 1 + ((tid + round) % (B - 1));
                    q = 1 + ((B - 1 - tid + round) % (B - 1));
                }
                if (p > q) { int t = p; p = q; q = t; }
                const double apq = sG[p * B + q];
                const double app = sG[p * B + p], aqq = sG[q * B + q];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    const double theta = (aqq - app) / (2.0 * apq);
                    double t;
                    if (fabs(theta) > 1e150) t = 0.5 / theta;
                    else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
                    c = 1.0 / sqrt(t * t + 1.0);
                    s = t * c;
                }
                sp[tid] = p;
                sq[tid] = q;
                sc[tid] = c;
                ss[tid] = s;
            }
            __syncthreads();
            // G <- J^T G J, one 2x2 sub-block (pair a rows, pair c columns) per work item
            for (int e = tid; e < half * half; e += nt) {
                const int a = e / half, c = e % half;
                const int pa = sp[a], qa = sq[a], pc = sp[c], qc = sq[c];
                const double ca = sc[a], sa = ss[a], cc = sc[c], scc = ss[c];
                const double g_pp = sG[pa * B + pc], g_pq = sG[pa * B + qc];
                const double g_qp = sG[qa * B + pc], g_qq = sG[qa * B + qc];
                // T = G_sub J_c
                const double t_pp = g_pp * cc - g_pq * scc, t_pq = g_pp * scc + g_pq * cc;
                const double t_qp = g_qp * cc - g_qq * scc, t_qq = g_qp * scc + g_qq * cc;
                // J_a^T T
                double n_pp = ca * t_pp - sa * t_qp, n_pq = ca * t_pq - sa * t_qq;
                double n_qp = sa * t_pp + ca * t_qp, n_qq = sa * t_pq + ca * t_qq;
                if (a == c) n_pq = n_qp = 0.0;
                sG[pa * B + pc] = n_pp;
                sG[pa * B + qc] = n_pq;
                sG[qa * B + pc] = n_qp;
                sG[qa * B + qc] = n_qq;
            }
            // V <- V J
            for (int e = tid; e < B * half; e += nt) {
                const int r = e / half, a = e % half;
                const int p = sp[a], q = sq[a];
                const double c = sc[a], s = ss[a];
                const double vp = V[r * B + p], vq = V[r * B + q];
                V[r * B + p] = c * vp - s * vq;
                V[r * B + q] = s * vp + c * vq;
            }
            __syncthreads();
        }
    }

    // order columns by descending eigenvalue (ties to the lower index) and fix each column's sign
    for (int col = tid; col < B; col += nt) {
        const double lam = sG[col * B + col];
        int rank = 0;
        for (int o = 0; o < B; ++o) {
            const double l2 = sG[o * B + o];
            rank += (l2 > lam) || (l2 == lam && o < col);
        }
        srank[col] = rank;
        int best = 0;
        double bv = -1.0;
        for (int r = 0; r < B; ++r) {
            const double a = fabs(V[r * B + col]);
            if (a > bv) { bv = a; best = r; }
        }
        ssign[col] = (V[best * B + col] < 0.0) ? -1.0 : 1.0;
    }
    __syncthreads();
    for (int e = tid; e < B * B; e += nt) {
        const int r = e / B, col = e % B;
        U[((int64_t)b * B + r) * B + srank[col]] = (float)(ssign[col] * V[r * B + col]);
    }
}


static size_t svd_v_bytes(int K, int B) { return align_up((size_t)K * B * sizeof(double), 256); }

size_t block_svd_workspace(int N, int K, int B)
{
    // eigenvectors [nb][B][B] + partial Gram matrices [nb][chunks][B][B], fp64
    return svd_v_bytes(K, B) + align_up((size_t)K * B * gram_chunks(N) * sizeof(double), 256);
}

int launch_block_svd(const void *W, int wdt, int N, int K, int64_t ldw, int B, const int32_t *perm,
                     float *U, void *ws, hipStream_t s)
{
    const int nb = K / B, nchunks = gram_chunks(N);
    double *V = reinterpret_cast<double *>(ws);
    double *partial = reinterpret_cast<double *>(reinterpret_cast<char *>(ws) +
                                                 svd_v_bytes(K, B));
    hipLaunchKernelGGL(k_gram, dim3(nb, nchunks), dim3(256), 0, s, W, wdt, N, K, ldw, B, perm,
                       partial);
    int rc = check_launch("gram");
    if (rc != W4A4_OK) return rc;
    const size_t lds = (size_t)B * B * sizeof(double);
    if ((rc = ensure_dynamic_lds((const void *)k_jacobi, lds, "jacobi"))) return rc;
    hipLaunchKernelGGL(k_jacobi, dim3(nb), dim3(256), lds, s, partial, nchunks, B, V, U);
    return check_launch("jacobi");
}

}  // namespace w4a4
