// Offline weight side: composite block rotation R_b = U_b . H_B, weight rotation W' = W[:, perm] R,
// per-output-channel int4 RTN and nibble packing, all on the device.
//
// The rotation and RTN follow the gist.science summary of arXiv 2605.28803 ("Metodologia", item 1:
// R = R_SVD . H with a normalized Hadamard H, applied block by block after the zigzag permutation)
// and the DiT builder flags on vnrobo.com ("Build DiT action head pack": --use-rtn --w-bits 4,
// --svd-rank 0). Weight codes and scales are integer/fp32 results of fp64 arithmetic, so every dot
// product here is evaluated in a fixed order (increasing index, separate multiply and add, no
// contraction) that makes them exactly reproducible.
#include "w4a4_internal.h"

namespace w4a4 {

// One thread per (b, i, j): R64[b][i][j] = sum_l U_b[i][l] * H[l][j], l increasing (U == NULL
// stands for U_b = I, giving R_b = H exactly); also the fp32 copy and the fp16 high/low split (MFMA
// operand order) consumed by the activation kernels.
__global__ void k_rotation(const float *__restrict__ U, int K, int B, double hinv,
                           double *__restrict__ R64, float *__restrict__ r32,
                           __half *__restrict__ rhi, __half *__restrict__ rlo)
{
#pragma clang fp contract(off)
    const int64_t total = (int64_t)K * B;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int j = (int)(idx % B);
    const int64_t bi = idx / B;  // b * B + i
    const int b = (int)(bi / B);
    const int i = (int)(bi % B);
    double s = 0.0;
    if (U) {
        const float *u = U + bi * B;
        for (int l = 0; l < B; ++l) {
            double h = hadamard_negative(l, j) ? -hinv : hinv;
            double p = (double)u[l] * h;
            s = s + p;
        }
    } else {
        s = hadamard_negative(i, j) ? -hinv : hinv;
    }
    R64[idx] = s;
    if (!r32) return;  // fp64 rotation only (the GPTQ Hessian's activation rotation)
    r32[idx] = (float)s;
    // split: hi = fp16(R), lo = fp16((R - hi) * 2^shift)
    __half hi = __float2half_rn((float)s);
    double rem = s - (double)__half2float(hi);
    __half lo = __float2half_rn((float)(rem * (double)(1 << ROT_LO_SHIFT)));
    const int64_t t = rot16_index(b, i, j, B);
    rhi[t] = hi;
    rlo[t] = lo;
}

int launch_rotation(const float *U, int K, int B, double hinv, double *R64, void *rot,
                    hipStream_t s)
{
    RotLayout L = rot_layout(K, B);
    char *base = reinterpret_cast<char *>(rot);
    float *r32 = rot ? reinterpret_cast<float *>(base) : nullptr;
    __half *rhi = rot ? reinterpret_cast<__half *>(base + L.r32) : nullptr;
    __half *rlo = rot ? reinterpret_cast<__half *>(base + L.r32 + L.r16) : nullptr;
    const int64_t total = (int64_t)K * B;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(k_rotation, dim3((unsigned)blocks), dim3(threads), 0, s, U, K, B, hinv, R64,
                       r32, rhi, rlo);
    return check_launch("rotation");
}

__global__ void k_fill_u64(unsigned long long *p, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

// Weight rotation, passes over the same fixed-order arithmetic:
//   PASS 0: per-row max |W'| (fp64 bits, atomic max of non-negative values is order independent);
//   PASS 1: s_w = fp32(max / 7), codes = clamp(rint(W' / s_w), -8, 7), packed two per byte;
//   PASS 2: the rotated rows themselves, fp64 [rows][K] into `wrot` (the GPTQ solver's weights, and
//           the rotated calibration activations its Hessian is built from).
// Workgroup = (ROWS output rows) x (a 256-position chunk of K, which holds whole blocks since the
// block divides 256 or equals it); each thread owns two adjacent positions (one output byte).
constexpr int WP_ROWS = 8;
constexpr int WP_CHUNK = 256;

template <int PASS>
__global__ __launch_bounds__(128) void k_weight_pack(const void *__restrict__ W, int wdt, int N,
                                                     int K, int64_t ldw, int B,
                                                     const int32_t *__restrict__ perm,
                                                     const double *__restrict__ R64,
                                                     unsigned long long *__restrict__ rowmax,
                                                     uint8_t *__restrict__ wq,
                                                     float *__restrict__ w_scale, int qmax,
                                                     double *__restrict__ wrot = nullptr)
{
#pragma clang fp contract(off)
    __shared__ double sW[WP_ROWS][WP_CHUNK];
    __shared__ double sMax[WP_ROWS][4];
    const int n0 = blockIdx.x * WP_ROWS;
    const int k0 = blockIdx.y * WP_CHUNK;
    const int kend = min(k0 + WP_CHUNK, K);
    const int tid = threadIdx.x;

    // gather W[n][perm[c]] for the chunk, widened to fp64 (exact)
    for (int e = tid; e < WP_ROWS * WP_CHUNK; e += blockDim.x) {
        int r = e / WP_CHUNK, c = e % WP_CHUNK;
        int n = n0 + r, k = k0 + c;
        double v = 0.0;
        if (n < N && k < kend) {
            int src = perm ? perm[k] : k;
            v = load_as_f64(W, wdt, (int64_t)n * ldw + src);
        }
        sW[r][c] = v;
    }
    __syncthreads();

    const int kp = k0 + 2 * tid;  // first of this thread's two positions
    const bool active = kp < kend;
    double acc[WP_ROWS][2];
#pragma unroll
    for (int r = 0; r < WP_ROWS; ++r) acc[r][0] = acc[r][1] = 0.0;
    if (active) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kp + h;
            const int b = k / B, j = k % B;
            const int cb = b * B - k0;  // chunk offset of the block start
            const double *Rb = R64 + (int64_t)b * B * B + j;
            for (int i = 0; i < B; ++i) {
                const double rij = Rb[(int64_t)i * B];
#pragma unroll
                for (int r = 0; r < WP_ROWS; ++r) {
                    double p = sW[r][cb + i] * rij;
                    acc[r][h] = acc[r][h] + p;
                }
            }
        }
    }

    if (PASS == 2) {
        if (!active) return;
#pragma unroll
        for (int r = 0; r < WP_ROWS; ++r) {
            const int n = n0 + r;
            if (n >= N) continue;
            wrot[(int64_t)n * K + kp] = acc[r][0];
            if (kp + 1 < kend) wrot[(int64_t)n * K + kp + 1] = acc[r][1];
        }
        return;
    }
    if (PASS == 0) {
        // row max over this workgroup's positions, then one atomic per row
        const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int r = 0; r < WP_ROWS; ++r) {
            double m = active ? fmax(fabs(acc[r][0]), fabs(acc[r][1])) : 0.0;
            for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
            if (lane == 0) sMax[r][wave] = m;
        }
        __syncthreads();
        if (tid < WP_ROWS && n0 + tid < N) {
            double m = 0.0;
            for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = fmax(m, sMax[tid][w]);
            atomicMax(&rowmax[n0 + tid], (unsigned long long)__double_as_longlong(m));
        }
    } else {
#pragma unroll
        for (int r = 0; r < WP_ROWS; ++r) {
            const int n = n0 + r;
            if (n >= N) continue;
            const double m = __longlong_as_double((long long)rowmax[n]);
            const float s = (m > 0.0) ? (float)(m / (double)qmax) : 1.0f;
            if (blockIdx.y == 0 && tid == 0) w_scale[n] = s;
            if (!active) continue;
            int q[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                double v = rint(acc[r][h] / (double)s);
                v = fmin(fmax(v, -(double)qmax - 1.0), (double)qmax);
                q[h] = (int)v;
            }
            if (qmax == 7)
                wq[(int64_t)n * (K / 2) + kp / 2] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
            else
                *reinterpret_cast<uint16_t *>(&wq[(int64_t)n * K + kp]) =
                    (uint16_t)((q[0] & 0xFF) | ((q[1] & 0xFF) << 8));
        }
    }
}

int launch_weight_pack(const void *W, int wdt, int N, int K, int64_t ldw, int B,
                       const int32_t *perm, const double *R64, unsigned long long *rowmax,
                       uint8_t *wq, float *w_scale, int bits, hipStream_t s)
{
    const int qmax = bits == 8 ? 127 : 7;
    hipLaunchKernelGGL(k_fill_u64, dim3((N + 255) / 256), dim3(256), 0, s, rowmax, (int64_t)N);
    dim3 grid((N + WP_ROWS - 1) / WP_ROWS, (K + WP_CHUNK - 1) / WP_CHUNK);
    hipLaunchKernelGGL(k_weight_pack<0>, grid, dim3(WP_CHUNK / 2), 0, s, W, wdt, N, K, ldw, B,
                       perm, R64, rowmax, wq, w_scale, qmax);
    hipLaunchKernelGGL(k_weight_pack<1>, grid, dim3(WP_CHUNK / 2), 0, s, W, wdt, N, K, ldw, B,
                       perm, R64, rowmax, wq, w_scale, qmax);
    return check_launch("weight pack");
}

// The GPTQ solver's weight side: per-row max |W'| (for the fixed RTN scales) and the fp64 rows W'.
int launch_weight_rowmax_rot(const void *W, int wdt, int N, int K, int64_t ldw, int B,
                             const int32_t *perm, const double *R64, unsigned long long *rowmax,
                             double *wrot, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_u64, dim3((N + 255) / 256), dim3(256), 0, s, rowmax, (int64_t)N);
    dim3 grid((N + WP_ROWS - 1) / WP_ROWS, (K + WP_CHUNK - 1) / WP_CHUNK);
    hipLaunchKernelGGL(k_weight_pack<0>, grid, dim3(WP_CHUNK / 2), 0, s, W, wdt, N, K, ldw, B,
                       perm, R64, rowmax, nullptr, nullptr, 7, nullptr);
    hipLaunchKernelGGL(k_weight_pack<2>, grid, dim3(WP_CHUNK / 2), 0, s, W, wdt, N, K, ldw, B,
                       perm, R64, nullptr, nullptr, nullptr, 7, wrot);
    return check_launch("weight row max + rotation");
}

int launch_rotate_rows_f64(const void *A, int adt, int rows, int K, int64_t lda, int B,
                           const int32_t *perm, const double *R64, double *out, hipStream_t s)
{
    if (rows == 0) return W4A4_OK;
    dim3 grid((rows + WP_ROWS - 1) / WP_ROWS, (K + WP_CHUNK - 1) / WP_CHUNK);
    hipLaunchKernelGGL(k_weight_pack<2>, grid, dim3(WP_CHUNK / 2), 0, s, A, adt, rows, K, lda, B,
                       perm, R64, nullptr, nullptr, nullptr, 7, out);
    return check_launch("rotate rows (fp64)");
}

}  // namespace w4a4
