// Runtime activation path: zigzag gather + block rotation + activation scale + int4 quantize + pack.
//
// x'[m][b*B + j] = sum_i X[m][perm[b*B + i]] * R_b[i][j] (R_b = U_b . H_B, gist.science summary,
// "Metodologia" item 1), then symmetric int4 codes with either the current denoising step's table
// scale (vnrobo.com "Y tuong paper": the runtime only looks up the step's scale) or a dynamic
// per-token scale (FoldQuantVLA summary, key change 2). The decision q = rint(x' * fp32(1/s)) is
// taken in fp32.
#include "w4a4_internal.h"

namespace w4a4 {

__global__ void k_fill_u32(uint32_t *p, uint32_t v, int64_t n)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

int launch_fill_u32(uint32_t *p, uint32_t value, int64_t count, hipStream_t s)
{
    if (count <= 0) return W4A4_OK;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, p, value,
                       count);
    return check_launch("fill");
}

__device__ __forceinline__ float step_scale(const float *table, int step)
{
    float s = table[step];
    return (s > 0.0f && s <= 3.402823466e38f) ? s : 1.0f;
}

// fp32(max / 7) divided in fp64 (exactly the fp32 quotient, the double rounding being innocuous
// for an fp32 dividend); 1.0f for a zero max.
__device__ __forceinline__ float scale_from_absmax(float amax)
{
    return amax > 0.0f ? (float)((double)amax / 7.0) : 1.0f;
}

__device__ __forceinline__ int quant_code(float x, float r)
{
    float y = x * r;
    float t = rintf(y);
    t = fminf(fmaxf(t, -8.0f), 7.0f);
    return (int)t;
}

// Workgroup = RQ_ROWS rows x one chunk of up to 256 positions (whole blocks); 128 threads, each
// owning two adjacent positions (one output byte).
constexpr int RQ_ROWS = 8;
constexpr int RQ_CHUNK = 256;

template <int MODE>
__global__ __launch_bounds__(128) void k_rotate_quant_valu(
    const void *__restrict__ X, int xdt, int M, int K, int64_t ldx, int B,
    const int32_t *__restrict__ perm, const float *__restrict__ R32, const float *__restrict__ table,
    int step, uint32_t *__restrict__ rowmax, uint8_t *__restrict__ xq, float *__restrict__ x_scale,
    float *__restrict__ xrot_dbg)
{
    __shared__ float sX[RQ_ROWS][RQ_CHUNK];
    __shared__ float sMax[RQ_ROWS][2];
    const int m0 = blockIdx.x * RQ_ROWS;
    const int k0 = blockIdx.y * RQ_CHUNK;
    const int kend = min(k0 + RQ_CHUNK, K);
    const int tid = threadIdx.x;

    for (int e = tid; e < RQ_ROWS * RQ_CHUNK; e += blockDim.x) {
        int r = e / RQ_CHUNK, c = e % RQ_CHUNK;
        int m = m0 + r, k = k0 + c;
        float v = 0.0f;
        if (m < M && k < kend) v = load_as_f32(X, xdt, (int64_t)m * ldx + (perm ? perm[k] : k));
        sX[r][c] = v;
    }
    __syncthreads();

    const int kp = k0 + 2 * tid;
    const bool active = kp < kend;
    float acc[RQ_ROWS][2];
#pragma unroll
    for (int r = 0; r < RQ_ROWS; ++r) acc[r][0] = acc[r][1] = 0.0f;
    if (active) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kp + h;
            const int b = k / B, j = k % B;
            const int cb = b * B - k0;
            const float *Rb = R32 + (int64_t)b * B * B + j;
            for (int i = 0; i < B; ++i) {
                const float rij = Rb[(int64_t)i * B];
#pragma unroll
                for (int r = 0; r < RQ_ROWS; ++r) acc[r][h] = fmaf(sX[r][cb + i], rij, acc[r][h]);
            }
        }
    }

    if (xrot_dbg && active && MODE != ACT_TOKEN_MAX && MODE != ACT_CALIB_MAX) {
#pragma unroll
        for (int r = 0; r < RQ_ROWS; ++r) {
            int m = m0 + r;
            if (m < M) {
                xrot_dbg[(int64_t)m * K + kp] = acc[r][0];
                xrot_dbg[(int64_t)m * K + kp + 1] = acc[r][1];
            }
        }
    }

    if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
        const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int r = 0; r < RQ_ROWS; ++r) {
            float m = active ? fmaxf(fabsf(acc[r][0]), fabsf(acc[r][1])) : 0.0f;
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            if (lane == 0) sMax[r][wave] = m;
        }
        __syncthreads();
        if (MODE == ACT_TOKEN_MAX) {
            if (tid < RQ_ROWS && m0 + tid < M)
                atomicMax(&rowmax[m0 + tid], __float_as_uint(fmaxf(sMax[tid][0], sMax[tid][1])));
        } else if (tid == 0) {
            float m = 0.0f;
            for (int r = 0; r < RQ_ROWS; ++r)
                if (m0 + r < M) m = fmaxf(m, fmaxf(sMax[r][0], sMax[r][1]));
            atomicMax(&rowmax[0], __float_as_uint(m));
        }
        return;
    }

#pragma unroll
    for (int r = 0; r < RQ_ROWS; ++r) {
        const int m = m0 + r;
        if (m >= M) continue;
        float s;
        if (MODE == ACT_PER_STEP) s = step_scale(table, step);
        else s = scale_from_absmax(__uint_as_float(rowmax[m]));
        if (blockIdx.y == 0 && tid == 0) {
            if (MODE == ACT_PER_STEP) {
                if (blockIdx.x == 0 && r == 0) x_scale[0] = s;
            } else {
                x_scale[m] = s;
            }
        }
        if (!active) continue;
        const float rcp = (float)(1.0 / (double)s);
        const int q0 = quant_code(acc[r][0], rcp);
        const int q1 = quant_code(acc[r][1], rcp);
        xq[(int64_t)m * (K / 2) + kp / 2] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    }
}

int launch_rotate_quant(const void *X, int xdt, int M, int K, int64_t ldx, int B,
                        const int32_t *perm, const void *rot, const float *table, int step,
                        ActMode mode, uint32_t *rowmax, uint8_t *xq, float *x_scale,
                        float *xrot_dbg, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    const float *R32 = reinterpret_cast<const float *>(rot);
    dim3 grid((M + RQ_ROWS - 1) / RQ_ROWS, (K + RQ_CHUNK - 1) / RQ_CHUNK);
    dim3 block(RQ_CHUNK / 2);
    switch (mode) {
    case ACT_PER_STEP:
        hipLaunchKernelGGL(k_rotate_quant_valu<ACT_PER_STEP>, grid, block, 0, s, X, xdt, M, K, ldx,
                           B, perm, R32, table, step, rowmax, xq, x_scale, xrot_dbg);
        break;
    case ACT_TOKEN_MAX:
        hipLaunchKernelGGL(k_rotate_quant_valu<ACT_TOKEN_MAX>, grid, block, 0, s, X, xdt, M, K, ldx,
                           B, perm, R32, table, step, rowmax, xq, x_scale, xrot_dbg);
        break;
    case ACT_TOKEN_QUANT:
        hipLaunchKernelGGL(k_rotate_quant_valu<ACT_TOKEN_QUANT>, grid, block, 0, s, X, xdt, M, K,
                           ldx, B, perm, R32, table, step, rowmax, xq, x_scale, xrot_dbg);
        break;
    case ACT_CALIB_MAX:
        hipLaunchKernelGGL(k_rotate_quant_valu<ACT_CALIB_MAX>, grid, block, 0, s, X, xdt, M, K, ldx,
                           B, perm, R32, table, step, rowmax, xq, x_scale, xrot_dbg);
        break;
    }
    return check_launch("rotate-quantize");
}

__global__ void k_scale_from_absmax(const uint32_t *amax, float *out)
{
    out[0] = scale_from_absmax(__uint_as_float(amax[0]));
}

int launch_scale_from_absmax(const uint32_t *amax, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_scale_from_absmax, dim3(1), dim3(1), 0, s, amax, out);
    return check_launch("scale from absmax");
}

}  // namespace w4a4
