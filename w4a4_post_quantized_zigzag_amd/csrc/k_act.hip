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

// ------------------------------------------------------------------ fp16 path on MFMA
//
// x'_b = x_b R_b for fp16 activations, evaluated as x'^T = R_b^T x^T with
// v_mfma_f32_16x16x32_f16: the A operand is R_b^T (16 output channels j x 32 inputs i), the B
// operand is the activation tile (32 inputs i x 16 tokens m), so each lane ends with 4 consecutive
// output channels of one token, which it quantizes and packs into two bytes. R_b is used as two
// fp16 parts, R ~= hi + lo * 2^-12: fp16 x fp16 products are exact in fp32, so the result carries
// fp32 accumulation error plus ~2^-22 relative from the split. Each wave keeps the R_b^T fragments
// of its B/4 output channels in registers and reuses them over all row tiles of the workgroup.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int MT = 64;  // token rows per tile

template <int MODE, int B, bool GATHER>
__global__ __launch_bounds__(256) void k_rq_mfma(
    const uint16_t *__restrict__ X, int64_t ldx, int M, int K, const int32_t *__restrict__ perm,
    const _Float16 *__restrict__ rhi, const _Float16 *__restrict__ rlo,
    const float *__restrict__ table, int step, uint32_t *__restrict__ rowmax,
    uint8_t *__restrict__ xq, float *__restrict__ x_scale, float *__restrict__ xrot_dbg,
    int rows_per_wg)
{
#pragma clang fp contract(off)
    constexpr int KK = B / 32;       // 32-wide k steps
    constexpr int JW = B / 4;        // output channels per wave
    constexpr int JF = JW / 16;      // 16-channel fragments per wave
    constexpr int LDSR = B + 8;      // halves per staged row (16-byte pad)
    __shared__ __attribute__((aligned(16))) uint16_t sx[MT * LDSR];
    __shared__ float smax[4][MT];

    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int jbase = wave * JW;

    v8h ahi[JF][KK], alo[JF][KK];
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int64_t off = ((int64_t)b * B + jbase + 16 * jf + r) * B + 32 * kk + 8 * g;
            ahi[jf][kk] = *reinterpret_cast<const v8h *>(rhi + off);
            alo[jf][kk] = *reinterpret_cast<const v8h *>(rlo + off);
        }

    float s_step = 1.0f, rcp_step = 1.0f;
    if (MODE == ACT_PER_STEP) {
        s_step = step_scale(table, step);
        rcp_step = (float)(1.0 / (double)s_step);
        if (blockIdx.x == 0 && b == 0 && tid == 0) x_scale[0] = s_step;
    }

    const int row_begin = blockIdx.x * rows_per_wg;
    const int row_end = min(M, row_begin + rows_per_wg);

    // Tile staging, prefetched one tile ahead into registers. Loads are unconditional from clamped
    // in-bounds rows (the clamped rows are zeroed when stored), so they stay in flight during the
    // previous tile's MFMA work.
    //  gather:     thread -> one source column (fixed for the kernel), rows tid/B + t*(256/B)
    //  contiguous: thread -> 16-byte chunks e = tid + t*256 of the tile (row e/(B/8), chunk e%(B/8))
    constexpr int RSTEP = 256 / B, NLD = MT / RSTEP;
    constexpr int C8 = B / 8, NCH = MT * C8 / 256;
    const int gi = tid % B, grr0 = tid / B;
    const int64_t gcol = GATHER ? (perm ? perm[b * B + gi] : b * B + gi) : 0;
    uint16_t pv[GATHER ? NLD : 1];
    uint4 pc[GATHER ? 1 : NCH];
    auto tile_load = [&](int m0) {
        if (GATHER) {
#pragma unroll
            for (int t = 0; t < NLD; ++t) {
                const int m = min(m0 + grr0 + t * RSTEP, row_end - 1);
                pv[t] = X[(int64_t)m * ldx + gcol];
            }
        } else {
#pragma unroll
            for (int t = 0; t < NCH; ++t) {
                const int e = tid + t * 256;
                const int m = min(m0 + e / C8, row_end - 1);
                pc[t] = *reinterpret_cast<const uint4 *>(X + (int64_t)m * ldx + b * B + 8 * (e % C8));
            }
        }
    };
    auto tile_store = [&](int m0) {
        if (GATHER) {
#pragma unroll
            for (int t = 0; t < NLD; ++t) {
                const int rr = grr0 + t * RSTEP;
                sx[rr * LDSR + gi] = (m0 + rr < row_end) ? pv[t] : (uint16_t)0;
            }
        } else {
#pragma unroll
            for (int t = 0; t < NCH; ++t) {
                const int e = tid + t * 256, rr = e / C8;
                const bool live = m0 + rr < row_end;
                const uint4 v = make_uint4(live ? pc[t].x : 0u, live ? pc[t].y : 0u,
                                           live ? pc[t].z : 0u, live ? pc[t].w : 0u);
                *reinterpret_cast<uint4 *>(&sx[rr * LDSR + 8 * (e % C8)]) = v;
            }
        }
    };

    if (row_begin < row_end) tile_load(row_begin);
    for (int m0 = row_begin; m0 < row_end; m0 += MT) {
        __syncthreads();
        tile_store(m0);
        __syncthreads();
        if (m0 + MT < row_end) tile_load(m0 + MT);
#pragma unroll 1
        for (int mf = 0; mf < MT / 16; ++mf) {
            v4f chi[JF], clo[JF];
#pragma unroll
            for (int jf = 0; jf < JF; ++jf) chi[jf] = clo[jf] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const v8h xb = *reinterpret_cast<const v8h *>(&sx[(mf * 16 + r) * LDSR + 32 * kk + 8 * g]);
#pragma unroll
                for (int jf = 0; jf < JF; ++jf) {
                    chi[jf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jf][kk], xb, chi[jf], 0, 0, 0);
                    clo[jf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[jf][kk], xb, clo[jf], 0, 0, 0);
                }
            }
            const int m = m0 + mf * 16 + r;
            const bool live = m < row_end;
            float v[JF][4];
#pragma unroll
            for (int jf = 0; jf < JF; ++jf)
#pragma unroll
                for (int i = 0; i < 4; ++i) v[jf][i] = chi[jf][i] + clo[jf][i] * (1.0f / (1 << ROT_LO_SHIFT));

            if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
                float a = 0.0f;
#pragma unroll
                for (int jf = 0; jf < JF; ++jf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) a = fmaxf(a, fabsf(v[jf][i]));
                a = fmaxf(a, __shfl_xor(a, 16));
                a = fmaxf(a, __shfl_xor(a, 32));
                if (g == 0) smax[wave][mf * 16 + r] = live ? a : 0.0f;
                continue;
            }
            if (!live) continue;
            const int jcol = b * B + jbase + 4 * g;
            if (xrot_dbg) {
#pragma unroll
                for (int jf = 0; jf < JF; ++jf)
                    *reinterpret_cast<float4 *>(&xrot_dbg[(int64_t)m * K + jcol + 16 * jf]) =
                        make_float4(v[jf][0], v[jf][1], v[jf][2], v[jf][3]);
            }
            float rcp = rcp_step;
            if (MODE == ACT_TOKEN_QUANT) {
                const float s = scale_from_absmax(__uint_as_float(rowmax[m]));
                rcp = (float)(1.0 / (double)s);
                if (b == 0 && wave == 0 && g == 0) x_scale[m] = s;
            }
#pragma unroll
            for (int jf = 0; jf < JF; ++jf) {
                const int q0 = quant_code(v[jf][0], rcp), q1 = quant_code(v[jf][1], rcp);
                const int q2 = quant_code(v[jf][2], rcp), q3 = quant_code(v[jf][3], rcp);
                const uint16_t packed = (uint16_t)((q0 & 0xF) | ((q1 & 0xF) << 4) |
                                                   ((q2 & 0xF) << 8) | ((q3 & 0xF) << 12));
                *reinterpret_cast<uint16_t *>(&xq[(int64_t)m * (K / 2) + (jcol + 16 * jf) / 2]) = packed;
            }
        }
        if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
            __syncthreads();
            if (tid < MT) {
                const int m = m0 + tid;
                const float a = fmaxf(fmaxf(smax[0][tid], smax[1][tid]), fmaxf(smax[2][tid], smax[3][tid]));
                if (MODE == ACT_TOKEN_MAX) {
                    if (m < row_end) atomicMax(&rowmax[m], __float_as_uint(a));
                } else {
                    // one atomic per tile: reduce the tile's rows within wave 0
                    float t = a;
                    for (int off = 32; off > 0; off >>= 1) t = fmaxf(t, __shfl_xor(t, off));
                    if (tid == 0) atomicMax(&rowmax[0], __float_as_uint(t));
                }
            }
        }
    }
}

// Zigzag gather of whole rows: Xp[m][j] = X[m][perm[j]] (fp16), one workgroup per row, the source
// row staged in LDS with 16-byte loads and the permuted row written with 16-byte stores.
template <bool VEC>
__global__ __launch_bounds__(256) void k_permute_rows(const uint16_t *__restrict__ X, int64_t ldx,
                                                      int K, const int32_t *__restrict__ perm,
                                                      uint16_t *__restrict__ Xp)
{
    extern __shared__ uint16_t srow[];
    const int m = blockIdx.x, tid = threadIdx.x;
    const uint16_t *xr = X + (int64_t)m * ldx;
    uint16_t *out = Xp + (int64_t)m * K;
    if (VEC) {
        for (int c = tid * 8; c < K; c += 256 * 8)
            *reinterpret_cast<uint4 *>(&srow[c]) = *reinterpret_cast<const uint4 *>(&xr[c]);
    } else {
        for (int c = tid; c < K; c += 256) srow[c] = xr[c];
    }
    __syncthreads();
    if (VEC) {
        for (int c = tid * 8; c < K; c += 256 * 8) {
            const int4 p0 = *reinterpret_cast<const int4 *>(&perm[c]);
            const int4 p1 = *reinterpret_cast<const int4 *>(&perm[c + 4]);
            uint4 v;
            v.x = (uint32_t)srow[p0.x] | ((uint32_t)srow[p0.y] << 16);
            v.y = (uint32_t)srow[p0.z] | ((uint32_t)srow[p0.w] << 16);
            v.z = (uint32_t)srow[p1.x] | ((uint32_t)srow[p1.y] << 16);
            v.w = (uint32_t)srow[p1.z] | ((uint32_t)srow[p1.w] << 16);
            *reinterpret_cast<uint4 *>(&out[c]) = v;
        }
    } else {
        for (int c = tid; c < K; c += 256) out[c] = srow[perm[c]];
    }
}

bool act_uses_permute_pass(int M, int K, int per_token)
{
    (void)M;
    // long rows make the in-kernel 2-byte gather touch a new cache line per element; a separate
    // coalesced permutation pass (its output stays in the 256 MB last-level cache) is then cheaper,
    // and per-token mode reads the permuted rows twice. The pass stages a whole row in LDS.
    if (K > 65536) return false;
    return K > 4096 || (per_token && K > 2048);
}

size_t act_permute_bytes(int M, int K) { return align_up((size_t)M * K * sizeof(uint16_t), 256); }

static int rq_rows_per_wg(int M, int nb)
{
    const int mt = (M + MT - 1) / MT;
    int rg = (512 + nb - 1) / nb;
    rg = max(1, min(rg, mt));
    return ((mt + rg - 1) / rg) * MT;
}

int launch_rotate_quant_mfma(const void *X, int M, int K, int64_t ldx, int B, const int32_t *perm,
                             const void *rot, const float *table, int step, ActMode mode,
                             uint32_t *rowmax, uint8_t *xq, float *x_scale, float *xrot_dbg,
                             const uint16_t *xperm, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    RotLayout L = rot_layout(K, B);
    const char *base = reinterpret_cast<const char *>(rot);
    const _Float16 *rhi = reinterpret_cast<const _Float16 *>(base + L.r32);
    const _Float16 *rlo = reinterpret_cast<const _Float16 *>(base + L.r32 + L.r16);
    const int nb = K / B;
    const int rpw = rq_rows_per_wg(M, nb);
    dim3 grid((M + rpw - 1) / rpw, nb);
    const uint16_t *src = xperm ? xperm : reinterpret_cast<const uint16_t *>(X);
    const int64_t ld = xperm ? K : ldx;
    // contiguous 16-byte tile loads need 16-byte aligned rows; otherwise gather element-wise
    const bool rows_aligned = ((uintptr_t)src % 16 == 0) && (ld % 8 == 0);
    const bool gather = ((perm != nullptr) && (xperm == nullptr)) || !rows_aligned;
    if (xperm) perm = nullptr;
#define W4A4_RQ(MODEV, BV, GV)                                                                     \
    hipLaunchKernelGGL((k_rq_mfma<MODEV, BV, GV>), grid, dim3(256), 0, s, src, ld, M, K, perm, rhi, \
                       rlo, table, step, rowmax, xq, x_scale, xrot_dbg, rpw)
#define W4A4_RQ_B(MODEV)                                                                           \
    if (B == 128) { if (gather) W4A4_RQ(MODEV, 128, true); else W4A4_RQ(MODEV, 128, false); }      \
    else { if (gather) W4A4_RQ(MODEV, 64, true); else W4A4_RQ(MODEV, 64, false); }
    switch (mode) {
    case ACT_PER_STEP: W4A4_RQ_B(ACT_PER_STEP) break;
    case ACT_TOKEN_MAX: W4A4_RQ_B(ACT_TOKEN_MAX) break;
    case ACT_TOKEN_QUANT: W4A4_RQ_B(ACT_TOKEN_QUANT) break;
    case ACT_CALIB_MAX: W4A4_RQ_B(ACT_CALIB_MAX) break;
    }
#undef W4A4_RQ_B
#undef W4A4_RQ
    return check_launch("rotate-quantize (mfma)");
}

int launch_permute_rows(const void *X, int M, int K, int64_t ldx, const int32_t *perm, uint16_t *xp,
                        hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    const size_t lds = (size_t)K * sizeof(uint16_t);
    const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0) &&
                     ((uintptr_t)perm % 16 == 0);
    const void *fn = vec ? (const void *)k_permute_rows<true> : (const void *)k_permute_rows<false>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(W4A4_ERR_HIP, "permute LDS request: %s", hipGetErrorString(e));
    }
    const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
    if (vec) hipLaunchKernelGGL(k_permute_rows<true>, dim3(M), dim3(256), lds, s, x, ldx, K, perm, xp);
    else hipLaunchKernelGGL(k_permute_rows<false>, dim3(M), dim3(256), lds, s, x, ldx, K, perm, xp);
    return check_launch("permute rows");
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
