// Runtime activation path: zigzag gather + block rotation + activation scale + int4 quantize + pack.
//
// x'[m][b*B + j] = sum_i X[m][perm[b*B + i]] * R_b[i][j] (R_b = U_b . H_B, gist.science summary,
// "Metodologia" item 1), then symmetric int4 codes with either the current denoising step's table
// scale (vnrobo.com "Y tuong paper": the runtime only looks up the step's scale) or a dynamic
// per-token scale (FoldQuantVLA summary, key change 2). The decision q = rint(x' * fp32(1/s)) is
// taken in fp32.
#include <cmath>

#include "rq_core.h"

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

// fp32(max / qmax) divided in fp64 (exactly the fp32 quotient, the double rounding being innocuous
// for an fp32 dividend); 1.0f for a zero max. qmax = 7 for int4 codes, 127 for the int8 codes of
// the W8A8 linears (Q8).
template <bool Q8>
__device__ __forceinline__ float scale_from_absmax_q(float amax)
{
    return amax > 0.0f ? (float)((double)amax / (Q8 ? 127.0 : 7.0)) : 1.0f;
}
__device__ __forceinline__ float scale_from_absmax(float amax) { return scale_from_absmax_q<false>(amax); }

template <bool Q8>
__device__ __forceinline__ int quant_code_q(float x, float r)
{
    float y = x * r;
    float t = rintf(y);
    t = fminf(fmaxf(t, Q8 ? -128.0f : -8.0f), Q8 ? 127.0f : 7.0f);
    return (int)t;
}
__device__ __forceinline__ int quant_code(float x, float r) { return quant_code_q<false>(x, r); }

// Workgroup = RQ_ROWS rows x one chunk of up to 256 positions (whole blocks); 128 threads, each
// owning two adjacent positions (one output byte).
constexpr int RQ_ROWS = 8;
constexpr int RQ_CHUNK = 256;

template <int MODE, bool Q8>
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
        float s, rcp;
        if (MODE == ACT_PER_STEP) {
            const StepScale ss = step_scale(table, step);
            s = ss.s;
            rcp = ss.rcp;
        } else {
            s = scale_from_absmax_q<Q8>(__uint_as_float(rowmax[m]));
            rcp = (float)(1.0 / (double)s);
        }
        if (blockIdx.y == 0 && tid == 0) {
            if (MODE == ACT_PER_STEP) {
                if (blockIdx.x == 0 && r == 0) x_scale[0] = s;
            } else {
                x_scale[m] = s;
            }
        }
        if (!active) continue;
        const int q0 = quant_code_q<Q8>(acc[r][0], rcp);
        const int q1 = quant_code_q<Q8>(acc[r][1], rcp);
        if (Q8)
            *reinterpret_cast<uint16_t *>(&xq[(int64_t)m * K + kp]) =
                (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
        else
            xq[(int64_t)m * (K / 2) + kp / 2] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    }
}

int launch_rotate_quant(const void *X, int xdt, int M, int K, int64_t ldx, int B,
                        const int32_t *perm, const void *rot, const float *table, int step,
                        ActMode mode, uint32_t *rowmax, uint8_t *xq, float *x_scale,
                        float *xrot_dbg, bool q8, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    const float *R32 = reinterpret_cast<const float *>(rot);
    dim3 grid((M + RQ_ROWS - 1) / RQ_ROWS, (K + RQ_CHUNK - 1) / RQ_CHUNK);
    dim3 block(RQ_CHUNK / 2);
#define W4A4_VALU(MODEV, QV)                                                                       \
    hipLaunchKernelGGL((k_rotate_quant_valu<MODEV, QV>), grid, block, 0, s, X, xdt, M, K, ldx, B,  \
                       perm, R32, table, step, rowmax, xq, x_scale, xrot_dbg)
    switch (mode) {
    case ACT_PER_STEP:
        if (q8) W4A4_VALU(ACT_PER_STEP, true); else W4A4_VALU(ACT_PER_STEP, false);
        break;
    case ACT_TOKEN_MAX: W4A4_VALU(ACT_TOKEN_MAX, false); break;
    case ACT_TOKEN_QUANT:
        if (q8) W4A4_VALU(ACT_TOKEN_QUANT, true); else W4A4_VALU(ACT_TOKEN_QUANT, false);
        break;
    case ACT_CALIB_MAX: W4A4_VALU(ACT_CALIB_MAX, false); break;
    }
#undef W4A4_VALU
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
constexpr int MT = 64;  // token rows per tile

template <int MODE, int B, bool GATHER, bool Q8, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_rq_mfma(
    const uint16_t *__restrict__ X, int64_t ldx, int M, int K, const int32_t *__restrict__ perm,
    const _Float16 *__restrict__ rhi, const _Float16 *__restrict__ rlo,
    const float *__restrict__ table, int step, uint32_t *__restrict__ rowmax,
    uint8_t *__restrict__ xq, float *__restrict__ x_scale, float *__restrict__ xrot_dbg,
    int rows_per_wg, int gstride)
{
#pragma clang fp contract(off)
    constexpr int KK = B / 32;       // 32-wide k steps
    constexpr int NT = 64 * NW;      // threads
    constexpr int JW = B / NW;       // output channels per wave
    constexpr int JF = JW / 16;      // 16-channel fragments per wave
    constexpr int MF = MT / 16;      // 16-token fragments per tile
    constexpr int LDSR = B + 8;      // halves per staged row (16-byte pad)
    constexpr int OB = Q8 ? B : B / 2;  // output code bytes per row of one block
    constexpr int OCH = MT * OB / 16;   // 16-byte output chunks per tile
    constexpr float LO = 1.0f / (1 << ROT_LO_SHIFT);
    const int64_t ldq = Q8 ? K : K / 2;
    __shared__ __attribute__((aligned(16))) uint16_t sx[MT * LDSR];
    __shared__ float smax[NW][MT];
    __shared__ __attribute__((aligned(16))) uint8_t sq[MT * OB];

    // Workgroup -> (row group, block). Workgroups are dealt round-robin to the 8 XCDs, each with
    // its own L2; consecutive workgroups of one XCD take the blocks of one row group, so a row
    // (whose zigzag gather spreads every block's channels over the whole row) is fetched into one
    // XCD's L2 only, not into all eight.
    const int nb = K / B, T = gridDim.x;
    const int per_x = T / 8, rm = T % 8, xcd = blockIdx.x % 8;
    const int lin = xcd * per_x + min(xcd, rm) + blockIdx.x / 8;
    const int b = lin % nb, rg = lin / nb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int jbase = wave * JW;

    // R_b^T fragments of this wave's output channels (high part pre-scaled by 2^12)
    v8h ahi[JF][KK], alo[JF][KK];
    load_rot_frags<JF, KK>(rhi, rlo, b, jbase, lane, B, ahi, alo);

    float rs_step = 0.0f;
    if (MODE == ACT_PER_STEP) {
        const StepScale ss = step_scale(table, step + b * gstride);
        rs_step = ss.rcp * LO;
        if (rg == 0 && (gstride || b == 0) && tid == 0) x_scale[b * gstride] = ss.s;
    }

    const int row_begin = rg * rows_per_wg;
    const int row_end = min(M, row_begin + rows_per_wg);

    // Tile staging, prefetched one tile ahead into registers. Loads are unconditional from clamped
    // in-bounds rows (the clamped rows are zeroed when stored), so they stay in flight during the
    // previous tile's MFMA work.
    //  gather:     thread -> one source column (fixed for the kernel), rows tid/B + t*(NT/B)
    //  contiguous: thread -> 16-byte chunks e = tid + t*NT of the tile (row e/(B/8), chunk e%(B/8))
    constexpr int RSTEP = NT / B, NLD = MT / RSTEP;
    constexpr int C8 = B / 8, NCH = MT * C8 / NT;
    static_assert(NLD * RSTEP == MT && NCH * NT == MT * C8 && JW % 16 == 0, "whole rounds");
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
                const int e = tid + t * NT;
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
                const int e = tid + t * NT, rr = e / C8;
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

        // acc[mf][jf] = 2^12 x' for tokens m0 + mf*16 + (lane % 16), channels jbase + 16 jf +
        // 4 (lane / 16) + 0..3: the streaming kernel's arithmetic, in the same order
        v4f acc[MF][JF];
        rotate_acc<MF, JF, KK>(ahi, alo, [&](int mf, int kk) {
            return *reinterpret_cast<const v8h *>(&sx[(mf * 16 + r) * LDSR + 8 * (4 * kk + g)]);
        }, acc);

#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            const int row = mf * 16 + r;
            const int m = m0 + row;
            const bool live = m < row_end;
            if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
                float a = 0.0f;
#pragma unroll
                for (int jf = 0; jf < JF; ++jf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) a = fmaxf(a, fabsf(acc[mf][jf][i]));
                a = fmaxf(a, __shfl_xor(a, 16));
                a = fmaxf(a, __shfl_xor(a, 32));
                if (g == 0) smax[wave][row] = live ? a * LO : 0.0f;
                continue;
            }
            const int jl = jbase + 4 * g;  // first of this lane's 4 channels within the block
            if (xrot_dbg && live) {
#pragma unroll
                for (int jf = 0; jf < JF; ++jf)
                    *reinterpret_cast<float4 *>(&xrot_dbg[(int64_t)m * K + b * B + jl + 16 * jf]) =
                        make_float4(acc[mf][jf][0] * LO, acc[mf][jf][1] * LO, acc[mf][jf][2] * LO,
                                    acc[mf][jf][3] * LO);
            }
            float rs = rs_step;
            if (MODE == ACT_TOKEN_QUANT) {
                const int mc = min(m, row_end - 1);
                const float sc = scale_from_absmax_q<Q8>(__uint_as_float(rowmax[mc]));
                rs = (float)(1.0 / (double)sc) * LO;
                if (b == 0 && wave == 0 && g == 0 && live) x_scale[m] = sc;
            }
#pragma unroll
            for (int jf = 0; jf < JF; ++jf) {
                if (Q8)
                    *reinterpret_cast<uint32_t *>(&sq[row * OB + jl + 16 * jf]) =
                        quant_pack4<true>(acc[mf][jf], rs);
                else
                    *reinterpret_cast<uint16_t *>(&sq[row * OB + (jl + 16 * jf) / 2]) =
                        (uint16_t)quant_pack4(acc[mf][jf], rs);
            }
        }
        __syncthreads();
        if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
            if (tid < MT) {
                const int m = m0 + tid;
                float a = smax[0][tid];
#pragma unroll
                for (int w = 1; w < NW; ++w) a = fmaxf(a, smax[w][tid]);
                if (MODE == ACT_TOKEN_MAX) {
                    if (m < row_end) atomicMax(&rowmax[m], __float_as_uint(a));
                } else {
                    // one atomic per tile: reduce the tile's rows within wave 0
                    float t = a;
                    for (int off = 32; off > 0; off >>= 1) t = fmaxf(t, __shfl_xor(t, off));
                    if (tid == 0) atomicMax(&rowmax[b * gstride], __float_as_uint(t));
                }
            }
        } else if (((uintptr_t)xq & 15) == 0) {
            // the tile's codes: 16-byte stores (OB / 16 chunks per row)
            for (int e = tid; e < OCH; e += NT) {
                const int row = e / (OB / 16), ch = e % (OB / 16);
                if (m0 + row < row_end)
                    *reinterpret_cast<uint4 *>(&xq[(int64_t)(m0 + row) * ldq + b * OB + 16 * ch]) =
                        *reinterpret_cast<const uint4 *>(&sq[row * OB + 16 * ch]);
            }
        } else {
            // xq without 16-byte alignment (allowed for int4 codes): byte stores
            for (int e = tid; e < MT * OB; e += NT) {
                const int row = e / OB, c = e % OB;
                if (m0 + row < row_end) xq[(int64_t)(m0 + row) * ldq + b * OB + c] = sq[row * OB + c];
            }
        }
    }
}

// ------------------------------------------------------------------ contiguous rows, LDS DMA ring
//
// Same arithmetic as k_rq_mfma for rows already in zigzag order (a permuted copy, or the caller's
// own layout), with the activation tiles streamed by global_load_lds_dwordx4 into a ring of
// RQ_STAGES LDS tiles so the next tile's loads are in flight while one is multiplied (two tiles:
// measured faster than three or four on the long-K per-token pass, 42.8 -> 41.1 us). The ring is
// synchronized with explicit vmcnt waits and plain s_barrier (a fenced barrier would drain every
// in-flight tile). Staged rows are XOR-swizzled by 16-byte chunk (chunk ^ (row % chunks_per_row)),
// which makes the 16 rows a fragment read touches hit 16 different bank groups.
constexpr int RQ_STAGES = 2;
constexpr int RQ_RING_MAX_ROWS = 1024;  // rows per workgroup (per-token scales staged in LDS)
constexpr int RQ_SMALL_M = 256;         // batches up to this many tokens use k_rq_small
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

__device__ __forceinline__ void rq_dma16(const void *gptr, uint32_t lds_addr)
{
    // one wave-wide 16-byte-per-lane DMA into LDS at lds_addr + 16 * lane (no VGPR written);
    // M0 holds the LDS base and needs one wait state before the LDS DMA reads it
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}

__device__ __forceinline__ void rq_wait_vmcnt(int n)
{
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// F6: the codes go out in the FP6 operand layout of the FP6 GEMM instead of packed int4 (B = 128,
// so a rotation block is one 128-k stage of that layout: xq is the operand, stage b its block b).
template <int MODE, int B, bool DBG, bool Q8, bool F6 = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_rq_ring(
    const uint16_t *__restrict__ X, int64_t ldx, int M, int K, const _Float16 *__restrict__ rhi,
    const _Float16 *__restrict__ rlo, const float *__restrict__ table, int step,
    uint32_t *__restrict__ rowmax, uint8_t *__restrict__ xq, float *__restrict__ x_scale,
    float *__restrict__ xrot_dbg, int rows_per_wg, int row_groups, int gstride)
{
#pragma clang fp contract(off)
    constexpr int NT = 64 * NW;  // threads
    constexpr int KK = B / 32, JW = B / NW, JF = JW / 16, MF = MT / 16;
    constexpr float LO = 1.0f / (1 << ROT_LO_SHIFT);
    constexpr int NXCD = 8;
    constexpr int ROWB = B * 2;                   // bytes per staged row
    constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
    constexpr int TILE = MT * ROWB;               // bytes per tile
    constexpr int QPW = TILE / 1024 / NW;         // DMA instructions per wave per tile
    static_assert(QPW * 1024 * NW == TILE && JF * 16 * NW == B, "whole DMA instructions and fragments per wave");
    constexpr int RPI = 1024 / ROWB;              // rows per DMA instruction
    constexpr int OB = Q8 ? B : B / 2;            // output code bytes per row of one block
    constexpr int OCH = MT * OB / 16;             // 16-byte output chunks per tile
    const int64_t ldq = Q8 ? K : K / 2;           // output row stride in bytes
    extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
    __shared__ float smax[NW][MT];
    __shared__ __attribute__((aligned(16))) uint8_t sq[MT * OB];
    __shared__ float srcp[MODE == ACT_TOKEN_QUANT ? RQ_RING_MAX_ROWS : 1];

    // Workgroup -> (block b, row group). Workgroups are dealt round-robin to the 8 XCDs, each with
    // its own L2; when the block count allows, all row groups of a block go to one XCD, one after
    // another, so that block's R_b fragments come into that L2 once and are hit by the rest.
    const int nb = K / B, wg = blockIdx.x;
    int b, rgi;
    if (nb % NXCD == 0) {
        const int x = wg % NXCD, i = wg / NXCD;
        b = NXCD * (i / row_groups) + x;
        rgi = i % row_groups;
    } else {
        b = wg / row_groups;
        rgi = wg % row_groups;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int jbase = wave * JW;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int row_begin = rgi * rows_per_wg;
    const int row_end = min(M, row_begin + rows_per_wg);
    const int ntiles = (row_end - row_begin + MT - 1) / MT;
    const uint32_t ring0 = (uint32_t)(uintptr_t)(const lds_u8_t *)ring;

    // DMA sources of this lane: instruction q covers tile rows (wave*QPW + q)*RPI + lane/CPR,
    // physical chunk lane % CPR holding logical chunk (lane % CPR) ^ (row % CPR)
    auto issue = [&](int t) {
        const uint32_t base = ring0 + (uint32_t)((t % RQ_STAGES) * TILE);
        const int m0 = row_begin + t * MT;
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            const int row = (uwave * QPW + q) * RPI + lane / CPR;
            const int c = (lane % CPR) ^ (row % CPR);
            const int m = min(m0 + row, row_end - 1);
            rq_dma16(X + (int64_t)m * ldx + b * B + 8 * c, base + (uint32_t)((uwave * QPW + q) * 1024));
        }
    };

    // the first tiles' loads go out before the set-up loads below, so the two latencies overlap
#pragma unroll
    for (int p = 0; p < RQ_STAGES - 1; ++p)
        if (p < ntiles) issue(p);

    // per-token reciprocal scales (times 2^-12) of this workgroup's rows, staged in LDS: a global
    // load inside the tile loop would make the compiler wait for every DMA issued before it
    if (MODE == ACT_TOKEN_QUANT) {
        for (int i = tid; i < row_end - row_begin; i += NT) {
            const float s = scale_from_absmax_q<Q8>(__uint_as_float(rowmax[row_begin + i]));
            srcp[i] = (float)(1.0 / (double)s) * LO;
            if (b == 0) x_scale[row_begin + i] = s;
        }
    }
    // R_b^T fragments of this wave's output channels (high part pre-scaled by 2^12)
    v8h ahi[JF][KK], alo[JF][KK];
    load_rot_frags<JF, KK>(rhi, rlo, b, jbase, lane, B, ahi, alo);
    float rs_step = 0.0f;
    if (MODE == ACT_PER_STEP) {
        const StepScale ss = step_scale(table, step + b * gstride);
        rs_step = ss.rcp * LO;
        if (rgi == 0 && (gstride || b == 0) && tid == 0) x_scale[b * gstride] = ss.s;
    }
    if (MODE == ACT_TOKEN_QUANT) __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int ahead = min(ntiles - 1 - t, RQ_STAGES - 2);
        asm volatile("" ::: "memory");
        rq_wait_vmcnt(ahead * QPW);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + RQ_STAGES - 1 < ntiles) issue(t + RQ_STAGES - 1);
        const uint8_t *tile = ring + (t % RQ_STAGES) * TILE;
        const int m0 = row_begin + t * MT;

        // acc[mf][jf] = 2^12 x' for tokens mf*16 + (lane % 16), channels jbase + 16 jf + 4 (lane / 16)
        // + 0..3; consecutive MFMAs go to different accumulators
        v4f acc[MF][JF];
        rotate_acc<MF, JF, KK>(ahi, alo, [&](int mf, int kk) {
            const int row = mf * 16 + r;
            const int c = (4 * kk + g) ^ (row % CPR);
            return *reinterpret_cast<const v8h *>(&tile[row * ROWB + 16 * c]);
        }, acc);

#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            const int row = mf * 16 + r;
            const int m = m0 + row;
            if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
                float a = 0.0f;
#pragma unroll
                for (int jf = 0; jf < JF; ++jf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) a = fmaxf(a, fabsf(acc[mf][jf][i]));
                a = fmaxf(a, __shfl_xor(a, 16));
                a = fmaxf(a, __shfl_xor(a, 32));
                if (g == 0) smax[wave][row] = (m < row_end) ? a * LO : 0.0f;
                continue;
            }
            const int jl = jbase + 4 * g;  // first of this lane's 4 channels within the block
            if (DBG && m < row_end) {
#pragma unroll
                for (int jf = 0; jf < JF; ++jf)
                    *reinterpret_cast<float4 *>(&xrot_dbg[(int64_t)m * K + b * B + jl + 16 * jf]) =
                        make_float4(acc[mf][jf][0] * LO, acc[mf][jf][1] * LO, acc[mf][jf][2] * LO,
                                    acc[mf][jf][3] * LO);
            }
            const float rs = (MODE == ACT_TOKEN_QUANT) ? srcp[min(m, row_end - 1) - row_begin] : rs_step;
#pragma unroll
            for (int jf = 0; jf < JF; ++jf) {
                if (Q8)
                    *reinterpret_cast<uint32_t *>(&sq[row * OB + jl + 16 * jf]) =
                        quant_pack4<true>(acc[mf][jf], rs);
                else
                    *reinterpret_cast<uint16_t *>(&sq[row * OB + (jl + 16 * jf) / 2]) =
                        (uint16_t)quant_pack4(acc[mf][jf], rs);
            }
        }
        // Tile epilogue after every wave's LDS writes (lgkmcnt(0) + plain barrier; the next write
        // to smax / sq comes after the next tile's barrier, by which time these reads are consumed)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
            if (tid < MT) {
                float a = smax[0][tid];
#pragma unroll
                for (int w = 1; w < NW; ++w) a = fmaxf(a, smax[w][tid]);
                if (MODE == ACT_TOKEN_MAX) {
                    if (m0 + tid < row_end) atomicMax(&rowmax[m0 + tid], __float_as_uint(a));
                } else {
                    float u = a;
                    for (int off = 32; off > 0; off >>= 1) u = fmaxf(u, __shfl_xor(u, off));
                    if (tid == 0) atomicMax(&rowmax[b * gstride], __float_as_uint(u));
                }
            }
        } else if (F6) {
            // thread -> (tile row, 32-k group): 16-byte head at row * 64 + 16 g of the stage block,
            // 8-byte tail at R2 * 64 + (g * R2 + row) * 8; with M odd the tile holding row M (the
            // last row group's last tile) writes that pad row as zeros
            static_assert(!F6 || (B == 128 && !Q8), "FP6 output: one 128-k stage per block, int4 codes");
            const int R2 = (M + 1) & ~1;
            uint8_t *blk = xq + (int64_t)b * R2 * 96;
            for (int e = tid; e < MT * 4; e += NT) {
                const int row = e >> 2, g = e & 3, m = m0 + row;
                const bool live = m < row_end;
                if (!live && !(m == M && (M & 1))) continue;
                uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
                if (live) f6_encode_group(*reinterpret_cast<const uint4 *>(&sq[row * OB + 16 * g]), w);
                *reinterpret_cast<uint4 *>(blk + (int64_t)m * 64 + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
                *reinterpret_cast<uint2 *>(blk + (int64_t)R2 * 64 + ((int64_t)g * R2 + m) * 8) =
                    make_uint2(w[4], w[5]);
            }
        } else {
            // codes of the tile: 16-byte stores (OB / 16 chunks per row)
            for (int e = tid; e < OCH; e += NT) {
                const int row = e / (OB / 16), ch = e % (OB / 16);
                if (m0 + row < row_end)
                    *reinterpret_cast<uint4 *>(&xq[(int64_t)(m0 + row) * ldq + b * OB + 16 * ch]) =
                        *reinterpret_cast<const uint4 *>(&sq[row * OB + 16 * ch]);
            }
        }
    }
}

// ------------------------------------------------------------------ few tokens
//
// With at most RQ_SMALL_M tokens there are too few row tiles to amortize a block's R_b fragments,
// and the launch is latency-bound; the grid is spread as wide as the work allows instead: one
// workgroup per (16-token slice, block) of NW waves, each holding the fragments of 1/NW of the
// block's output channels (8 waves for block 128, 4 for block 64). The slice's inputs X[m][perm[b*B + i]] are gathered with 2-byte loads
// (no permuted copy, no alignment needed; copying whole rows to LDS first moves more bytes per CU
// and measured slower) and staged in LDS as the MFMA B operand.
template <int MODE, int B, bool DBG, bool Q8, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_rq_small(
    const uint16_t *__restrict__ X, int64_t ldx, int M, int K, const int32_t *__restrict__ perm,
    const _Float16 *__restrict__ rhi, const _Float16 *__restrict__ rlo,
    const float *__restrict__ table, int step, uint32_t *__restrict__ rowmax,
    uint8_t *__restrict__ xq, float *__restrict__ x_scale, float *__restrict__ xrot_dbg,
    int gstride)
{
#pragma clang fp contract(off)
    // NW waves, each with B / NW output channels of the block
    constexpr int KK = B / 32, JW = B / NW, JF = JW / 16;
    static_assert(JF >= 1, "at least one 16-channel fragment per wave");
    constexpr int LDSR = B + 8;         // halves per staged row (16-byte pad)
    constexpr int RSTEP = 64 * NW / B;  // rows gathered per pass of the workgroup
    constexpr int PER = 16 / RSTEP;     // gathered elements per thread
    constexpr float LO = 1.0f / (1 << ROT_LO_SHIFT);
    __shared__ __attribute__((aligned(16))) uint16_t sx[16 * LDSR];
    __shared__ float smax[NW][16];

    // workgroup -> (16-token slice, block); with 8 | nb the slices of a block share an XCD (and
    // its L2, where the block's fragments are then fetched once)
    const int nb = K / B, ns = gridDim.x / nb, wg = blockIdx.x;
    int b, si;
    if (nb % 8 == 0) {
        const int i = wg / 8;
        b = 8 * (i / ns) + wg % 8;
        si = i % ns;
    } else {
        b = wg / ns;
        si = wg % ns;
    }
    const int m0 = si * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int jbase = wave * JW;

    // gather: thread -> input column tid % B of the block, rows tid / B + RSTEP * i (clamped).
    // Issue order: the permutation entry, then the R_b fragments (independent of it), then the
    // gathers that need it -- loads retire in order, so the wait for the entry does not also wait
    // for the fragments, and their latency overlaps the entry's.
    // The entry is loaded unconditionally (from any readable word, here the rotation operand, when
    // the identity is meant) and the identity is selected only where the address is formed:
    // consuming the loaded value right away, as a branch's join would, waits for it at once.
    const int gc = tid % B, gr0 = tid / B;
    const int32_t *pidx = perm ? perm + (b * B + gc) : reinterpret_cast<const int32_t *>(rhi);
    const int praw = *pidx;
    __builtin_amdgcn_sched_barrier(0);
    v8h ahi[JF][KK], alo[JF][KK];
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int64_t off = rot16_fragment(b, jbase / 16 + jf, kk, lane, B);
            ahi[jf][kk] = *reinterpret_cast<const v8h *>(rhi + off);
            alo[jf][kk] = *reinterpret_cast<const v8h *>(rlo + off);
        }
    __builtin_amdgcn_sched_barrier(0);
    const int64_t src_col = perm ? (int64_t)praw : (int64_t)(b * B + gc);
    uint16_t xv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int m = min(m0 + gr0 + RSTEP * i, M - 1);
        xv[i] = X[(int64_t)m * ldx + src_col];
    }
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ahi[jf][kk] = ahi[jf][kk] * (_Float16)(1 << ROT_LO_SHIFT);
    float rs = 0.0f;
    if (MODE == ACT_PER_STEP) {
        const StepScale ss = step_scale(table, step + b * gstride);
        rs = ss.rcp * LO;
        if (si == 0 && (gstride || b == 0) && tid == 0) x_scale[b * gstride] = ss.s;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int rr = gr0 + RSTEP * i;
        sx[rr * LDSR + gc] = (m0 + rr < M) ? xv[i] : (uint16_t)0;
    }
    __syncthreads();

    // acc[jf] = 2^12 x' for token m0 + (lane % 16), channels jbase + 16 jf + 4 (lane / 16) + 0..3
    v4f acc[JF];
#pragma unroll
    for (int jf = 0; jf < JF; ++jf) acc[jf] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const v8h xb = *reinterpret_cast<const v8h *>(&sx[r * LDSR + 32 * kk + 8 * g]);
#pragma unroll
        for (int jf = 0; jf < JF; ++jf)
            acc[jf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[jf][kk], xb, acc[jf], 0, 0, 0);
#pragma unroll
        for (int jf = 0; jf < JF; ++jf)
            acc[jf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jf][kk], xb, acc[jf], 0, 0, 0);
    }

    const int m = m0 + r;
    if (MODE == ACT_TOKEN_MAX || MODE == ACT_CALIB_MAX) {
        float a = 0.0f;
#pragma unroll
        for (int jf = 0; jf < JF; ++jf)
#pragma unroll
            for (int i = 0; i < 4; ++i) a = fmaxf(a, fabsf(acc[jf][i]));
        a = fmaxf(a, __shfl_xor(a, 16));
        a = fmaxf(a, __shfl_xor(a, 32));
        if (g == 0) smax[wave][r] = (m < M) ? a * LO : 0.0f;
        __syncthreads();
        if (tid < 16) {
            float u = smax[0][tid];
#pragma unroll
            for (int w = 1; w < NW; ++w) u = fmaxf(u, smax[w][tid]);
            if (MODE == ACT_TOKEN_MAX) {
                if (m0 + tid < M) atomicMax(&rowmax[m0 + tid], __float_as_uint(u));
            } else {
#pragma unroll
                for (int off = 8; off > 0; off >>= 1) u = fmaxf(u, __shfl_xor(u, off));
                if (tid == 0) atomicMax(&rowmax[b * gstride], __float_as_uint(u));
            }
        }
        return;
    }
    if (m >= M) return;
    const int jl = jbase + 4 * g;
    if (DBG) {
#pragma unroll
        for (int jf = 0; jf < JF; ++jf)
            *reinterpret_cast<float4 *>(&xrot_dbg[(int64_t)m * K + b * B + jl + 16 * jf]) =
                make_float4(acc[jf][0] * LO, acc[jf][1] * LO, acc[jf][2] * LO, acc[jf][3] * LO);
    }
    if (MODE == ACT_TOKEN_QUANT) {
        const float s = scale_from_absmax_q<Q8>(__uint_as_float(rowmax[m]));
        rs = (float)(1.0 / (double)s) * LO;
        if (b == 0 && wave == 0 && g == 0) x_scale[m] = s;
    }
#pragma unroll
    for (int jf = 0; jf < JF; ++jf) {
        if (Q8)
            *reinterpret_cast<uint32_t *>(&xq[(int64_t)m * K + b * B + jl + 16 * jf]) =
                quant_pack4<true>(acc[jf], rs);
        else
            *reinterpret_cast<uint16_t *>(&xq[(int64_t)m * (K / 2) + (b * B + jl + 16 * jf) / 2]) =
                (uint16_t)quant_pack4(acc[jf], rs);
    }
}

// ------------------------------------------------------------------ Hadamard-only rotation
//
// The rotation with U_b = I, R_b = H_B: the plain block Walsh-Hadamard transform (the
// FoldQuantVLA summary's block Hadamard, the DuQuant-style rotation without the SVD factor). No
// rotation operand is read, so a workgroup stages whole rows of X in LDS with coalesced loads,
// gathers each block's zigzag inputs from LDS and applies the transform as log2(B) butterfly stages
// in fp64: a quad of 4 lanes per (row, block) unit with B / 4 values each, the low index bits inside
// a lane and the two high bits across the quad (exchanged with quad-permute DPP moves, plain VALU
// work), scaled once by fp64(1/sqrt(B)). Each value is the fp32 rounding of an fp64 result a few
// ulps from the exact x'. The oracle rounds the same real number, so the two agree unless x' lies
// within ~2^-45 (relative) of an fp32 rounding boundary, or the block's signed sum cancels to a
// value comparable to the oracle's own fp64 rounding.
// Per-token mode takes the row maximum in the same workgroup, with no second pass over HBM: the
// first sweep keeps HD_KEEP rounds of results in registers, and the second recomputes any further
// rounds from LDS.
constexpr int HD_UNITS = 64;  // (row, block) units per round of the workgroup: 64 quads
constexpr int HD_KEEP = 2;
constexpr int HD_MAX_LDS = 128 * 1024;  // staged rows; the entry point rejects larger K

__device__ __forceinline__ double hd_load(const uint16_t *p, int i)
{
    return (double)__half2float(__ushort_as_half(p[i]));
}
__device__ __forceinline__ double hd_load(const float *p, int i) { return (double)p[i]; }

// x from the lane of this quad selected by the quad-permute control CTRL (both 32-bit halves)
template <int CTRL>
__device__ __forceinline__ double quad_dpp(double x)
{
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm(1, 0, 3, 2)
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm(2, 3, 0, 1)

template <int MODE, int B, typename XT, bool DBG>
__global__ __launch_bounds__(256) void k_rq_hadamard(
    const XT *__restrict__ X, int64_t ldx, int M, int K, int rows_per_wg, int vec_load, double hinv,
    const int32_t *__restrict__ perm, const float *__restrict__ table, int step,
    uint8_t *__restrict__ xq, float *__restrict__ x_scale, float *__restrict__ xrot_dbg)
{
#pragma clang fp contract(off)
    constexpr int EPT = B / 4;  // values per lane
    extern __shared__ __attribute__((aligned(16))) unsigned char hd_smem[];
    XT *srow = reinterpret_cast<XT *>(hd_smem);
    __shared__ uint32_t smax[HD_UNITS];
    const int tid = threadIdx.x, t4 = tid & 3, slot = tid >> 2;
    const int row0 = blockIdx.x * rows_per_wg;
    const int nrows = min(rows_per_wg, M - row0);
    const int nb = K / B;
    const int units = nrows * nb;

    if (vec_load) {
        constexpr int VE = 16 / sizeof(XT);
        const int cpr = K / VE;
        for (int c = tid; c < nrows * cpr; c += 256) {
            const int rr = c / cpr, cc = c % cpr;
            *reinterpret_cast<uint4 *>(&srow[(int64_t)rr * K + VE * cc]) =
                *reinterpret_cast<const uint4 *>(&X[(int64_t)(row0 + rr) * ldx + VE * cc]);
        }
    } else {
        for (int c = tid; c < nrows * K; c += 256) {
            const int rr = c / K, cc = c % K;
            srow[(int64_t)rr * K + cc] = X[(int64_t)(row0 + rr) * ldx + cc];
        }
    }
    if (tid < HD_UNITS) smax[tid] = 0u;
    __syncthreads();

    // the lane's EPT values of unit u (row u / nb, block u % nb): inputs EPT * t4 + e of the block
    auto transform = [&](int u, float (&out)[EPT]) {
        const int rr = u / nb, b = u % nb;
        const XT *xr = srow + (int64_t)rr * K;
        double v[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int j = b * B + EPT * t4 + e;
            v[e] = hd_load(xr, perm ? perm[j] : j);
        }
#pragma unroll
        for (int d = 1; d < EPT; d <<= 1)
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (!(e & d)) {
                    const double a = v[e], c = v[e + d];
                    v[e] = a + c;
                    v[e + d] = a - c;
                }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const double p = quad_dpp<DPP_QUAD_XOR1>(v[e]);
            v[e] = (t4 & 1) ? p - v[e] : v[e] + p;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const double p = quad_dpp<DPP_QUAD_XOR2>(v[e]);
            v[e] = (t4 & 2) ? p - v[e] : v[e] + p;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) out[e] = (float)(v[e] * hinv);
    };
    // quantize the unit with r = fp32(1/s) and store its EPT codes (EPT / 2 contiguous bytes)
    auto emit = [&](int u, const float (&x)[EPT], float r) {
        const int m = row0 + u / nb, col = (u % nb) * B + EPT * t4;
        if (DBG) {
#pragma unroll
            for (int e = 0; e < EPT; ++e) xrot_dbg[(int64_t)m * K + col + e] = x[e];
        }
        uint32_t w[EPT / 8];
#pragma unroll
        for (int k = 0; k < EPT / 8; ++k) {
            uint32_t t = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) t |= (uint32_t)(quant_code(x[8 * k + e], r) & 0xF) << (4 * e);
            w[k] = t;
        }
        uint8_t *dst = xq + (int64_t)m * (K / 2) + col / 2;
        if (EPT == 32) *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1 % (EPT / 8)], w[2 % (EPT / 8)], w[3 % (EPT / 8)]);
        else *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1 % (EPT / 8)]);
    };

    if (MODE == ACT_PER_STEP) {
        const StepScale ss = step_scale(table, step);
        const float r = ss.rcp;
        if (blockIdx.x == 0 && tid == 0) x_scale[0] = ss.s;
        for (int u = slot; u < units; u += HD_UNITS) {
            float x[EPT];
            transform(u, x);
            emit(u, x, r);
        }
        return;
    }

    // per token: row maxima first (kept results for the first HD_KEEP rounds), then quantize
    float keep[HD_KEEP][EPT];
    auto row_max = [&](int u, const float (&x)[EPT]) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) a = fmaxf(a, fabsf(x[e]));
        a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), DPP_QUAD_XOR1, 0xF, 0xF, false)));
        a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), DPP_QUAD_XOR2, 0xF, 0xF, false)));
        if (t4 == 0) atomicMax(&smax[u / nb], __float_as_uint(a));
    };
#pragma unroll
    for (int k = 0; k < HD_KEEP; ++k) {
        const int u = slot + k * HD_UNITS;
        if (u < units) {
            transform(u, keep[k]);
            row_max(u, keep[k]);
        }
    }
    for (int u = slot + HD_KEEP * HD_UNITS; u < units; u += HD_UNITS) {
        float x[EPT];
        transform(u, x);
        row_max(u, x);
    }
    __syncthreads();
    auto finish = [&](int u, const float (&x)[EPT]) {
        const int rr = u / nb;
        const float s = scale_from_absmax(__uint_as_float(smax[rr]));
        if (u % nb == 0 && t4 == 0) x_scale[row0 + rr] = s;
        emit(u, x, (float)(1.0 / (double)s));
    };
#pragma unroll
    for (int k = 0; k < HD_KEEP; ++k) {
        const int u = slot + k * HD_UNITS;
        if (u < units) finish(u, keep[k]);
    }
    for (int u = slot + HD_KEEP * HD_UNITS; u < units; u += HD_UNITS) {
        float x[EPT];
        transform(u, x);
        finish(u, x);
    }
}

size_t hadamard_lds_bytes(int M, int K, int B, int x_dtype, int *rows_per_wg)
{
    const int nb = K / B;
    int r = max(1, min(HD_UNITS / nb, M / 256));
    if (rows_per_wg) *rows_per_wg = r;
    return (size_t)r * K * (x_dtype == W4A4_F16 ? 2 : 4);
}

int launch_rotate_quant_hadamard(const void *X, int x_dtype, int M, int K, int64_t ldx, int B,
                                 const int32_t *perm, const float *table, int step, uint8_t *xq,
                                 float *x_scale, float *xrot_dbg, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    int rpw = 1;
    const size_t lds = hadamard_lds_bytes(M, K, B, x_dtype, &rpw);
    const int esz = x_dtype == W4A4_F16 ? 2 : 4;
    const int vec = ((uintptr_t)X % 16 == 0) && ((ldx * esz) % 16 == 0) && ((K * esz) % 16 == 0);
    const double hinv = 1.0 / std::sqrt((double)B);
    dim3 grid((M + rpw - 1) / rpw);
    const bool per_step = table != nullptr;
#define W4A4_HD_LAUNCH(MODEV, BV, XTV, DV)                                                         \
    do {                                                                                           \
        const int lrc = ensure_dynamic_lds((const void *)k_rq_hadamard<MODEV, BV, XTV, DV>, lds,   \
                                           "Hadamard rotate");                                     \
        if (lrc != W4A4_OK) return lrc;                                                            \
        hipLaunchKernelGGL((k_rq_hadamard<MODEV, BV, XTV, DV>), grid, dim3(256), lds, s,           \
                           reinterpret_cast<const XTV *>(X), ldx, M, K, rpw, vec, hinv, perm,      \
                           table, step, xq, x_scale, xrot_dbg);                                    \
    } while (0)
#define W4A4_HD_D(MODEV, BV, XTV)                                                                  \
    if (xrot_dbg) W4A4_HD_LAUNCH(MODEV, BV, XTV, true); else W4A4_HD_LAUNCH(MODEV, BV, XTV, false);
#define W4A4_HD_X(MODEV, BV)                                                                       \
    if (x_dtype == W4A4_F16) { W4A4_HD_D(MODEV, BV, uint16_t) } else { W4A4_HD_D(MODEV, BV, float) }
#define W4A4_HD_B(MODEV)                                                                           \
    if (B == 128) { W4A4_HD_X(MODEV, 128) } else { W4A4_HD_X(MODEV, 64) }
    if (per_step) { W4A4_HD_B(ACT_PER_STEP) } else { W4A4_HD_B(ACT_TOKEN_QUANT) }
#undef W4A4_HD_B
#undef W4A4_HD_X
#undef W4A4_HD_D
#undef W4A4_HD_LAUNCH
    return check_launch("rotate-quantize (Hadamard)");
}

// Zigzag gather of whole rows: Xp[m][j] = X[m][perm[j]] (fp16), one workgroup per row, the source
// row staged in LDS with 16-byte loads and the permuted row written with 16-byte stores. The
// workgroup of row m also clears zero_row[m] (the per-token maxima the next pass accumulates), when
// given, which saves a separate fill launch.
template <bool VEC>
__global__ __launch_bounds__(256) void k_permute_rows(const uint16_t *__restrict__ X, int64_t ldx,
                                                      int K, const int32_t *__restrict__ perm,
                                                      uint16_t *__restrict__ Xp,
                                                      uint32_t *__restrict__ zero_row)
{
    extern __shared__ uint16_t srow[];
    const int m = blockIdx.x, tid = threadIdx.x;
    if (zero_row && tid == 0) zero_row[m] = 0u;
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
            // entries outside [0, K) (not a permutation) read a clamped element, never past the row
            auto at = [&](int i) { return (uint32_t)srow[min(max(i, 0), K - 1)]; };
            uint4 v;
            v.x = at(p0.x) | (at(p0.y) << 16);
            v.y = at(p0.z) | (at(p0.w) << 16);
            v.z = at(p1.x) | (at(p1.y) << 16);
            v.w = at(p1.z) | (at(p1.w) << 16);
            *reinterpret_cast<uint4 *>(&out[c]) = v;
        }
    } else {
        for (int c = tid; c < K; c += 256) out[c] = srow[min(max(perm[c], 0), K - 1)];
    }
}

bool act_uses_permute_pass(int M, int K, int per_token)
{
    // The in-kernel gather issues one 2-byte load per element, each from a different cache line of
    // a long row; a coalesced permutation pass (its output stays in the 256 MB last-level cache)
    // followed by 16-byte DMA tile loads wins once the batch is a few MB, and earlier in per-token
    // mode, which reads the rows twice (and where the pass also clears the row maxima). The pass
    // stages a whole row in LDS.
    if (K > 65536 || M <= RQ_SMALL_M) return false;  // few tokens: gathered in the kernel
    const int64_t elems = (int64_t)M * K;
    return per_token ? (K >= 2048 || elems >= (1 << 20)) : (elems >= (1 << 22));
}

size_t act_permute_bytes(int M, int K) { return align_up((size_t)M * K * sizeof(uint16_t), 256); }

static int rq_rows_per_wg(int M, int nb)
{
    const int mt = (M + MT - 1) / MT;
    int rg = (512 + nb - 1) / nb;
    rg = max(1, min(rg, mt));
    return ((mt + rg - 1) / rg) * MT;
}

bool rq_ring_path(int M, const void *X, int64_t ldx, const int32_t *perm, const uint16_t *xperm,
                  int K)
{
    if (M <= RQ_SMALL_M && !xperm) return false;
    const uint16_t *src = xperm ? xperm : reinterpret_cast<const uint16_t *>(X);
    const int64_t ld = xperm ? K : ldx;
    const bool rows_aligned = ((uintptr_t)src % 16 == 0) && (ld % 8 == 0);
    return rows_aligned && (xperm || !perm);
}

int launch_rotate_quant_mfma(const void *X, int M, int K, int64_t ldx, int B, const int32_t *perm,
                             const void *rot, const float *table, int step, ActMode mode,
                             uint32_t *rowmax, uint8_t *xq, float *x_scale, float *xrot_dbg,
                             const uint16_t *xperm, bool q8, hipStream_t s, int gstride, bool f6)
{
    if (M == 0) return W4A4_OK;
    if (f6 && (!rq_ring_path(M, X, ldx, perm, xperm, K) || B != 128 || q8 || xrot_dbg ||
               (uintptr_t)xq % 16 != 0 || (mode != ACT_PER_STEP && mode != ACT_TOKEN_QUANT)))
        return fail(W4A4_ERR_UNSUPPORTED, "FP6 activation output needs the streaming kernel");
    RotLayout L = rot_layout(K, B);
    const char *base = reinterpret_cast<const char *>(rot);
    const _Float16 *rhi = reinterpret_cast<const _Float16 *>(base + L.r32);
    const _Float16 *rlo = reinterpret_cast<const _Float16 *>(base + L.r32 + L.r16);
    const int nb = K / B;
    // Every family below is instantiated for both code widths in the quantizing modes (per-step,
    // per-token second pass) and for int4 only in the max-only passes, which write no codes.
    if (M <= RQ_SMALL_M && !xperm) {
        dim3 grid_s(((M + 15) / 16) * nb);
        const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
        // block 128: 8 waves of 16 channels (2.88 vs 3.00 us per launch on the DiT up-projection
        // than 4 waves of 32: half the fragment loads per lane, twice the waves in flight)
#define W4A4_SMALL(MODEV, BV, DV, QV)                                                              \
    hipLaunchKernelGGL((k_rq_small<MODEV, BV, DV, QV, (BV == 128 ? 8 : 4)>), grid_s,               \
                       dim3(BV == 128 ? 512 : 256), 0, s, x, ldx, M, K, perm, rhi, rlo, table,     \
                       step, rowmax, xq, x_scale, xrot_dbg, gstride)
#define W4A4_SMALL_B(MODEV, DV, QV)                                                                \
    if (B == 128) W4A4_SMALL(MODEV, 128, DV, QV); else W4A4_SMALL(MODEV, 64, DV, QV);
#define W4A4_SMALL_Q(MODEV)                                                                        \
    if (xrot_dbg) { if (q8) { W4A4_SMALL_B(MODEV, true, true) } else { W4A4_SMALL_B(MODEV, true, false) } } \
    else { if (q8) { W4A4_SMALL_B(MODEV, false, true) } else { W4A4_SMALL_B(MODEV, false, false) } }
        switch (mode) {
        case ACT_PER_STEP: W4A4_SMALL_Q(ACT_PER_STEP) break;
        case ACT_TOKEN_MAX: W4A4_SMALL_B(ACT_TOKEN_MAX, false, false) break;
        case ACT_TOKEN_QUANT: W4A4_SMALL_Q(ACT_TOKEN_QUANT) break;
        case ACT_CALIB_MAX: W4A4_SMALL_B(ACT_CALIB_MAX, false, false) break;
        }
#undef W4A4_SMALL_Q
#undef W4A4_SMALL_B
#undef W4A4_SMALL
        return check_launch("rotate-quantize (few tokens)");
    }
    const int rpw = rq_rows_per_wg(M, nb);
    dim3 grid(((M + rpw - 1) / rpw) * nb);  // (row group, block) pairs, XCD-aware in the kernel
    const uint16_t *src = xperm ? xperm : reinterpret_cast<const uint16_t *>(X);
    const int64_t ld = xperm ? K : ldx;
    // contiguous 16-byte tile loads need 16-byte aligned rows; otherwise gather element-wise
    const bool rows_aligned = ((uintptr_t)src % 16 == 0) && (ld % 8 == 0);
    const bool gather = ((perm != nullptr) && (xperm == nullptr)) || !rows_aligned;
    if (xperm) perm = nullptr;
    if (!gather && ((uintptr_t)xq % 16 == 0)) {
        // rows in zigzag order: LDS DMA ring (rows per workgroup capped by the staged scales)
        const int rpw_r = min(rpw, RQ_RING_MAX_ROWS);
        const int groups = (M + rpw_r - 1) / rpw_r;
        dim3 grid_r(groups * nb);
        const size_t lds = (size_t)RQ_STAGES * MT * B * sizeof(uint16_t);
    // block 128: 8 waves of 16 channels (twice the waves in flight on the same tiles)
#define W4A4_RING_K(MODEV, BV, DV, QV, FV)                                                         \
    do {                                                                                           \
        constexpr int RNW = BV == 128 ? 8 : 4;                                                     \
        const int lrc = ensure_dynamic_lds((const void *)k_rq_ring<MODEV, BV, DV, QV, FV, RNW>,    \
                                           lds, "rotate-quantize");                                \
        if (lrc != W4A4_OK) return lrc;                                                            \
        hipLaunchKernelGGL((k_rq_ring<MODEV, BV, DV, QV, FV, RNW>), grid_r, dim3(64 * RNW), lds,   \
                           s, src, ld, M, K, rhi, rlo, table, step, rowmax, xq, x_scale, xrot_dbg, \
                           rpw_r, groups, gstride);                                                \
    } while (0)
#define W4A4_RING(MODEV, BV, DV, QV) W4A4_RING_K(MODEV, BV, DV, QV, false)
#define W4A4_RING_F6(MODEV) W4A4_RING_K(MODEV, 128, false, false, true)
#define W4A4_RING_B(MODEV, DV, QV)                                                                 \
    if (B == 128) W4A4_RING(MODEV, 128, DV, QV); else W4A4_RING(MODEV, 64, DV, QV);
#define W4A4_RING_Q(MODEV)                                                                         \
    if (xrot_dbg) { if (q8) { W4A4_RING_B(MODEV, true, true) } else { W4A4_RING_B(MODEV, true, false) } } \
    else { if (q8) { W4A4_RING_B(MODEV, false, true) } else { W4A4_RING_B(MODEV, false, false) } }
        if (f6) {
            if (mode == ACT_PER_STEP) W4A4_RING_F6(ACT_PER_STEP);
            else W4A4_RING_F6(ACT_TOKEN_QUANT);
            return check_launch("rotate-quantize (ring, FP6 output)");
        }
        switch (mode) {
        case ACT_PER_STEP: W4A4_RING_Q(ACT_PER_STEP) break;
        case ACT_TOKEN_MAX: W4A4_RING_B(ACT_TOKEN_MAX, false, false) break;
        case ACT_TOKEN_QUANT: W4A4_RING_Q(ACT_TOKEN_QUANT) break;
        case ACT_CALIB_MAX: W4A4_RING_B(ACT_CALIB_MAX, false, false) break;
        }
#undef W4A4_RING_Q
#undef W4A4_RING_B
#undef W4A4_RING_F6
#undef W4A4_RING
#undef W4A4_RING_K
        return check_launch("rotate-quantize (ring)");
    }
    // block 128: 8 waves of 16 channels (each thread gathers half as many inputs per tile)
#define W4A4_RQ(MODEV, BV, GV, QV)                                                                 \
    hipLaunchKernelGGL((k_rq_mfma<MODEV, BV, GV, QV, (BV == 128 ? 8 : 4)>), grid,                  \
                       dim3(BV == 128 ? 512 : 256), 0, s, src, ld, M, K, perm, rhi, rlo, table,     \
                       step, rowmax, xq, x_scale, xrot_dbg, rpw, gstride)
#define W4A4_RQ_B(MODEV, QV)                                                                       \
    if (B == 128) { if (gather) W4A4_RQ(MODEV, 128, true, QV); else W4A4_RQ(MODEV, 128, false, QV); } \
    else { if (gather) W4A4_RQ(MODEV, 64, true, QV); else W4A4_RQ(MODEV, 64, false, QV); }
#define W4A4_RQ_Q(MODEV)                                                                           \
    if (q8) { W4A4_RQ_B(MODEV, true) } else { W4A4_RQ_B(MODEV, false) }
    switch (mode) {
    case ACT_PER_STEP: W4A4_RQ_Q(ACT_PER_STEP) break;
    case ACT_TOKEN_MAX: W4A4_RQ_B(ACT_TOKEN_MAX, false) break;
    case ACT_TOKEN_QUANT: W4A4_RQ_Q(ACT_TOKEN_QUANT) break;
    case ACT_CALIB_MAX: W4A4_RQ_B(ACT_CALIB_MAX, false) break;
    }
#undef W4A4_RQ_Q
#undef W4A4_RQ_B
#undef W4A4_RQ
    return check_launch("rotate-quantize (mfma)");
}

int launch_permute_rows(const void *X, int M, int K, int64_t ldx, const int32_t *perm, uint16_t *xp,
                        uint32_t *zero_row, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    const size_t lds = (size_t)K * sizeof(uint16_t);
    const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0) &&
                     ((uintptr_t)perm % 16 == 0);
    const void *fn = vec ? (const void *)k_permute_rows<true> : (const void *)k_permute_rows<false>;
    if (int rc = ensure_dynamic_lds(fn, lds, "permute")) return rc;
    const uint16_t *x = reinterpret_cast<const uint16_t *>(X);
    if (vec)
        hipLaunchKernelGGL(k_permute_rows<true>, dim3(M), dim3(256), lds, s, x, ldx, K, perm, xp,
                           zero_row);
    else
        hipLaunchKernelGGL(k_permute_rows<false>, dim3(M), dim3(256), lds, s, x, ldx, K, perm, xp,
                           zero_row);
    return check_launch("permute rows");
}

// count scales (one per calibration group: the whole linear, or each rotation block)
__global__ void k_scale_from_absmax(const uint32_t *amax, float *out, int q8, int count)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    out[i] = q8 ? scale_from_absmax_q<true>(__uint_as_float(amax[i]))
                : scale_from_absmax(__uint_as_float(amax[i]));
}

int launch_scale_from_absmax(const uint32_t *amax, float *out, bool q8, hipStream_t s, int count)
{
    hipLaunchKernelGGL(k_scale_from_absmax, dim3((count + 255) / 256), dim3(256), 0, s, amax, out,
                       q8 ? 1 : 0, count);
    return check_launch("scale from absmax");
}

}  // namespace w4a4
