// W4A4 GEMM: packed int4 activations [M][K/2] x packed int4 weights [N][K/2] -> int32 on int8 MFMA,
// with the dequantization (per-token or per-step activation scale, per-output-channel weight
// scale), optional GELU / residual epilogue and the fp16 store fused into the tile's epilogue.
//
// CDNA4 has no int4 matrix instruction and its FP4 format (e2m1) does not hold the uniform int4
// grid, so nibbles are widened to int8 in registers right before v_mfma_i32_16x16x64_i8. The
// widening keeps each nibble in the high half of its byte, (v << 4) & 0xF0F0F0F0 for the even
// codes and v & 0xF0F0F0F0 for the odd ones, so every int8 operand equals 16 * code exactly and the
// MFMA sums 256 * q * p; an arithmetic shift right by 8 recovers the exact integer sum
// (|sum| <= 64 K, so 256 * 64 K stays below 2^31 for the at most 2^16 k values of one split). Both
// operands go through the same even/odd reordering of k, so the dot products match.
#include <cmath>
#include <type_traits>

#include "rq_core.h"

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int MAX_K_SPLIT = 1 << 16;  // 256 * 64 * 2^16 = 2^30 fits int32
constexpr int SMALL_M = 64;           // rows up to which the weight-streaming kernel is used
// tile kinds of the software-pipelined GEMM (k_gemm_sp) in the GEMM plan
enum SpKind { SP_128x192 = 11, SP_128x128 = 12, SP_64x128 = 13 };

// Tile order of the tiled GEMM kernels. Dispatch id i runs on XCD i % 8, and XCD x takes a
// contiguous 1/8 of the order. The order walks bands of `band` column tiles, row-major inside a
// band, so the tiles of one XCD form a compact block: its L2 holds a few activation row tiles and a
// few weight column tiles, each read by several of its workgroups (band = 1 is column-major: one
// XCD then reads every activation row tile once, all from the last-level cache or HBM).
__device__ __forceinline__ void xcd_tile(int id, int tiles_m, int tiles_n, int band, int &tm,
                                         int &tn)
{
    const int T = tiles_m * tiles_n;
    const int per_x = T / 8, rm = T % 8, x = id % 8;
    const int lin = x * per_x + min(x, rm) + id / 8;
    const int b = lin / (band * tiles_m);
    const int w = min(band, tiles_n - b * band);  // the last band may be narrower
    const int r = lin - b * band * tiles_m;
    tm = r / w;
    tn = b * band + r % w;
}

// Band width that minimizes the operand bytes one XCD's block of tiles touches: about
// rows * bm + band * bn per k, with rows * band = its share of the tiles.
static int tile_band(int tiles_m, int tiles_n, int bm, int bn)
{
    const double per_x = (double)tiles_m * (double)tiles_n / 8.0;
    const int g = (int)std::lround(std::sqrt(per_x * (double)bm / (double)bn));
    return std::max(1, std::min(g, tiles_n));
}

__device__ __forceinline__ void widen16(const uint4 &p, uint4 &lo, uint4 &hi)
{
    // 16 packed bytes (k = 0..31 of a half step) -> 32 int8 values, two dwords per packed dword
    lo.x = (p.x << 4) & 0xF0F0F0F0u; lo.y = p.x & 0xF0F0F0F0u;
    lo.z = (p.y << 4) & 0xF0F0F0F0u; lo.w = p.y & 0xF0F0F0F0u;
    hi.x = (p.z << 4) & 0xF0F0F0F0u; hi.y = p.z & 0xF0F0F0F0u;
    hi.z = (p.w << 4) & 0xF0F0F0F0u; hi.w = p.w & 0xF0F0F0F0u;
}

// Load 16 packed bytes of row `row` at packed byte offset `kb`; zero outside [0, rows) x [0, kbend).
template <bool VEC>
__device__ __forceinline__ uint4 load_packed16(const uint8_t *__restrict__ base, int rows, int row,
                                               int64_t ld, int kb, int kbend)
{
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row >= rows) return v;
    const uint8_t *p = base + (int64_t)row * ld + kb;
    if (VEC && kb + 16 <= kbend) {
        v = *reinterpret_cast<const uint4 *>(p);
    } else {
        uint32_t w[4] = {0, 0, 0, 0};
        for (int t = 0; t < 16; ++t)
            if (kb + t < kbend) w[t >> 2] |= (uint32_t)p[t] << (8 * (t & 3));
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return v;
}

// Branch-free 16-byte load for the aligned path: out-of-range items read row 0 / byte 0 of the same
// operand (always in bounds) and report valid = false, so the caller zeroes them when it consumes
// the data. Keeping the load unconditional lets it stay in flight across the MFMA work.
__device__ __forceinline__ uint4 load16_clamped(const uint8_t *__restrict__ base, int rows, int row,
                                                int64_t ld, int kb, int kbend, bool &valid)
{
    valid = (row < rows) && (kb < kbend);
    const int64_t off = valid ? (int64_t)row * ld + kb : 0;
    return *reinterpret_cast<const uint4 *>(base + off);
}

__device__ __forceinline__ uint4 zero_unless(const uint4 &v, bool valid)
{
    return make_uint4(valid ? v.x : 0u, valid ? v.y : 0u, valid ? v.z : 0u, valid ? v.w : 0u);
}

// erf-GELU, v * Phi(v), in fp32 with one branch-free path: for w = min(|v|, 6),
// Phi(-w) = exp(-w^2/2) * g(w) where g(w) = 0.5 erfc(w / sqrt 2) exp(w^2 / 2) is a degree-7
// polynomial in t = 1 / (1 + 0.3 w) (relative least-squares fit on [0, 6], relative error 1.6e-7;
// fit_gelu_tail.py beside this file regenerates the coefficients), and Phi(v) = 1 - Phi(-w) for
// v >= 0. Beyond |v| = 6 the tail is below 1e-9 and leaves GELU unchanged at fp16 resolution. The
// result is within about 1e-6 relative of the exact value, so after the fp16 rounding it equals
// the correctly rounded GELU or its neighbour; it costs two transcendental and about 15 other VALU
// operations, several times less than a library erf with range branches.
__device__ __forceinline__ float gelu_erf(float v)
{
    // min(|v|, 6) in one v_med3_f32 (for NaN v the result is NaN through the exponential below)
    const float w = __builtin_amdgcn_fmed3f(fabsf(v), 0.0f, 6.0f);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3f, w, 1.0f));
    float p = 0.0311708786f;
    p = fmaf(p, t, -0.220824048f);
    p = fmaf(p, t, 0.48928532f);
    p = fmaf(p, t, -0.294268399f);
    p = fmaf(p, t, 0.306398928f);
    p = fmaf(p, t, 0.0590155609f);
    p = fmaf(p, t, 0.129963309f);
    p = fmaf(p, t, -0.000741627882f);
    const float e = __builtin_amdgcn_exp2f((v * v) * -0.721347520444482f);  // exp(-v^2/2)
    const float tail = p * e;                                               // Phi(-|v|)
    return v * (v >= 0.0f ? 1.0f - tail : tail);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v)
{
    return __half_as_ushort(__float2half_rn(v));
}

// Two fp32 values rounded to fp16 (to nearest even, v_cvt_pk_f16_f32), packed low value first.
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi)
{
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t h = __builtin_convertvector(f2_t{lo, hi}, h2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// The dequantization is specified as a chain of fp32 roundings followed by one fp16 rounding.
// The compiler may otherwise fuse "fp16(a * b)" or "fp16(a * b + c)" into one mixed-precision
// instruction that rounds once, which differs at fp16 ties; pinning each fp32 intermediate in a
// register keeps every rounding where it is written.
__device__ __forceinline__ float fp32_value(float x)
{
    // not volatile: the value stays opaque to instruction selection, but the scheduler may still
    // interleave the epilogue's per-element chains (volatile statements keep their program order,
    // which serialized every element's GELU behind the previous one's)
    asm("" : "+v"(x));
    return x;
}

// Dequantize one accumulator with scales already in registers and store it as fp16.
__device__ __forceinline__ void store_scaled(const GemmEpilogue &epi, int m, int n, int32_t v,
                                             float sx, float sw)
{
#pragma clang fp contract(off)
    float y = fp32_value((float)v * sx);
    y = fp32_value(y * sw);
    if (epi.mode == W4A4_EPI_GELU) y = fp32_value(gelu_erf(y));
    else if (epi.mode == W4A4_EPI_RESIDUAL)
        y = fp32_value(y + __half2float(__ushort_as_half(epi.residual[(int64_t)m * epi.ldr + n])));
    epi.Y[(int64_t)m * epi.ldy + n] = f32_to_f16_bits(y);
}

// Dequantize one accumulator and store it (shared by every GEMM variant).
__device__ __forceinline__ void store_output(const GemmEpilogue &epi, int m, int n, int N,
                                             int32_t v)
{
#pragma clang fp contract(off)
    if (epi.mode == GEMM_OUT_I32) {
        epi.acc_out[(int64_t)m * N + n] = v;
        return;
    }
    const float sx = epi.x_scale_per_token ? epi.x_scale[m] : epi.x_scale[0];
    store_scaled(epi, m, n, v, sx, epi.w_scale[n]);
}

// Small-M GEMM (M <= 16 * MF <= 64): the weights are streamed once from HBM, so the kernel is built
// for memory-level parallelism. A workgroup owns 16 output columns; its 4 waves split K, each wave
// issuing the loads of a whole chunk of 128-k windows before computing. Each lane loads 16 packed
// bytes of its operand row per window (lane = row (lane % 16) x k-quarter (lane / 16)) and widens
// them into the two int8 operands of two v_mfma_i32_16x16x64_i8; both operands use the same
// widening, so each MFMA pairs identical k. The 4 partial tiles are added exactly in LDS.
// Q8: int8 operands (W8A8), one code per byte: a 64-byte window is 64 k and its 16 bytes per lane
// are already the MFMA operand, so there is one MFMA per window and no scaling by 256.
constexpr int SM_CHUNK = 4;  // 64-byte windows whose loads are in flight together

template <int MF, bool VEC, bool Q8>
__global__ __launch_bounds__(256) void k_gemm_smallm(const uint8_t *__restrict__ xq,
                                                     const uint8_t *__restrict__ wq, int M, int N,
                                                     int K, GemmEpilogue epi)
{
#pragma clang fp contract(off)
    __shared__ int32_t red[4][MF * 16][17];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int ldp = Q8 ? K : K / 2;  // bytes per operand row
    const int windows = (ldp + 63) / 64;
    const int per_wave = (windows + 3) / 4;
    const int w_begin = wave * per_wave, w_end = min(windows, w_begin + per_wave);

    // Epilogue operands are fetched first, so their latency hides under the operand loads (with
    // unconditional loads on selected addresses, as in the wide kernel). The epilogue thread owns
    // column n0 + (tid % 16) and rows tid / 16 + 16 f.
    const int ecol = threadIdx.x & 15, erow = threadIdx.x >> 4;
    const int en = min(n0 + ecol, N - 1);
    const bool scaled = epi.mode != GEMM_OUT_I32;
    const bool has_res = epi.mode == W4A4_EPI_RESIDUAL;
    const float *stand_in = reinterpret_cast<const float *>(wq);
    const float e_sw = *(scaled ? epi.w_scale + en : stand_in);
    float e_sx[MF];
    uint16_t e_res[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
        const int m = min(erow + 16 * f, M - 1);
        e_sx[f] = *(scaled ? epi.x_scale + (epi.x_scale_per_token ? m : 0) : stand_in);
        e_res[f] = *(has_res ? epi.residual + (int64_t)m * epi.ldr + en
                             : reinterpret_cast<const uint16_t *>(wq));
    }

    v4i total[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) total[f] = v4i{0, 0, 0, 0};

    for (int wc = w_begin; wc < w_end; wc += SM_CHUNK) {
        const int nc = min(SM_CHUNK, w_end - wc);  // live windows of this chunk (wave-uniform)
        uint4 bq[SM_CHUNK], aq[SM_CHUNK][MF];
        bool bv[SM_CHUNK], av[SM_CHUNK][MF];
#pragma unroll
        for (int c = 0; c < SM_CHUNK; ++c) {
            if (c >= nc) continue;
            const int kb = (wc + c) * 64 + 16 * g;
            if (VEC) {
                bq[c] = load16_clamped(wq, N, n0 + r, ldp, kb, ldp, bv[c]);
            } else {
                bq[c] = load_packed16<false>(wq, N, n0 + r, ldp, kb, ldp);
                bv[c] = true;
            }
#pragma unroll
            for (int f = 0; f < MF; ++f) {
                if (VEC) {
                    aq[c][f] = load16_clamped(xq, M, f * 16 + r, ldp, kb, ldp, av[c][f]);
                } else {
                    aq[c][f] = load_packed16<false>(xq, M, f * 16 + r, ldp, kb, ldp);
                    av[c][f] = true;
                }
            }
        }
        v4i acc[MF];
#pragma unroll
        for (int f = 0; f < MF; ++f) acc[f] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < SM_CHUNK; ++c) {
            if (c >= nc) continue;
            if (Q8) {
                uint4 b = zero_unless(bq[c], bv[c]);
#pragma unroll
                for (int f = 0; f < MF; ++f) {
                    uint4 a = zero_unless(aq[c][f], av[c][f]);
                    acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<v4i *>(&a),
                                                                   *reinterpret_cast<v4i *>(&b),
                                                                   acc[f], 0, 0, 0);
                }
                continue;
            }
            uint4 b0, b1;
            widen16(zero_unless(bq[c], bv[c]), b0, b1);
#pragma unroll
            for (int f = 0; f < MF; ++f) {
                uint4 a0, a1;
                widen16(zero_unless(aq[c][f], av[c][f]), a0, a1);
                acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<v4i *>(&a0),
                                                               *reinterpret_cast<v4i *>(&b0),
                                                               acc[f], 0, 0, 0);
                acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<v4i *>(&a1),
                                                               *reinterpret_cast<v4i *>(&b1),
                                                               acc[f], 0, 0, 0);
            }
        }
        // fold the chunk (at most 512 k, so 256 * 64 * 512 fits) into the exact running sum;
        // int8 sums are exact as they stand
#pragma unroll
        for (int f = 0; f < MF; ++f) total[f] += Q8 ? acc[f] : (acc[f] >> 8);
    }
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][f * 16 + 4 * g + i][r] = total[f][i];
    __syncthreads();
    const int n = n0 + ecol;
#pragma unroll
    for (int f = 0; f < MF; ++f) {
        const int m = erow + 16 * f;
        if (m >= M || n >= N) continue;
        const int32_t v = red[0][m][ecol] + red[1][m][ecol] + red[2][m][ecol] + red[3][m][ecol];
        if (!scaled) {
            epi.acc_out[(int64_t)m * N + n] = v;
            continue;
        }
        float y = fp32_value((float)v * e_sx[f]);
        y = fp32_value(y * e_sw);
        if (epi.mode == W4A4_EPI_GELU) y = fp32_value(gelu_erf(y));
        else if (epi.mode == W4A4_EPI_RESIDUAL) y = fp32_value(y + __half2float(__ushort_as_half(e_res[f])));
        epi.Y[(int64_t)m * epi.ldy + n] = f32_to_f16_bits(y);
    }
}

// Small-M GEMM with 16 * NF output columns per workgroup, for aligned operands (16-byte rows and
// pointers). Every workgroup reads the whole activation, so with NF weight fragments per activation
// fragment the activation is loaded and widened N / (16 NF) times instead of N / 16 times, and each
// widened activation fragment feeds 2 NF MFMAs. Rows at or beyond M or N are read from clamped (in
// bounds) addresses and not zeroed: their products only reach accumulator rows and columns that are
// never stored. Packed rows are a whole number of 64-byte windows (other K go to k_gemm_smallm),
// so nothing is zeroed. The WV waves of a workgroup split K, so a short grid (few wide tiles) still
// keeps several waves per SIMD streaming. Each wave sums its k range in one int32 accumulator, exact
// while a wave covers at most 2^16 k (256 * 64 * 2^16 = 2^30); the waves' partial tiles are added
// in LDS with integer atomics, which are exact in any order.
template <int MF, int NF, int WV, int CH, bool Q8>
__global__ __launch_bounds__(64 * WV) void k_gemm_smallm_wide(const uint8_t *__restrict__ xq,
                                                              const uint8_t *__restrict__ wq, int M,
                                                              int N, int K, GemmEpilogue epi)
{
#pragma clang fp contract(off)
    constexpr int NT = 64 * WV, NC = 16 * NF, LDR = NC + 4, RS = NT / NC;
    constexpr int ER = (MF * 16 + RS - 1) / RS;  // output rows per thread
    __shared__ int32_t red[MF * 16 * LDR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * NC;
    const int ldp = Q8 ? K : K / 2;  // bytes per operand row
    const int windows = ldp / 64;
    const int per_wave = (windows + WV - 1) / WV;
    const int w_begin = wave * per_wave, w_end = min(windows, w_begin + per_wave);

    for (int i = threadIdx.x; i < MF * 16 * LDR; i += NT) red[i] = 0;
    __syncthreads();

    // Epilogue operands first: this thread owns column n0 + tid % NC and rows tid / NC + RS j.
    // The loads are unconditional, on selected addresses (a word of the packed weights stands in
    // for an operand the mode does not have; its value is never used): a load inside a branch on
    // the mode would be waited for at the branch's join, before the first operand load issues.
    const int ecol = threadIdx.x % NC, erow = threadIdx.x / NC;
    const int en = min(n0 + ecol, N - 1);
    const bool scaled = epi.mode != GEMM_OUT_I32;
    const bool has_res = epi.mode == W4A4_EPI_RESIDUAL;
    const float *stand_in = reinterpret_cast<const float *>(wq);
    const float e_sw = *(scaled ? epi.w_scale + en : stand_in);
    float e_sx[ER];
    uint16_t e_res[ER];
#pragma unroll
    for (int j = 0; j < ER; ++j) {
        const int m = min(erow + RS * j, M - 1);
        e_sx[j] = *(scaled ? epi.x_scale + (epi.x_scale_per_token ? m : 0) : stand_in);
        e_res[j] = *(has_res ? epi.residual + (int64_t)m * epi.ldr + en
                             : reinterpret_cast<const uint16_t *>(wq));
    }

    const uint8_t *wrow[NF], *xrow[MF];
#pragma unroll
    for (int j = 0; j < NF; ++j) wrow[j] = wq + (int64_t)min(n0 + 16 * j + r, N - 1) * ldp + 16 * g;
#pragma unroll
    for (int f = 0; f < MF; ++f) xrow[f] = xq + (int64_t)min(16 * f + r, M - 1) * ldp + 16 * g;

    v4i acc[MF][NF];
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[f][j] = v4i{0, 0, 0, 0};

    // One chunk = CH windows. compute() consumes a chunk's loaded operands; nc = live windows.
    auto compute = [&](const uint4 (&bq)[CH][NF], const uint4 (&aq)[CH][MF], int nc) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (c >= nc) continue;
            if (Q8) {
#pragma unroll
                for (int f = 0; f < MF; ++f)
#pragma unroll
                    for (int j = 0; j < NF; ++j)
                        acc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            *reinterpret_cast<const v4i *>(&aq[c][f]),
                            *reinterpret_cast<const v4i *>(&bq[c][j]), acc[f][j], 0, 0, 0);
                continue;
            }
            // all fragments widened first, then the MF * NF products of the even k before those of
            // the odd k, so no MFMA waits for the result of the one just issued
            uint4 b0[NF], b1[NF], a0[MF], a1[MF];
#pragma unroll
            for (int j = 0; j < NF; ++j) widen16(bq[c][j], b0[j], b1[j]);
#pragma unroll
            for (int f = 0; f < MF; ++f) widen16(aq[c][f], a0[f], a1[f]);
#pragma unroll
            for (int f = 0; f < MF; ++f)
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    acc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        *reinterpret_cast<v4i *>(&a0[f]), *reinterpret_cast<v4i *>(&b0[j]),
                        acc[f][j], 0, 0, 0);
#pragma unroll
            for (int f = 0; f < MF; ++f)
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    acc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        *reinterpret_cast<v4i *>(&a1[f]), *reinterpret_cast<v4i *>(&b1[j]),
                        acc[f][j], 0, 0, 0);
        }
    };
    // t counts the wave's windows; positions past its range re-read its last window (in bounds,
    // never consumed), so the prefetch loads are unconditional and the compiler can count the
    // ones still in flight.
    const int cnt = max(w_end - w_begin, 0);
    auto window = [&](int t) { return w_begin + min(t, cnt - 1); };
    auto load = [&](uint4 (&bq)[CH][NF], uint4 (&aq)[CH][MF], int t0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int kb = window(t0 + c) * 64;
#pragma unroll
            for (int j = 0; j < NF; ++j) bq[c][j] = *reinterpret_cast<const uint4 *>(wrow[j] + kb);
#pragma unroll
            for (int f = 0; f < MF; ++f) aq[c][f] = *reinterpret_cast<const uint4 *>(xrow[f] + kb);
        }
    };
    uint4 bq0[CH][NF], aq0[CH][MF];
    if (per_wave >= 2 * CH) {
        // two register sets: the next chunk's loads are in flight while this one computes
        uint4 bq1[CH][NF], aq1[CH][MF];
        if (cnt > 0) {
            load(bq0, aq0, 0);
            for (int t = 0;;) {
                // the scheduling barriers keep the next chunk's loads ahead of this chunk's work
                // (the scheduler would otherwise sink them next to their use)
                load(bq1, aq1, t + CH);
                __builtin_amdgcn_sched_barrier(0);
                compute(bq0, aq0, cnt - t);
                t += CH;
                if (t >= cnt) break;
                load(bq0, aq0, t + CH);
                __builtin_amdgcn_sched_barrier(0);
                compute(bq1, aq1, cnt - t);
                t += CH;
                if (t >= cnt) break;
            }
        }
    } else {
        for (int t = 0; t < cnt; t += CH) {
            const int nc = cnt - t;  // live windows (wave-uniform): only those are loaded
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                if (c >= nc) continue;
                const int kb = window(t + c) * 64;
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    bq0[c][j] = *reinterpret_cast<const uint4 *>(wrow[j] + kb);
#pragma unroll
                for (int f = 0; f < MF; ++f)
                    aq0[c][f] = *reinterpret_cast<const uint4 *>(xrow[f] + kb);
            }
            compute(bq0, aq0, nc);
        }
    }
    // accumulator lane layout: row 4 g + i of fragment f, column r of fragment j
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                atomicAdd(&red[(f * 16 + 4 * g + i) * LDR + j * 16 + r],
                          Q8 ? acc[f][j][i] : (acc[f][j][i] >> 8));
    __syncthreads();
    const int n = n0 + ecol;
    if (n >= N) return;
#pragma unroll
    for (int j = 0; j < ER; ++j) {
        const int m = erow + RS * j;
        if (m >= M) break;
        const int32_t v = red[m * LDR + ecol];
        if (!scaled) {
            epi.acc_out[(int64_t)m * N + n] = v;
            continue;
        }
        float y = fp32_value((float)v * e_sx[j]);
        y = fp32_value(y * e_sw);
        if (epi.mode == W4A4_EPI_GELU) y = fp32_value(gelu_erf(y));
        else if (epi.mode == W4A4_EPI_RESIDUAL) y = fp32_value(y + __half2float(__ushort_as_half(e_res[j])));
        epi.Y[(int64_t)m * epi.ldy + n] = f32_to_f16_bits(y);
    }
}

// Large-M GEMM. A BM x BN tile per workgroup of WAVES_M x WAVES_N waves, each wave a
// (BM/WAVES_M) x (BN/WAVES_N) tile of 16x16 fragments. Operands stay packed in LDS (two stages of
// 128 k: 64 bytes per row), so LDS traffic per MFMA is half that of staging int8; each wave widens
// the fragments it reads (3 VALU ops per packed dword), which overlaps with the MFMA pipe.
// Per stage and wave: FM*FN*2 v_mfma_i32_16x16x64_i8. Global loads of stage s+2 are issued right
// after the barrier of stage s and stored to LDS after the compute of stage s+1. The 16-byte chunks
// of a staged row are XOR-swizzled by row so fragment reads and staging writes spread over banks.
// Tiles are assigned so that the workgroups of one XCD (dispatch id mod 8) share weight tiles.
constexpr int BG_KS = 128;            // k per stage
constexpr int BG_ROWB = BG_KS / 2;    // packed bytes per staged row

__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ ((row >> 1) & 3)) * 16; }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm_big(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ wq, int M, int N, int K,
    int k_split, int tiles_m, int tiles_n, GemmEpilogue epi, int32_t *__restrict__ partial)
{
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int A_IT = BM * 4 / NT, B_IT = BN * 4 / NT;  // 16-byte staging items per thread
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * BG_ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * BG_ROWB];

    // XCD-aware tile order: dispatch id i runs on XCD i % 8; XCD x owns a contiguous range of the
    // n-major tile order, so tiles sharing weight columns share that XCD's L2.
    const int T = tiles_m * tiles_n;
    const int id = blockIdx.x;
    const int q = T / 8, rm = T % 8, x = id % 8;
    const int lin = x * q + min(x, rm) + id / 8;
    const int tn = lin / tiles_m, tm = lin % tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int ldp = K / 2;
    const int kb_begin = blockIdx.y * (k_split / 2);
    const int kb_end = min(kb_begin + k_split / 2, ldp);
    const int stages = (kb_end - kb_begin + BG_ROWB - 1) / BG_ROWB;

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    uint4 ra[A_IT], rb[B_IT];
    bool va[A_IT], vb[B_IT];
    auto gload = [&](int st) {
        const int kb = kb_begin + st * BG_ROWB;
#pragma unroll
        for (int t = 0; t < A_IT; ++t) {
            const int item = tid + t * NT;
            if (VEC) {
                ra[t] = load16_clamped(xq, M, m0 + (item >> 2), ldp, kb + 16 * (item & 3), kb_end, va[t]);
            } else {
                ra[t] = load_packed16<false>(xq, M, m0 + (item >> 2), ldp, kb + 16 * (item & 3), kb_end);
                va[t] = true;
            }
        }
#pragma unroll
        for (int t = 0; t < B_IT; ++t) {
            const int item = tid + t * NT;
            if (VEC) {
                rb[t] = load16_clamped(wq, N, n0 + (item >> 2), ldp, kb + 16 * (item & 3), kb_end, vb[t]);
            } else {
                rb[t] = load_packed16<false>(wq, N, n0 + (item >> 2), ldp, kb + 16 * (item & 3), kb_end);
                vb[t] = true;
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int t = 0; t < A_IT; ++t) {
            const int item = tid + t * NT, row = item >> 2;
            *reinterpret_cast<uint4 *>(&sA[buf][row * BG_ROWB + swz(row, item & 3)]) = zero_unless(ra[t], va[t]);
        }
#pragma unroll
        for (int t = 0; t < B_IT; ++t) {
            const int item = tid + t * NT, row = item >> 2;
            *reinterpret_cast<uint4 *>(&sB[buf][row * BG_ROWB + swz(row, item & 3)]) = zero_unless(rb[t], vb[t]);
        }
    };

    const int fr = lane & 15, fg = lane >> 4;
    if (stages > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    if (stages > 1) gload(1);
    for (int st = 0; st < stages; ++st) {
        const int buf = st & 1;
        v4i b0[FN], b1[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WTN + j * 16 + fr;
            const uint4 p = *reinterpret_cast<const uint4 *>(&sB[buf][row * BG_ROWB + swz(row, fg)]);
            uint4 lo, hi;
            widen16(p, lo, hi);
            b0[j] = *reinterpret_cast<v4i *>(&lo);
            b1[j] = *reinterpret_cast<v4i *>(&hi);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 16 + fr;
            const uint4 p = *reinterpret_cast<const uint4 *>(&sA[buf][row * BG_ROWB + swz(row, fg)]);
            uint4 lo, hi;
            widen16(p, lo, hi);
            const v4i a0 = *reinterpret_cast<v4i *>(&lo), a1 = *reinterpret_cast<v4i *>(&hi);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0[j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1[j], acc[i][j], 0, 0, 0);
            }
        }
        if (st + 1 < stages) lstore(buf ^ 1);
        __syncthreads();
        if (st + 2 < stages) gload(st + 2);
    }

    if (partial || epi.mode == GEMM_OUT_I32) {
        int32_t *dst = partial ? partial + (int64_t)blockIdx.y * M * N : epi.acc_out;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WTN + j * 16 + fr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * WTM + i * 16 + 4 * fg + r;
                    if (m < M && n < N) dst[(int64_t)m * N + n] = acc[i][j][r] >> 8;
                }
            }
        return;
    }
    // scales of this lane's columns and rows, loaded once
    float wsc[FN], xsc[FM][4];
#pragma unroll
    for (int j = 0; j < FN; ++j) wsc[j] = epi.w_scale[min(n0 + wn * WTN + j * 16 + fr, N - 1)];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            xsc[i][r] = epi.x_scale_per_token
                            ? epi.x_scale[min(m0 + wm * WTM + i * 16 + 4 * fg + r, M - 1)]
                            : epi.x_scale[0];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 16 + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WTM + i * 16 + 4 * fg + r;
                if (m < M && n < N) store_scaled(epi, m, n, acc[i][j][r] >> 8, xsc[i][r], wsc[j]);
            }
        }
    }
}

// Group-wise small-M GEMM (M <= 16 * MF): one 128-k rotation block per window. The 4 waves take
// the blocks of a group of 4 * SMG_G in turn (wave w: blocks c0 + 4 i + w), each leaving the exact
// int32 partial tile of its block in LDS; then every thread folds the partials of its outputs into
// fp32 in block order with one fused multiply-add per block, y = fma(float(acc_g), s_g, y), and
// the epilogue scales by the weight scale. Operands must be 16-byte aligned with K % 128 == 0.
constexpr int SMG_G = 2;  // blocks per wave per group

template <int MF>
__global__ __launch_bounds__(256) void k_gemm_smallm_g(const uint8_t *__restrict__ xq,
                                                       const uint8_t *__restrict__ wq, int M,
                                                       int N, int K, GemmEpilogue epi)
{
#pragma clang fp contract(off)
    __shared__ int32_t part[4 * SMG_G][MF * 16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int ldp = K / 2, nb = K / 128;
    const int ecol = tid & 15, erow = tid >> 4;
    const int en = min(n0 + ecol, N - 1);
    const float e_sw = epi.w_scale[en];
    const bool has_res = epi.mode == W4A4_EPI_RESIDUAL;
    uint16_t e_res[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f)  // unconditional load on a selected address (see the wide kernel)
        e_res[f] = *(has_res ? epi.residual + (int64_t)min(erow + 16 * f, M - 1) * epi.ldr + en
                             : reinterpret_cast<const uint16_t *>(wq));
    float y[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) y[f] = 0.0f;

    for (int c0 = 0; c0 < nb; c0 += 4 * SMG_G) {
        uint4 bq[SMG_G], aq[SMG_G][MF];
        bool bv[SMG_G], av[SMG_G][MF];
#pragma unroll
        for (int i = 0; i < SMG_G; ++i) {
            const int blk = c0 + 4 * i + wave;
            const int kb = min(blk, nb - 1) * 64 + 16 * g;
            bq[i] = load16_clamped(wq, N, n0 + r, ldp, kb, ldp, bv[i]);
#pragma unroll
            for (int f = 0; f < MF; ++f) aq[i][f] = load16_clamped(xq, M, f * 16 + r, ldp, kb, ldp, av[i][f]);
        }
#pragma unroll
        for (int i = 0; i < SMG_G; ++i) {
            if (c0 + 4 * i + wave >= nb) continue;
            uint4 b0, b1;
            widen16(zero_unless(bq[i], bv[i]), b0, b1);
#pragma unroll
            for (int f = 0; f < MF; ++f) {
                uint4 a0, a1;
                widen16(zero_unless(aq[i][f], av[i][f]), a0, a1);
                v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<v4i *>(&a0),
                                                                *reinterpret_cast<v4i *>(&b0),
                                                                v4i{0, 0, 0, 0}, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<v4i *>(&a1),
                                                           *reinterpret_cast<v4i *>(&b1), acc, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < 4; ++t) part[4 * i + wave][f * 16 + 4 * g + t][r] = acc[t] >> 8;
            }
        }
        __syncthreads();
        for (int j = 0; j < 4 * SMG_G && c0 + j < nb; ++j) {
            const float sg = epi.x_scale[c0 + j];
#pragma unroll
            for (int f = 0; f < MF; ++f) y[f] = fmaf((float)part[j][erow + 16 * f][ecol], sg, y[f]);
        }
        __syncthreads();
    }
    const int n = n0 + ecol;
#pragma unroll
    for (int f = 0; f < MF; ++f) {
        const int m = erow + 16 * f;
        if (m >= M || n >= N) continue;
        float t = fp32_value(y[f] * e_sw);
        if (epi.mode == W4A4_EPI_GELU) t = fp32_value(gelu_erf(t));
        else if (epi.mode == W4A4_EPI_RESIDUAL) t = fp32_value(t + __half2float(__ushort_as_half(e_res[f])));
        epi.Y[(int64_t)m * epi.ldy + n] = f32_to_f16_bits(t);
    }
}

// Pipelined variant of the large-M GEMM for K and the k split multiples of 128 with 16-byte
// aligned operands. Operand tiles go from global memory straight into a ring of NSTAGE LDS stages
// with global_load_lds_dwordx4 (no staging registers), so NSTAGE-1 stages of loads are in flight
// while one stage is multiplied. The workgroup synchronizes with a plain s_barrier after waiting
// only for the loads of the stage about to be read (s_waitcnt vmcnt), instead of the full drain a
// fenced barrier implies. Each wave instruction fills 1 KB of LDS (lane L -> bytes 16L..16L+15);
// a lane picks its global source so that the LDS image is the same XOR-swizzled layout the
// fragment reads expect. Rows past M / N are clamped to the last row: they only feed outputs that
// are never stored.
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// One wave-wide 16-byte-per-lane DMA from global memory into LDS at lds_addr + 16 * lane. Written
// as inline assembly so the compiler does not treat later LDS reads as depending on it (it would
// drain every outstanding load); the kernel orders it with explicit vmcnt waits and barriers. The
// instruction writes no VGPR; M0 carries the LDS base (with the one wait state an M0 write needs
// before an LDS DMA reads it).
__device__ __forceinline__ void dma_to_lds16(const void *gptr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}

// 4 bytes per lane from global memory into LDS at lds_addr + 4 * lane (same counter as the above)
__device__ __forceinline__ void dma_to_lds4(const void *gptr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)(const lds_u8_t *)p;
}

__device__ __forceinline__ void wait_vmcnt(int n)
{
    // s_waitcnt with lgkmcnt and expcnt at their no-wait values; n is a small compile-time count
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// s_waitcnt vmcnt(N) for a compile-time N <= 63 (the count's low four bits at 3:0, its high two
// bits at 15:14; expcnt and lgkmcnt at their no-wait values).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds six bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Epilogue kinds of the pipelined kernel (compile-time, so each variant is straight-line code).
enum { PE_NONE = W4A4_EPI_NONE, PE_GELU = W4A4_EPI_GELU, PE_RESIDUAL = W4A4_EPI_RESIDUAL,
       PE_INT32 = 3 };

// Q8: int8 operands (W8A8): a staged 64-byte row is 64 k, each fragment read is already an MFMA
// operand (one v_mfma_i32_16x16x64_i8 per fragment pair and stage, no widening) and the sums are
// not scaled by 256.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int PE, bool VEC_OUT, bool Q8,
          bool GS = false, bool RQN = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
// the fused rotate-quantize tiles run two workgroups per CU: keep their registers within two waves
// per SIMD (the up projection's GELU form otherwise takes 260 with the interleaved epilogue)
__attribute__((amdgpu_waves_per_eu(RQN ? 2 : 1))) void k_gemm_pipe(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ wq, int M, int N, int K,
    int k_split, int tiles_m, int tiles_n, int band, GemmEpilogue epi,
    int32_t *__restrict__ partial)
{
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int A_BYTES = BM * BG_ROWB, B_BYTES = BN * BG_ROWB, STAGE = A_BYTES + B_BYTES;
    // DMA instructions (1 KB chunks of 16 rows) per wave and stage. When the A tile's chunks do not
    // divide among the waves (80-row tiles), chunk q of wave w is chunk q * NW + w and the first
    // waves take one more; each wave then waits for its own count.
    constexpr int NCA = A_BYTES / 1024;
    constexpr bool AWHOLE = NCA % NW == 0;
    constexpr int QA = (NCA + NW - 1) / NW, QB = B_BYTES / 1024 / NW;
    constexpr int L = QA + QB;
    constexpr int SHIFT = Q8 ? 0 : 8;  // int4 operands enter the MFMA as 16 * code
    static_assert(NCA * 1024 == A_BYTES && QB * 1024 * NW == B_BYTES, "whole KB chunks");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, band, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int ldp = Q8 ? K : K / 2;  // bytes per operand row
    const int split_bytes = Q8 ? k_split : k_split / 2;
    const int kb_begin = blockIdx.y * split_bytes;
    const int kb_end = min(kb_begin + split_bytes, ldp);
    const int stages = (kb_end - kb_begin) / BG_ROWB;

    // per-lane DMA sources: instruction q of this wave covers staged rows achunk(q)*16 + lane/4,
    // physical chunk lane%4, which holds logical chunk (lane%4) ^ swizzle(row)
    auto achunk = [&](int q) { return AWHOLE ? wave * QA + q : q * NW + wave; };
    const int uwave_a = __builtin_amdgcn_readfirstlane(wave);
    const int qa_w = AWHOLE ? QA : (NCA - uwave_a + NW - 1) / NW;  // A chunks this wave loads
    const int lw = AWHOLE ? L : qa_w + QB;
    const uint8_t *srcA[QA];
    const uint8_t *srcB[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int row = min(achunk(q), NCA - 1) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 1) & 3);
        srcA[q] = xq + (int64_t)min(m0 + row, M - 1) * ldp + kb_begin + 16 * c;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int row = (wave * QB + q) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 1) & 3);
        srcB[q] = wq + (int64_t)min(n0 + row, N - 1) * ldp + kb_begin + 16 * c;
    }
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = lds_address(smem);
    auto issue = [&](int st) {
        const uint32_t base = lds0 + (uint32_t)((st % NSTAGE) * STAGE);
        const int koff = st * BG_ROWB;
#pragma unroll
        for (int q = 0; q < QA; ++q)
            if (AWHOLE || q < qa_w)
                dma_to_lds16(srcA[q] + koff,
                             base + (uint32_t)((AWHOLE ? uwave * QA + q : q * NW + uwave) * 1024));
#pragma unroll
        for (int q = 0; q < QB; ++q)
            dma_to_lds16(srcB[q] + koff, base + (uint32_t)(A_BYTES + (uwave * QB + q) * 1024));
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    // GS (group-wise scales): a stage is one 128-k rotation block; its exact partial is folded into
    // yf with one fused multiply-add by the block's scale (epi.x_scale[block]), in block order
    float yf[GS ? FM : 1][GS ? FN : 1][4];
    if (GS) {
#pragma unroll
        for (int i = 0; i < (GS ? FM : 1); ++i)
#pragma unroll
            for (int j = 0; j < (GS ? FN : 1); ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) yf[i][j][r] = 0.0f;
    }

#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
        if (p < stages) issue(p);

    const int fr = lane & 15, fg = lane >> 4;
    for (int st = 0; st < stages; ++st) {
        // stages st+1 .. st+NSTAGE-2 may still be in flight; stage st must have landed
        const int ahead = min(stages - 1 - st, NSTAGE - 2);
        asm volatile("" ::: "memory");
        wait_vmcnt(ahead * lw);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (st + NSTAGE - 1 < stages) issue(st + NSTAGE - 1);
        const uint8_t *sA = smem + (st % NSTAGE) * STAGE;
        const uint8_t *sB = sA + A_BYTES;
        uint4 pb[FN], pa[FM];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WTN + j * 16 + fr;
            pb[j] = *reinterpret_cast<const uint4 *>(&sB[row * BG_ROWB + swz(row, fg)]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 16 + fr;
            pa[i] = *reinterpret_cast<const uint4 *>(&sA[row * BG_ROWB + swz(row, fg)]);
        }
        if (Q8) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        *reinterpret_cast<const v4i *>(&pb[j]), *reinterpret_cast<const v4i *>(&pa[i]),
                        acc[i][j], 0, 0, 0);
            continue;
        }
        v4i b0[FN], b1[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            uint4 lo, hi;
            widen16(pb[j], lo, hi);
            b0[j] = *reinterpret_cast<v4i *>(&lo);
            b1[j] = *reinterpret_cast<v4i *>(&hi);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            uint4 lo, hi;
            widen16(pa[i], lo, hi);
            const v4i a0 = *reinterpret_cast<v4i *>(&lo), a1 = *reinterpret_cast<v4i *>(&hi);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0[j], a0, GS ? v4i{0, 0, 0, 0} : acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1[j], a1, acc[i][j], 0, 0, 0);
            }
        }
        if (GS) {
            const float sg = epi.x_scale[st];
#pragma unroll
            for (int i = 0; i < (GS ? FM : 1); ++i)
#pragma unroll
                for (int j = 0; j < (GS ? FN : 1); ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        yf[i][j][r] = fmaf((float)(acc[i][j][r] >> 8), sg, yf[i][j][r]);
        }
        // Schedule: all fragment reads first, the B widening and the first A widening, then each
        // MFMA followed by up to two VALU ops (the next A fragment's widening) so the VALU work
        // overlaps the matrix pipe instead of running between blocks of MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 12 * FN + 12, 0);
#pragma unroll
        for (int t = 0; t < FM * FN * 2; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (t < (FM - 1) * FN * 2) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
    }

    // The weight fragment is the MFMA's A operand and the activation fragment its B operand, so
    // the accumulator of fragment (i, j) holds, in lane (fr, fg), output row
    // m = m0 + wm * WTM + 16 i + fr and the four consecutive output columns
    // n = n0 + wn * WTN + 16 j + 4 fg + 0..3: each lane dequantizes and stores 8 contiguous bytes.
    const int mrow = m0 + wm * WTM + fr, ncol = n0 + wn * WTN + 4 * fg;
    if (PE == PE_INT32) {
        int32_t *dst = partial ? partial + (int64_t)blockIdx.y * M * N : epi.acc_out;
        // four consecutive columns per lane: one 16-byte store when the rows allow it
        const bool vec4 = (N % 4 == 0) && ((uintptr_t)dst % 16 == 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int m = mrow + i * 16, n = ncol + j * 16;
                if (m >= M) continue;
                if (vec4 && n + 3 < N) {
                    *reinterpret_cast<int4 *>(&dst[(int64_t)m * N + n]) =
                        make_int4(acc[i][j][0] >> SHIFT, acc[i][j][1] >> SHIFT,
                                  acc[i][j][2] >> SHIFT, acc[i][j][3] >> SHIFT);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) dst[(int64_t)m * N + n + r] = acc[i][j][r] >> SHIFT;
                }
            }
        return;
    } else if (VEC_OUT) {
#pragma clang fp contract(off)
        // Staged epilogue (Y and residual rows 16-byte aligned, N % 8 == 0, checked by the host):
        // the output tile goes through LDS so that global memory sees whole 128-byte lines. Each
        // lane's accumulator holds four consecutive columns of one row, so a direct store from
        // the fragment layout writes 16 rows x 32 bytes per instruction, a quarter line per row,
        // and the partial-line writes cost several times the bytes they carry. The ring is free
        // once every wave has passed the last stage's fragment reads.
        constexpr int TP = BN * 2 + 16;  // LDS row pitch in bytes (the pad spreads the fragment
                                         // writes of 16 rows over all banks)
        constexpr int CPR = BN / 8;      // 16-byte chunks per tile row
        constexpr int NT = NW * 64;
        const int rows_here = min(BM, M - m0), cols_here = min(BN, N - n0);
        // RQN: when this tile's 128 columns are rotation block rb of the next linear's input, the
        // finished fp16 tile is rotated and quantized here as well. The fragments of R_rb and the
        // step scale are loaded first, so their latency hides under the dequantization.
        static_assert(!RQN || (BN == 128 && 128 % (NW * 16) == 0 && !Q8 && !GS),
                      "fused rotate-quantize: 128-column int4 tiles");
        constexpr int RJF = RQN ? 128 / (NW * 16) : 1;  // 16-channel fragments of R per wave
        const bool rq_tile = RQN && n0 >= epi.rq.col0 && n0 < epi.rq.col0 + epi.rq.kn;
        const int rb = RQN ? (n0 - epi.rq.col0) / 128 : 0;
        v8h rqh[RJF][4], rql[RJF][4];
        StepScale rss{0.0f, 0.0f};
        if (RQN && rq_tile) {
            load_rot_frags<RJF, 4>(epi.rq.rhi, epi.rq.rlo, rb, wave * RJF * 16, lane, 128, rqh, rql);
            rss = step_scale(epi.rq.table, epi.rq.step);
        }
        // keep those loads here: left to itself the scheduler sinks them next to the rotation (to
        // shorten their registers' lives) and the whole L2 latency shows after the dequantization
        if (RQN) __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        if (PE == PE_RESIDUAL) {
            // every chunk is loaded from a clamped in-bounds address with no branch, all loads of a
            // thread before its LDS writes (chunks past M or N hold stand-in values, never stored)
            static_assert((BM * CPR) % NT == 0, "whole rounds of residual chunks");
            constexpr int RC = BM * CPR / NT;
            uint4 rv[RC];
#pragma unroll
            for (int t = 0; t < RC; ++t) {
                const int c = tid + t * NT, r = c / CPR, cc = c % CPR;
                rv[t] = *reinterpret_cast<const uint4 *>(
                    epi.residual + (int64_t)min(m0 + r, M - 1) * epi.ldr + min(n0 + cc * 8, N - 8));
            }
#pragma unroll
            for (int t = 0; t < RC; ++t) {
                const int c = tid + t * NT, r = c / CPR, cc = c % CPR;
                *reinterpret_cast<uint4 *>(&smem[r * TP + cc * 16]) = rv[t];
            }
            __syncthreads();
        }
        float xsc[FM];
        float wsc[FN][4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            xsc[i] = GS ? 0.0f
                        : epi.x_scale_per_token ? epi.x_scale[min(mrow + i * 16, M - 1)] : epi.x_scale[0];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = ncol + j * 16;  // N % 8 == 0: a clamped column is a whole float4
            const float4 w4 = *reinterpret_cast<const float4 *>(epi.w_scale + min(n, N - 4));
            wsc[j][0] = w4.x; wsc[j][1] = w4.y; wsc[j][2] = w4.z; wsc[j][3] = w4.w;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int rl = wm * WTM + i * 16 + fr;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int cl = wn * WTN + j * 16 + 4 * fg;
                uint2 *cell = reinterpret_cast<uint2 *>(&smem[rl * TP + cl * 2]);
                uint2 rv = make_uint2(0u, 0u);
                if (PE == PE_RESIDUAL) rv = *cell;
                const uint32_t rh[2] = {rv.x, rv.y};
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (GS) {
                        y[r] = fp32_value(yf[GS ? i : 0][GS ? j : 0][r] * wsc[j][r]);
                    } else {
                        y[r] = fp32_value((float)(acc[i][j][r] >> SHIFT) * xsc[i]);
                        y[r] = fp32_value(y[r] * wsc[j][r]);
                    }
                    if (PE == PE_GELU) y[r] = fp32_value(gelu_erf(y[r]));
                    if (PE == PE_RESIDUAL)
                        y[r] = fp32_value(y[r] + __half2float(__ushort_as_half(
                                                     (uint16_t)(rh[r >> 1] >> (16 * (r & 1))))));
                }
                *cell = make_uint2(f32x2_to_f16x2(y[0], y[1]), f32x2_to_f16x2(y[2], y[3]));
            }
        }
        __syncthreads();
        uint8_t *sq = smem + BM * TP;  // RQN: the tile's codes, 64 bytes per row
        if (RQN && rq_tile) {
            // x' = y R_rb on the fp16 tile exactly as the streaming rotate-quantize computes it:
            // lane inputs are 8 consecutive columns 8 (4 kk + fg) of row 16 mf + fr
            v4f racc[BM / 16][RJF];
            rotate_acc<BM / 16, RJF, 4>(rqh, rql, [&](int mf, int kk) {
                return *reinterpret_cast<const v8h *>(&smem[(mf * 16 + fr) * TP + 16 * (4 * kk + fg)]);
            }, racc);
            const float rs = rss.rcp * (1.0f / (1 << ROT_LO_SHIFT));
#pragma unroll
            for (int mf = 0; mf < BM / 16; ++mf)
#pragma unroll
                for (int jf = 0; jf < RJF; ++jf)
                    *reinterpret_cast<uint16_t *>(&sq[(mf * 16 + fr) * 64 + (wave * RJF * 16 + 16 * jf + 4 * fg) / 2]) =
                        (uint16_t)quant_pack4(racc[mf][jf], rs);
        }
        // the fp16 tile, unless it only feeds the next linear (its codes are written below) and the
        // caller does not need it
        const bool store_tile = !(RQN && rq_tile && !epi.rq.store_y);
        if (store_tile) {
#pragma unroll 4
            for (int c = tid; c < BM * CPR; c += NT) {
                const int r = c / CPR, cc = c % CPR;
                const uint4 v = *reinterpret_cast<const uint4 *>(&smem[r * TP + cc * 16]);
                if (r < rows_here && cc * 8 < cols_here)
                    *reinterpret_cast<uint4 *>(epi.Y + (int64_t)(m0 + r) * epi.ldy + n0 + cc * 8) = v;
            }
        }
        if (RQN && rq_tile) {
            __syncthreads();  // every wave's codes are in LDS
            const int64_t ldq = epi.rq.kn / 2;
            for (int c = tid; c < BM * 4; c += NT) {
                const int r = c >> 2, ch = c & 3;
                if (r < rows_here)
                    *reinterpret_cast<uint4 *>(epi.rq.xq + (int64_t)(m0 + r) * ldq + rb * 64 + 16 * ch) =
                        *reinterpret_cast<const uint4 *>(&sq[r * 64 + 16 * ch]);
            }
            if (m0 == 0 && rb == 0 && tid == 0) epi.rq.x_scale[0] = rss.s;
        }
    } else {
#pragma clang fp contract(off)
        // element path (rows not 16-byte aligned): each lane dequantizes and stores its four
        // columns one fp16 at a time
        float xsc[FM];
        float wsc[FN][4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            xsc[i] = GS ? 0.0f
                        : epi.x_scale_per_token ? epi.x_scale[min(mrow + i * 16, M - 1)] : epi.x_scale[0];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = ncol + j * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) wsc[j][r] = epi.w_scale[min(n + r, N - 1)];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = mrow + i * 16;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = ncol + j * 16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (n + r >= N) continue;
                    float y;
                    if (GS) {
                        y = fp32_value(yf[GS ? i : 0][GS ? j : 0][r] * wsc[j][r]);
                    } else {
                        y = fp32_value((float)(acc[i][j][r] >> SHIFT) * xsc[i]);
                        y = fp32_value(y * wsc[j][r]);
                    }
                    if (PE == PE_GELU) y = fp32_value(gelu_erf(y));
                    if (PE == PE_RESIDUAL)
                        y = fp32_value(y + __half2float(__ushort_as_half(
                                               epi.residual[(int64_t)m * epi.ldr + n + r])));
                    epi.Y[(int64_t)m * epi.ldy + n + r] = f32_to_f16_bits(y);
                }
            }
        }
    }
}

// Software-pipelined large-M GEMM for packed int4 operands (K and the k split multiples of 128,
// 16-byte aligned operands), the kernel for batches of a few thousand tokens whose grids hold about
// one tile per compute unit. Eight waves, two per SIMD: waves 0-3 and 4-7 form two k groups, and
// wave (g, c) owns columns [c BN/4, (c+1) BN/4) of the tile for the k half g of every 128-k stage
// (the low or high 8 bytes of each lane's 16-byte fragment, i.e. one of the two MFMAs a packed
// fragment pair feeds). One SIMD thus always holds a second wave whose matrix work can run while
// the first widens nibbles, reads LDS or waits. Operand stages go from global memory into an
// NS-stage LDS ring with global_load_lds_dwordx4, issued by the waves of group 0 only; a barrier
// after their load waits publishes each stage to all eight waves. A stage's fragments are read one
// iteration ahead; the steady-state loop waits with a compile-time load count; the epilogue
// operands are fetched before the loop. At the end each group hands the partial sums of the tile
// rows the other group finalizes through LDS (int32 adds are exact in any order), and each wave
// dequantizes and stores half of its fragments.
// At iteration s the ring holds stage s (already in registers), s+1 (being read) and up to NS-2
// stages in flight; the slot refilled at iteration s held stage s-1, whose fragment reads every
// wave finished before the barrier of iteration s.
template <int BM, int BN, int NS, int KS, int PE, bool VO, bool ST = false, bool RQN = false,
          bool RMAP = false>
__global__ __launch_bounds__(512) void k_gemm_sp(const uint8_t *__restrict__ xq,
                                                 const uint8_t *__restrict__ wq, int M, int N,
                                                 int K, int k_split, int tiles_m, int tiles_n,
                                                 int band,
                                                 GemmEpilogue epi, int32_t *__restrict__ partial)
{
    constexpr int NC = 4;  // column waves per k group
    constexpr int WTN = BN / NC;
    constexpr int FM = BM / 16, FN = WTN / 16;
    constexpr int FMH = FM / 2;  // fragment rows each k group finalizes
    // a ring slot holds KS sub-stages of 128 k, each [A rows x 64 B][B rows x 64 B]
    constexpr int A_BYTES = BM * BG_ROWB, B_BYTES = BN * BG_ROWB, STAGE = A_BYTES + B_BYTES;
    constexpr int SLOT = KS * STAGE;
    constexpr int QA = A_BYTES / 1024 / NC, QB = B_BYTES / 1024 / NC;  // DMA instrs per sub-stage
    constexpr int L = KS * (QA + QB);                                  // DMA instrs per slot
    constexpr int NF = FM + FN;
    constexpr bool RES_EARLY = (PE == PE_RESIDUAL) && (FMH * FN <= 16) && !RMAP;
    static_assert(QA * 1024 * NC == A_BYTES && QB * 1024 * NC == B_BYTES, "whole KB per wave");
    static_assert(NS >= 2 && FN >= 1 && FM % 2 == 0, "ring of at least two slots");
    static_assert((size_t)BM * BN * 4 <= (size_t)NS * SLOT, "partial sums fit in the ring");
    // ST (staged output): the fp16 tile goes through LDS after the exchange area, for 16-byte
    // stores of whole row segments instead of each lane's 8 bytes
    constexpr int XCH_BYTES = 2 * (BM / 32) * (BN / 64) * 4 * 64 * 16;
    constexpr int STP = BN * 2 + 16;  // staged row pitch in bytes (pad spreads the banks)
    static_assert(!ST || (VO && (size_t)XCH_BYTES + (size_t)BM * STP <= (size_t)NS * SLOT),
                  "staged tile fits in the ring after the exchange");
    // RQN: the next linear's rotate-quantize of the staged tile (a 128-column rotation block), its
    // codes staged after the tile (64 bytes per row)
    static_assert(!RQN || (ST && BN == 128 && PE != PE_INT32 &&
                           (size_t)XCH_BYTES + (size_t)BM * (STP + 64) <= (size_t)NS * SLOT),
                  "fused rotate-quantize: staged 128-column tiles");
    // RMAP (residual column map epi.res_cols): the tile's residual is gathered row by row into LDS
    // after the codes area, and the epilogue reads it from there in the fragment layout. The tile's
    // map entries and gather order sit in LDS past the ring (2 x BN ints).
    constexpr int RES_OFF = XCH_BYTES + BM * STP + (RQN ? BM * 64 : 0);
    constexpr int RPT = BM * BN / 512;  // residual elements each thread gathers
    static_assert(!RMAP || (ST && PE == PE_RESIDUAL && BN <= 512 && 512 % BN == 0 &&
                            (size_t)RES_OFF + (size_t)BM * STP <= (size_t)NS * SLOT),
                  "mapped residual: staged tiles with room for the residual tile");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, band, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wc = wave & 3, kgrp = wave >> 2;
    const int ugrp = __builtin_amdgcn_readfirstlane(kgrp);
    const int ldp = K / 2;
    const int kb_begin = blockIdx.y * (k_split / 2);
    const int kb_end = min(kb_begin + k_split / 2, ldp);
    const int stages = (kb_end - kb_begin) / (BG_ROWB * KS);  // ring slots of KS sub-stages
    const int fr = lane & 15, fg = lane >> 4;
    // this wave finalizes fragment rows i = kgrp * FMH .. kgrp * FMH + FMH - 1
    const int mrow = m0 + kgrp * FMH * 16 + fr, ncol = n0 + wc * WTN + 4 * fg;

    // epilogue operands first: their latency hides under the operand stream
    float xsc[FMH];
    float wsc[FN][4];
    uint32_t rsd[RES_EARLY ? FMH : 1][RES_EARLY ? FN : 1][2];
    if (PE != PE_INT32) {
#pragma unroll
        for (int i = 0; i < FMH; ++i)
            xsc[i] = epi.x_scale_per_token ? epi.x_scale[min(mrow + i * 16, M - 1)] : epi.x_scale[0];
        // VO (N % 4 == 0, aligned rows, checked by the host): one vector load per operand from a
        // clamped in-bounds column, with no branch, so the loads stay in flight under the main
        // loop (columns past N are computed from stand-in values and never stored)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = ncol + j * 16;
            if (VO) {
                const float4 w4 = *reinterpret_cast<const float4 *>(epi.w_scale + min(n, N - 4));
                wsc[j][0] = w4.x; wsc[j][1] = w4.y; wsc[j][2] = w4.z; wsc[j][3] = w4.w;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) wsc[j][r] = epi.w_scale[min(n + r, N - 1)];
            }
        }
        if (RES_EARLY) {
#pragma unroll
            for (int i = 0; i < (RES_EARLY ? FMH : 1); ++i)
#pragma unroll
                for (int j = 0; j < (RES_EARLY ? FN : 1); ++j) {
                    const int m = min(mrow + i * 16, M - 1), n = ncol + j * 16;
                    const uint16_t *src = epi.residual + (int64_t)m * epi.ldr;
                    if (VO) {
                        const uint2 v = *reinterpret_cast<const uint2 *>(src + min(n, N - 4));
                        rsd[i][j][0] = v.x; rsd[i][j][1] = v.y;
                    } else {
                        uint32_t e[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) e[r] = src[min(n + r, N - 1)];
                        rsd[i][j][0] = e[0] | (e[1] << 16); rsd[i][j][1] = e[2] | (e[3] << 16);
                    }
                }
        }
    }

    // RMAP: thread -> tile column rcol and rows tid / BN + r (512 / BN) of the residual gather,
    // issued in the last main-loop iteration under that iteration's matrix work. rcol is the
    // tile's gather order at tid % BN (the identity without epi.res_order): lanes that gather
    // adjacent source columns share cache lines. Columns and map entries are clamped into range.
    int rcol = tid % BN;
    const int rrow0 = tid / BN;
    uint16_t rgv[RMAP ? RPT : 1];

    const uint8_t *srcA[QA];
    const uint8_t *srcB[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int row = (wc * QA + q) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 1) & 3);
        srcA[q] = xq + (int64_t)min(m0 + row, M - 1) * ldp + kb_begin + 16 * c;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int row = (wc * QB + q) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 1) & 3);
        srcB[q] = wq + (int64_t)min(n0 + row, N - 1) * ldp + kb_begin + 16 * c;
    }
    const int uwc = __builtin_amdgcn_readfirstlane(wc);
    const uint32_t lds0 = lds_address(smem);
    if (RMAP && __builtin_amdgcn_readfirstlane(wave) == 0) {
        // the tile's map entries and gather order into LDS past the ring, loaded by wave 0 ahead of
        // its first stages (so the first stage's wait and barrier cover them); columns past N
        // repeat column N - 1
#pragma unroll
        for (int q = 0; q < BN / 64; ++q) {
            const int n = min(n0 + q * 64 + lane, N - 1);
            dma_to_lds4(epi.res_cols + n, lds0 + (uint32_t)(NS * SLOT + q * 256));
            if (epi.res_order)
                dma_to_lds4(epi.res_order + n, lds0 + (uint32_t)(NS * SLOT + BN * 4 + q * 256));
        }
    }
    auto issue = [&](int st) {
        if (ugrp != 0) return;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t base = lds0 + (uint32_t)((st % NS) * SLOT + ks * STAGE);
            const int koff = (st * KS + ks) * BG_ROWB;
#pragma unroll
            for (int q = 0; q < QA; ++q)
                dma_to_lds16(srcA[q] + koff, base + (uint32_t)((uwc * QA + q) * 1024));
#pragma unroll
            for (int q = 0; q < QB; ++q)
                dma_to_lds16(srcB[q] + koff, base + (uint32_t)(A_BYTES + (uwc * QB + q) * 1024));
        }
    };
    // this group's 8 bytes of each fragment: A rows 16 i + fr (all tile rows), B rows of this
    // wave's columns
    const int half = 8 * kgrp;
    auto read_frags = [&](int st, uint2 (&F)[KS][NF]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint8_t *sA = smem + (st % NS) * SLOT + ks * STAGE;
            const uint8_t *sB = sA + A_BYTES;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wc * WTN + j * 16 + fr;
                F[ks][FM + j] =
                    *reinterpret_cast<const uint2 *>(&sB[row * BG_ROWB + swz(row, fg) + half]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = i * 16 + fr;
                F[ks][i] = *reinterpret_cast<const uint2 *>(&sA[row * BG_ROWB + swz(row, fg) + half]);
            }
        }
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    // 8 packed bytes -> the 16 int8 operand bytes 16 * code (the order widen16 gives either half)
    auto widen8 = [](const uint2 &p) {
        return v4i{(int)((p.x << 4) & 0xF0F0F0F0u), (int)(p.x & 0xF0F0F0F0u),
                   (int)((p.y << 4) & 0xF0F0F0F0u), (int)(p.y & 0xF0F0F0F0u)};
    };
    auto compute = [&](const uint2 (&F)[KS][NF]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            v4i b[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) b[j] = widen8(F[ks][FM + j]);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v4i a = widen8(F[ks][i]);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[j], a, acc[i][j], 0, 0, 0);
            }
        }
    };
    // Iteration s: wait until slot s has landed (with every slot up to s+NS-2 issued, exactly
    // NS-2 younger slots may stay in flight; near the end it waits for everything), barrier (slot s
    // is visible to all waves, and every wave has finished reading slot s-1), refill slot s-1's
    // place with slot s+NS-1, then read slot s's fragments and compute.
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < stages) issue(p);
    uint2 F[KS][NF];
    for (int s = 0; s < stages; ++s) {
        asm volatile("" ::: "memory");
        if (s + NS - 2 <= stages - 1 && ugrp == 0) wait_vm<(NS - 2) * L>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + NS - 1 < stages) issue(s + NS - 1);
        if (RMAP && s == stages - 1) {
            const int *sig = reinterpret_cast<const int *>(smem + NS * SLOT);
            if (epi.res_order) rcol = min(max(sig[BN + tid % BN] - n0, 0), BN - 1);
            const int rsrc = min(max(sig[rcol], 0), N - 1);
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int m = min(m0 + rrow0 + r * (512 / BN), M - 1);
                rgv[r] = epi.residual[(int64_t)m * epi.ldr + rsrc];
            }
        }
        read_frags(s, F);
        compute(F);
    }

    // RQN: when this tile's 128 columns are rotation block rb of the next linear's input, each
    // wave rotates 16 of its channels once the fp16 tile is staged. The R_rb fragments and the
    // step scale are loaded here, so their latency hides under the exchange and the dequantization.
    const bool rq_tile = RQN && n0 >= epi.rq.col0 && n0 < epi.rq.col0 + epi.rq.kn;
    const int rb = RQN ? (n0 - epi.rq.col0) / 128 : 0;
    v8h rqh[1][4], rql[1][4];
    StepScale rss{0.0f, 0.0f};
    if (RQN && rq_tile) {
        load_rot_frags<1, 4>(epi.rq.rhi, epi.rq.rlo, rb, wave * 16, lane, 128, rqh, rql);
        rss = step_scale(epi.rq.table, epi.rq.step);
    }
    if (RQN) __builtin_amdgcn_sched_barrier(0);

    // Exchange the k groups' partial sums through LDS: group g keeps fragment rows i in its half
    // and sends the other half. Slot layout: [sender group][fragment row in half][FN][column wave]
    // x 64 lanes x 16 bytes. The group index is made a compile-time constant (one copy of the
    // epilogue per group) so that the accumulators stay in registers.
    __syncthreads();  // every wave is past its last fragment read
    if (RMAP) {
        // the gathered residual tile, row pitch STP like the staged output; read after the
        // exchange barrier inside finish
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *reinterpret_cast<uint16_t *>(smem + RES_OFF + (rrow0 + r * (512 / BN)) * STP + 2 * rcol) =
                rgv[r];
    }
    auto finish = [&](auto G) {
        constexpr int g = decltype(G)::value, other = 1 - g;
        int4 *xch = reinterpret_cast<int4 *>(smem);
#pragma unroll
        for (int ih = 0; ih < FMH; ++ih)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int slot = ((g * FMH + ih) * FN + j) * NC + wc;
                const v4i v = acc[other * FMH + ih][j];
                xch[slot * 64 + lane] = make_int4(v[0], v[1], v[2], v[3]);
            }
        __syncthreads();
#pragma unroll
        for (int ih = 0; ih < FMH; ++ih)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int slot = ((other * FMH + ih) * FN + j) * NC + wc;
                const int4 v = xch[slot * 64 + lane];
                v4i &a = acc[g * FMH + ih][j];
                a[0] += v.x; a[1] += v.y; a[2] += v.z; a[3] += v.w;
            }
        if (PE == PE_INT32) {
            int32_t *dst = partial ? partial + (int64_t)blockIdx.y * M * N : epi.acc_out;
            const bool vec4 = (N % 4 == 0) && ((uintptr_t)dst % 16 == 0);
#pragma unroll
            for (int ih = 0; ih < FMH; ++ih)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const v4i &a = acc[g * FMH + ih][j];
                    const int m = mrow + ih * 16, n = ncol + j * 16;
                    if (m >= M) continue;
                    if (vec4 && n + 3 < N) {
                        *reinterpret_cast<int4 *>(&dst[(int64_t)m * N + n]) =
                            make_int4(a[0] >> 8, a[1] >> 8, a[2] >> 8, a[3] >> 8);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N) dst[(int64_t)m * N + n + r] = a[r] >> 8;
                    }
                }
            return;
        }
        {
#pragma clang fp contract(off)
#pragma unroll
        for (int ih = 0; ih < FMH; ++ih) {
            const int m = mrow + ih * 16;
            uint32_t rl[FN][2];
            if (PE == PE_RESIDUAL) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (RES_EARLY) {
                        rl[j][0] = rsd[RES_EARLY ? ih : 0][RES_EARLY ? j : 0][0];
                        rl[j][1] = rsd[RES_EARLY ? ih : 0][RES_EARLY ? j : 0][1];
                        continue;
                    }
                    if (RMAP) {
                        const int rloc = (g * FMH + ih) * 16 + fr, cloc = wc * WTN + j * 16 + 4 * fg;
                        const uint2 v = *reinterpret_cast<const uint2 *>(smem + RES_OFF + rloc * STP +
                                                                         2 * cloc);
                        rl[j][0] = v.x; rl[j][1] = v.y;
                        continue;
                    }
                    const int n = ncol + j * 16;
                    const uint16_t *src = epi.residual + (int64_t)min(m, M - 1) * epi.ldr;
                    if (VO) {
                        const uint2 v = *reinterpret_cast<const uint2 *>(src + min(n, N - 4));
                        rl[j][0] = v.x; rl[j][1] = v.y;
                    } else {
                        uint32_t e[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) e[r] = src[min(n + r, N - 1)];
                        rl[j][0] = e[0] | (e[1] << 16); rl[j][1] = e[2] | (e[3] << 16);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const v4i &a = acc[g * FMH + ih][j];
                const int n = ncol + j * 16;
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    y[r] = fp32_value((float)(a[r] >> 8) * xsc[ih]);
                    y[r] = fp32_value(y[r] * wsc[j][r]);
                    if (PE == PE_GELU) y[r] = fp32_value(gelu_erf(y[r]));
                    if (PE == PE_RESIDUAL) {
                        const uint32_t hv = rl[j][r >> 1] >> (16 * (r & 1));
                        y[r] = fp32_value(y[r] + __half2float(__ushort_as_half((uint16_t)hv)));
                    }
                }
                if (ST) {
                    const int rl = (g * FMH + ih) * 16 + fr, cl = wc * WTN + j * 16 + 4 * fg;
                    *reinterpret_cast<uint2 *>(smem + XCH_BYTES + rl * STP + cl * 2) =
                        make_uint2(f32x2_to_f16x2(y[0], y[1]), f32x2_to_f16x2(y[2], y[3]));
                    continue;
                }
                if (m >= M) continue;
                uint16_t *dst = epi.Y + (int64_t)m * epi.ldy + n;
                if (VO) {
                    if (n >= N) continue;
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(f32x2_to_f16x2(y[0], y[1]),
                                                                 f32x2_to_f16x2(y[2], y[3]));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) dst[r] = f32_to_f16_bits(y[r]);
                }
            }
        }
        }
    };
    if (ugrp == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, 1>{});
    if constexpr (ST && PE != PE_INT32) {
        __syncthreads();  // every wave's part of the tile is in LDS
        constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
        const int rows_here = min(BM, M - m0), cols_here = min(BN, N - n0);
        uint8_t *sq = smem + XCH_BYTES + BM * STP;  // RQN: the tile's codes
        if (RQN && rq_tile) {
            // x' = y R_rb on the staged fp16 tile with the streaming rotate-quantize's arithmetic
            // and order: lane inputs are 8 consecutive columns 8 (4 kk + fg) of row 16 mf + fr
            v4f racc[BM / 16][1];
            rotate_acc<BM / 16, 1, 4>(rqh, rql, [&](int mf, int kk) {
                return *reinterpret_cast<const v8h *>(smem + XCH_BYTES + (mf * 16 + fr) * STP +
                                                      16 * (4 * kk + fg));
            }, racc);
            const float rs = rss.rcp * (1.0f / (1 << ROT_LO_SHIFT));
#pragma unroll
            for (int mf = 0; mf < BM / 16; ++mf)
                *reinterpret_cast<uint16_t *>(&sq[(mf * 16 + fr) * 64 + (wave * 16 + 4 * fg) / 2]) =
                    (uint16_t)quant_pack4(racc[mf][0], rs);
        }
        // the fp16 tile, unless it only feeds the next linear and the caller does not need it
        const bool store_tile = !(RQN && rq_tile && !epi.rq.store_y);
        if (store_tile) {
#pragma unroll 2
            for (int c = tid; c < BM * CPR; c += 512) {
                const int r = c / CPR, cc = c % CPR;
                const uint4 v = *reinterpret_cast<const uint4 *>(smem + XCH_BYTES + r * STP + cc * 16);
                if (r < rows_here && cc * 8 < cols_here)
                    *reinterpret_cast<uint4 *>(epi.Y + (int64_t)(m0 + r) * epi.ldy + n0 + cc * 8) = v;
            }
        }
        if (RQN && rq_tile) {
            __syncthreads();  // every wave's codes are in LDS
            const int64_t ldq = epi.rq.kn / 2;
            for (int c = tid; c < BM * 4; c += 512) {
                const int r = c >> 2, ch = c & 3;
                if (r < rows_here)
                    *reinterpret_cast<uint4 *>(epi.rq.xq + (int64_t)(m0 + r) * ldq + rb * 64 + 16 * ch) =
                        *reinterpret_cast<const uint4 *>(&sq[r * 64 + 16 * ch]);
            }
            if (m0 == 0 && rb == 0 && tid == 0) epi.rq.x_scale[0] = rss.s;
        }
    }
}

// Split-K reduction of exact int32 partials, then the same epilogue.
__global__ void k_splitk_epilogue(const int32_t *__restrict__ partial, int splits, int M, int N,
                                  GemmEpilogue epi)
{
#pragma clang fp contract(off)
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)M * N) return;
    const int m = (int)(idx / N), n = (int)(idx % N);
    int32_t v = 0;
    for (int s = 0; s < splits; ++s) v += partial[(int64_t)s * M * N + idx];
    store_output(epi, m, n, N, v);
}

// Same reduction four columns at a time (N % 4 == 0, 16-byte aligned partials, and 8-byte fp16
// rows / 16-byte weight scales, checked by the host): vector loads of the partials and the
// epilogue operands, one 8-byte store per thread.
__global__ void k_splitk_epilogue4(const int32_t *__restrict__ partial, int splits, int M, int N,
                                   GemmEpilogue epi)
{
#pragma clang fp contract(off)
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t MN = (int64_t)M * N;
    if (g >= MN / 4) return;
    const int64_t idx = g * 4;
    const int m = (int)(idx / N), n = (int)(idx % N);
    int4 v = *reinterpret_cast<const int4 *>(partial + idx);
    for (int sp = 1; sp < splits; ++sp) {
        const int4 t = *reinterpret_cast<const int4 *>(partial + sp * MN + idx);
        v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
    }
    if (epi.mode == GEMM_OUT_I32) {
        *reinterpret_cast<int4 *>(epi.acc_out + idx) = v;
        return;
    }
    const float sx = epi.x_scale_per_token ? epi.x_scale[m] : epi.x_scale[0];
    const float4 w4 = *reinterpret_cast<const float4 *>(epi.w_scale + n);
    const int32_t a[4] = {v.x, v.y, v.z, v.w};
    const float ws[4] = {w4.x, w4.y, w4.z, w4.w};
    uint32_t rh[2] = {0u, 0u};
    if (epi.mode == W4A4_EPI_RESIDUAL) {
        const uint2 r = *reinterpret_cast<const uint2 *>(epi.residual + (int64_t)m * epi.ldr + n);
        rh[0] = r.x; rh[1] = r.y;
    }
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        y[r] = fp32_value((float)a[r] * sx);
        y[r] = fp32_value(y[r] * ws[r]);
        if (epi.mode == W4A4_EPI_GELU) y[r] = fp32_value(gelu_erf(y[r]));
        else if (epi.mode == W4A4_EPI_RESIDUAL)
            y[r] = fp32_value(y[r] + __half2float(__ushort_as_half((uint16_t)(rh[r >> 1] >> (16 * (r & 1))))));
    }
    *reinterpret_cast<uint2 *>(epi.Y + (int64_t)m * epi.ldy + n) =
        make_uint2(f32x2_to_f16x2(y[0], y[1]), f32x2_to_f16x2(y[2], y[3]));
}

// ------------------------------------------------------------------ FP6 matrix-core operands
//
// The OCP E3M2 six-bit float (the "bf6" operand format of v_mfma_scale_f32_16x16x128_f8f6f4) holds
// every integer in [-8, 7] exactly, and the FP6 matrix instructions run at twice the int8 rate with
// no widening work. Products of two codes are exact integers and so is every partial sum of them
// below 2^24 in the fp32 accumulator (|sum| <= 64 K with K <= 2^18), so the accumulator holds the
// same integer as the int32 path and the epilogue gives the same bits.
//
// Operand layout of a [rows][K] code matrix (K % 128 == 0, R2 = rows rounded up to even, the pad
// row all zeros): per 128-k stage, four groups of 32 consecutive k, each group's codes as 6-bit
// fields (code i at bits 6i..6i+5 of a 192-bit little-endian string) -- the lane image of one MFMA
// operand fragment. Stage s is one block of R2 * 96 bytes at s * R2 * 96: the first 16 bytes of
// each group ("head") at row * 64 + 16 * group, then the last 8 bytes ("tail") at R2 * 64 +
// (group * R2 + row) * 8. A tile's stage is thus a few contiguous runs (whole cache lines for the
// loads into LDS). Heads are staged in LDS like packed int4 rows (XOR-swizzled 64-byte rows) and
// read with one 16-byte access; tails are staged group-major, so the 16 lanes reading one group's
// tails touch 128 contiguous bytes: one conflict-free 8-byte access.
constexpr int F6_KS = 128;         // k per stage
constexpr int F6_MAX_K = 1 << 18;  // 64 * 2^18 = 2^24: every partial sum is exact in fp32

__host__ __device__ inline int f6_rows2(int rows) { return (rows + 1) & ~1; }

// One thread per (32-k group, row, 128-k stage), groups fastest: the four threads of a row read
// its 64 packed bytes of the stage and write its 64 head bytes (consecutive rows are contiguous
// in the stage block), each also one 8-byte tail (consecutive rows of a group are contiguous);
// zeros for the pad row.
__global__ __launch_bounds__(256) void k_codes_to_f6(const uint8_t *__restrict__ q, int rows, int K,
                                                     uint8_t *__restrict__ out)
{
    const int R2 = f6_rows2(rows);
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)R2 * (K / 32)) return;
    const int g = (int)(t & 3);
    const int row = (int)((t >> 2) % R2);
    const int st = (int)((t >> 2) / R2);
    uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    if (row < rows)
        f6_encode_group(*reinterpret_cast<const uint4 *>(q + (int64_t)row * (K / 2) + 64 * st + 16 * g), w);
    uint8_t *blk = out + (int64_t)st * R2 * 96;
    *reinterpret_cast<uint4 *>(blk + (int64_t)row * 64 + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2 *>(blk + (int64_t)R2 * 64 + ((int64_t)g * R2 + row) * 8) =
        make_uint2(w[4], w[5]);
}

int launch_codes_to_f6(const uint8_t *q, int rows, int K, uint8_t *out, hipStream_t s)
{
    const int64_t threads = (int64_t)f6_rows2(rows) * (K / 32);
    if (threads == 0) return W4A4_OK;
    hipLaunchKernelGGL(k_codes_to_f6, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, q,
                       rows, K, out);
    return check_launch("codes to fp6");
}

typedef int v8i __attribute__((ext_vector_type(8)));

// Pipelined FP6 GEMM: the int4 pipelined kernel's structure (LDS ring of NSTAGE stages filled by
// global_load_lds_dwordx4, vmcnt waits + plain barriers, XCD-aware tile order), one
// v_mfma_scale_f32_16x16x128_f8f6f4 per fragment pair and stage with unit E8M0 scales (127), both
// operands bf6 (format 3). xf / wf are FP6 operands of M / N rows; LDS stage image: A heads
// [BM][64] swizzled, A tails [4][BM][8], B heads [BN][64], B tails [4][BN][8].
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int PE, bool VEC_OUT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm_f6(
    const uint8_t *__restrict__ xf, const uint8_t *__restrict__ wf, int M, int N, int K,
    int k_split, int tiles_m, int tiles_n, int band, GemmEpilogue epi,
    int32_t *__restrict__ partial)
{
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int AH = BM * 64, AT = BM * 32, BH = BN * 64, BT = BN * 32;
    constexpr int STAGE = AH + AT + BH + BT;
    constexpr int NI = STAGE / 1024;  // 1 KB DMA instructions per stage
    constexpr int Q = NI / NW;        // ... per wave
    constexpr int IAH = BM / 16, IAT = BM / 32, IBH = BN / 16;  // instruction ranges
    static_assert(BM % 128 == 0 && BN % 128 == 0, "whole-KB tail instructions");
    static_assert(Q * NW == NI, "whole DMA instructions per wave");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, band, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int R2x = f6_rows2(M), R2w = f6_rows2(N);
    const int st_split = k_split / F6_KS;
    const int st_begin = blockIdx.y * st_split;
    const int stages = min(st_split, K / F6_KS - st_begin);

    // per-lane DMA source of each of this wave's instructions at stage 0 of the split, and the
    // byte step from one stage to the next (one stage block of the operand)
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t *src[Q];
    int64_t sstep[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int ii = uwave * Q + q;
        const bool is_a = ii < IAH + IAT;
        const int i2 = is_a ? ii : ii - IAH - IAT;
        const int nh = is_a ? IAH : IBH;
        const int r0 = is_a ? m0 : n0, rows = is_a ? M : N, R2 = is_a ? R2x : R2w;
        const int bm = is_a ? BM : BN;
        const uint8_t *blk = (is_a ? xf : wf) + (int64_t)st_begin * R2 * 96;
        sstep[q] = (int64_t)R2 * 96;
        if (i2 < nh) {
            const int row = i2 * 16 + (lane >> 2);
            const int c = (lane & 3) ^ ((row >> 1) & 3);
            src[q] = blk + (int64_t)min(r0 + row, rows - 1) * 64 + 16 * c;
        } else {
            const int t = i2 - nh, g = t / (bm / 128), part = t % (bm / 128);
            const int row = min(r0 + part * 128 + 2 * lane, R2 - 2);
            src[q] = blk + (int64_t)R2 * 64 + ((int64_t)g * R2 + row) * 8;
        }
    }
    const uint32_t lds0 = lds_address(smem);
    auto issue = [&](int st) {
        const uint32_t base = lds0 + (uint32_t)((st % NSTAGE) * STAGE);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            dma_to_lds16(src[q] + st * sstep[q], base + (uint32_t)((uwave * Q + q) * 1024));
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
        if (p < stages) issue(p);

    const int fr = lane & 15, fg = lane >> 4;
    for (int st = 0; st < stages; ++st) {
        const int ahead = min(stages - 1 - st, NSTAGE - 2);
        asm volatile("" ::: "memory");
        // wait until at most `ahead` stages of loads are in flight (a smaller count where the ring
        // cannot hold that many: only ever a longer wait)
        if (ahead <= 0) wait_vm<0>();
        else if (ahead == 1) wait_vm<Q>();
        else if (ahead == 2) wait_vm<(NSTAGE > 3 ? 2 * Q : 0)>();
        else if (ahead == 3) wait_vm<(NSTAGE > 4 ? 3 * Q : 0)>();
        else wait_vm<(NSTAGE > 5 ? 4 * Q : 0)>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (st + NSTAGE - 1 < stages) issue(st + NSTAGE - 1);
        const uint8_t *sA = smem + (st % NSTAGE) * STAGE;
        const uint8_t *sAt = sA + AH, *sB = sA + AH + AT, *sBt = sB + BH;
        v8i fb[FN], fa[FM];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WTN + j * 16 + fr;
            const uint4 h = *reinterpret_cast<const uint4 *>(&sB[row * 64 + swz(row, fg)]);
            const uint2 t = *reinterpret_cast<const uint2 *>(&sBt[(fg * BN + row) * 8]);
            fb[j] = v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)t.x, (int)t.y, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 16 + fr;
            const uint4 h = *reinterpret_cast<const uint4 *>(&sA[row * 64 + swz(row, fg)]);
            const uint2 t = *reinterpret_cast<const uint2 *>(&sAt[(fg * BM + row) * 8]);
            fa[i] = v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)t.x, (int)t.y, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[j], fa[i], acc[i][j], 3, 3,
                                                                             0, 127, 0, 127);
        // every fragment read of the stage first, then the MFMAs: one LDS latency per stage
        // instead of one per activation fragment
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FM + FN), 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * (FM + FN), 0);  // tail register moves
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);        // MFMA
    }

    // lane (fr, fg) of fragment (i, j): output row m0 + wm * WTM + 16 i + fr, columns
    // n0 + wn * WTN + 16 j + 4 fg + 0..3 (the weight fragment is the MFMA's A operand)
    const int mrow = m0 + wm * WTM + fr, ncol = n0 + wn * WTN + 4 * fg;
    if (PE == PE_INT32) {
        int32_t *dst = partial ? partial + (int64_t)blockIdx.y * M * N : epi.acc_out;
        const bool vec4 = (N % 4 == 0) && ((uintptr_t)dst % 16 == 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int m = mrow + i * 16, n = ncol + j * 16;
                if (m >= M) continue;
                int v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = (int)acc[i][j][r];
                if (vec4 && n + 3 < N) {
                    *reinterpret_cast<int4 *>(&dst[(int64_t)m * N + n]) = make_int4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) dst[(int64_t)m * N + n + r] = v[r];
                }
            }
        return;
    } else {
#pragma clang fp contract(off)
        float xsc[FM];
        float wsc[FN][4];
        uint32_t rsd[FM][FN][2];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            xsc[i] = epi.x_scale_per_token ? epi.x_scale[min(mrow + i * 16, M - 1)] : epi.x_scale[0];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = ncol + j * 16;
            if (VEC_OUT && n + 3 < N) {
                const float4 w4 = *reinterpret_cast<const float4 *>(epi.w_scale + n);
                wsc[j][0] = w4.x; wsc[j][1] = w4.y; wsc[j][2] = w4.z; wsc[j][3] = w4.w;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) wsc[j][r] = epi.w_scale[min(n + r, N - 1)];
            }
        }
        auto residual4 = [&](int m, int n, uint32_t (&h)[2]) {
            const uint16_t *rs = epi.residual + (int64_t)min(m, M - 1) * epi.ldr;
            if (VEC_OUT && n + 3 < N) {
                const uint2 v = *reinterpret_cast<const uint2 *>(rs + n);
                h[0] = v.x; h[1] = v.y;
            } else {
                uint32_t e[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = rs[min(n + r, N - 1)];
                h[0] = e[0] | (e[1] << 16); h[1] = e[2] | (e[3] << 16);
            }
        };
        if (PE == PE_RESIDUAL && VEC_OUT) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) residual4(mrow + i * 16, ncol + j * 16, rsd[i][j]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = mrow + i * 16;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = ncol + j * 16;
                float y[4];
                if (PE == PE_RESIDUAL && !VEC_OUT) residual4(m, n, rsd[i][j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // the accumulator is an exact integer: (float)(int) of it is itself
                    y[r] = fp32_value(acc[i][j][r] * xsc[i]);
                    y[r] = fp32_value(y[r] * wsc[j][r]);
                    if (PE == PE_GELU) y[r] = fp32_value(gelu_erf(y[r]));
                    if (PE == PE_RESIDUAL) {
                        const uint32_t hv = rsd[i][j][r >> 1] >> (16 * (r & 1));
                        y[r] = fp32_value(y[r] + __half2float(__ushort_as_half((uint16_t)hv)));
                    }
                }
                if (m >= M) continue;
                uint16_t *dst = epi.Y + (int64_t)m * epi.ldy + n;
                if (VEC_OUT && n + 3 < N) {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(f32x2_to_f16x2(y[0], y[1]),
                                                                 f32x2_to_f16x2(y[2], y[3]));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) dst[r] = f32_to_f16_bits(y[r]);
                }
            }
        }
    }
}

struct GemmPlan {
    // 0 small-M; 1 = 256x256, 2 = 128x256, 3 = 128x128, 4 = 64x128, 5 = 80x128 (k_gemm_pipe /
    // k_gemm_big);
    // SP_* (k_gemm_sp, packed int4 with K % 128 == 0 and aligned operands)
    int kind;
    int bm, bn, splits, k_split;
};

// Pick the tile shape and k split with the smallest estimated time: full rounds of 256 compute
// units (one workgroup per unit) times the per-tile time, plus the write and read of split-K
// partials. kg is the k granularity of a stage (128 for packed int4, 64 for int8 operands); sp
// allows the software-pipelined kernel, whose per-stage times were measured on MI355X.
static GemmPlan plan_gemm(int M, int N, int K, int kg, bool pipe, bool sp = false,
                          bool gelu = false, bool bn128_pipe = false)
{
    GemmPlan best{0, 0, 16, 1, K};
    if (M <= SMALL_M) return best;
    // Per tile kind, times measured on MI355X (microseconds; tile sweeps over the 1600-token stack
    // linears and the prefill and long-K projections):
    //   f     launch, first operand loads and epilogue of one workgroup
    //   s     one 128-k stage of one workgroup alone on its CU
    //   beta  slowdown of each stage per extra workgroup sharing the CU (occ > 1: co-resident
    //         workgroups overlap one another's loads, epilogues and matrix work)
    //   e     each further round of workgroups on a CU
    //   occ   workgroups one CU holds at once (LDS and registers)
    //   gran  k granularity of the ring (a k split is a whole number of it)
    // (The 80-row tile takes the 64-row tile's f and beta and s scaled by its area; on the stack's
    // QKV projection this predicts 11.6 us against 11.5 us measured.)
    // Per CU: w = ceil(tiles * splits / 256) workgroups, co = min(w, occ) of them at once:
    //   t = f + stages * s * (1 + beta (co - 1)) * w / co + (ceil(w / occ) - 1) e
    // plus, for the GELU epilogue, its VALU time per output a thread owns (exposed once per
    // workgroup when it runs alone on its CU, co times when co workgroups finish together), and
    // for a K split the int32 partials written and read back plus the reduction launch.
    struct Cand { int kind, bm, bn, threads, occ; double f, s, beta, e; int gran; };
    const Cand cands[] = {{1, 256, 256, 512, 1, 3.7, 1.79, 0.0, 3.0, kg},
                          {2, 128, 256, 512, 1, 6.0, 1.01, 0.0, 3.0, kg},
                          {3, 128, 128, 256, 2, 4.6, 0.61, 0.68, 3.0, kg},
                          {4, 64, 128, 256, 3, 3.9, 0.49, 0.57, 3.0, kg},
                          {5, 80, 128, 256, 3, 3.9, 0.61, 0.57, 3.0, kg},
                          {SP_128x128, 128, 128, 512, 1, 6.96, 0.58, 0.0, 2.95, 256},
                          {SP_64x128, 64, 128, 512, 1, 5.3, 0.2875, 0.0, 3.05, 512}};
    const int ncand = sp ? 7 : 5;
    double best_t = 1e30;
    for (int ci = 0; ci < ncand; ++ci) {
        const Cand &c = cands[ci];
        if ((c.kind == 4 || c.kind == 5) && !pipe) continue;
        // the fused rotate-quantize tiles: 128 columns, pipelined or split-group
        if (bn128_pipe && c.kind != 3 && c.kind != 4 && c.kind != 5 && c.kind != SP_64x128)
            continue;
        if (c.kind >= SP_128x128 && K % c.gran) continue;  // whole ring slots only
        const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        // up to 256 splits: K <= 2^24 then always fits pieces of at most MAX_K_SPLIT k, the most
        // one int32 accumulator of the tile kernels holds
        for (int splits = 1; splits <= 256; splits *= 2) {
            if ((c.kind == 4 || c.kind == 5) && splits > 1) continue;
            int k_split = ((K + splits - 1) / splits + c.gran - 1) / c.gran * c.gran;
            if (k_split > MAX_K_SPLIT) continue;
            const int real_splits = (K + k_split - 1) / k_split;
            if (real_splits != splits) continue;
            if (splits > 1 && k_split < 1024) continue;
            const double stages = k_split / (double)BG_KS;
            const double w = std::ceil(tiles * splits / 256.0);
            const double co = std::min(w, (double)c.occ);
            double t = c.f + stages * c.s * (1.0 + c.beta * (co - 1.0)) * w / co +
                       (std::ceil(w / c.occ) - 1.0) * c.e;
            if (gelu) {
                const double per_thread = (double)c.bm * c.bn / c.threads;
                t += c.occ == 1 ? 0.065 * per_thread
                                : 0.031 * per_thread * (w <= c.occ ? co : 1.0);
            }
            if (splits > 1)
                t += (2.0 * splits * M * (double)N * 4 + M * (double)N * 2) / 5e12 * 1e6 + 2.0;
            if (t < best_t * 0.98) {
                best_t = t;
                best = GemmPlan{c.kind, c.bm, c.bn, splits, k_split};
            }
        }
    }
    return best;
}

size_t gemm_workspace(int M, int N, int K, bool q8)
{
    // the launch plans with or without the pipelined kernel (operand alignment decides): enough
    // for either
    size_t need = 0;
    for (int pipe = 0; pipe < 3; ++pipe)
        for (int gelu = 0; gelu < 2; ++gelu) {
            GemmPlan p = plan_gemm(M, N, K, q8 ? BG_ROWB : BG_KS, pipe != 0, pipe == 2 && !q8,
                                   gelu != 0);
            if (p.splits > 1)
                need = std::max(need, (size_t)p.splits * (size_t)M * (size_t)N * sizeof(int32_t));
        }
    return need;
}

template <int BM, int BN, int WM, int WN>
static void launch_big(bool vec, dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq,
                       int M, int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                       int32_t *partial)
{
    const dim3 block(64 * WM * WN);
    if (vec)
        hipLaunchKernelGGL((k_gemm_big<BM, BN, WM, WN, true>), grid, block, 0, s, xq, wq, M, N, K,
                           k_split, tm, tn, epi, partial);
    else
        hipLaunchKernelGGL((k_gemm_big<BM, BN, WM, WN, false>), grid, block, 0, s, xq, wq, M, N,
                           K, k_split, tm, tn, epi, partial);
}

// Operand stages in the pipelined kernel's LDS ring. Three measured faster than four on the
// 1600-token shapes (1600x3072x1024 GEMM 10.6 -> 10.3 us; mixed W4A4/W8A8 stack 11.04 -> 10.93 ms
// per pass) and two slower on the int8-operand ones; the 256x256 tile takes two (see launch_pipe).
constexpr int PIPE_STAGES = 3;

template <int BM, int BN, int WM, int WN, int PE, bool VO, bool Q8, bool GS = false,
          bool RQN = false, int NS = PIPE_STAGES>
static int launch_pipe_e(dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq, int M,
                         int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                         int32_t *partial, int band = 0)
{
    // the staged epilogue reuses the ring for the output tile (BM rows of BN fp16 plus a pad) and,
    // with the fused rotate-quantize, for the tile's codes (64 bytes per row) after it
    const size_t ring = (size_t)NS * (BM + BN) * BG_ROWB;
    const size_t tile = (PE != PE_INT32 && VO) ? (size_t)BM * (BN * 2 + 16) + (RQN ? BM * 64 : 0) : 0;
    const size_t lds = ring > tile ? ring : tile;
    const void *fn = (const void *)k_gemm_pipe<BM, BN, WM, WN, NS, PE, VO, Q8, GS, RQN>;
    if (int rc = ensure_dynamic_lds(fn, lds, "gemm")) return rc;
    hipLaunchKernelGGL((k_gemm_pipe<BM, BN, WM, WN, NS, PE, VO, Q8, GS, RQN>), grid,
                       dim3(64 * WM * WN), lds, s, xq, wq, M, N, K, k_split, tm, tn,
                       band > 0 ? band : tile_band(tm, tn, BM, BN), epi, partial);
    return W4A4_OK;
}

// the 128-column tiles with the next linear's rotate-quantize in the staged epilogue. When only
// some column tiles carry it (the next linear's input is part of the output), the tiles go to the
// XCDs in row bands (every XCD gets all column tiles of its rows), so that extra epilogue work is
// spread evenly instead of landing on the XCDs that own those columns.
// Ring depths measured on the 1600-token stack shapes (K = 1024): three stages for the GELU and
// residual epilogues (up GEMM 18.8 -> 18.1 us against four; two stages no faster), two for the plain
// one (the QKV projection, pass about 0.7 % shorter than with three).
template <int BM, int WM, int WN>
static int launch_pipe_rq(dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq, int M,
                          int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi)
{
    const int band = (epi.rq.col0 > 0 || epi.rq.kn < N) ? tn : 0;
    if (epi.mode == W4A4_EPI_GELU)
        return launch_pipe_e<BM, 128, WM, WN, PE_GELU, true, false, false, true, 3>(
            grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
    if (epi.mode == W4A4_EPI_RESIDUAL)
        return launch_pipe_e<BM, 128, WM, WN, PE_RESIDUAL, true, false, false, true, 3>(
            grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
    return launch_pipe_e<BM, 128, WM, WN, PE_NONE, true, false, false, true, 2>(
        grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
}

template <int BM, int BN, int WM, int WN, bool Q8, bool GS = false, int NS = PIPE_STAGES>
static int launch_pipe_t(dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq, int M,
                         int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                         int32_t *partial)
{
    if (!GS && (partial || epi.mode == GEMM_OUT_I32))
        return launch_pipe_e<BM, BN, WM, WN, PE_INT32, false, Q8, false, false, NS>(grid, s, xq, wq, M, N, K, k_split,
                                                                 tm, tn, epi, partial);
    // staged epilogue: whole 16-byte chunks of Y / residual rows and 16-byte weight-scale loads
    const bool vo = (N % 8 == 0) && (epi.ldy % 8 == 0) && ((uintptr_t)epi.Y % 16 == 0) &&
                    ((uintptr_t)epi.w_scale % 16 == 0) &&
                    (epi.mode != W4A4_EPI_RESIDUAL ||
                     (epi.ldr % 8 == 0 && (uintptr_t)epi.residual % 16 == 0));
#define W4A4_PIPE_E(PEV)                                                                           \
    return vo ? launch_pipe_e<BM, BN, WM, WN, PEV, true, Q8, GS, false, NS>(grid, s, xq, wq, M, N, K, k_split, \
                                                                 tm, tn, epi, partial)             \
              : launch_pipe_e<BM, BN, WM, WN, PEV, false, Q8, GS, false, NS>(grid, s, xq, wq, M, N, K,        \
                                                                  k_split, tm, tn, epi, partial);
    if (epi.mode == W4A4_EPI_GELU) { W4A4_PIPE_E(PE_GELU) }
    if (epi.mode == W4A4_EPI_RESIDUAL) { W4A4_PIPE_E(PE_RESIDUAL) }
    W4A4_PIPE_E(PE_NONE)
#undef W4A4_PIPE_E
}

template <bool Q8>
static int launch_pipe(int kind, dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq,
                       int M, int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                       int32_t *partial)
{
    // 256x256 tiles on a two-stage ring (64 KB of operands): measured faster than three or four
    // stages on the prefill projection (34.3 -> 32.7 us) and the 8192^3 GEMM (401 -> 389 us)
    if (kind == 1)
        return launch_pipe_t<256, 256, 2, 4, Q8, false, 2>(grid, s, xq, wq, M, N, K, k_split, tm,
                                                           tn, epi, partial);
    // the GELU epilogue is VALU-heavy: with two waves per SIMD (8 waves on the same tile) one
    // wave's epilogue runs under the other's matrix work
    if (kind == 2 && !partial && epi.mode == W4A4_EPI_GELU)
        return launch_pipe_t<128, 256, 2, 4, Q8>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi,
                                                 partial);
    if (kind == 2)
        return launch_pipe_t<128, 256, 1, 4, Q8>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi,
                                                 partial);
    if (kind == 4)
        return launch_pipe_t<64, 128, 1, 4, Q8>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi,
                                                partial);
    if (kind == 5)
        return launch_pipe_t<80, 128, 1, 4, Q8>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi,
                                                partial);
    return launch_pipe_t<128, 128, 2, 2, Q8>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, partial);
}

// ---- software-pipelined GEMM launch (plan kinds SP_*)

// Whether a split-group tile kind has LDS room to gather a mapped residual tile next to its staged
// output and codes (k_gemm_sp's RMAP form).
template <int BM, int BN, int NS, int KS>
constexpr bool sp_rmap_fits()
{
    constexpr size_t xch = 2 * (BM / 32) * (BN / 64) * 4 * 64 * 16, stp = BN * 2 + 16;
    return BN <= 512 && 512 % BN == 0 &&
           xch + BM * stp + BM * 64 + BM * stp <= (size_t)NS * KS * (BM + BN) * BG_ROWB;
}
static bool sp_kind_maps_residual(int kind) { return kind == SP_64x128; }

template <int BM, int BN, int NS, int KS, int PE, bool VO, bool ST = false, bool RQN = false,
          bool RMAP = false>
static int launch_sp_e(dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq, int M,
                       int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                       int32_t *partial, int band = 0)
{
    // RMAP: the tile's map entries and gather order (2 x BN ints) past the ring
    const size_t lds = (size_t)NS * KS * (BM + BN) * BG_ROWB + (RMAP ? 2 * BN * sizeof(int) : 0);
    const void *fn = (const void *)k_gemm_sp<BM, BN, NS, KS, PE, VO, ST, RQN, RMAP>;
    if (int rc = ensure_dynamic_lds(fn, lds, "gemm")) return rc;
    hipLaunchKernelGGL((k_gemm_sp<BM, BN, NS, KS, PE, VO, ST, RQN, RMAP>), grid, dim3(512), lds, s, xq,
                       wq, M, N, K, k_split, tm, tn, band > 0 ? band : tile_band(tm, tn, BM, BN),
                       epi, partial);
    return W4A4_OK;
}

// The split-group GEMM with the next linear's rotate-quantize in the staged epilogue (no K split;
// the caller has checked the staged-store conditions). A launch whose rotated columns are only part
// of N orders its tiles by row band, as the pipelined form does.
template <int BM, int NS, int KS>
static int launch_sp_rq(dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq, int M,
                        int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi)
{
    const int band = (epi.rq.col0 > 0 || epi.rq.kn < N) ? tn : 0;
    if (epi.mode == W4A4_EPI_GELU)
        return launch_sp_e<BM, 128, NS, KS, PE_GELU, true, true, true>(
            grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
    if (epi.mode == W4A4_EPI_RESIDUAL && epi.res_cols) {
        if constexpr (sp_rmap_fits<BM, 128, NS, KS>())
            return launch_sp_e<BM, 128, NS, KS, PE_RESIDUAL, true, true, true, true>(
                grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
        return fail(W4A4_ERR_UNSUPPORTED, "mapped residual needs the staged split-group epilogue");
    }
    if (epi.mode == W4A4_EPI_RESIDUAL)
        return launch_sp_e<BM, 128, NS, KS, PE_RESIDUAL, true, true, true>(
            grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
    return launch_sp_e<BM, 128, NS, KS, PE_NONE, true, true, true>(
        grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, nullptr, band);
}

template <int BM, int BN, int NS, int KS>
static int launch_sp_t(dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq, int M,
                       int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                       int32_t *partial)
{
    if (partial || epi.mode == GEMM_OUT_I32)
        return launch_sp_e<BM, BN, NS, KS, PE_INT32, false>(grid, s, xq, wq, M, N, K, k_split, tm,
                                                            tn, epi, partial);
    // 4-column groups: 8-byte Y / residual accesses and 16-byte weight-scale loads
    const bool vo = (N % 4 == 0) && (epi.ldy % 4 == 0) && ((uintptr_t)epi.Y % 8 == 0) &&
                    ((uintptr_t)epi.w_scale % 16 == 0) &&
                    (epi.mode != W4A4_EPI_RESIDUAL ||
                     (epi.ldr % 4 == 0 && (uintptr_t)epi.residual % 8 == 0));
    // whole 16-byte row segments of Y: the output tile is staged in LDS
    const bool st = vo && (N % 8 == 0) && (epi.ldy % 8 == 0) && ((uintptr_t)epi.Y % 16 == 0);
#define W4A4_SP_E(PEV)                                                                             \
    if (st) return launch_sp_e<BM, BN, NS, KS, PEV, true, true>(grid, s, xq, wq, M, N, K, k_split, \
                                                                tm, tn, epi, partial);             \
    return vo ? launch_sp_e<BM, BN, NS, KS, PEV, true>(grid, s, xq, wq, M, N, K, k_split, tm, tn,   \
                                                       epi, partial)                               \
              : launch_sp_e<BM, BN, NS, KS, PEV, false>(grid, s, xq, wq, M, N, K, k_split, tm, tn,  \
                                                        epi, partial);
    if (epi.mode == W4A4_EPI_GELU) { W4A4_SP_E(PE_GELU) }
    if (epi.mode == W4A4_EPI_RESIDUAL && epi.res_cols) {
        // launch_gemm routes a residual column map here only for such kinds and staged stores
        if constexpr (sp_rmap_fits<BM, BN, NS, KS>()) {
            if (st)
                return launch_sp_e<BM, BN, NS, KS, PE_RESIDUAL, true, true, false, true>(
                    grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, partial);
        }
        return fail(W4A4_ERR_UNSUPPORTED, "mapped residual needs the staged split-group epilogue");
    }
    if (epi.mode == W4A4_EPI_RESIDUAL) { W4A4_SP_E(PE_RESIDUAL) }
    W4A4_SP_E(PE_NONE)
#undef W4A4_SP_E
}

// Launch one software-pipelined GEMM tile kind (also the tile sweep's entry point).
int launch_gemm_sp_kind(int kind, dim3 grid, hipStream_t s, const uint8_t *xq, const uint8_t *wq,
                        int M, int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                        int32_t *partial)
{
    switch (kind) {
    case SP_128x128:
        return launch_sp_t<128, 128, 4, 2>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, partial);
    case SP_64x128:  // two ring slots: measured faster than three (long-K 43.1 -> 42.2 us)
        return launch_sp_t<64, 128, 2, 4>(grid, s, xq, wq, M, N, K, k_split, tm, tn, epi, partial);
    default:
        return fail(W4A4_ERR_ARG, "unknown GEMM tile kind %d", kind);
    }
}

// Group-wise GEMM (per rotation block activation scales in epi.x_scale[K / 128]): the grouped
// small-M kernel for M <= 64, else the pipelined kernel with GS (one block per stage, no K split,
// the 128-row tiles whose registers hold the fp32 accumulators). The caller guarantees
// K % 128 == 0 and 16-byte aligned operands.
int launch_gemm_grouped(const uint8_t *xq, const uint8_t *wq, int M, int N, int K,
                        const GemmEpilogue &epi, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    if (M <= SMALL_M) {
        dim3 g((N + 15) / 16);
        const int mf = (M + 15) / 16;
        if (mf == 1) hipLaunchKernelGGL(k_gemm_smallm_g<1>, g, dim3(256), 0, s, xq, wq, M, N, K, epi);
        else if (mf == 2) hipLaunchKernelGGL(k_gemm_smallm_g<2>, g, dim3(256), 0, s, xq, wq, M, N, K, epi);
        else if (mf == 3) hipLaunchKernelGGL(k_gemm_smallm_g<3>, g, dim3(256), 0, s, xq, wq, M, N, K, epi);
        else hipLaunchKernelGGL(k_gemm_smallm_g<4>, g, dim3(256), 0, s, xq, wq, M, N, K, epi);
        return check_launch("gemm grouped small-M");
    }
    // 128 x 256 tiles unless 128 x 128 tiles take fewer rounds of 256 compute units at their
    // (lower) per-tile efficiency
    const int tm = (M + 127) / 128, tn2 = (N + 255) / 256, tn3 = (N + 127) / 128;
    const double t2 = std::ceil(tm * (double)tn2 / 256.0) * 2.0 / 0.85;
    const double t3 = std::ceil(tm * (double)tn3 / 256.0) * 1.0 / 0.6;
    int rc;
    if (t2 <= t3)
        rc = launch_pipe_t<128, 256, 1, 4, false, true>(dim3(tm * tn2, 1), s, xq, wq, M, N, K, K, tm,
                                                        tn2, epi, nullptr);
    else
        rc = launch_pipe_t<128, 128, 2, 2, false, true>(dim3(tm * tn3, 1), s, xq, wq, M, N, K, K, tm,
                                                        tn3, epi, nullptr);
    if (rc != W4A4_OK) return rc;
    return check_launch("gemm grouped");
}

// Shape of the wide small-M kernel, measured on MI355X: as many column fragments per workgroup as
// still give 256 workgroups (wider tiles read and widen the activation fewer times), 8 waves
// splitting K up to K = 8192 (short weight streams want more waves in flight), 4 beyond (each wave
// streams longer, and the larger tiles fit in its registers with a two-chunk prefetch).
struct SmallmShape { int nf, wv; };
static SmallmShape smallm_shape(int N, int K)
{
    const int nf = N >= 4 * 4096 ? 4 : (N >= 2 * 4096 ? 2 : 1);
    return SmallmShape{nf, K <= 8192 ? 8 : 4};
}

template <int MF>
static void launch_smallm_wide(SmallmShape sh, bool q8, hipStream_t s, const uint8_t *xq,
                               const uint8_t *wq, int M, int N, int K, const GemmEpilogue &epi)
{
    // (column fragments, waves, windows per chunk)
#define W4A4_WIDE(NFV, WVV, CHV)                                                                   \
    {                                                                                              \
        const dim3 g((N + 16 * NFV - 1) / (16 * NFV)), b(64 * WVV);                                \
        if (q8) hipLaunchKernelGGL((k_gemm_smallm_wide<MF, NFV, WVV, CHV, true>), g, b, 0, s, xq,   \
                                   wq, M, N, K, epi);                                              \
        else hipLaunchKernelGGL((k_gemm_smallm_wide<MF, NFV, WVV, CHV, false>), g, b, 0, s, xq, wq, \
                                M, N, K, epi);                                                     \
        return;                                                                                    \
    }
    if (sh.wv == 8) {
        if (sh.nf == 4) W4A4_WIDE(4, 8, 2)
        if (sh.nf == 2) W4A4_WIDE(2, 8, 1)
        W4A4_WIDE(1, 8, 4)
    }
    if (sh.nf == 4) W4A4_WIDE(4, 4, 2)
    if (sh.nf == 2) W4A4_WIDE(2, 4, 4)
    W4A4_WIDE(1, 4, 4)
#undef W4A4_WIDE
}

// q8: int8 operands [rows][K] (W8A8); the caller guarantees K % 64 == 0 and 16-byte aligned
// operands for them.
size_t gemm_mapped_residual_workspace(int M, int N, int K)
{
    return align_up(gemm_workspace(M, N, K, false), 256) + align_up((size_t)M * N * 2, 256);
}

int launch_gemm(const uint8_t *xq, const uint8_t *wq, int M, int N, int K, const GemmEpilogue &epi_in,
                void *ws, size_t ws_bytes, hipStream_t s, bool q8, bool *rq_done)
{
    if (rq_done) *rq_done = false;
    if (M == 0) return W4A4_OK;
    GemmEpilogue epi = epi_in;
    if (epi.mode != W4A4_EPI_RESIDUAL || !epi.res_cols) epi.res_cols = epi.res_order = nullptr;
    const int row_bytes = q8 ? K : K / 2;
    const bool vec = (row_bytes % 16 == 0) && ((uintptr_t)xq % 16 == 0) && ((uintptr_t)wq % 16 == 0);
    const bool pipe = q8 || (vec && K % BG_KS == 0);
    GemmPlan p = plan_gemm(M, N, K, q8 ? BG_ROWB : BG_KS, pipe, pipe && !q8,
                           epi.mode == W4A4_EPI_GELU);
    // the next linear's rotate-quantize in the epilogue: a 128-column pipelined or split-group tile
    // plan without a K split, the staged (16-byte) epilogue, 128-aligned columns; else the caller
    // runs it
    const bool vo_rows = (N % 8 == 0) && (epi.ldy % 8 == 0) && ((uintptr_t)epi.Y % 16 == 0) &&
                         ((uintptr_t)epi.w_scale % 16 == 0) &&
                         (epi.mode != W4A4_EPI_RESIDUAL ||
                          (epi.ldr % 8 == 0 && (uintptr_t)epi.residual % 16 == 0));
    const bool fuse = epi.rq.xq && !q8 && pipe && vo_rows && epi.mode != GEMM_OUT_I32 &&
                      epi.rq.col0 % 128 == 0 && epi.rq.kn % 128 == 0 &&
                      (uintptr_t)epi.rq.xq % 16 == 0;
    GemmPlan f{};
    const bool fused = fuse && [&] {
        f = plan_gemm(M, N, K, BG_KS, true, true, epi.mode == W4A4_EPI_GELU, true);
        return (f.kind == 3 || f.kind == 4 || f.kind == 5 || sp_kind_maps_residual(f.kind)) &&
               f.splits == 1;
    }();
    // A residual column map is read in the split-group kernel's staged epilogue; any other plan
    // gets the residual gathered into the workspace (after the split-K partials) first.
    if (epi.res_cols) {
        const bool in_kernel = fused ? sp_kind_maps_residual(f.kind)
                                     : (!q8 && sp_kind_maps_residual(p.kind) && p.splits == 1 &&
                                        vo_rows);
        if (!in_kernel) {
            const size_t off = align_up(gemm_workspace(M, N, K, q8), 256);
            if (!ws || ws_bytes < off + align_up((size_t)M * N * 2, 256))
                return fail(W4A4_ERR_WORKSPACE, "gemm with a residual map needs %zu workspace bytes",
                            off + align_up((size_t)M * N * 2, 256));
            uint16_t *gathered = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + off);
            const int rc = launch_permute_rows(epi.residual, M, N, epi.ldr, epi.res_cols, gathered,
                                               nullptr, s);
            if (rc != W4A4_OK) return rc;
            epi.residual = gathered;
            epi.ldr = N;
            epi.res_cols = epi.res_order = nullptr;
        }
    }
    if (fused) {
        const int tm = (M + f.bm - 1) / f.bm, tn = (N + f.bn - 1) / f.bn;
        const dim3 grid(tm * tn, 1);
        int rc;
        if (f.kind == SP_64x128)  // a two-slot ring (96 KB): measured faster here than three
            rc = launch_sp_rq<64, 2, 4>(grid, s, xq, wq, M, N, K, f.k_split, tm, tn, epi);
        else if (f.kind == 4)
            rc = launch_pipe_rq<64, 1, 4>(grid, s, xq, wq, M, N, K, f.k_split, tm, tn, epi);
        else if (f.kind == 5)
            rc = launch_pipe_rq<80, 1, 4>(grid, s, xq, wq, M, N, K, f.k_split, tm, tn, epi);
        else
            rc = launch_pipe_rq<128, 2, 2>(grid, s, xq, wq, M, N, K, f.k_split, tm, tn, epi);
        if (rc != W4A4_OK) return rc;
        if (rq_done) *rq_done = true;
        return check_launch("gemm + next rotate-quantize");
    }
    // the small-M kernels cover at most SMALL_M rows: a plan without a tile kernel beyond that
    // would leave rows unwritten, so it is refused loudly (no such plan exists for K <= 2^24)
    if (p.kind == 0 && M > SMALL_M)
        return fail(W4A4_ERR_UNSUPPORTED, "no GEMM tile plan for M = %d, N = %d, K = %d", M, N, K);
    if (p.kind == 0) {
        const int mf = (M + 15) / 16;
        // the wide kernel: whole 64-byte windows and at most 2^16 k per wave (4 waves)
        if (vec && row_bytes % 64 == 0 && (q8 || K <= 4 * MAX_K_SPLIT)) {
            const SmallmShape sh = smallm_shape(N, K);
            if (mf == 1) launch_smallm_wide<1>(sh, q8, s, xq, wq, M, N, K, epi);
            else if (mf == 2) launch_smallm_wide<2>(sh, q8, s, xq, wq, M, N, K, epi);
            else if (mf == 3) launch_smallm_wide<3>(sh, q8, s, xq, wq, M, N, K, epi);
            else launch_smallm_wide<4>(sh, q8, s, xq, wq, M, N, K, epi);
            return check_launch("gemm small-M");
        }
        dim3 g((N + 15) / 16);
#define W4A4_SMALLM_Q(MFV, QV)                                                                     \
    if (vec) hipLaunchKernelGGL((k_gemm_smallm<MFV, true, QV>), g, dim3(256), 0, s, xq, wq, M, N, K, \
                                epi);                                                              \
    else hipLaunchKernelGGL((k_gemm_smallm<MFV, false, QV>), g, dim3(256), 0, s, xq, wq, M, N, K, epi);
#define W4A4_SMALLM(MFV)                                                                           \
    if (q8) { W4A4_SMALLM_Q(MFV, true) } else { W4A4_SMALLM_Q(MFV, false) }
        if (mf == 1) { W4A4_SMALLM(1) }
        else if (mf == 2) { W4A4_SMALLM(2) }
        else if (mf == 3) { W4A4_SMALLM(3) }
        else { W4A4_SMALLM(4) }
#undef W4A4_SMALLM
#undef W4A4_SMALLM_Q
        return check_launch("gemm small-M");
    }
    int32_t *partial = nullptr;
    if (p.splits > 1) {
        const size_t need = gemm_workspace(M, N, K, q8);
        if (!ws || ws_bytes < need)
            return fail(W4A4_ERR_WORKSPACE, "gemm needs %zu workspace bytes", need);
        partial = reinterpret_cast<int32_t *>(ws);
    }
    const int tm = (M + p.bm - 1) / p.bm, tn = (N + p.bn - 1) / p.bn;
    dim3 grid(tm * tn, p.splits);
    if (q8) {
        int rc = launch_pipe<true>(p.kind, grid, s, xq, wq, M, N, K, p.k_split, tm, tn, epi, partial);
        if (rc != W4A4_OK) return rc;
    } else if (p.kind >= SP_128x192) {
        int rc = launch_gemm_sp_kind(p.kind, grid, s, xq, wq, M, N, K, p.k_split, tm, tn, epi,
                                     partial);
        if (rc != W4A4_OK) return rc;
    } else if (pipe) {
        int rc = launch_pipe<false>(p.kind, grid, s, xq, wq, M, N, K, p.k_split, tm, tn, epi, partial);
        if (rc != W4A4_OK) return rc;
    } else if (p.kind == 1)
        launch_big<256, 256, 2, 4>(vec, grid, s, xq, wq, M, N, K, p.k_split, tm, tn, epi, partial);
    else if (p.kind == 2)
        launch_big<128, 256, 1, 4>(vec, grid, s, xq, wq, M, N, K, p.k_split, tm, tn, epi, partial);
    else
        launch_big<128, 128, 2, 2>(vec, grid, s, xq, wq, M, N, K, p.k_split, tm, tn, epi, partial);
    int rc = check_launch("gemm");
    if (rc != W4A4_OK || p.splits <= 1) return rc;
    const int64_t total = (int64_t)M * N;
    const bool out_vec = (epi.mode == GEMM_OUT_I32)
                             ? ((uintptr_t)epi.acc_out % 16 == 0)
                             : ((epi.ldy % 4 == 0) && ((uintptr_t)epi.Y % 8 == 0) &&
                                ((uintptr_t)epi.w_scale % 16 == 0) &&
                                (epi.mode != W4A4_EPI_RESIDUAL ||
                                 (epi.ldr % 4 == 0 && (uintptr_t)epi.residual % 8 == 0)));
    if (N % 4 == 0 && (uintptr_t)partial % 16 == 0 && out_vec)
        hipLaunchKernelGGL(k_splitk_epilogue4, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256),
                           0, s, partial, p.splits, M, N, epi);
    else
        hipLaunchKernelGGL(k_splitk_epilogue, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                           s, partial, p.splits, M, N, epi);
    return check_launch("gemm split-k epilogue");
}

// ---- FP6 GEMM launch

// Tile shape and k split of the FP6 GEMM. The kernel is bound by the latency of its loads into
// LDS (the ring holds two or more stages in flight, and at the FP6 matrix rate a stage's MFMAs take
// less time than its loads), so the model counts stages: full rounds of 256 compute units (one
// workgroup per CU) times the stages of one split times the time of one stage, measured on MI355X
// for each tile (256 x 256: 1.4 us, 128 x 256: 0.95 us, 128 x 128: 0.55 us),
// plus a fixed launch / epilogue cost and the write and read of split-K partials.
static GemmPlan plan_gemm_f6(int M, int N, int K)
{
    struct Cand { int kind, bm, bn; double t_stage; };
    const Cand cands[] = {{1, 256, 256, 1.4e-6}, {2, 128, 256, 0.95e-6}, {3, 128, 128, 0.55e-6}};
    GemmPlan best{3, 128, 128, 1, K};
    double best_t = 1e30;
    for (const Cand &c : cands) {
        const double tiles = (double)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        for (int splits = 1; splits <= 16; splits *= 2) {
            const int k_split = ((K + splits - 1) / splits + F6_KS - 1) / F6_KS * F6_KS;
            if ((K + k_split - 1) / k_split != splits) continue;
            if (splits > 1 && k_split < 1024) continue;
            const double rounds = std::ceil(tiles * splits / 256.0);
            const double t_c = rounds * (k_split / F6_KS) * c.t_stage + 4e-6;
            const double t_r = splits > 1 ? (2.0 * splits * M * (double)N * 4 + M * (double)N * 2) / 5e12 + 2e-6 : 0.0;
            if (t_c + t_r < best_t * 0.98) {
                best_t = t_c + t_r;
                best = GemmPlan{c.kind, c.bm, c.bn, splits, k_split};
            }
        }
    }
    return best;
}

size_t gemm_f6_workspace(int M, int N, int K)
{
    const GemmPlan p = plan_gemm_f6(M, N, K);
    return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

template <int BM, int BN, int WM, int WN, int NS, int PE, bool VO>
static int launch_f6_e(dim3 grid, hipStream_t s, const uint8_t *xf, const uint8_t *wf, int M,
                       int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                       int32_t *partial)
{
    const size_t lds = (size_t)NS * (BM + BN) * 96;
    const void *fn = (const void *)k_gemm_f6<BM, BN, WM, WN, NS, PE, VO>;
    if (int rc = ensure_dynamic_lds(fn, lds, "fp6 gemm")) return rc;
    hipLaunchKernelGGL((k_gemm_f6<BM, BN, WM, WN, NS, PE, VO>), grid, dim3(64 * WM * WN), lds, s,
                       xf, wf, M, N, K, k_split, tm, tn, tile_band(tm, tn, BM, BN), epi, partial);
    return W4A4_OK;
}

template <int BM, int BN, int WM, int WN, int NS>
static int launch_f6_t(dim3 grid, hipStream_t s, const uint8_t *xf, const uint8_t *wf, int M,
                       int N, int K, int k_split, int tm, int tn, const GemmEpilogue &epi,
                       int32_t *partial)
{
    if (partial || epi.mode == GEMM_OUT_I32)
        return launch_f6_e<BM, BN, WM, WN, NS, PE_INT32, false>(grid, s, xf, wf, M, N, K, k_split,
                                                                 tm, tn, epi, partial);
    const bool vo = (epi.ldy % 4 == 0) && ((uintptr_t)epi.Y % 8 == 0) &&
                    ((uintptr_t)epi.w_scale % 16 == 0) &&
                    (epi.mode != W4A4_EPI_RESIDUAL ||
                     (epi.ldr % 4 == 0 && (uintptr_t)epi.residual % 8 == 0));
#define W4A4_F6_E(PEV)                                                                             \
    return vo ? launch_f6_e<BM, BN, WM, WN, NS, PEV, true>(grid, s, xf, wf, M, N, K, k_split, tm,   \
                                                           tn, epi, partial)                       \
              : launch_f6_e<BM, BN, WM, WN, NS, PEV, false>(grid, s, xf, wf, M, N, K, k_split, tm,  \
                                                            tn, epi, partial);
    if (epi.mode == W4A4_EPI_GELU) { W4A4_F6_E(PE_GELU) }
    if (epi.mode == W4A4_EPI_RESIDUAL) { W4A4_F6_E(PE_RESIDUAL) }
    W4A4_F6_E(PE_NONE)
#undef W4A4_F6_E
}

// FP6 operands (see the layout above); the caller guarantees K % 128 == 0, K <= F6_MAX_K and
// 16-byte aligned operands.
int launch_gemm_f6(const uint8_t *xf, const uint8_t *wf, int M, int N, int K,
                   const GemmEpilogue &epi, void *ws, size_t ws_bytes, hipStream_t s)
{
    if (M == 0) return W4A4_OK;
    const GemmPlan p = plan_gemm_f6(M, N, K);
    int32_t *partial = nullptr;
    if (p.splits > 1) {
        const size_t need = gemm_f6_workspace(M, N, K);
        if (!ws || ws_bytes < need)
            return fail(W4A4_ERR_WORKSPACE, "fp6 gemm needs %zu workspace bytes", need);
        partial = reinterpret_cast<int32_t *>(ws);
    }
    const int tm = (M + p.bm - 1) / p.bm, tn = (N + p.bn - 1) / p.bn;
    const dim3 grid(tm * tn, p.splits);
    int rc;
    if (p.kind == 1)  // two stages: measured faster than three (prefill 30.4 -> 28.7 us)
        rc = launch_f6_t<256, 256, 2, 4, 2>(grid, s, xf, wf, M, N, K, p.k_split, tm, tn, epi, partial);
    else if (p.kind == 2)
        rc = launch_f6_t<128, 256, 1, 4, 4>(grid, s, xf, wf, M, N, K, p.k_split, tm, tn, epi, partial);
    else
        rc = launch_f6_t<128, 128, 2, 2, 4>(grid, s, xf, wf, M, N, K, p.k_split, tm, tn, epi, partial);
    if (rc != W4A4_OK) return rc;
    rc = check_launch("fp6 gemm");
    if (rc != W4A4_OK || p.splits <= 1) return rc;
    const int64_t total = (int64_t)M * N;
    const bool out_vec = (epi.mode == GEMM_OUT_I32)
                             ? ((uintptr_t)epi.acc_out % 16 == 0)
                             : ((epi.ldy % 4 == 0) && ((uintptr_t)epi.Y % 8 == 0) &&
                                ((uintptr_t)epi.w_scale % 16 == 0) &&
                                (epi.mode != W4A4_EPI_RESIDUAL ||
                                 (epi.ldr % 4 == 0 && (uintptr_t)epi.residual % 8 == 0)));
    if (N % 4 == 0 && (uintptr_t)partial % 16 == 0 && out_vec)
        hipLaunchKernelGGL(k_splitk_epilogue4, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256),
                           0, s, partial, p.splits, M, N, epi);
    else
        hipLaunchKernelGGL(k_splitk_epilogue, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                           s, partial, p.splits, M, N, epi);
    return check_launch("fp6 gemm split-k epilogue");
}

}  // namespace w4a4
